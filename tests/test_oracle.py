"""Pins for the fp64 attention oracle (CPU only).

The oracle computes plain attention (PipeThreader OSDI'25 summary page,
"FlashAttention-3" paragraph: acc_s = Q K^T, softmax -> P, O = P V). Nothing
here compares it with itself: each test checks it against something fixed
independently -- hand-derived closed forms, a 50-digit mpmath brute force,
a numpy/scipy library special case, or an exact mathematical invariant.
``test_planted_mistakes_are_caught`` compiles mutated copies of the oracle
(dropped scale, wrong sign, off-by-one mask, transposed operand, ...) and
requires each to fail at least one of these pins.
"""

import json
import math
import os
import shutil
import tempfile

import numpy as np
import pytest
import scipy.special

from software_pipelined_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits, gen_decode, gen_qkv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")


def _bits(x):
    a = np.asarray(x, dtype=np.float32)
    b = f32_to_bf16_bits(a)
    assert np.array_equal(bf16_bits_to_f32(b), a), "fixture values must be exact in bf16"
    return b


def _run(orc, q, k, v, causal, scale, lib=None):
    return orc.attn_fwd(q, k, v, causal, scale, lib=lib)


# ---------------------------------------------------------------- pins as checks
# Each check raises AssertionError on failure; tests call them on the real
# oracle, the mutation test calls them on planted-mistake builds.

def check_closed_forms(orc, lib=None):
    cases = json.load(open(GOLDEN))["cases"]
    env = {"e": math.e, "exp": math.exp, "log": math.log, "__builtins__": {}}
    for c in cases:
        N, d = c["N"], c["d"]
        q = _bits(c["q"]).reshape(1, 1, N, d)
        k = _bits(c["k"]).reshape(1, 1, N, d)
        v = _bits(c["v"]).reshape(1, 1, N, d)
        for mode, causal in (("full", False), ("causal", True)):
            out, lse = _run(orc, q, k, v, causal, c["scale"], lib)
            exp_o = np.array([[eval(f, env) for f in row] for row in c[mode]["O"]])
            exp_l = np.array([eval(f, env) for f in c[mode]["LSE"]])
            np.testing.assert_allclose(out[0, 0], exp_o, rtol=1e-14, atol=1e-14,
                                       err_msg=f"{c['name']} {mode} O")
            np.testing.assert_allclose(lse[0, 0], exp_l, rtol=1e-14, atol=1e-14,
                                       err_msg=f"{c['name']} {mode} LSE")


def _mp_attention(qf, kf, vf, causal, scale):
    """50-digit brute force, written independently of the oracle: LSE first as
    log(sum exp(s)), then O as sum exp(s - LSE) v (no max subtraction)."""
    import mpmath as mp
    mp.mp.dps = 50
    B, H, N, d = qf.shape
    out = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    sig = mp.mpf(float(np.float32(scale)))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                keys = range(i + 1) if causal else range(N)
                s = [sig * mp.fsum(mp.mpf(float(qf[b, h, i, c])) * mp.mpf(float(kf[b, h, j, c]))
                                   for c in range(d)) for j in keys]
                L = mp.log(mp.fsum(mp.exp(x) for x in s))
                lse[b, h, i] = float(L)
                for c in range(d):
                    out[b, h, i, c] = float(mp.fsum(mp.exp(x - L) * mp.mpf(float(vf[b, h, j, c]))
                                                    for x, j in zip(s, keys)))
    return out, lse


def check_mpmath(orc, lib=None, shapes=None):
    shapes = shapes or [(1, 1, 1, 1), (1, 2, 2, 2), (2, 1, 3, 4), (1, 1, 5, 8), (1, 1, 8, 4),
                        (1, 1, 17, 8), (2, 2, 5, 2)]
    for n, (B, H, N, d) in enumerate(shapes):
        q, k, v = gen_qkv(B, H, N, d, seed=100 + n)
        qf, kf, vf = (bf16_bits_to_f32(x).astype(np.float64) for x in (q, k, v))
        for causal in (False, True):
            scale = np.float32(1.0 / math.sqrt(d)) if n % 2 == 0 else np.float32(0.731)
            out, lse = _run(orc, q, k, v, causal, scale, lib)
            ref_o, ref_l = _mp_attention(qf, kf, vf, causal, scale)
            np.testing.assert_allclose(out, ref_o, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lse, ref_l, rtol=1e-12, atol=1e-13)


def _scipy_attention(q, k, v, causal, scale):
    qf, kf, vf = (bf16_bits_to_f32(x).astype(np.float64) for x in (q, k, v))
    s = float(np.float32(scale)) * (qf @ np.swapaxes(kf, -1, -2))
    if causal:
        N = q.shape[2]
        s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
    p = scipy.special.softmax(s, axis=-1)
    return p @ vf, scipy.special.logsumexp(s, axis=-1)


def check_library(orc, lib=None):
    for (B, H, N, d, seed) in [(1, 2, 200, 64, 7), (2, 1, 129, 128, 8), (1, 1, 64, 256, 9)]:
        q, k, v = gen_qkv(B, H, N, d, seed)
        for causal in (False, True):
            out, lse = _run(orc, q, k, v, causal, 1.0 / math.sqrt(d), lib)
            ref_o, ref_l = _scipy_attention(q, k, v, causal, 1.0 / math.sqrt(d))
            np.testing.assert_allclose(out, ref_o, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(lse, ref_l, rtol=1e-12, atol=1e-12)


def check_constant_v(orc, lib=None):
    """V rows all equal c  =>  O_i = c exactly (weights sum to one)."""
    B, H, N, d = 1, 2, 37, 8
    q, k, _ = gen_qkv(B, H, N, d, seed=11)
    c = _bits(np.linspace(-3.5, 3.5, d).astype(np.float32))
    v = np.broadcast_to(c, (B, H, N, d)).copy()
    for causal in (False, True):
        out, _ = _run(orc, q, k, v, causal, 0.3, lib)
        np.testing.assert_allclose(out, np.broadcast_to(bf16_bits_to_f32(c), out.shape),
                                   rtol=1e-13, atol=1e-13)


def check_causal_row0(orc, lib=None):
    """Causal row 0 sees key 0 only: O_0 = V_0, LSE_0 = scale * q_0 . k_0."""
    B, H, N, d = 2, 2, 9, 16
    q, k, v = gen_qkv(B, H, N, d, seed=12)
    out, lse = _run(orc, q, k, v, True, 0.25, lib)
    qf, kf, vf = (bf16_bits_to_f32(x).astype(np.float64) for x in (q, k, v))
    np.testing.assert_array_equal(out[:, :, 0], vf[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.25 * np.einsum("bhc,bhc->bh", qf[:, :, 0], kf[:, :, 0]),
                               rtol=1e-14, atol=1e-14)


def check_zero_keys(orc, lib=None):
    """K = 0: uniform weights. O_i = mean of visible V rows; LSE_i = ln |J_i|."""
    B, H, N, d = 1, 1, 23, 4
    q, _, v = gen_qkv(B, H, N, d, seed=13)
    k = np.zeros_like(q)
    vf = bf16_bits_to_f32(v).astype(np.float64)
    out, lse = _run(orc, q, k, v, False, 0.5, lib)
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(vf[0, 0].mean(0), (N, d)), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.full(N, math.log(N)), rtol=1e-14)
    out, lse = _run(orc, q, k, v, True, 0.5, lib)
    cm = np.cumsum(vf[0, 0], axis=0) / np.arange(1, N + 1)[:, None]
    np.testing.assert_allclose(out[0, 0], cm, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.log(np.arange(1, N + 1)), rtol=1e-14, atol=1e-15)


def check_lse_bounds(orc, lib=None):
    """max_j s_ij <= LSE_i <= max_j s_ij + ln |J_i|."""
    B, H, N, d = 1, 2, 50, 32
    q, k, v = gen_qkv(B, H, N, d, seed=14, key_stress=True)
    qf, kf = (bf16_bits_to_f32(x).astype(np.float64) for x in (q, k))
    for causal in (False, True):
        _, lse = _run(orc, q, k, v, causal, 0.2, lib)
        s = float(np.float32(0.2)) * qf @ np.swapaxes(kf, -1, -2)
        if causal:
            s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
        m = s.max(-1)
        cnt = np.arange(1, N + 1) if causal else np.full(N, N)
        assert np.all(lse >= m - 1e-12)
        assert np.all(lse <= m + np.log(cnt) + 1e-12)


def check_key_shift(orc, lib=None):
    """K_j -> K_j + c for every j: O unchanged, LSE_i shifts by scale * q_i . c."""
    B, H, N, d = 1, 1, 40, 8
    q, k, v = gen_qkv(B, H, N, d, seed=15)
    # small integers keep k + c exact in bf16
    kint = _bits(np.round(bf16_bits_to_f32(k) * 4))
    c = np.array([1, -2, 3, 0, -1, 2, -3, 1], dtype=np.float32)
    k2 = _bits(bf16_bits_to_f32(kint) + c)
    qf = bf16_bits_to_f32(q).astype(np.float64)
    for causal in (False, True):
        o1, l1 = _run(orc, q, kint, v, causal, 0.125, lib)
        o2, l2 = _run(orc, q, k2, v, causal, 0.125, lib)
        np.testing.assert_allclose(o2, o1, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(l2 - l1, 0.125 * (qf @ c.astype(np.float64)), rtol=1e-11, atol=1e-11)


def check_permutations(orc, lib=None):
    """Non-causal: permuting K and V rows together changes nothing; permuting
    (b, h) slices permutes the outputs."""
    B, H, N, d = 2, 3, 31, 8
    q, k, v = gen_qkv(B, H, N, d, seed=16)
    o1, l1 = _run(orc, q, k, v, False, 0.4, lib)
    perm = np.random.default_rng(0).permutation(N)
    o2, l2 = _run(orc, q, k[:, :, perm], v[:, :, perm], False, 0.4, lib)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=1e-13, atol=1e-13)
    hp = [2, 0, 1]
    o3, l3 = _run(orc, q[:, hp][::-1].copy(), k[:, hp][::-1].copy(), v[:, hp][::-1].copy(), True, 0.4, lib)
    o4, l4 = _run(orc, q, k, v, True, 0.4, lib)
    np.testing.assert_array_equal(o3, o4[:, hp][::-1])
    np.testing.assert_array_equal(l3, l4[:, hp][::-1])


def check_causal_is_truncation(orc, lib=None):
    """Causal row i equals full attention of query i over keys 0..i."""
    B, H, N, d = 1, 1, 12, 8
    q, k, v = gen_qkv(B, H, N, d, seed=17)
    oc, lc = _run(orc, q, k, v, True, 0.3, lib)
    for i in (0, 1, 5, N - 1):
        qi = np.repeat(q[:, :, i:i + 1], i + 1, axis=2)
        of, lf = _run(orc, qi, k[:, :, :i + 1].copy(), v[:, :, :i + 1].copy(), False, 0.3, lib)
        np.testing.assert_allclose(oc[0, 0, i], of[0, 0, 0], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lc[0, 0, i], lf[0, 0, 0], rtol=1e-14, atol=1e-14)


def check_linear_in_v(orc, lib=None):
    """O(V1 + V2) = O(V1) + O(V2) when V1 + V2 is exact in bf16."""
    B, H, N, d = 1, 1, 33, 8
    q, k, _ = gen_qkv(B, H, N, d, seed=18)
    rng = np.random.default_rng(1)
    v1 = rng.integers(-8, 8, size=(B, H, N, d)).astype(np.float32)
    v2 = rng.integers(-8, 8, size=(B, H, N, d)).astype(np.float32)
    for causal in (False, True):
        o1, _ = _run(orc, q, k, _bits(v1), causal, 0.2, lib)
        o2, _ = _run(orc, q, k, _bits(v2), causal, 0.2, lib)
        o3, _ = _run(orc, q, k, _bits(v1 + v2), causal, 0.2, lib)
        np.testing.assert_allclose(o3, o1 + o2, rtol=1e-12, atol=1e-12)


def check_dominant_key(orc, lib=None):
    """One key's logit exceeds all others by >= 50: O_i = V_{j*} within e^-50 * N * max|V|."""
    B, H, N, d = 1, 1, 16, 4
    _, _, v = gen_qkv(B, H, N, d, seed=19)
    q = _bits(np.ones((B, H, N, d), dtype=np.float32))
    kk = np.zeros((B, H, N, d), dtype=np.float32)
    kk[0, 0, 5] = 64.0  # logit 0.25 * 4 * 64 = 64 vs 0 for the rest
    out, lse = _run(orc, q, _bits(kk), v, False, 0.25, lib)
    vf = bf16_bits_to_f32(v).astype(np.float64)
    bound = math.exp(-50) * N * np.abs(vf).max()
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(vf[0, 0, 5], (N, d)), rtol=0, atol=bound)
    np.testing.assert_allclose(lse[0, 0], 64.0 + np.log1p((N - 1) * np.exp(-64.0)), rtol=1e-15)


def check_row_subset(orc, lib=None):
    """Selected rows equal the same rows of a full run (rows are independent)."""
    B, H, N, d = 2, 2, 45, 16
    q, k, v = gen_qkv(B, H, N, d, seed=20)
    for causal in (False, True):
        o, l = orc.attn_fwd(q, k, v, causal, 0.25, lib=lib)
        rows = np.array([0, 3, 44, 45, 90, 179])
        os_, ls = orc.attn_fwd_rows(q, k, v, causal, 0.25, rows, lib=lib)
        np.testing.assert_array_equal(os_, o.reshape(-1, d)[rows])
        np.testing.assert_array_equal(ls, l.reshape(-1)[rows])


# ---------------------------------------------------------------- decoding pins
# The decoding entry point: Nq query rows against Nkv keys, every key visible.

def _mp_decode(qf, kf, vf, scale):
    """50-digit brute force of the rectangular case, independent of the oracle."""
    import mpmath as mp
    mp.mp.dps = 50
    B, H, Nq, d = qf.shape
    Nkv = kf.shape[2]
    out = np.zeros((B, H, Nq, d))
    lse = np.zeros((B, H, Nq))
    sig = mp.mpf(float(np.float32(scale)))
    for b in range(B):
        for h in range(H):
            for i in range(Nq):
                s = [sig * mp.fsum(mp.mpf(float(qf[b, h, i, c])) * mp.mpf(float(kf[b, h, j, c]))
                                   for c in range(d)) for j in range(Nkv)]
                L = mp.log(mp.fsum(mp.exp(x) for x in s))
                lse[b, h, i] = float(L)
                for c in range(d):
                    out[b, h, i, c] = float(mp.fsum(mp.exp(x - L) * mp.mpf(float(vf[b, h, j, c]))
                                                    for j, x in enumerate(s)))
    return out, lse


def check_decode_mpmath(orc, lib=None):
    shapes = [(1, 1, 1, 1, 1), (1, 2, 1, 5, 4), (2, 1, 3, 2, 2), (1, 1, 2, 17, 8), (2, 2, 1, 7, 3),
              (1, 3, 4, 9, 2)]
    for n, (B, H, Nq, Nkv, d) in enumerate(shapes):
        q, k, v = gen_decode(B, H, Nq, Nkv, d, seed=300 + n)
        qf, kf, vf = (bf16_bits_to_f32(x).astype(np.float64) for x in (q, k, v))
        scale = np.float32(1.0 / math.sqrt(d)) if n % 2 == 0 else np.float32(0.613)
        out, lse = orc.attn_decode(q, k, v, scale, lib=lib)
        ref_o, ref_l = _mp_decode(qf, kf, vf, scale)
        np.testing.assert_allclose(out, ref_o, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, ref_l, rtol=1e-12, atol=1e-13)


def check_decode_uniform_and_constant(orc, lib=None):
    # K = 0: every weight equal, O = mean of V over the whole cache, LSE = ln Nkv
    B, H, Nq, Nkv, d = 2, 3, 2, 11, 4
    q, k, v = gen_decode(B, H, Nq, Nkv, d, seed=7)
    out, lse = orc.attn_decode(q, np.zeros_like(k), v, 0.5, lib=lib)
    vf = bf16_bits_to_f32(v).astype(np.float64)
    np.testing.assert_allclose(out, np.broadcast_to(vf.mean(axis=2, keepdims=True), out.shape),
                               rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, np.full(lse.shape, math.log(Nkv)), rtol=1e-14, atol=1e-14)
    # V constant per (b, h): O equals that constant whatever the weights
    cst = _bits(np.arange(B * H * d, dtype=np.float32).reshape(B, H, 1, d) * 0.25)
    vc = np.ascontiguousarray(np.broadcast_to(cst, (B, H, Nkv, d)))
    out, _ = orc.attn_decode(q, k, vc, 0.9, lib=lib)
    np.testing.assert_allclose(out, np.broadcast_to(bf16_bits_to_f32(cst).astype(np.float64), out.shape),
                               rtol=1e-13, atol=1e-13)


def check_decode_grouped_heads(orc, lib=None):
    # Grouped K/V heads (G query heads per K/V head, query head h reading K/V
    # head h // G) are, by definition, attention with each K/V head repeated G
    # times; since a group's query heads are adjacent in memory, the same
    # numbers come from the grouped-free call over Hkv heads of G * Nq rows
    # (the reshape the decoding entry point documents), bit for bit
    for (B, H, Hkv, Nq, Nkv, d) in [(2, 4, 2, 1, 9, 4), (1, 8, 1, 3, 5, 2), (1, 6, 3, 2, 17, 8)]:
        G = H // Hkv
        q, k, v = gen_decode(B, H, Nq, Nkv, d, seed=40 + H, Hkv=Hkv)
        assert k.shape == (B, Hkv, Nkv, d)
        ref_o, ref_l = orc.attn_decode(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), 0.37, lib=lib)
        o, l = orc.attn_decode(q.reshape(B, Hkv, G * Nq, d), k, v, 0.37, lib=lib)
        assert np.array_equal(o.reshape(B, H, Nq, d), ref_o) and np.array_equal(l.reshape(B, H, Nq), ref_l)


ALL_CHECKS = [check_closed_forms, check_mpmath, check_library, check_constant_v, check_causal_row0,
              check_zero_keys, check_lse_bounds, check_key_shift, check_permutations,
              check_causal_is_truncation, check_linear_in_v, check_dominant_key, check_row_subset,
              check_decode_mpmath, check_decode_uniform_and_constant, check_decode_grouped_heads]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(oracle_mod, check):
    check(oracle_mod)


def test_empty_and_bad_arguments(oracle_mod):
    q = np.zeros((1, 1, 0, 8), dtype=np.uint16)
    o, l = oracle_mod.attn_fwd(q, q, q, False, 1.0)
    assert o.shape == (1, 1, 0, 8) and l.shape == (1, 1, 0)
    q, k, v = gen_qkv(1, 1, 4, 8, seed=1)
    with pytest.raises(ValueError):
        oracle_mod.attn_fwd_rows(q, k, v, False, 1.0, rows=np.array([4]))
    with pytest.raises(ValueError):
        oracle_mod.attn_fwd_rows(q, k[:, :, :3], v, False, 1.0)


# Each mutation is a plausible slip in the oracle's arithmetic; every one must
# be caught by some pin above.
MUTATIONS = {
    "dropped_scale": ("double s = sigma * dot;", "double s = dot;"),
    "lse_without_max": ("*lse_out = m + log(l);", "*lse_out = log(l);"),
    "wrong_sign_in_exp": ("w[j] = exp(w[j] - m);", "w[j] = exp(m - w[j]);"),
    "causal_excludes_diagonal": ("int64_t nvis = causal ? i + 1 : N;", "int64_t nvis = causal ? (i > 0 ? i : 1) : N;"),
    "q_used_as_keys": ("const uint16_t* kj = k + j * d;", "const uint16_t* kj = q + j * d;"),
    "no_normalisation": ("w[j] = w[j] / l;", "w[j] = w[j];"),
    "transposed_v_index": ("out_row[c] += w[j] * widen_bf16(vj[c]);",
                           "out_row[c] += w[j] * widen_bf16(v[c * d + (j % d)]);"),
    "log2_lse": ("*lse_out = m + log(l);", "*lse_out = m + log2(l);"),
    "scale_squared": ("double sigma = (double)scale;", "double sigma = (double)scale * (double)scale;"),
    "decode_kv_head_stride": ("k + bh * Nkv * d, v + bh * Nkv * d", "k + bh * Nq * d, v + bh * Nq * d"),
    "decode_row_split": ("int64_t bh = r / Nq, i = r % Nq;", "int64_t bh = r % (B * H), i = r / (B * H);"),
    "decode_scale_dropped": ("const double sigma = scale;", "const double sigma = 1.0;"),
}


def test_planted_mistakes_are_caught(oracle_mod):
    src = open(oracle_mod.SOURCE_PATH).read()
    tmp = tempfile.mkdtemp()
    fast_checks = [c for c in ALL_CHECKS if c is not check_mpmath]  # the decoding brute force is small
    try:
        for name, (old, new) in MUTATIONS.items():
            assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
            path = os.path.join(tmp, f"{name}.c")
            open(path, "w").write(src.replace(old, new))
            lib = oracle_mod.bind(oracle_mod.compile_source(path, os.path.join(tmp, f"lib{name}.so")))
            caught = []
            for chk in fast_checks:
                try:
                    chk(oracle_mod, lib=lib)
                except (AssertionError, ArithmeticError, ValueError):
                    caught.append(chk.__name__)
            assert caught, f"planted mistake '{name}' passed every pin"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
