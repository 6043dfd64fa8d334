"""Pins for the fp64 attention-backward oracle (CPU only).

The backward is the derivative of the forward definition (the attention
backward the Twill write-up schedules in its section 3.2; the pages do not
restate it). Nothing here compares the oracle's backward with itself or with
its own formulas retyped: each check fixes it against something independent
-- 50-digit central finite differences of the forward definition, torch's
autograd of a plain fp64 attention, or exact identities of the gradient.
``test_planted_bwd_mistakes_are_caught`` compiles mutated copies of the
oracle and requires each to fail at least one of these pins.
"""

import os
import shutil
import tempfile

import numpy as np
import pytest

from software_pipelined_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits, gen_dout, gen_qkv


def _f64(x):
    return bf16_bits_to_f32(x).astype(np.float64)


def _bwd(orc, q, k, v, do, causal, scale, lib=None):
    return orc.attn_bwd(q, k, v, do, causal, scale, lib=lib)


# ---------------------------------------------------------------- independent references

def _mp_loss(qf, kf, vf, dof, causal, scale, mp):
    """sum_ic dO_ic O_ic for the forward definition, in mpmath."""
    B, H, N, d = len(qf), len(qf[0]), len(qf[0][0]), len(qf[0][0][0])
    total = mp.mpf(0)
    for b in range(B):
        for h in range(H):
            for i in range(N):
                js = range(i + 1) if causal else range(N)
                s = [scale * mp.fsum(qf[b][h][i][c] * kf[b][h][j][c] for c in range(d)) for j in js]
                m = max(s)
                w = [mp.exp(x - m) for x in s]
                l = mp.fsum(w)
                for c in range(d):
                    o = mp.fsum(w[t] * vf[b][h][j][c] for t, j in enumerate(js)) / l
                    total += dof[b][h][i][c] * o
    return total


def check_bwd_finite_differences(orc, lib=None):
    """Central differences at 50 digits (step 1e-20) of the forward definition."""
    import mpmath
    mp = mpmath.mp
    shapes = [((1, 1, 3, 2), False, 0.7), ((1, 2, 4, 3), True, 0.5), ((2, 1, 2, 2), False, -1.25),
              ((1, 1, 5, 2), True, 1.0)]
    with mpmath.workdps(50):
        hstep = mp.mpf("1e-20")
        for n, (shape, causal, sc) in enumerate(shapes):
            B, H, N, d = shape
            q, k, v = gen_qkv(B, H, N, d, seed=60 + n)
            do = gen_dout(B, H, N, d, seed=60 + n)
            scale = float(np.float32(sc))
            dq, dk, dv = _bwd(orc, q, k, v, do, causal, scale, lib)
            base = [[[[[mp.mpf(float(x)) for x in row] for row in hh] for hh in bb] for bb in _f64(a)]
                    for a in (q, k, v, do)]
            sc_mp = mp.mpf(scale)
            for which, grad in ((0, dq), (1, dk), (2, dv)):
                for idx in np.ndindex(B, H, N, d):
                    b, h, i, c = idx
                    plus = [[[[x for x in row] for row in hh] for hh in bb] for bb in base[which]]
                    minus = [[[[x for x in row] for row in hh] for hh in bb] for bb in base[which]]
                    plus[b][h][i][c] += hstep
                    minus[b][h][i][c] -= hstep
                    args_p = list(base[:3])
                    args_m = list(base[:3])
                    args_p[which] = plus
                    args_m[which] = minus
                    fd = (_mp_loss(*args_p, base[3], causal, sc_mp, mp) -
                          _mp_loss(*args_m, base[3], causal, sc_mp, mp)) / (2 * hstep)
                    got = grad[idx]
                    assert abs(got - float(fd)) <= 1e-12 + 1e-11 * abs(float(fd)), \
                        f"shape {shape} causal {causal} grad {which} at {idx}: {got} vs {float(fd)}"


def _torch_grads(q, k, v, do, causal, scale):
    import torch
    Q, K, V, dO = (torch.tensor(_f64(x), dtype=torch.float64) for x in (q, k, v, do))
    for t in (Q, K, V):
        t.requires_grad_(True)
    S = scale * torch.matmul(Q, K.transpose(-1, -2).contiguous())
    if causal:
        N = Q.shape[2]
        S = S.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), diagonal=1), float("-inf"))
    O = torch.matmul(torch.softmax(S, dim=-1), V)
    (O * dO).sum().backward()
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


def check_bwd_torch_autograd(orc, lib=None):
    """torch.autograd of a plain fp64 attention (library differentiation)."""
    for n, (shape, causal, sc) in enumerate([((1, 2, 48, 16), False, 0.25), ((1, 2, 48, 16), True, 0.25),
                                             ((2, 1, 100, 8), True, -0.4), ((1, 1, 33, 64), False, 0.125)]):
        B, H, N, d = shape
        q, k, v = gen_qkv(B, H, N, d, seed=80 + n)
        do = gen_dout(B, H, N, d, seed=80 + n)
        scale = float(np.float32(sc))
        got = _bwd(orc, q, k, v, do, causal, scale, lib)
        ref = _torch_grads(q, k, v, do, causal, scale)
        for name, g, r in zip(("dq", "dk", "dv"), got, ref):
            np.testing.assert_allclose(g, r, rtol=1e-10, atol=1e-12 * max(1.0, np.abs(r).max()),
                                       err_msg=f"{name} {shape} causal={causal}")


def check_bwd_identities(orc, lib=None):
    """Exact identities of the gradient.

    Rows of P sum to one and rows of dS sum to zero, so per head
    sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i; dO = 0 gives zero gradients;
    a V constant over keys makes every dS zero, so dQ = dK = 0; with the
    causal mask query 0 sees only key 0, so dQ_0 = 0.
    """
    B, H, N, d = 2, 2, 37, 8
    q, k, v = gen_qkv(B, H, N, d, seed=91)
    do = gen_dout(B, H, N, d, seed=91)
    for causal in (False, True):
        dq, dk, dv = _bwd(orc, q, k, v, do, causal, 0.375, lib)
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12 * np.abs(dk).sum())
        np.testing.assert_allclose(dv.sum(axis=2), _f64(do).sum(axis=2), rtol=1e-12, atol=1e-12)
        if causal:
            np.testing.assert_allclose(dq[:, :, 0, :], 0.0, atol=1e-13)
        zero = np.zeros_like(do)
        for g in _bwd(orc, q, k, v, zero, causal, 0.375, lib):
            assert np.all(g == 0.0)
        vc = np.ascontiguousarray(np.broadcast_to(v[:, :, :1, :], v.shape))
        dq, dk, dv = _bwd(orc, q, k, vc, do, causal, 0.375, lib)
        np.testing.assert_allclose(dq, 0.0, atol=1e-12)
        np.testing.assert_allclose(dk, 0.0, atol=1e-12)
        np.testing.assert_allclose(dv.sum(axis=2), _f64(do).sum(axis=2), rtol=1e-12, atol=1e-12)


def check_bwd_row_subset(orc, lib=None):
    """Selected query/key rows equal the same rows of a full run."""
    B, H, N, d = 2, 3, 29, 8
    q, k, v = gen_qkv(B, H, N, d, seed=93)
    do = gen_dout(B, H, N, d, seed=93)
    for causal in (False, True):
        full = [x.reshape(B * H * N, d) for x in _bwd(orc, q, k, v, do, causal, 0.3, lib)]
        qrows = np.array([0, 5, N - 1, N, 2 * N + 7, B * H * N - 1])
        krows = np.array([3, N + 1, 3 * N + 28, 4 * N])
        dq, dk, dv = orc.attn_bwd_rows(q, k, v, do, causal, 0.3, qrows, krows, lib=lib)
        assert np.array_equal(dq, full[0][qrows])
        assert np.array_equal(dk, full[1][krows]) and np.array_equal(dv, full[2][krows])


ALL_BWD_CHECKS = [check_bwd_finite_differences, check_bwd_torch_autograd, check_bwd_identities,
                  check_bwd_row_subset]


@pytest.mark.parametrize("check", ALL_BWD_CHECKS, ids=lambda f: f.__name__)
def test_bwd_oracle_pin(oracle_mod, check):
    check(oracle_mod)


def test_bwd_bad_arguments(oracle_mod):
    q, k, v = gen_qkv(1, 1, 4, 8, seed=1)
    do = gen_dout(1, 1, 4, 8, seed=1)
    with pytest.raises(ValueError):
        oracle_mod.attn_bwd_rows(q, k, v, do, False, 1.0, qrows=np.array([4]))
    with pytest.raises(ValueError):
        oracle_mod.attn_bwd_rows(q, k, v, do, False, 1.0, krows=np.array([-1]))
    with pytest.raises(ValueError):
        oracle_mod.attn_bwd_rows(q, k, v, do[:, :, :3], False, 1.0)


# Plausible slips in the backward's arithmetic; each must fail some pin.
BWD_MUTATIONS = {
    "dq_drops_D": ("double ds = w[j] * (dp - D);", "double ds = w[j] * dp;"),
    "dkdv_drops_D": ("double ds = p * (dp - D[i]);", "double ds = p * dp;"),
    "dk_uses_k": ("dk_row[c] += sigma * ds * widen_bf16(q[i * d + c]);",
                  "dk_row[c] += sigma * ds * widen_bf16(k[i * d + c]);"),
    "dq_without_scale": ("dq_row[c] += sigma * ds * widen_bf16(k[j * d + c]);",
                         "dq_row[c] += ds * widen_bf16(k[j * d + c]);"),
    "dv_uses_ds": ("dv_row[c] += p * widen_bf16(dout[i * d + c]);",
                   "dv_row[c] += ds * widen_bf16(dout[i * d + c]);"),
    "causal_keys_see_every_query": ("for (int64_t i = causal ? j : 0; i < N; ++i) {",
                                    "for (int64_t i = 0; i < N; ++i) {"),
    "lse_sign": ("double p = exp(sigma * dot - lse[i]);", "double p = exp(sigma * dot + lse[i]);"),
    "D_uses_v": ("acc += widen_bf16(dout[i * d + c]) * o_row[c];",
                 "acc += widen_bf16(dout[i * d + c]) * widen_bf16(v[i * d + c]);"),
}


def test_planted_bwd_mistakes_are_caught(oracle_mod):
    src = open(oracle_mod.SOURCE_PATH).read()
    tmp = tempfile.mkdtemp()
    checks = ALL_BWD_CHECKS
    try:
        for name, (old, new) in BWD_MUTATIONS.items():
            assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
            path = os.path.join(tmp, f"{name}.c")
            open(path, "w").write(src.replace(old, new))
            lib = oracle_mod.bind(oracle_mod.compile_source(path, os.path.join(tmp, f"lib{name}.so")))
            caught = []
            for chk in checks:
                try:
                    chk(oracle_mod, lib=lib)
                except (AssertionError, ArithmeticError, ValueError):
                    caught.append(chk.__name__)
            assert caught, f"planted mistake '{name}' passed every pin"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
