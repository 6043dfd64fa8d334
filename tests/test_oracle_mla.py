"""Pins for the fp64 MLA-decoding oracle (CPU only).

The oracle evaluates the absorbed MLA decoding operator: every query head
attends to one shared cache of latent rows, keys being whole rows and values
their first Dv entries. It is pinned against the split-KV decoding oracle
(itself pinned by brute force and closed forms) for the case where every head
has that one cache as its K and V, against a 50-digit brute force, and by
exact invariants; mutated copies of its source must each fail a pin.
"""

import math
import os
import shutil
import tempfile

import numpy as np
import pytest

from software_pipelined_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits, gen_mla


def _f64(x):
    return bf16_bits_to_f32(x).astype(np.float64)


def check_equals_decoding_with_shared_kv(orc, lib=None):
    """Dv = Dk: MLA is decoding with the cache as every head's K and V; Dv < Dk:
    the first Dv columns of that result (values are a prefix of the rows)."""
    for (B, H, N, Dk, Dv, sc) in [(2, 3, 17, 8, 8, 0.3), (1, 4, 40, 12, 5, -0.7), (2, 2, 1, 6, 6, 1.0)]:
        q, kv = gen_mla(B, H, N, Dk, seed=N + Dk)
        kh = np.ascontiguousarray(np.broadcast_to(kv[:, None], (B, H, N, Dk)))
        ref_o, ref_l = orc.attn_decode(q[:, :, None, :], kh, kh, sc)
        out, lse = orc.mla_decode(q, kv, Dv, sc, lib=lib)
        np.testing.assert_allclose(out, ref_o[:, :, 0, :Dv], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse, ref_l[:, :, 0], rtol=1e-13, atol=1e-14)


def check_mpmath(orc, lib=None):
    import mpmath
    with mpmath.workdps(50):
        for (B, H, N, Dk, Dv) in [(1, 2, 5, 4, 3), (2, 1, 3, 3, 3)]:
            q, kv = gen_mla(B, H, N, Dk, seed=7 + N)
            sc = float(np.float32(0.41))
            out, lse = orc.mla_decode(q, kv, Dv, sc, lib=lib)
            qf, kf = _f64(q), _f64(kv)
            for b in range(B):
                for h in range(H):
                    s = [mpmath.mpf(sc) * mpmath.fsum(mpmath.mpf(float(qf[b, h, c])) * float(kf[b, j, c])
                                                      for c in range(Dk)) for j in range(N)]
                    m = max(s)
                    w = [mpmath.exp(x - m) for x in s]
                    l = mpmath.fsum(w)
                    for c in range(Dv):
                        o = mpmath.fsum(w[j] * float(kf[b, j, c]) for j in range(N)) / l
                        assert abs(float(o) - out[b, h, c]) <= 1e-13 * max(1.0, abs(float(o)))
                    assert abs(float(m + mpmath.log(l)) - lse[b, h]) <= 1e-13 * max(1.0, abs(float(m)))


def check_invariants(orc, lib=None):
    """q = 0: uniform weights, out = mean of the value prefix, lse = ln N;
    rows of the same sequence share one cache, other sequences do not matter."""
    B, H, N, Dk, Dv = 2, 3, 9, 6, 4
    q, kv = gen_mla(B, H, N, Dk, seed=3)
    out, lse = orc.mla_decode(np.zeros_like(q), kv, Dv, 0.5, lib=lib)
    np.testing.assert_allclose(out, np.broadcast_to(_f64(kv)[:, None, :, :Dv].mean(axis=2), out.shape),
                               rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, math.log(N), rtol=1e-14)
    out0, _ = orc.mla_decode(q, kv, Dv, 0.5, lib=lib)
    kv2 = kv.copy()
    kv2[1] = f32_to_bf16_bits(np.full((N, Dk), 0.25, dtype=np.float32))
    out2, _ = orc.mla_decode(q, kv2, Dv, 0.5, lib=lib)
    assert np.array_equal(out0[0], out2[0]) and not np.allclose(out0[1], out2[1])
    rows = np.array([0, 4, B * H - 1])
    o_r, l_r = orc.mla_decode_rows(q, kv, Dv, 0.5, rows, lib=lib)
    assert np.array_equal(o_r, out0.reshape(-1, Dv)[rows])


ALL_MLA_CHECKS = [check_equals_decoding_with_shared_kv, check_mpmath, check_invariants]


@pytest.mark.parametrize("check", ALL_MLA_CHECKS, ids=lambda f: f.__name__)
def test_mla_oracle_pin(oracle_mod, check):
    check(oracle_mod)


MLA_MUTATIONS = {
    "value_from_wrong_offset": ("o[c] += p * widen_bf16(kvb[j * Dk + c]);", "o[c] += p * widen_bf16(kvb[j * Dk + c + (Dk - Dv)]);"),
    "per_head_cache": ("const uint16_t* kvb = kv + (r / H) * N * Dk;", "const uint16_t* kvb = kv + (r % B) * N * Dk;"),
    "key_truncated_to_value": ("for (int64_t c = 0; c < Dk; ++c) dot +=", "for (int64_t c = 0; c < Dv; ++c) dot +="),
    "scale_dropped": ("w[j] = sg * dot;", "w[j] = dot;"),
    "lse_without_max": ("lse[t] = m + log(l);", "lse[t] = log(l);"),
}


def test_planted_mla_mistakes_are_caught(oracle_mod):
    src = open(oracle_mod.SOURCE_PATH).read()
    tmp = tempfile.mkdtemp()
    try:
        for name, (old, new) in MLA_MUTATIONS.items():
            assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
            path = os.path.join(tmp, f"{name}.c")
            open(path, "w").write(src.replace(old, new))
            lib = oracle_mod.bind(oracle_mod.compile_source(path, os.path.join(tmp, f"lib{name}.so")))
            caught = []
            for chk in ALL_MLA_CHECKS:
                try:
                    chk(oracle_mod, lib=lib)
                except (AssertionError, ArithmeticError, ValueError):
                    caught.append(chk.__name__)
            assert caught, f"planted mistake '{name}' passed every pin"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
