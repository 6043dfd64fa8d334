"""Pins for the fp64 Mamba2 ChunkScan oracle (CPU only).

The oracle evaluates, per output step, the chunk-local sum the PipeThreader
summary page describes in its Mamba2 running example (cb scaled by the
exponential decay from dA and by dt, multiplied with x). Each check fixes it
against something independent of that sum: the state-space recurrence the
chunked form comes from (a state reset at each chunk start, advanced one step
at a time), numpy/scipy library products for special cases, and exact
invariants. ``test_planted_chunkscan_mistakes_are_caught`` compiles mutated
copies of the oracle and requires each to fail at least one pin.
"""

import os
import shutil
import tempfile

import numpy as np
import pytest
import scipy.linalg

from software_pipelined_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits, gen_chunk_scan


def _f64(x):
    return bf16_bits_to_f32(x).astype(np.float64)


def check_recurrence(orc, lib=None):
    """cb = C B^T from small integer factors (exact in bf16); the oracle must
    equal the step-by-step recurrence h_t = exp(dA_t) h_{t-1} + dt_t B_t x_t^T,
    y_t = C_t h_t, with h reset to zero at every chunk start and
    dA_t = dA_cumsum_t - dA_cumsum_{t-1} inside the chunk."""
    rng = np.random.default_rng(5)
    for (B, S, H, P, L, N) in [(1, 37, 2, 3, 16, 2), (2, 64, 1, 4, 32, 3), (1, 10, 3, 2, 4, 2)]:
        x, _, dt, dacs = gen_chunk_scan(B, S, H, P, L, seed=S)
        nc = (S + L - 1) // L
        C = rng.integers(-1, 2, size=(B, nc * L, N)).astype(np.float64)
        Bm = rng.integers(-1, 2, size=(B, nc * L, N)).astype(np.float64)
        C[:, S:] = 0.0
        Bm[:, S:] = 0.0
        cbf = np.einsum("bcmn,bckn->bcmk", C.reshape(B, nc, L, N), Bm.reshape(B, nc, L, N))
        cb = f32_to_bf16_bits(cbf.astype(np.float32))
        assert np.array_equal(_f64(cb), cbf)
        out = orc.chunk_scan(x, cb, dt, dacs, L, lib=lib)
        xf = _f64(x)
        ref = np.zeros((B, S, H, P))
        for b in range(B):
            for h in range(H):
                for c in range(nc):
                    state = np.zeros((N, P))
                    prev = 0.0
                    for m in range(L):
                        s = c * L + m
                        if s >= S:
                            break
                        cur = float(dacs[b, h, c, m])
                        state = np.exp(cur - prev) * state + float(dt[b, h, c, m]) * np.outer(Bm[b, s], xf[b, s, h])
                        prev = cur
                        ref[b, s, h] = C[b, s] @ state
        np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12 * max(1.0, np.abs(ref).max()))


def check_no_decay_is_masked_matmul(orc, lib=None):
    """dA_cumsum = 0 and dt = 1: each chunk's output is tril(cb) @ x."""
    B, S, H, P, L = 2, 50, 2, 5, 16
    x, cb, _, _ = gen_chunk_scan(B, S, H, P, L, seed=9)
    nc = (S + L - 1) // L
    ones = np.ones((B, H, nc, L), dtype=np.float32)
    out = orc.chunk_scan(x, cb, ones, np.zeros_like(ones), L, lib=lib)
    xf, cbf = _f64(x), _f64(cb)
    for b in range(B):
        for c in range(nc):
            s0, s1 = c * L, min(S, (c + 1) * L)
            n = s1 - s0
            A = np.tril(cbf[b, c, :n, :n])
            for h in range(H):
                np.testing.assert_allclose(out[b, s0:s1, h], A @ xf[b, s0:s1, h], rtol=1e-12, atol=1e-12)


def check_identity_cb(orc, lib=None):
    """cb = I: out_s = dt_s x_s (the decay of a step to itself is 1)."""
    B, S, H, P, L = 1, 40, 3, 4, 16
    x, _, dt, dacs = gen_chunk_scan(B, S, H, P, L, seed=10)
    nc = (S + L - 1) // L
    eye = f32_to_bf16_bits(np.broadcast_to(np.eye(L, dtype=np.float32), (B, nc, L, L)).copy())
    out = orc.chunk_scan(x, eye, dt, dacs, L, lib=lib)
    dts = dt.transpose(0, 2, 3, 1).reshape(B, nc * L, H)[:, :S].astype(np.float64)
    np.testing.assert_allclose(out, dts[..., None] * _f64(x), rtol=1e-14, atol=0)


def check_constant_step_toeplitz(orc, lib=None):
    """One chunk with dA_cumsum_m = a (m + 1): the decay matrix is the lower
    Toeplitz matrix of exp(a i), built with scipy."""
    B, S, H, P, L = 1, 32, 1, 6, 32
    x, cb, dt, _ = gen_chunk_scan(B, S, H, P, L, seed=11)
    a = -0.37
    dacs = (a * (np.arange(L) + 1.0)).astype(np.float32).reshape(1, 1, 1, L)
    out = orc.chunk_scan(x, cb, dt, dacs, L, lib=lib)
    # the oracle sees the float32 running sums; build the matrix from them exactly as rounded
    steps = np.float64(dacs[0, 0, 0])
    T = np.tril(np.exp(steps[:, None] - steps[None, :]))
    T_ref = np.tril(scipy.linalg.toeplitz(np.exp(a * np.arange(L))))
    np.testing.assert_allclose(T, T_ref, rtol=1e-5)  # the float32 rounding of a(m + 1)
    ref = (_f64(cb[0, 0]) * T * dt[0, 0, 0].astype(np.float64)[None, :]) @ _f64(x[0, :, 0])
    np.testing.assert_allclose(out[0, :, 0], ref, rtol=1e-12, atol=1e-13)


def check_chunks_are_independent(orc, lib=None):
    """Changing x or cb in chunk 1 leaves every other chunk's output unchanged
    bit for bit, and changes chunk 1's."""
    B, S, H, P, L = 1, 48, 2, 3, 16
    x, cb, dt, dacs = gen_chunk_scan(B, S, H, P, L, seed=12)
    base = orc.chunk_scan(x, cb, dt, dacs, L, lib=lib)
    x2 = x.copy()
    x2[:, 16:32] = f32_to_bf16_bits(np.full((1, 16, H, P), 0.5, dtype=np.float32))
    cb2 = cb.copy()
    cb2[:, 1] = f32_to_bf16_bits(np.full((1, L, L), -1.0, dtype=np.float32))
    for xx, cc in ((x2, cb), (x, cb2)):
        out = orc.chunk_scan(xx, cc, dt, dacs, L, lib=lib)
        assert np.array_equal(out[:, :16], base[:, :16]) and np.array_equal(out[:, 32:], base[:, 32:])
        assert not np.allclose(out[:, 16:32], base[:, 16:32])


def check_row_subset(orc, lib=None):
    B, S, H, P, L = 2, 70, 3, 4, 32
    x, cb, dt, dacs = gen_chunk_scan(B, S, H, P, L, seed=13)
    full = orc.chunk_scan(x, cb, dt, dacs, L, lib=lib).reshape(-1, P)
    rows = np.array([0, 5, 31 * H + 1, 32 * H, S * H - 1, S * H, B * S * H - 1])
    assert np.array_equal(orc.chunk_scan_rows(x, cb, dt, dacs, L, rows, lib=lib), full[rows])


ALL_CS_CHECKS = [check_recurrence, check_no_decay_is_masked_matmul, check_identity_cb,
                 check_constant_step_toeplitz, check_chunks_are_independent, check_row_subset]


@pytest.mark.parametrize("check", ALL_CS_CHECKS, ids=lambda f: f.__name__)
def test_chunkscan_oracle_pin(oracle_mod, check):
    check(oracle_mod)


def test_chunkscan_bad_arguments(oracle_mod):
    x, cb, dt, dacs = gen_chunk_scan(1, 20, 2, 4, 8, seed=1)
    with pytest.raises(ValueError):
        oracle_mod.chunk_scan_rows(x, cb, dt, dacs, 8, rows=np.array([40]))
    with pytest.raises(ValueError):
        oracle_mod.chunk_scan(x, cb[:, :2], dt, dacs, 8)


CS_MUTATIONS = {
    "future_steps_included": ("for (int64_t k = 0; k <= m; ++k) {", "for (int64_t k = 0; k < L && c * L + k < S; ++k) {"),
    "diagonal_excluded": ("for (int64_t k = 0; k <= m; ++k) {", "for (int64_t k = 0; k < m; ++k) {"),
    "decay_sign": ("exp((double)da_c[m] - (double)da_c[k])", "exp((double)da_c[k] - (double)da_c[m])"),
    "dt_dropped": ("* (double)dt_c[k];", ";"),
    "dt_of_output_step": ("* (double)dt_c[k];", "* (double)dt_c[m];"),
    "chunk_offset_dropped": ("x + ((b * S + c * L + k) * H + h) * P;", "x + ((b * S + k) * H + h) * P;"),
    "cb_transposed": ("double w = widen_bf16(cb_row[k])", "double w = widen_bf16(cb[((b * nc + c) * L + k) * L + m])"),
}


def test_planted_chunkscan_mistakes_are_caught(oracle_mod):
    src = open(oracle_mod.SOURCE_PATH).read()
    tmp = tempfile.mkdtemp()
    try:
        for name, (old, new) in CS_MUTATIONS.items():
            assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
            path = os.path.join(tmp, f"{name}.c")
            open(path, "w").write(src.replace(old, new))
            lib = oracle_mod.bind(oracle_mod.compile_source(path, os.path.join(tmp, f"lib{name}.so")))
            caught = []
            for chk in ALL_CS_CHECKS:
                try:
                    chk(oracle_mod, lib=lib)
                except (AssertionError, ArithmeticError, ValueError):
                    caught.append(chk.__name__)
            assert caught, f"planted mistake '{name}' passed every pin"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
