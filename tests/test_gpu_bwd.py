"""Parity of the attention backward (attn_bwd) with the fp64 oracle (GPU).

Every call goes through the C ABI: the forward (attn_fwd) makes out and lse
from the seeded q, k, v, then attn_bwd takes them with the seeded dO.
Expected values come only from the oracle's backward, which recomputes the
forward itself in fp64.

Acceptance bar, per gradient X in (dq, dk, dv), relative to the reference's
own scale (the gradients' magnitudes vary with N and d):
    max |X - X_ref|  <= 1e-2 * max |X_ref|  + 1e-5
    mean |X - X_ref| <= 5e-3 * mean |X_ref| + 1e-5
The products run on bf16 operands with fp32 accumulation; P and dS are
rounded to bf16 (relative error up to 2^-9 = 1.95e-3 per term, rms
2^-9/sqrt(3) = 1.1e-3) before the dV, dK and dQ contractions. A gradient
element is a sum of many such terms of mixed sign, so its relative error has
about the per-term rms, 1-2e-3 (the mean bar, 5e-3, leaves 2.5x over that);
the worst element over a few million is a few rms, 3-4e-3 measured, under
the max bar with 2.5x to spare. The absolute floor covers gradients that
vanish in exact arithmetic (one visible key: dP - D = 0), where the fp32
difference of two O(10) dot products leaves O(1e-6) residue.
"""

import sys

import numpy as np
import pytest

from software_pipelined_amd import inputs as I

from gpu_helpers import ensure_built, to_device

pytestmark = pytest.mark.gpu

GRAD_MAX_REL = 1e-2
GRAD_MEAN_REL = 5e-3
GRAD_ABS_FLOOR = 1e-5


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    ensure_built()


def run_bwd(q, k, v, do, causal, scale, workspace=None):
    """Forward then backward on the GPU; returns numpy (dq, dk, dv)."""
    import torch
    from software_pipelined_amd import attn
    tq, tk, tv, tdo = (to_device(x) for x in (q, k, v, do))
    sc = float(np.float32(scale))
    out, lse = attn.attn_forward(tq, tk, tv, causal=causal, scale=sc)
    dq, dk, dv = attn.attn_backward(tq, tk, tv, out, lse, tdo, causal=causal, scale=sc, workspace=workspace)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()


def compare_grads(got, ref, what):
    stats = {}
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert np.isfinite(g).all(), f"{what}: non-finite {name}"
        err = np.abs(g.astype(np.float64) - r)
        scale_max = float(np.abs(r).max()) if r.size else 0.0
        scale_mean = float(np.abs(r).mean()) if r.size else 0.0
        e_max = float(err.max()) if err.size else 0.0
        e_mean = float(err.mean()) if err.size else 0.0
        stats[name] = (e_max / max(scale_max, 1e-30), e_mean / max(scale_mean, 1e-30))
        assert e_max <= GRAD_MAX_REL * scale_max + GRAD_ABS_FLOOR, \
            f"{what}: {name} max abs err {e_max:.3e} vs scale {scale_max:.3e}"
        assert e_mean <= GRAD_MEAN_REL * scale_mean + GRAD_ABS_FLOOR, \
            f"{what}: {name} mean abs err {e_mean:.3e} vs mean {scale_mean:.3e}"
    _say(f"{what}: " + ", ".join(f"{n} max/mean rel {a:.2e}/{b:.2e}" for n, (a, b) in stats.items()))
    return stats


SHAPES = [
    # (B, H, N, d, causal)
    (1, 1, 1, 64, False),
    (1, 1, 1, 128, True),
    (1, 2, 32, 64, False),
    (1, 2, 32, 128, True),
    (1, 1, 100, 128, False),    # ragged: one 128-row tile, 4 query blocks, last ragged
    (2, 1, 257, 64, True),      # ragged key tiles and query blocks, causal
    (1, 2, 384, 128, False),    # three full tiles
    (1, 1, 500, 128, True),
    (2, 2, 300, 64, False),
    (1, 1, 1, 256, False),
    (1, 2, 100, 256, True),     # d = 256: one wave per SIMD, ragged blocks
    (2, 1, 300, 256, False),
    (1, 1, 1, 128, False),      # d = 128 without the mask (ping-pong dQ): one key block
    (1, 3, 65, 128, False),     # two key blocks, the second holding one key
    (2, 2, 1000, 128, False),   # 16 key blocks, ragged last block and query tile
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b%d_h%d_n%d_d%d_%s" % (*s[:4], "c" if s[4] else "f"))
def test_bwd_matches_oracle(oracle_mod, shape):
    B, H, N, d, causal = shape
    _say(f"case bwd {shape}")
    seed = 700 + B + H + N + d
    q, k, v = I.gen_qkv(B, H, N, d, seed=seed)
    do = I.gen_dout(B, H, N, d, seed=seed)
    scale = I.default_scale(d)
    got = run_bwd(q, k, v, do, causal, scale)
    ref = oracle_mod.attn_bwd(q, k, v, do, causal, scale)
    compare_grads(got, ref, f"bwd {shape}")


def test_bwd_negative_scale_and_stress_keys(oracle_mod):
    B, H, N, d = 1, 2, 200, 64
    _say("case bwd negative scale / stressed keys")
    q, k, v = I.gen_qkv(B, H, N, d, seed=71, key_stress=True)
    do = I.gen_dout(B, H, N, d, seed=71)
    for causal in (False, True):
        for scale in (np.float32(-0.125), np.float32(0.125), np.float32(0.0)):
            got = run_bwd(q, k, v, do, causal, scale)
            ref = oracle_mod.attn_bwd(q, k, v, do, causal, scale)
            compare_grads(got, ref, f"bwd scale {scale} causal {causal}")


def test_bwd_workload_causal_2k_sampled(oracle_mod):
    """The causal N=2048 d=128 workload at full size: dQ on sampled query rows
    of every head, dK and dV on sampled key rows of two heads."""
    cfg = I.CAUSAL_2K
    _say(f"case bwd workload {cfg.name}")
    q, k, v = I.gen_qkv(cfg.B, cfg.H, cfg.N, cfg.d, seed=cfg.seed)
    do = I.gen_dout(cfg.B, cfg.H, cfg.N, cfg.d, seed=cfg.seed)
    got = [x.reshape(-1, cfg.d) for x in run_bwd(q, k, v, do, cfg.causal, cfg.scale)]
    qrows = I.sample_rows(cfg.B, cfg.H, cfg.N, per_head=6, seed=31)
    heads = (0, cfg.B * cfg.H - 1)
    krows = np.concatenate([h * cfg.N + I.sample_rows(1, 1, cfg.N, per_head=24, seed=32 + h) for h in heads])
    dq, dk, dv = oracle_mod.attn_bwd_rows(q, k, v, do, cfg.causal, cfg.scale, qrows, krows)
    compare_grads((got[0][qrows], got[1][krows], got[2][krows]), (dq, dk, dv), cfg.name)


def _sampled_parity(oracle_mod, B, H, N, d, causal, seed, key_heads, what):
    q, k, v = I.gen_qkv(B, H, N, d, seed=seed)
    do = I.gen_dout(B, H, N, d, seed=seed)
    scale = I.default_scale(d)
    got = [x.reshape(-1, d) for x in run_bwd(q, k, v, do, causal, scale)]
    qrows = I.sample_rows(B, H, N, per_head=4, seed=seed + 1)
    krows = np.concatenate([h * N + I.sample_rows(1, 1, N, per_head=24, seed=seed + 2 + h) for h in key_heads])
    dq, dk, dv = oracle_mod.attn_bwd_rows(q, k, v, do, causal, scale, qrows, krows)
    compare_grads((got[0][qrows], got[1][krows], got[2][krows]), (dq, dk, dv), what)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_bwd_many_heads_wide_dkdv_workgroups(oracle_mod, causal):
    """B*H*ceil(N/256) >= 1024: the dK/dV kernel runs 8-wave workgroups."""
    _say(f"case bwd b4_h64_n1000_d128 causal={causal}")
    _sampled_parity(oracle_mod, 4, 64, 1000, 128, causal, 41, (0, 255), f"bwd b4_h64_n1000 causal={causal}")


def test_bwd_workload_16k_sampled(oracle_mod):
    """The N=16384 d=128 workload at full size, as the benchmark times it:
    dQ on sampled rows of every head, dK and dV on sampled key rows of every
    head."""
    cfg = I.HEADLINE
    _say(f"case bwd workload {cfg.name}")
    _sampled_parity(oracle_mod, cfg.B, cfg.H, cfg.N, cfg.d, cfg.causal, cfg.seed, tuple(range(cfg.B * cfg.H)),
                    cfg.name)


def test_bwd_workload_d64_causal_8k_sampled(oracle_mod):
    """The causal N=8192 d=64 workload with every 7th key scaled by 8, at full
    size as the benchmark times it: dQ and dK/dV on sampled rows of every
    head."""
    cfg = I.CAUSAL_8K_STRESS
    _say(f"case bwd workload {cfg.name}")
    q, k, v = I.gen_config(cfg)
    do = I.gen_dout(cfg.B, cfg.H, cfg.N, cfg.d, seed=cfg.seed)
    got = [x.reshape(-1, cfg.d) for x in run_bwd(q, k, v, do, cfg.causal, cfg.scale)]
    qrows = I.sample_rows(cfg.B, cfg.H, cfg.N, per_head=3, seed=51)
    heads = range(cfg.B * cfg.H)
    krows = np.concatenate([h * cfg.N + I.sample_rows(1, 1, cfg.N, per_head=6, seed=52 + h) for h in heads])
    dq, dk, dv = oracle_mod.attn_bwd_rows(q, k, v, do, cfg.causal, cfg.scale, qrows, krows)
    compare_grads((got[0][qrows], got[1][krows], got[2][krows]), (dq, dk, dv), cfg.name)


def test_bwd_workload_d256_causal_4k_sampled(oracle_mod):
    """The causal N=4096 d=256 workload at full size: dQ on sampled query rows
    of every head, dK and dV on sampled key rows of every head."""
    cfg = I.CAUSAL_4K_D256
    _say(f"case bwd workload {cfg.name}")
    _sampled_parity(oracle_mod, cfg.B, cfg.H, cfg.N, cfg.d, cfg.causal, cfg.seed, tuple(range(cfg.B * cfg.H)),
                    cfg.name)


def test_bwd_d256_negative_scale(oracle_mod):
    B, H, N, d = 1, 1, 160, 256
    _say("case bwd d256 negative scale / stressed keys")
    q, k, v = I.gen_qkv(B, H, N, d, seed=73, key_stress=True)
    do = I.gen_dout(B, H, N, d, seed=73)
    for causal in (False, True):
        got = run_bwd(q, k, v, do, causal, np.float32(-0.0625))
        ref = oracle_mod.attn_bwd(q, k, v, do, causal, np.float32(-0.0625))
        compare_grads(got, ref, f"bwd d256 scale -0.0625 causal {causal}")


def test_bwd_reuses_one_workspace(oracle_mod):
    import torch
    from software_pipelined_amd import attn
    st, need = attn.attn_bwd_workspace_size(2, 2, 300, 128)
    assert st == attn.ATTN_OK
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    for shape in ((2, 2, 300, 128, False), (1, 1, 70, 128, True)):
        B, H, N, d, causal = shape
        _say(f"case bwd workspace reuse {shape}")
        q, k, v = I.gen_qkv(B, H, N, d, seed=950 + N)
        do = I.gen_dout(B, H, N, d, seed=950 + N)
        got = run_bwd(q, k, v, do, causal, I.default_scale(d), workspace=ws)
        ref = oracle_mod.attn_bwd(q, k, v, do, causal, I.default_scale(d))
        compare_grads(got, ref, f"bwd reuse {shape}")


def test_bwd_is_deterministic():
    q, k, v = I.gen_qkv(1, 2, 700, 128, seed=5)
    do = I.gen_dout(1, 2, 700, 128, seed=5)
    a = run_bwd(q, k, v, do, True, I.default_scale(128))
    b = run_bwd(q, k, v, do, True, I.default_scale(128))
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
