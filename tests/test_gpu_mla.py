"""Parity of MLA decoding (mla_decode) with the fp64 oracle (GPU).

Every call goes through the C ABI; inputs come from the seeded generator and
expected values only from the oracle. Bar: the split-KV decoding bar of the
attention outputs (O max abs <= 1e-2, mean <= 1e-3, LSE max abs <= 1e-3).
"""

import sys

import numpy as np
import pytest

from software_pipelined_amd import inputs as I

from gpu_helpers import compare, ensure_built, to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    ensure_built()


def run_mla(q, kv, scale, workspace=None):
    import torch
    from software_pipelined_amd import attn
    out, lse = attn.mla_decode_torch(to_device(q), to_device(kv), float(np.float32(scale)), workspace=workspace)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


SHAPES = [
    # (B, H, N)
    (1, 64, 1),        # one cache row
    (1, 64, 33),       # one block, its second half holds one key
    (1, 64, 96),       # the second half of the last block holds no key
    (2, 128, 100),
    (1, 128, 1000),    # several blocks per chunk, ragged tail
    (3, 64, 2049),
    (2, 192, 500),     # three 64-head workgroups per (sequence, chunk)
    (1, 256, 700),     # four
    (300, 64, 128),    # one chunk per sequence (the whole cache), more workgroups than CUs
    # enough sequences for 64-head workgroups (fewer take 16-head ones), with ragged tails
    (64, 128, 1000),
    (128, 64, 2049),   # the last block's second half holds no key
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b%d_h%d_n%d" % s)
def test_mla_matches_oracle(oracle_mod, shape):
    B, H, N = shape
    _say(f"case mla {shape}")
    q, kv = I.gen_mla(B, H, N, 576, seed=400 + N)
    scale = np.float32(1.0 / np.sqrt(192.0))
    out, lse = run_mla(q, kv, scale)
    ro, rl = oracle_mod.mla_decode(q, kv, 512, scale)
    _say(str(compare(out, lse, ro, rl, f"mla {shape}")))


@pytest.mark.parametrize("cfg", I.MLA_CONFIGS, ids=lambda c: c.name)
def test_mla_workloads(oracle_mod, cfg):
    _say(f"case mla workload {cfg.name}")
    q, kv = I.gen_mla(cfg.B, cfg.H, cfg.N, cfg.Dk, cfg.seed)
    out, lse = run_mla(q, kv, cfg.scale)
    ro, rl = oracle_mod.mla_decode(q, kv, cfg.Dv, cfg.scale)
    _say(str(compare(out, lse, ro, rl, cfg.name)))


def test_mla_negative_scale_and_reuse(oracle_mod):
    import torch
    from software_pipelined_amd import attn
    st, need = attn.mla_decode_workspace_size(2, 128, 3000)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    for shape, scale in (((2, 128, 3000), np.float32(-0.09)), ((1, 64, 77), np.float32(0.2)),
                         ((1, 64, 300), np.float32(0.0))):
        B, H, N = shape
        _say(f"case mla reuse {shape} scale {scale}")
        q, kv = I.gen_mla(B, H, N, 576, seed=17 + N)
        out, lse = run_mla(q, kv, scale, workspace=ws)
        ro, rl = oracle_mod.mla_decode(q, kv, 512, scale)
        _say(str(compare(out, lse, ro, rl, f"mla {shape}")))


@pytest.mark.parametrize("shape", [(1, 64, 65536), (64, 128, 512)], ids=lambda s: "b%d_h%d_n%d" % s)
def test_mla_long_cache_and_many_rows(oracle_mod, shape):
    """A 65,536-row cache for one sequence (256 chunks: the workgroup-per-row
    merge) and 64 sequences of 128 heads over 512 rows (8,192 merged rows)."""
    B, H, N = shape
    _say(f"case mla {shape}")
    q, kv = I.gen_mla(B, H, N, 576, seed=900 + B)
    scale = np.float32(1.0 / np.sqrt(192.0))
    out, lse = run_mla(q, kv, scale)
    ro, rl = oracle_mod.mla_decode(q, kv, 512, scale)
    _say(str(compare(out, lse, ro, rl, f"mla {shape}")))


def test_mla_near_one_hot_rows(oracle_mod):
    """The 64 rotary values (key only, not part of the value) of every
    seventh cache row scaled by 16 (exact in bf16): those rows' scores grow
    about 5x, so most heads put nearly all their weight on a few rows, the
    case where rounding of P and of the partials matters most, while the
    values keep unit scale (the bar is absolute)."""
    B, H, N = 2, 128, 3000
    _say(f"case mla stressed rows {(B, H, N)}")
    q, kv = I.gen_mla(B, H, N, 576, seed=77)
    kvf = I.bf16_bits_to_f32(kv)
    kvf[:, ::7, 512:] *= np.float32(16.0)
    kv = I.f32_to_bf16_bits(kvf)
    scale = np.float32(1.0 / np.sqrt(192.0))
    out, lse = run_mla(q, kv, scale)
    ro, rl = oracle_mod.mla_decode(q, kv, 512, scale)
    _say(str(compare(out, lse, ro, rl, "mla stressed rows")))


def test_mla_is_deterministic():
    q, kv = I.gen_mla(2, 128, 1500, 576, seed=3)
    a = run_mla(q, kv, 0.07)
    b = run_mla(q, kv, 0.07)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
