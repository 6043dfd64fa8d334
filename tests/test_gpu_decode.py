"""Parity of the split-KV decoding path with the fp64 oracle (GPU).

Every call goes through the C ABI (``attn_fwd_decode`` via ctypes, with a
workspace sized by ``attn_decode_workspace_size``). Inputs come from the
seeded generator; expected values only from the oracle's decoding entry.
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


def run_decode(q, k, v, scale, workspace=None):
    import torch
    from software_pipelined_amd import attn
    out, lse = attn.attn_decode(to_device(q), to_device(k), to_device(v),
                                scale=float(np.float32(scale)), workspace=workspace)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


SHAPES = [
    # (B, H, Nq, Nkv, d)
    (1, 2, 1, 1, 64),        # one key
    (1, 1, 1, 33, 128),      # two key blocks, fewer than the chunks: empty chunks
    (2, 3, 1, 1000, 128),    # ragged last block
    (1, 2, 5, 257, 64),      # several query rows
    (1, 1, 33, 100, 128),    # two query tiles, the second ragged
    (2, 2, 1, 64, 256),
    (1, 1, 3, 4095, 256),
    (3, 1, 32, 2049, 64),
    (16, 16, 1, 200, 128),   # chunks of 2, 2 and 3 blocks (d = 128: three-slot rings), ragged tail
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b%d_h%d_nq%d_nkv%d_d%d" % s)
def test_decode_matches_oracle(oracle_mod, shape):
    B, H, Nq, Nkv, d = shape
    _say(f"case decode {shape}")
    q, k, v = I.gen_decode(B, H, Nq, Nkv, d, seed=500 + sum(shape))
    scale = I.default_scale(d)
    out, lse = run_decode(q, k, v, scale)
    ro, rl = oracle_mod.attn_decode(q, k, v, scale)
    _say(str(compare(out, lse, ro, rl, f"decode {shape}")))


def oracle_grouped(oracle_mod, q, k, v, scale):
    """The oracle's decoding with grouped K/V heads by their definition: each
    K/V head repeated for the H / Hkv query heads that read it."""
    G = q.shape[1] // k.shape[1]
    return oracle_mod.attn_decode(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), scale)


@pytest.mark.parametrize("cfg", I.DECODE_CONFIGS, ids=lambda c: c.name)
def test_decode_workloads_all_rows(oracle_mod, cfg):
    _say(f"case decode workload {cfg.name}")
    q, k, v = I.gen_decode_config(cfg)
    out, lse = run_decode(q, k, v, cfg.scale)
    ro, rl = oracle_grouped(oracle_mod, q, k, v, cfg.scale)
    _say(str(compare(out, lse, ro, rl, cfg.name)))


GROUPED = [
    # (B, H, Hkv, Nq, Nkv, d)
    (1, 4, 2, 1, 300, 128),    # two query heads per K/V head
    (2, 8, 1, 2, 1000, 64),    # all heads on one K/V head, two query rows each
    (1, 16, 4, 9, 257, 128),   # 36 query rows per K/V head: two query tiles
    (1, 8, 2, 1, 4095, 256),
]


@pytest.mark.parametrize("shape", GROUPED, ids=lambda s: "b%d_h%d_kv%d_nq%d_nkv%d_d%d" % s)
def test_decode_grouped_kv_heads(oracle_mod, shape):
    """Grouped K/V heads through the torch wrapper (one call over Hkv heads of
    G * Nq query rows), against the oracle with each K/V head repeated."""
    B, H, Hkv, Nq, Nkv, d = shape
    _say(f"case decode grouped {shape}")
    q, k, v = I.gen_decode(B, H, Nq, Nkv, d, seed=700 + sum(shape), Hkv=Hkv)
    scale = I.default_scale(d)
    out, lse = run_decode(q, k, v, scale)
    ro, rl = oracle_grouped(oracle_mod, q, k, v, scale)
    _say(str(compare(out, lse, ro, rl, f"decode grouped {shape}")))


@pytest.mark.parametrize("shape", [(1, 1, 1, 100000, 64), (1, 8, 2, 131072, 128)],
                         ids=lambda s: "b%d_h%d_nq%d_nkv%d_d%d" % s)
def test_decode_long_caches(oracle_mod, shape):
    """Long caches: one head of d = 64 takes the largest chunk count the merge
    handles (2048 chunks); 8 heads of d = 128 against 131072 keys."""
    B, H, Nq, Nkv, d = shape
    _say(f"case decode long cache {shape}")
    q, k, v = I.gen_decode(B, H, Nq, Nkv, d, seed=31 + d)
    out, lse = run_decode(q, k, v, I.default_scale(d))
    ro, rl = oracle_mod.attn_decode(q, k, v, I.default_scale(d))
    _say(str(compare(out, lse, ro, rl, f"decode {shape}")))


def test_decode_negative_scale_and_stress_keys(oracle_mod):
    # a negative scale, and every 7th key scaled by 8 (near-one-hot rows)
    B, H, Nq, Nkv, d = 2, 2, 2, 700, 64
    _say(f"case decode negative scale / stressed keys")
    q, k, v = I.gen_decode(B, H, Nq, Nkv, d, seed=77)
    kf = I.bf16_bits_to_f32(k)
    kf[:, :, ::7, :] *= np.float32(8.0)
    k = I.f32_to_bf16_bits(kf)
    for scale in (np.float32(-0.125), np.float32(0.125), np.float32(0.0)):
        out, lse = run_decode(q, k, v, scale)
        ro, rl = oracle_mod.attn_decode(q, k, v, scale)
        _say(str(compare(out, lse, ro, rl, f"decode scale {scale}")))


def test_decode_reuses_one_workspace(oracle_mod):
    # two calls in a row on one workspace buffer, the second smaller; stale
    # partials from the first call must not leak into the second
    import torch
    from software_pipelined_amd import attn
    st, need = attn.attn_decode_workspace_size(4, 8, 1, 4096, 128)
    assert st == attn.ATTN_OK
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    for shape in ((4, 8, 1, 4096, 128), (1, 3, 2, 500, 128)):
        B, H, Nq, Nkv, d = shape
        _say(f"case decode workspace reuse {shape}")
        q, k, v = I.gen_decode(B, H, Nq, Nkv, d, seed=900 + B)
        out, lse = run_decode(q, k, v, I.default_scale(d), workspace=ws)
        ro, rl = oracle_mod.attn_decode(q, k, v, I.default_scale(d))
        _say(str(compare(out, lse, ro, rl, f"decode reuse {shape}")))


def test_decode_is_deterministic():
    q, k, v = I.gen_decode(2, 4, 1, 3000, 128, seed=5)
    a = run_decode(q, k, v, I.default_scale(128))
    b = run_decode(q, k, v, I.default_scale(128))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
