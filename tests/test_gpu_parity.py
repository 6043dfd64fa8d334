"""Parity of the HIP attention-forward path with the fp64 oracle (GPU).

Every call goes through the C ABI (libattn.so via ctypes). Inputs come from
the seeded generator; expected values come only from the oracle, computed on
the host in the same process.
"""

import math
import sys

import numpy as np
import pytest

from software_pipelined_amd import inputs as I

from gpu_helpers import LSE_MAX_ABS, O_MAX_ABS, O_MEAN_ABS, compare, ensure_built, run_gpu

pytestmark = pytest.mark.gpu



def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    ensure_built()


def _oracle_full(oracle_mod, q, k, v, causal, scale):
    return oracle_mod.attn_fwd(q, k, v, causal, scale)


@pytest.mark.parametrize("causal", [False, True])
def test_small_workload_all_rows(oracle_mod, causal):
    cfg = I.SMALL
    _say(f"case small {cfg.name} causal={causal}")
    q, k, v = I.gen_config(cfg)
    out, lse = run_gpu(q, k, v, causal, cfg.scale)
    ro, rl = _oracle_full(oracle_mod, q, k, v, causal, cfg.scale)
    _say(str(compare(out, lse, ro, rl, cfg.name)))


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_multi_tile_all_rows(oracle_mod, d, causal):
    # N spans several query tiles and KV blocks with a ragged tail; B*H > 1.
    B, H, N = 2, 3, 777
    _say(f"case ragged B{B} H{H} N{N} d{d} causal={causal}")
    q, k, v = I.gen_qkv(B, H, N, d, seed=40 + d)
    scale = I.default_scale(d)
    out, lse = run_gpu(q, k, v, causal, scale)
    ro, rl = _oracle_full(oracle_mod, q, k, v, causal, scale)
    _say(str(compare(out, lse, ro, rl, f"ragged d{d}")))


@pytest.mark.parametrize("N", [1, 2, 3, 17, 31, 32, 33, 63, 64, 65, 127, 129, 255, 257])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_tiny_and_odd_lengths(oracle_mod, N, d):
    for causal in (False, True):
        _say(f"case tiny N{N} d{d} causal={causal}")
        q, k, v = I.gen_qkv(1, 2, N, d, seed=N * 7 + d)
        out, lse = run_gpu(q, k, v, causal, I.default_scale(d))
        ro, rl = _oracle_full(oracle_mod, q, k, v, causal, I.default_scale(d))
        compare(out, lse, ro, rl, f"N{N} d{d} causal={causal}")


@pytest.mark.parametrize("cfg", I.CONFIGS, ids=lambda c: c.name)
def test_full_size_workloads_every_row(oracle_mod, cfg):
    """Each workload at its full size, in the launch configuration the
    benchmark times, against the oracle on every row: O max abs error over
    all B*H*N*d elements, O mean abs error over all of them, LSE max abs
    error over all B*H*N rows, no NaN or Inf. The oracle runs in chunks of
    heads (its memory stays bounded and every chunk prints a line)."""
    _say(f"case full-size {cfg.name}: GPU run")
    q, k, v = I.gen_config(cfg)
    out, lse = run_gpu(q, k, v, cfg.causal, cfg.scale)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    B, H, N, d = cfg.B, cfg.H, cfg.N, cfg.d
    o2 = out.reshape(B * H, N, d)
    l2 = lse.reshape(B * H, N)
    # heads per oracle call: about 2^22 output elements
    hpc = max(1, (1 << 22) // (N * d))
    o_max = o_sum = l_max = 0.0
    for h0 in range(0, B * H, hpc):
        h1 = min(B * H, h0 + hpc)
        rows = np.arange(h0 * N, h1 * N, dtype=np.int64)
        ro, rl = oracle_mod.attn_fwd_rows(q, k, v, cfg.causal, cfg.scale, rows)
        e = np.abs(o2[h0:h1].reshape(-1, d).astype(np.float64) - ro)
        o_max = max(o_max, float(e.max()))
        o_sum += float(e.sum())
        l_max = max(l_max, float(np.abs(l2[h0:h1].reshape(-1).astype(np.float64) - rl).max()))
        if h1 == B * H or (h0 // hpc) % 8 == 0:
            _say(f"{cfg.name}: heads {h0}..{h1 - 1} of {B * H}: O max {o_max:.3e}, LSE max {l_max:.3e}")
    o_mean = o_sum / (B * H * N * d)
    _say(f"{cfg.name} every row: O max {o_max:.3e} mean {o_mean:.3e} LSE max {l_max:.3e}")
    assert o_max <= O_MAX_ABS, f"{cfg.name}: O max abs {o_max:.3e}"
    assert o_mean <= O_MEAN_ABS, f"{cfg.name}: O mean abs {o_mean:.3e}"
    assert l_max <= LSE_MAX_ABS, f"{cfg.name}: LSE max abs {l_max:.3e}"
    if cfg.causal:
        # causal row 0 sees only key 0: O_0 = V_0 bit for bit (its weight is
        # 1 exactly in bf16, and O is normalised with that weight)
        v0 = I.bf16_bits_to_f32(v)[:, :, 0]
        _say(f"{cfg.name} causal row 0: {int((out[:, :, 0] != v0).any(axis=-1).sum())} of {B * H} heads "
             f"differ from V_0")
        np.testing.assert_array_equal(out[:, :, 0], v0)


@pytest.mark.parametrize("d", [64, 128])
def test_long_sequence_sampled_rows(oracle_mod, d):
    """A sequence 8x the longest workload (N = 131072, one head): the block
    loop runs 1024-2048 blocks and row and element offsets pass 2^24; checked
    on sampled rows, both masks."""
    N = 1 << 17
    q, k, v = I.gen_qkv(1, 1, N, d, seed=2024 + d)
    for causal in (False, True):
        _say(f"case long N{N} d{d} causal={causal}")
        out, lse = run_gpu(q, k, v, causal, I.default_scale(d))
        assert np.isfinite(out).all() and np.isfinite(lse).all()
        rows = I.sample_rows(1, 1, N, per_head=48, seed=d)
        ro, rl = oracle_mod.attn_fwd_rows(q, k, v, causal, I.default_scale(d), rows)
        compare(out.reshape(-1, d)[rows], lse.reshape(-1)[rows], ro, rl, f"long N{N} d{d} causal={causal}")


def test_every_variant_matches_oracle(oracle_mod):
    from software_pipelined_amd import attn
    for vid in range(attn.attn_num_variants()):
        info = attn.attn_variant_info(vid)
        d = info["head_dim"]
        for causal in (False, True):
            _say(f"case variant {attn.attn_variant_name(vid)} causal={causal}")
            q, k, v = I.gen_qkv(1, 2, 300, d, seed=vid + 70)
            out, lse = run_gpu(q, k, v, causal, I.default_scale(d), variant=vid)
            ro, rl = _oracle_full(oracle_mod, q, k, v, causal, I.default_scale(d))
            compare(out, lse, ro, rl, attn.attn_variant_name(vid))


def test_stress_keys_max_tracking(oracle_mod):
    """Every 7th key scaled by 8 (near one-hot rows, frequent max jumps)."""
    for d in (64, 128):
        for causal in (False, True):
            q, k, v = I.gen_qkv(2, 2, 1000, d, seed=90, key_stress=True)
            out, lse = run_gpu(q, k, v, causal, I.default_scale(d))
            ro, rl = _oracle_full(oracle_mod, q, k, v, causal, I.default_scale(d))
            compare(out, lse, ro, rl, f"stress d{d} causal={causal}")


def test_negative_and_odd_scales(oracle_mod):
    q, k, v = I.gen_qkv(1, 2, 200, 128, seed=91)
    for scale in (-0.088, 0.3, -1.7, 1e-3, 0.0, -0.0):
        for causal in (False, True):
            out, lse = run_gpu(q, k, v, causal, scale)
            ro, rl = _oracle_full(oracle_mod, q, k, v, causal, scale)
            compare(out, lse, ro, rl, f"scale {scale}")


def test_invariants_on_gpu(oracle_mod):
    d, N = 128, 300
    q, k, v = I.gen_qkv(1, 2, N, d, seed=92)
    # constant V -> O equals that constant (within bf16 P rounding)
    c = I.f32_to_bf16_bits(np.linspace(-2, 2, d).astype(np.float32))
    vc = np.broadcast_to(c, v.shape).copy()
    for causal in (False, True):
        out, _ = run_gpu(q, k, vc, causal, I.default_scale(d))
        np.testing.assert_allclose(out, np.broadcast_to(I.bf16_bits_to_f32(c), out.shape),
                                   rtol=0, atol=2.0 * 2 ** -9)
    # K = 0 -> uniform weights: O = mean of visible V rows, LSE = ln |J_i|
    kz = np.zeros_like(k)
    vf = I.bf16_bits_to_f32(v).astype(np.float64)
    out, lse = run_gpu(q, kz, v, False, 0.1)
    np.testing.assert_allclose(out, np.broadcast_to(vf.mean(axis=2, keepdims=True), out.shape), atol=1e-5)
    np.testing.assert_allclose(lse, math.log(N), atol=1e-5)
    out, lse = run_gpu(q, kz, v, True, 0.1)
    cm = np.cumsum(vf, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    np.testing.assert_allclose(out, cm, atol=1e-5)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(np.arange(1, N + 1)), lse.shape), atol=1e-5)
    # causal row 0 -> O_0 = V_0 exactly, LSE_0 = scale * q_0 . k_0
    out, lse = run_gpu(q, k, v, True, I.default_scale(d))
    np.testing.assert_array_equal(out[:, :, 0], vf[:, :, 0].astype(np.float32))
    qf, kf = (I.bf16_bits_to_f32(x).astype(np.float64) for x in (q, k))
    np.testing.assert_allclose(lse[:, :, 0], float(I.default_scale(d)) * np.einsum("bhc,bhc->bh", qf[:, :, 0], kf[:, :, 0]),
                               atol=1e-4)


def test_deterministic_bitwise():
    q, k, v = I.gen_qkv(2, 4, 1500, 128, seed=93)
    for causal in (False, True):
        o1, l1 = run_gpu(q, k, v, causal, I.default_scale(128))
        o2, l2 = run_gpu(q, k, v, causal, I.default_scale(128))
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


def test_runs_on_caller_stream(oracle_mod):
    import torch
    from software_pipelined_amd import attn
    from gpu_helpers import to_device
    q, k, v = I.gen_qkv(1, 2, 500, 64, seed=94)
    s = torch.cuda.Stream()
    dq, dk, dv = to_device(q), to_device(k), to_device(v)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        out, lse = attn.attn_forward(dq, dk, dv, causal=True)
    s.synchronize()
    ro, rl = oracle_mod.attn_fwd(q, k, v, True, I.default_scale(64))
    compare(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, "side stream")


def test_device_pointer_errors():
    import torch
    from software_pipelined_amd import attn
    q = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros((1, 1, 64, 128), dtype=torch.float32, device="cuda")
    l = torch.zeros((1, 1, 64), dtype=torch.float32, device="cuda")
    p = q.data_ptr()
    assert attn.attn_fwd(p + 2, p, p, o.data_ptr(), l.data_ptr(), 1, 1, 64, 128, 0, 0.1, None) == attn.ATTN_ERR_MISALIGNED
    assert attn.attn_fwd(p, p, p, o.data_ptr(), l.data_ptr(), 1, 1, 64, 96, 0, 0.1, None) == attn.ATTN_ERR_HEAD_DIM
    assert attn.attn_fwd(p, p, p, o.data_ptr(), l.data_ptr(), 1, 1, 64, 128, 0, float("nan"), None) == attn.ATTN_ERR_BAD_SCALE
    assert attn.attn_fwd_variant(0, p, p, p, o.data_ptr(), l.data_ptr(), 1, 1, 64, 128, 0, 0.1, None) == attn.ATTN_ERR_BAD_SHAPE
    # outputs untouched on error
    assert float(o.abs().sum()) == 0.0


def test_overlapped_schedules_match_simple_schedule_bitwise():
    """Every schedule (deeper rings, pipelined, ping-pong) runs the same
    per-block arithmetic as the double-buffered simple kernel of the same
    tiling, only overlapped; any LDS-ring or wait hazard shows up as a bit
    difference."""
    from software_pipelined_amd import attn
    # reference per (head dim, keys per block): the double-buffered simple
    # schedule; the per-row arithmetic depends only on those two
    refs, pairs = {}, []
    for i in range(attn.attn_num_variants()):
        info = attn.attn_variant_info(i)
        name = attn.attn_variant_name(i)
        if "_st2_" in name and name.endswith("_simple"):
            refs.setdefault((info["head_dim"], info["block_n"]), i)
    for i in range(attn.attn_num_variants()):
        info = attn.attn_variant_info(i)
        ref = refs.get((info["head_dim"], info["block_n"]))
        if ref is not None and ref != i:
            pairs.append((i, ref))
    assert pairs
    for vid, ref in pairs:
        d = attn.attn_variant_info(vid)["head_dim"]
        for causal in (False, True):
            for N in (1, 100, 1000):
                _say(f"case differential {attn.attn_variant_name(vid)} vs {attn.attn_variant_name(ref)} "
                     f"N{N} causal={causal}")
                q, k, v = I.gen_qkv(2, 2, N, d, seed=N + d, key_stress=True)
                o1, l1 = run_gpu(q, k, v, causal, I.default_scale(d), variant=vid)
                o2, l2 = run_gpu(q, k, v, causal, I.default_scale(d), variant=ref)
                np.testing.assert_array_equal(o1, o2)
                np.testing.assert_array_equal(l1, l2)
