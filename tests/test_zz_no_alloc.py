"""The no-allocation decoding entry (attn_fwd_decode_static) against the
workspace entry (attn_fwd_decode) it shares its kernels with, through the C
ABI, and against the oracle: two calls in a row on one GPU, the second with
a smaller shape (the fixed scratch keeps the first call's contents). The
size limit is checked on the CPU."""

import numpy as np
import pytest

from software_pipelined_amd import inputs as I

from gpu_helpers import LSE_MAX_ABS, O_MAX_ABS, O_MEAN_ABS, ensure_built, to_device


def _say(msg):
    print(msg, flush=True)


def _lib():
    ensure_built()
    from software_pipelined_amd import attn
    attn.load_library()
    return attn


def test_static_decode_rejects_shapes_beyond_its_scratch():
    attn = _lib()
    cap = attn.attn_decode_static_max_bytes()
    assert cap == 16 << 20
    P = 1 << 20  # never dereferenced: the size check comes before any HIP call
    # 64 query rows of 128 heads against 64k keys need far more than 16 MiB
    st, need = attn.attn_decode_workspace_size(4, 128, 64, 65536, 128)
    assert st == attn.ATTN_OK and need > cap
    assert attn.attn_fwd_decode_static(P, P, P, P, P, 4, 128, 64, 65536, 128, 0.1, None) == attn.ATTN_ERR_TOO_LARGE
    assert attn.attn_fwd_decode_static(0, P, P, P, P, 1, 32, 1, 4096, 128, 0.1, None) == attn.ATTN_ERR_NULL_PTR
    assert attn.attn_fwd_decode_static(P, P, P, P, P, 1, 32, 1, 4096, 96, 0.1, None) == attn.ATTN_ERR_HEAD_DIM
    assert attn.attn_fwd_decode_static(P, P, P, P, P, 1, 32, 1, 0, 128, 0.1, None) == attn.ATTN_ERR_BAD_SHAPE
    assert attn.attn_fwd_decode_static(P + 4, P, P, P, P, 1, 32, 1, 4096, 128, 0.1, None) == attn.ATTN_ERR_MISALIGNED
    assert attn.attn_fwd_decode_static(0, 0, 0, 0, 0, 0, 32, 1, 4096, 128, 0.1, None) == attn.ATTN_OK


@pytest.mark.gpu
def test_static_decode_matches_workspace_entry_twice(oracle_mod):
    import torch
    attn = _lib()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    stream = torch.cuda.current_stream()
    # the first shape fills 14.1 of the 16 MiB, the second is smaller; the
    # oracle checks every 7th query row of the first and every row of the second
    for (B, H, Nq, Nkv, d, seed, step) in ((32, 32, 7, 4096, 128, 12, 7), (2, 8, 3, 1000, 64, 13, 1)):
        _say(f"case decode static B{B} H{H} Nq{Nq} Nkv{Nkv} d{d}")
        q, k, v = I.gen_decode(B, H, Nq, Nkv, d, seed)
        tq, tk, tv = to_device(q), to_device(k), to_device(v)
        scale = float(I.default_scale(d))
        st, need = attn.attn_decode_workspace_size(B, H, Nq, Nkv, d)
        assert st == attn.ATTN_OK and need <= attn.attn_decode_static_max_bytes()
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        outs = []
        for static in (False, True):
            out = torch.full((B, H, Nq, d), float("nan"), dtype=torch.float32, device="cuda")
            lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device="cuda")
            args = (tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), out.data_ptr(), lse.data_ptr(),
                    B, H, Nq, Nkv, d, scale)
            if static:
                st = attn.attn_fwd_decode_static(*args, stream.cuda_stream)
            else:
                st = attn.attn_fwd_decode(*args, ws.data_ptr(), need, stream.cuda_stream)
            _say(f"  {'static' if static else 'workspace'} entry status {st}")
            assert st == attn.ATTN_OK
            torch.cuda.synchronize()
            outs.append((out.cpu().numpy(), lse.cpu().numpy()))
        # same kernels, same chunk plan: bit-identical to the workspace entry
        np.testing.assert_array_equal(outs[0][0], outs[1][0])
        np.testing.assert_array_equal(outs[0][1], outs[1][1])
        rows = np.arange(0, B * H * Nq, step)
        ro, rl = oracle_mod.attn_decode_rows(q, k, v, scale, rows=rows)
        o, l = outs[1]
        e = np.abs(o.reshape(-1, d)[rows].astype(np.float64) - ro)
        le = np.abs(l.reshape(-1)[rows].astype(np.float64) - rl)
        _say(f"  O max {e.max():.3e} mean {e.mean():.3e} LSE max {le.max():.3e}")
        assert np.isfinite(o).all() and np.isfinite(l).all()
        assert e.max() <= O_MAX_ABS and e.mean() <= O_MEAN_ABS and le.max() <= LSE_MAX_ABS
