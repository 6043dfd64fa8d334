"""The decoding, backward, ChunkScan and MLA entry points enqueue on the
caller's stream (GPU). Each runs on a side stream while the default stream
is left alone; only the side stream is synchronised before the results are
read, and they must equal, bit for bit, the same call made on the default
stream."""

import numpy as np
import pytest

from software_pipelined_amd import inputs as I

from gpu_helpers import ensure_built, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    ensure_built()


def _on_side_stream_equals_default(fn):
    import torch
    torch.cuda.synchronize()
    ref = [t.cpu() for t in fn(None)]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        got = fn(s)
    s.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b.cpu())


def test_decode_on_caller_stream():
    from software_pipelined_amd import attn
    q, k, v = (to_device(x) for x in I.gen_decode(2, 4, 1, 3000, 128, seed=61))
    _on_side_stream_equals_default(lambda s: attn.attn_decode(q, k, v, stream=s))


def test_backward_on_caller_stream():
    from software_pipelined_amd import attn
    q, k, v = (to_device(x) for x in I.gen_qkv(1, 2, 700, 128, seed=62))
    do = to_device(I.gen_dout(1, 2, 700, 128, seed=62))
    out, lse = attn.attn_forward(q, k, v, causal=True)
    _on_side_stream_equals_default(lambda s: attn.attn_backward(q, k, v, out, lse, do, causal=True, stream=s))


def test_chunk_scan_on_caller_stream():
    import torch
    from software_pipelined_amd import attn
    x, cb, dt, dacs = I.gen_chunk_scan(1, 700, 4, 64, 256, seed=63)
    tx, tcb = to_device(x), to_device(cb)
    tdt, tda = torch.from_numpy(dt).to("cuda"), torch.from_numpy(dacs).to("cuda")
    _on_side_stream_equals_default(lambda s: [attn.mamba_chunk_scan(tx, tcb, tdt, tda, 256, stream=s)])


def test_mla_on_caller_stream():
    from software_pipelined_amd import attn
    q, kv = (to_device(x) for x in I.gen_mla(2, 64, 1500, 576, seed=64))
    _on_side_stream_equals_default(lambda s: attn.mla_decode_torch(q, kv, 0.07, stream=s))


def _busy(stream):
    """Queue a long spin on `stream` so that work enqueued after it runs late."""
    import torch
    with torch.cuda.stream(stream):
        torch.cuda._sleep(100_000_000)


@pytest.mark.parametrize("entry", ["decode", "backward", "mla"])
def test_wrappers_keep_their_buffers_for_a_non_current_stream(entry):
    """The torch wrappers allocate outputs and workspaces on the current
    stream but enqueue on the caller's. With the caller's stream held back by
    a spin, the current stream then churns the caching allocator (same sizes,
    filled with garbage) before the call's kernels have run; the results must
    still equal those of the same call on the current stream."""
    import torch
    from software_pipelined_amd import attn
    if entry == "decode":
        q, k, v = (to_device(x) for x in I.gen_decode(2, 4, 1, 3000, 128, seed=65))
        fn = lambda s: list(attn.attn_decode(q, k, v, stream=s))
    elif entry == "backward":
        q, k, v = (to_device(x) for x in I.gen_qkv(1, 2, 700, 128, seed=66))
        do = to_device(I.gen_dout(1, 2, 700, 128, seed=66))
        out, lse = attn.attn_forward(q, k, v, causal=True)
        fn = lambda s: attn.attn_backward(q, k, v, out, lse, do, causal=True, stream=s)
    else:
        q, kv = (to_device(x) for x in I.gen_mla(2, 64, 1500, 576, seed=67))
        fn = lambda s: list(attn.mla_decode_torch(q, kv, 0.07, stream=s))
    torch.cuda.synchronize()
    ref = [t.cpu() for t in fn(None) if t is not None]
    s = torch.cuda.Stream()
    _busy(s)
    got = [t for t in fn(s) if t is not None]
    sizes = [t.numel() * t.element_size() for t in got] + [64 << 20]
    junk = [torch.full((n,), 0x7F, dtype=torch.uint8, device="cuda") for n in sizes for _ in range(2)]
    s.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b.cpu())
    del junk
