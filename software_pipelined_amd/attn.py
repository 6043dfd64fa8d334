"""Thin Python binding of ``libattn.so`` (C ABI declared in include/attn.h).

Argument marshalling only: every step of the attention forward, decoding,
backward and MLA decoding and of the Mamba2 ChunkScan runs in the HIP kernels. The low-level functions take raw device
pointers and sizes with the same names and argument order as the C entry
points; ``attn_forward``, ``attn_decode``, ``attn_backward``,
``mla_decode_torch`` and ``mamba_chunk_scan`` are
convenience wrappers that allocate outputs (and workspaces) with torch
(device memory and streams are all torch is used for) and call them.

There is no fallback: if the compiled library is missing or fails to load,
every call raises.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")

ATTN_OK = 0
ATTN_ERR_NULL_PTR = 1
ATTN_ERR_BAD_SHAPE = 2
ATTN_ERR_HEAD_DIM = 3
ATTN_ERR_BAD_SCALE = 4
ATTN_ERR_MISALIGNED = 5
ATTN_ERR_HIP = 6
ATTN_ERR_WORKSPACE = 8
ATTN_ERR_TOO_LARGE = 9

_lib = None

_FWD_ARGS = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
             ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
             ctypes.c_void_p]


class AttnError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"attn status {status}: {attn_strerror(status)}")


def load_library():
    """Load libattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FileNotFoundError(
            f"{LIB_PATH} is missing: build it first (python -m software_pipelined_amd.build)")
    # torch first: its bundled HIP runtime has the same soname as the one the
    # library links, so loaded first it serves both. Loaded the other way
    # round, the process holds two HIP runtimes, and torch's device pointers
    # and streams are foreign to the library's (every launch then fails).
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd.argtypes = _FWD_ARGS
    lib.attn_fwd_variant.restype = ctypes.c_int
    lib.attn_fwd_variant.argtypes = [ctypes.c_int] + _FWD_ARGS
    lib.attn_strerror.restype = ctypes.c_char_p
    lib.attn_strerror.argtypes = [ctypes.c_int]
    lib.attn_num_variants.restype = ctypes.c_int
    lib.attn_num_variants.argtypes = []
    lib.attn_variant_name.restype = ctypes.c_char_p
    lib.attn_variant_name.argtypes = [ctypes.c_int]
    lib.attn_variant_info.restype = ctypes.c_int
    lib.attn_variant_info.argtypes = [ctypes.c_int] + [ctypes.POINTER(ctypes.c_int)] * 5
    lib.attn_default_variant.restype = ctypes.c_int
    lib.attn_default_variant.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.attn_decode_workspace_size.restype = ctypes.c_int
    lib.attn_decode_workspace_size.argtypes = [ctypes.c_int] * 5 + [ctypes.POINTER(ctypes.c_size_t)]
    lib.attn_bwd_workspace_size.restype = ctypes.c_int
    lib.attn_bwd_workspace_size.argtypes = [ctypes.c_int] * 4 + [ctypes.POINTER(ctypes.c_size_t)]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int] * 5 + [
        ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.mla_decode_workspace_size.restype = ctypes.c_int
    lib.mla_decode_workspace_size.argtypes = [ctypes.c_int] * 3 + [ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_decode.restype = ctypes.c_int
    lib.mla_decode.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int] * 3 + [
        ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.chunk_scan.restype = ctypes.c_int
    lib.chunk_scan.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + [ctypes.c_void_p]
    lib.attn_fwd_decode.restype = ctypes.c_int
    lib.attn_fwd_decode.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + [
        ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.attn_decode_static_max_bytes.restype = ctypes.c_size_t
    lib.attn_decode_static_max_bytes.argtypes = []
    lib.attn_fwd_decode_static.restype = ctypes.c_int
    lib.attn_fwd_decode_static.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + [
        ctypes.c_float, ctypes.c_void_p]
    lib.attn_probe_mfma.restype = ctypes.c_int
    lib.attn_probe_mfma.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p, ctypes.c_void_p]
    _lib = lib
    return lib


# ------------------------------------------------------------ C entry points

def attn_fwd(q, k, v, out, lse, B, H, N, d, causal, scale, stream) -> int:
    """Same arguments as the C ``attn_fwd``: device pointers (ints), sizes, stream handle."""
    return load_library().attn_fwd(q, k, v, out, lse, B, H, N, d, int(causal), float(scale), stream)


def attn_fwd_variant(id, q, k, v, out, lse, B, H, N, d, causal, scale, stream) -> int:
    return load_library().attn_fwd_variant(id, q, k, v, out, lse, B, H, N, d, int(causal),
                                           float(scale), stream)


def attn_strerror(status: int) -> str:
    return load_library().attn_strerror(status).decode()


def attn_num_variants() -> int:
    return load_library().attn_num_variants()


def attn_variant_name(id: int):
    r = load_library().attn_variant_name(id)
    return None if r is None else r.decode()


def attn_variant_info(id: int) -> dict:
    vals = [ctypes.c_int() for _ in range(5)]
    st = load_library().attn_variant_info(id, *[ctypes.byref(x) for x in vals])
    if st != ATTN_OK:
        raise AttnError(st)
    keys = ("head_dim", "block_m", "block_n", "waves", "lds_bytes")
    return dict(zip(keys, (x.value for x in vals)))


def attn_default_variant(d: int, causal: bool) -> int:
    return load_library().attn_default_variant(d, int(causal))


def attn_decode_workspace_size(B, H, Nq, Nkv, d):
    """(status, bytes) as returned through the C ``attn_decode_workspace_size``."""
    n = ctypes.c_size_t(0)
    st = load_library().attn_decode_workspace_size(B, H, Nq, Nkv, d, ctypes.byref(n))
    return st, n.value


def attn_fwd_decode(q, k, v, out, lse, B, H, Nq, Nkv, d, scale, workspace, workspace_bytes,
                    stream) -> int:
    """Same arguments as the C ``attn_fwd_decode``: device pointers (ints), sizes, stream."""
    return load_library().attn_fwd_decode(q, k, v, out, lse, B, H, Nq, Nkv, d, float(scale),
                                          workspace, workspace_bytes, stream)


def attn_probe_mfma(mode, blocks, iters, out, stream) -> int:
    """Same arguments as the C ``attn_probe_mfma`` (include/attn_probe.h): the
    matrix-core stream used to measure the sustained MFMA rate and clock."""
    return load_library().attn_probe_mfma(mode, blocks, iters, out, stream)


def attn_decode_static_max_bytes() -> int:
    return load_library().attn_decode_static_max_bytes()


def attn_fwd_decode_static(q, k, v, out, lse, B, H, Nq, Nkv, d, scale, stream) -> int:
    """Same arguments as the C ``attn_fwd_decode_static`` (no workspace: the
    library's fixed per-GPU scratch holds the chunk partials)."""
    return load_library().attn_fwd_decode_static(q, k, v, out, lse, B, H, Nq, Nkv, d, float(scale), stream)


# ------------------------------------------------------------ torch convenience

def _check_buffer(t, name, shape, dtype, device):
    """A caller-supplied output or workspace: a contiguous tensor of the given
    shape and dtype on the inputs' GPU (its data pointer goes to the kernels)."""
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_workspace(ws, device):
    """A workspace: contiguous and on the inputs' GPU; returns its size in
    bytes (the C entry point reports one that is too small)."""
    if not ws.is_cuda or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    return ws.numel() * ws.element_size()


def _used_on(stream, *tensors):
    """Tell torch's caching allocator that the kernels enqueued on ``stream``
    use these tensors: buffers allocated here (on the current stream) are then
    not handed out again before that stream's work is done, even when
    ``stream`` is not the current one."""
    for t in tensors:
        t.record_stream(stream)


def attn_bwd_workspace_size(B, H, N, d):
    """(status, bytes) as returned through the C ``attn_bwd_workspace_size``."""
    n = ctypes.c_size_t(0)
    st = load_library().attn_bwd_workspace_size(B, H, N, d, ctypes.byref(n))
    return st, n.value


def attn_bwd(q, k, v, out, lse, dout, dq, dk, dv, B, H, N, d, causal, scale, workspace,
             workspace_bytes, stream) -> int:
    """Same arguments as the C ``attn_bwd``: device pointers (ints), sizes, stream."""
    return load_library().attn_bwd(q, k, v, out, lse, dout, dq, dk, dv, B, H, N, d, int(bool(causal)),
                                   float(scale), workspace, workspace_bytes, stream)


def attn_backward(q, k, v, out, lse, dout, causal: bool = False, scale=None, dq=None, dk=None, dv=None,
                  workspace=None, stream=None):
    """Attention backward for torch tensors: (dq, dk, dv) float32 [B, H, N, d].

    q, k, v, dout: contiguous bfloat16 [B, H, N, d] on the GPU; out (float32
    [B, H, N, d]) and lse (float32 [B, H, N]) are the forward's outputs for
    the same q, k, v, causal and scale. Buffers not given (and the workspace
    of ``attn_bwd_workspace_size`` bytes) are allocated with torch.
    """
    import torch

    for t in (q, k, v, dout):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError("q, k, v, dout must be contiguous 4-d bfloat16 tensors on the GPU")
    B, H, N, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or dout.shape != q.shape:
        raise ValueError("q, k, v, dout must share one [B, H, N, d] shape")
    if out.dtype != torch.float32 or tuple(out.shape) != (B, H, N, d) or not out.is_contiguous():
        raise ValueError("out must be the forward's contiguous float32 [B, H, N, d] output")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous():
        raise ValueError("lse must be the forward's contiguous float32 [B, H, N] output")
    for t in (k, v, dout, out, lse):
        if t.device != q.device:
            raise ValueError("every tensor must be on q's GPU")
    if scale is None:
        scale = float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))
    st, need = attn_bwd_workspace_size(B, H, N, d)
    if st != ATTN_OK:
        raise AttnError(st)
    made = []
    grads = []
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        if g is None:
            g = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
            made.append(g)
        else:
            _check_buffer(g, name, (B, H, N, d), torch.float32, q.device)
        grads.append(g)
    dq, dk, dv = grads
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        made.append(workspace)
    ws_bytes = _check_workspace(workspace, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    _used_on(stream, *made)
    st = attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                  dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, causal, scale,
                  workspace.data_ptr(), ws_bytes, stream.cuda_stream)
    if st != ATTN_OK:
        raise AttnError(st)
    return dq, dk, dv


def mla_decode_workspace_size(B, H, N):
    """(status, bytes) as returned through the C ``mla_decode_workspace_size``."""
    n = ctypes.c_size_t(0)
    st = load_library().mla_decode_workspace_size(B, H, N, ctypes.byref(n))
    return st, n.value


def mla_decode(q, kv, out, lse, B, H, N, scale, workspace, workspace_bytes, stream) -> int:
    """Same arguments as the C ``mla_decode``: device pointers (ints), sizes, stream."""
    return load_library().mla_decode(q, kv, out, lse, B, H, N, float(scale), workspace, workspace_bytes, stream)


def mla_decode_torch(q, kv, scale, out=None, lse=None, workspace=None, stream=None):
    """MLA decoding for torch tensors: q bfloat16 [B, H, 576], kv bfloat16
    [B, N, 576] (values: the first 512 of each row). Returns (out float32
    [B, H, 512], lse float32 [B, H])."""
    import torch

    if q.dtype != torch.bfloat16 or kv.dtype != torch.bfloat16 or q.dim() != 3 or kv.dim() != 3:
        raise ValueError("q [B, H, 576] and kv [B, N, 576] must be bfloat16")
    B, H, Dk = q.shape
    N = kv.shape[1]
    if Dk != 576 or kv.shape[0] != B or kv.shape[2] != 576 or not q.is_contiguous() or not kv.is_contiguous():
        raise ValueError("q [B, H, 576] and kv [B, N, 576], contiguous")
    if not q.is_cuda or kv.device != q.device:
        raise ValueError("q and kv must be on one GPU")
    st, need = mla_decode_workspace_size(B, H, N)
    if st != ATTN_OK:
        raise AttnError(st)
    made = []
    if out is None:
        out = torch.empty((B, H, 512), dtype=torch.float32, device=q.device)
        made.append(out)
    else:
        _check_buffer(out, "out", (B, H, 512), torch.float32, q.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
        made.append(lse)
    else:
        _check_buffer(lse, "lse", (B, H), torch.float32, q.device)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        made.append(workspace)
    ws_bytes = _check_workspace(workspace, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    _used_on(stream, *made)
    st = mla_decode(q.data_ptr(), kv.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, scale,
                    workspace.data_ptr(), ws_bytes, stream.cuda_stream)
    if st != ATTN_OK:
        raise AttnError(st)
    return out, lse


def chunk_scan(x, cb, dt, dA_cumsum, out, B, S, H, P, L, stream) -> int:
    """Same arguments as the C ``chunk_scan``: device pointers (ints), sizes, stream."""
    return load_library().chunk_scan(x, cb, dt, dA_cumsum, out, B, S, H, P, L, stream)


def mamba_chunk_scan(x, cb, dt, dA_cumsum, L: int, out=None, stream=None):
    """Mamba2 ChunkScan for torch tensors: out float32 [B, S, H, P].

    x: bfloat16 [B, S, H, P]; cb: bfloat16 [B, nc, L, L]; dt, dA_cumsum:
    float32 [B, H, nc, L] (nc = ceil(S / L)); all contiguous on the GPU.
    """
    import torch

    if x.dtype != torch.bfloat16 or cb.dtype != torch.bfloat16 or x.dim() != 4:
        raise ValueError("x and cb must be bfloat16, x [B, S, H, P]")
    B, S, H, P = x.shape
    nc = (S + L - 1) // L
    if tuple(cb.shape) != (B, nc, L, L) or tuple(dt.shape) != (B, H, nc, L) or dt.shape != dA_cumsum.shape:
        raise ValueError("cb must be [B, nc, L, L] and dt, dA_cumsum [B, H, nc, L]")
    for t in (x, cb, dt, dA_cumsum):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("inputs must be contiguous GPU tensors")
    if dt.dtype != torch.float32 or dA_cumsum.dtype != torch.float32:
        raise ValueError("dt and dA_cumsum must be float32")
    for t in (cb, dt, dA_cumsum):
        if t.device != x.device:
            raise ValueError("every tensor must be on x's GPU")
    made = []
    if out is None:
        out = torch.empty((B, S, H, P), dtype=torch.float32, device=x.device)
        made.append(out)
    else:
        _check_buffer(out, "out", (B, S, H, P), torch.float32, x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    _used_on(stream, *made)
    st = chunk_scan(x.data_ptr(), cb.data_ptr(), dt.data_ptr(), dA_cumsum.data_ptr(), out.data_ptr(),
                    B, S, H, P, L, stream.cuda_stream)
    if st != ATTN_OK:
        raise AttnError(st)
    return out


def attn_forward(q, k, v, causal: bool = False, scale=None, out=None, lse=None, variant=None,
                 stream=None):
    """Attention forward on torch tensors already on the GPU.

    q, k, v: bfloat16 [B, H, N, d], contiguous, on a HIP device. Returns
    (out float32 [B, H, N, d], lse float32 [B, H, N]). ``scale`` defaults to
    float32(1/sqrt(d)). The kernel is enqueued on ``stream`` (default: torch's
    current stream) and the call returns without synchronising.
    """
    import torch

    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("q, k, v must be bfloat16")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be on the GPU")
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one GPU")
    B, H, N, d = q.shape
    if scale is None:
        scale = float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))
    made = []
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
        made.append(out)
    else:
        _check_buffer(out, "out", (B, H, N, d), torch.float32, q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        made.append(lse)
    else:
        _check_buffer(lse, "lse", (B, H, N), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    _used_on(stream, *made)
    handle = stream.cuda_stream
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
            B, H, N, d, causal, scale, handle)
    st = attn_fwd(*args) if variant is None else attn_fwd_variant(variant, *args)
    if st != ATTN_OK:
        raise AttnError(st)
    return out, lse


def attn_decode(q, k, v, scale=None, out=None, lse=None, workspace=None, stream=None):
    """Split-KV decoding on torch tensors already on the GPU.

    q: bfloat16 [B, H, Nq, d]; k, v: bfloat16 [B, Hkv, Nkv, d], contiguous,
    with Hkv dividing H (Hkv < H: grouped K/V heads, query head h reading K/V
    head h // (H / Hkv); the G = H / Hkv query heads of a group are adjacent
    in q, so the C entry point is called with Hkv heads of G * Nq query rows
    on the same buffers). Every query sees every key. Returns (out float32
    [B, H, Nq, d], lse float32 [B, H, Nq]); out, lse and the workspace (a
    uint8 tensor of at least ``attn_decode_workspace_size(B, Hkv, G * Nq, Nkv,
    d)`` bytes) are allocated with torch when not given. Enqueued on ``stream`` (default: torch's current stream).
    """
    import torch

    for t in (q, k, v):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError("q, k, v must be contiguous 4-d bfloat16 tensors on the GPU")
    B, H, Nq, d = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    if (tuple(k.shape) != (B, Hkv, Nkv, d) or k.shape != v.shape or Hkv < 1 or H % Hkv != 0):
        raise ValueError("k and v must be [B, Hkv, Nkv, d] with q's B and d and Hkv dividing q's H")
    G = H // Hkv  # query heads per K/V head: (H, Nq) -> (Hkv, G * Nq) over the same memory
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one GPU")
    if scale is None:
        scale = float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))
    st, need = attn_decode_workspace_size(B, Hkv, G * Nq, Nkv, d)
    if st != ATTN_OK:
        raise AttnError(st)
    made = []
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=torch.float32, device=q.device)
        made.append(out)
    else:
        _check_buffer(out, "out", (B, H, Nq, d), torch.float32, q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
        made.append(lse)
    else:
        _check_buffer(lse, "lse", (B, H, Nq), torch.float32, q.device)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        made.append(workspace)
    ws_bytes = _check_workspace(workspace, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    _used_on(stream, *made)
    st = attn_fwd_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                         B, Hkv, G * Nq, Nkv, d, scale, workspace.data_ptr(), ws_bytes,
                         stream.cuda_stream)
    if st != ATTN_OK:
        raise AttnError(st)
    return out, lse
