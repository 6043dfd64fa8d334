"""Python access to the fp64 oracle (``attn_oracle.c``): attention forward,
decoding, backward and MLA decoding, and Mamba2 ChunkScan.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path. It loads the C
oracle through ctypes and shares nothing with the HIP library.

The computation is the plain definition of attention (PipeThreader OSDI'25
summary page, "FlashAttention-3" paragraph: acc_s = Q K^T, softmax gives P,
O = P V), with the readings for scale, causal mask and log-sum-exp stated in
the C file's header.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def compile_source(src: str, out_path: str) -> str:
    """Compile one oracle C source into a shared library at ``out_path``.

    No ``-march=native`` and no fast-math: the library is built in one
    container and run on another host, and IEEE semantics are required.
    """
    tmp = out_path + ".tmp"
    cmd = ["gcc", "-O3", "-fopenmp", "-fno-fast-math", "-fPIC", "-shared", "-std=c11",
           src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


def build(force: bool = True) -> str:
    """Compile the C oracle into ``oracle/liboracle.so`` (gcc + OpenMP)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    return compile_source(_SRC, _LIB_PATH)


SOURCE_PATH = _SRC


def bind(path: str):
    """Load a compiled oracle library from ``path`` and declare its signatures."""
    lib = ctypes.CDLL(path)
    lib.oracle_attn_fwd_rows.restype = ctypes.c_int
    lib.oracle_attn_fwd_rows.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int, ctypes.c_float,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
    ]
    lib.oracle_attn_decode_rows.restype = ctypes.c_int
    lib.oracle_attn_decode_rows.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_float,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
    ]
    lib.oracle_attn_bwd_rows.restype = ctypes.c_int
    lib.oracle_attn_bwd_rows.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int, ctypes.c_float,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
    ]
    lib.oracle_chunk_scan_rows.restype = ctypes.c_int
    lib.oracle_chunk_scan_rows.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
    ]
    lib.oracle_mla_decode_rows.restype = ctypes.c_int
    lib.oracle_mla_decode_rows.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_float, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
    ]
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = bind(_LIB_PATH)
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def attn_fwd_rows(q, k, v, causal: bool, scale, rows=None, threads: int = 0, lib=None):
    """fp64 attention forward for selected rows.

    q, k, v: uint16 bf16 bit arrays [B, H, N, d]. ``rows``: flat row ids
    (b*H + h)*N + i, or None for every row. ``scale`` is converted to float32,
    the exact value the GPU path receives.
    Returns (out [n_rows, d] float64, lse [n_rows] float64).
    """
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    B, H, N, d = q.shape
    if rows is None:
        n_rows = B * H * N
        rows_ptr = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows = rows.size
        rows_ptr = rows.ctypes.data
    out = np.empty((n_rows, d), dtype=np.float64)
    lse = np.empty((n_rows,), dtype=np.float64)
    rc = (lib or _load()).oracle_attn_fwd_rows(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H, N, d, int(bool(causal)),
        float(np.float32(scale)), rows_ptr, n_rows, out.ctypes.data, lse.ctypes.data, int(threads))
    if rc < 0:
        raise ValueError("oracle rejected its arguments")
    if rc > 0:
        raise ArithmeticError(f"{rc} softmax rows failed the sum-to-one self-check")
    return out, lse


def attn_fwd(q, k, v, causal: bool, scale, threads: int = 0, lib=None):
    """fp64 attention forward over every row: (out [B,H,N,d], lse [B,H,N])."""
    B, H, N, d = q.shape
    out, lse = attn_fwd_rows(q, k, v, causal, scale, None, threads, lib)
    return out.reshape(B, H, N, d), lse.reshape(B, H, N)


def attn_decode_rows(q, k, v, scale, rows=None, threads: int = 0, lib=None):
    """fp64 decoding attention: q [B, H, Nq, d] against k, v [B, H, Nkv, d],
    every query seeing every key. ``rows``: flat query-row ids (b*H + h)*Nq + i,
    or None for all. Returns (out [n_rows, d] float64, lse [n_rows] float64)."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape or q.shape[:2] != k.shape[:2] \
            or q.shape[3] != k.shape[3]:
        raise ValueError("q must be [B, H, Nq, d] and k, v one [B, H, Nkv, d] shape")
    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    if rows is None:
        n_rows = B * H * Nq
        rows_ptr = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows = rows.size
        rows_ptr = rows.ctypes.data
    out = np.empty((n_rows, d), dtype=np.float64)
    lse = np.empty((n_rows,), dtype=np.float64)
    rc = (lib or _load()).oracle_attn_decode_rows(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H, Nq, Nkv, d,
        float(np.float32(scale)), rows_ptr, n_rows, out.ctypes.data, lse.ctypes.data, int(threads))
    if rc < 0:
        raise ValueError("oracle rejected its arguments")
    if rc > 0:
        raise ArithmeticError(f"{rc} softmax rows failed the sum-to-one self-check")
    return out, lse


def attn_decode(q, k, v, scale, threads: int = 0, lib=None):
    """fp64 decoding attention over every query row: (out [B,H,Nq,d], lse [B,H,Nq])."""
    B, H, Nq, d = q.shape
    out, lse = attn_decode_rows(q, k, v, scale, None, threads, lib)
    return out.reshape(B, H, Nq, d), lse.reshape(B, H, Nq)


def attn_bwd_rows(q, k, v, dout, causal: bool, scale, qrows=None, krows=None, threads: int = 0,
                  lib=None):
    """fp64 attention backward (gradient of the forward) for selected rows.

    q, k, v, dout: uint16 bf16 bit arrays [B, H, N, d]; dout is the upstream
    gradient of O. ``qrows``: flat query-row ids whose dQ is wanted;
    ``krows``: flat key-row ids whose dK and dV are wanted (None = all rows).
    Returns (dq [n_q, d], dk [n_k, d], dv [n_k, d]) as float64.
    """
    arrs = [np.ascontiguousarray(x, dtype=np.uint16) for x in (q, k, v, dout)]
    if arrs[0].ndim != 4 or any(a.shape != arrs[0].shape for a in arrs):
        raise ValueError("q, k, v, dout must share one [B, H, N, d] shape")
    B, H, N, d = arrs[0].shape

    def sel(rows):
        if rows is None:
            return None, B * H * N, None
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        return rows, rows.size, rows.ctypes.data

    qrows, n_q, qp = sel(qrows)
    krows, n_k, kp = sel(krows)
    dq = np.empty((n_q, d), dtype=np.float64)
    dk = np.empty((n_k, d), dtype=np.float64)
    dv = np.empty((n_k, d), dtype=np.float64)
    rc = (lib or _load()).oracle_attn_bwd_rows(
        arrs[0].ctypes.data, arrs[1].ctypes.data, arrs[2].ctypes.data, arrs[3].ctypes.data,
        B, H, N, d, int(bool(causal)), float(np.float32(scale)), qp, n_q, dq.ctypes.data,
        kp, n_k, dk.ctypes.data, dv.ctypes.data, int(threads))
    if rc < 0:
        raise ValueError("oracle rejected its arguments")
    if rc > 0:
        raise ArithmeticError(f"{rc} softmax rows failed the sum-to-one self-check")
    return dq, dk, dv


def attn_bwd(q, k, v, dout, causal: bool, scale, threads: int = 0, lib=None):
    """fp64 attention backward over every row: (dq, dk, dv), each [B, H, N, d]."""
    B, H, N, d = q.shape
    dq, dk, dv = attn_bwd_rows(q, k, v, dout, causal, scale, None, None, threads, lib)
    return dq.reshape(B, H, N, d), dk.reshape(B, H, N, d), dv.reshape(B, H, N, d)


def chunk_scan_rows(x, cb, dt, dacs, L: int, rows=None, threads: int = 0, lib=None):
    """fp64 Mamba2 ChunkScan for selected output rows.

    x: uint16 bf16 bits [B, S, H, P]; cb: uint16 bf16 bits [B, nc, L, L];
    dt, dacs: float32 [B, H, nc, L]. ``rows``: flat ids (b*S + s)*H + h, or
    None for all. Returns out [n_rows, P] float64.
    """
    x = np.ascontiguousarray(x, dtype=np.uint16)
    cb = np.ascontiguousarray(cb, dtype=np.uint16)
    dt = np.ascontiguousarray(dt, dtype=np.float32)
    dacs = np.ascontiguousarray(dacs, dtype=np.float32)
    B, S, H, P = x.shape
    nc = (S + L - 1) // L
    if cb.shape != (B, nc, L, L) or dt.shape != (B, H, nc, L) or dacs.shape != dt.shape:
        raise ValueError("cb must be [B, nc, L, L] and dt, dacs [B, H, nc, L]")
    if rows is None:
        n_rows, rows_ptr = B * S * H, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows, rows_ptr = rows.size, rows.ctypes.data
    out = np.empty((n_rows, P), dtype=np.float64)
    rc = (lib or _load()).oracle_chunk_scan_rows(
        x.ctypes.data, cb.ctypes.data, dt.ctypes.data, dacs.ctypes.data, B, S, H, P, L, rows_ptr, n_rows,
        out.ctypes.data, int(threads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return out


def chunk_scan(x, cb, dt, dacs, L: int, threads: int = 0, lib=None):
    """fp64 ChunkScan over every row: out [B, S, H, P]."""
    return chunk_scan_rows(x, cb, dt, dacs, L, None, threads, lib).reshape(x.shape)


def mla_decode_rows(q, kv, Dv: int, scale, rows=None, threads: int = 0, lib=None):
    """fp64 MLA decoding: q [B, H, Dk] against one shared cache kv [B, N, Dk]
    (keys: all Dk values of a row; values: its first Dv). ``rows``: flat
    (b*H + h) ids or None. Returns (out [n_rows, Dv], lse [n_rows]) float64."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    kv = np.ascontiguousarray(kv, dtype=np.uint16)
    if q.ndim != 3 or kv.ndim != 3 or q.shape[0] != kv.shape[0] or q.shape[2] != kv.shape[2]:
        raise ValueError("q must be [B, H, Dk] and kv [B, N, Dk]")
    B, H, Dk = q.shape
    N = kv.shape[1]
    if rows is None:
        n_rows, rows_ptr = B * H, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows, rows_ptr = rows.size, rows.ctypes.data
    out = np.empty((n_rows, Dv), dtype=np.float64)
    lse = np.empty((n_rows,), dtype=np.float64)
    rc = (lib or _load()).oracle_mla_decode_rows(q.ctypes.data, kv.ctypes.data, B, H, N, Dk, Dv,
                                                 float(np.float32(scale)), rows_ptr, n_rows, out.ctypes.data,
                                                 lse.ctypes.data, int(threads))
    if rc < 0:
        raise ValueError("oracle rejected its arguments")
    if rc > 0:
        raise ArithmeticError(f"{rc} softmax rows failed the sum-to-one self-check")
    return out, lse


def mla_decode(q, kv, Dv: int, scale, threads: int = 0, lib=None):
    """fp64 MLA decoding over every head: (out [B, H, Dv], lse [B, H])."""
    B, H, _ = q.shape
    out, lse = mla_decode_rows(q, kv, Dv, scale, None, threads, lib)
    return out.reshape(B, H, Dv), lse.reshape(B, H)
