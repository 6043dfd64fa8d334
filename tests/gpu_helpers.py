"""Shared helpers of the GPU tests: upload seeded inputs, run the HIP path
through the C ABI, and compare with the fp64 oracle at the stated bar.

Acceptance bar (fp32 outputs from bf16 inputs): O max abs error <= 1e-2,
O mean abs error <= 1e-3, LSE max abs error <= 1e-3, and no NaN/Inf.
"""

import numpy as np

O_MAX_ABS = 1e-2
O_MEAN_ABS = 1e-3
LSE_MAX_ABS = 1e-3


def ensure_built():
    from software_pipelined_amd import attn, build
    import os
    if not os.path.exists(attn.LIB_PATH):
        build.build_library()
    return attn.load_library()


def to_device(bits):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to("cuda")


def run_gpu(q, k, v, causal, scale, variant=None):
    """Run attention forward on numpy bf16 bit arrays; return numpy (out, lse)."""
    import torch
    from software_pipelined_amd import attn
    dq, dk, dv = to_device(q), to_device(k), to_device(v)
    out, lse = attn.attn_forward(dq, dk, dv, causal=causal, scale=float(np.float32(scale)),
                                 variant=variant)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def compare(out, lse, ref_o, ref_l, what=""):
    """Assert the acceptance bar; return the error statistics."""
    assert np.isfinite(out).all(), f"{what}: non-finite O"
    assert np.isfinite(lse).all(), f"{what}: non-finite LSE"
    err = np.abs(out.astype(np.float64) - ref_o)
    lerr = np.abs(lse.astype(np.float64) - ref_l)
    stats = dict(o_max=float(err.max()) if err.size else 0.0,
                 o_mean=float(err.mean()) if err.size else 0.0,
                 lse_max=float(lerr.max()) if lerr.size else 0.0)
    assert stats["o_max"] <= O_MAX_ABS, f"{what}: O max abs {stats['o_max']:.3e}"
    assert stats["o_mean"] <= O_MEAN_ABS, f"{what}: O mean abs {stats['o_mean']:.3e}"
    assert stats["lse_max"] <= LSE_MAX_ABS, f"{what}: LSE max abs {stats['lse_max']:.3e}"
    return stats
