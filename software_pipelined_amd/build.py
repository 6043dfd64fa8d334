"""Build step for the HIP library ``libattn.so`` (gfx950 only).

Compiles the kernel sources in ``csrc/`` (attention forward, split-KV decoding,
backward, Mamba2 ChunkScan, MLA decoding; shared device helpers in
``attn_common.h``) with one hipcc call into ``software_pipelined_amd/libattn.so``.
Packed FP32 VALU forms are disabled for all device code.
"""

from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", f) for f in
        ("attn_fwd.hip", "attn_decode.hip", "attn_bwd.hip", "chunk_scan.hip", "mla_decode.hip")]
LIB = os.path.join(PKG, "libattn.so")
INCLUDE = os.path.join(ROOT, "include")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise FileNotFoundError("hipcc not found (ROCm toolchain required)")


def compile_cmd(out: str, extra=()) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-I", INCLUDE, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # device code never sees NaN (masking uses -inf, inputs are finite):
            # lets v_max_f32 / v_max3_f32 skip NaN-quieting canonicalisation
            "-Xarch_device", "-fno-honor-nans",
            # MFMA results in VGPRs: with one wave per SIMD the compiler
            # otherwise keeps accumulators in AGPRs and copies O back and forth
            # every block for the VALU rescale; the Q fragments are parked in
            # AGPRs explicitly instead
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            *extra, *SRCS, "-o", out]


def build_library(verbose: bool = False) -> str:
    """Compile libattn.so in place (always recompiles)."""
    tmp = LIB + ".tmp"
    proc = subprocess.run(compile_cmd(tmp), capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + proc.stdout + proc.stderr)
    if verbose:
        print(proc.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
