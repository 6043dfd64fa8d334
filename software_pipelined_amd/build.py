"""Build step for the HIP library ``libattn.so`` (gfx950 only).

Compiles the kernel sources in ``csrc/`` (attention forward -- entry points
plus one variant table per head dimension --, split-KV decoding, backward,
Mamba2 ChunkScan, MLA decoding; shared device helpers in ``attn_common.h``)
one hipcc process per source, in parallel, then links them into
``software_pipelined_amd/libattn.so``. Packed FP32 VALU forms are disabled
for all device code.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC_NAMES = ("attn_fwd.hip", "attn_fwd_d64.hip", "attn_fwd_d128.hip", "attn_fwd_d256.hip", "attn_decode.hip",
             "attn_bwd.hip", "chunk_scan.hip", "mla_decode.hip", "clock_probe.hip")
SRCS = [os.path.join(PKG, "csrc", f) for f in SRC_NAMES]
LIB = os.path.join(PKG, "libattn.so")
INCLUDE = os.path.join(ROOT, "include")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise FileNotFoundError("hipcc not found (ROCm toolchain required)")


FLAGS = ["-O3", "-std=c++17", "-fPIC",
         "-I", INCLUDE, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # device code never sees NaN (masking uses -inf, inputs are finite):
         # lets v_max_f32 / v_max3_f32 skip NaN-quieting canonicalisation
         "-Xarch_device", "-fno-honor-nans",
         # MFMA results in VGPRs: with one wave per SIMD the compiler
         # otherwise keeps accumulators in AGPRs and copies O back and forth
         # every block for the VALU rescale; the Q fragments are parked in
         # AGPRs explicitly instead
         "-mllvm", "-amdgpu-mfma-vgpr-form"]


def compile_cmd(src: str, obj: str, extra=()) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", *FLAGS, *extra, "-c", src, "-o", obj]


def link_cmd(objs, out: str) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out]


def build_library(verbose: bool = False, jobs: int = 0) -> str:
    """Compile libattn.so in place (always recompiles every source)."""
    jobs = jobs or min(len(SRCS), os.cpu_count() or 1)
    with tempfile.TemporaryDirectory(prefix="attn_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in SRCS]

        def one(pair):
            src, obj = pair
            return subprocess.run(compile_cmd(src, obj), capture_output=True, text=True)

        with ThreadPoolExecutor(max_workers=jobs) as ex:
            procs = list(ex.map(one, zip(SRCS, objs)))
        errs = [p.stdout + p.stderr for p in procs if p.returncode != 0]
        if errs:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
        if verbose:
            for p in procs:
                print(p.stderr)
        tmp_lib = LIB + ".tmp"
        proc = subprocess.run(link_cmd(objs, tmp_lib), capture_output=True, text=True)
        if proc.returncode != 0:
            raise RuntimeError("link failed:\n" + proc.stdout + proc.stderr)
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
