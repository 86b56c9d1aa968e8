"""Build libsage.so (the HIP kernels and the C ABI) in-tree for gfx950.

Usage: python -m quantized_attention_video_02_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libsage.so")
SOURCES = ["sage_api.hip", "sage_quant.hip", "sage_attn.hip", "sage_bwd.hip"]
HEADERS = ["sage_common.h", "sage_device.h"]

# -ffp-contract=off: no implicit fused multiply-adds, so the quantization pass
# rounds exactly as documented (fused operations are written out explicitly).
# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
HIPFLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
            "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"]


# The backward sweeps run one wave per SIMD with more live values than the
# 256 registers vector instructions can address.  By default the compiler puts
# the MFMA results (S, dP, the per-tile products) in the accumulation
# registers, and every vector use then costs a move out of them; this option
# keeps MFMA results in ordinary VGPRs (the compiled dQ loop: 1246 vector
# instructions per tile instead of 1422, no spills).
SOURCE_FLAGS = {"sage_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: libsage needs ROCm (hipcc) to build")


def build(verbose: bool = False, jobs: int = 3) -> str:
    """Compile every source for gfx950 and link libsage.so (always rebuilds)."""
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [cc, *HIPFLAGS, *SOURCE_FLAGS.get(src, []), "-I", INCLUDE, "-c", os.path.join(CSRC, src),
               "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def is_stale() -> bool:
    if not os.path.exists(LIB_PATH):
        return True
    t = os.path.getmtime(LIB_PATH)
    deps = [os.path.join(CSRC, s) for s in SOURCES + HEADERS] + [os.path.join(INCLUDE, "sage.h")]
    return any(os.path.getmtime(p) > t for p in deps)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
