"""Build libqgemv.so (gfx950) in-tree with hipcc.

    python -m block_dequant_gemv_amd.build

Flags:
  --offload-arch=gfx950           MI355X only; no other targets, no host fallback.
  -ffp-contract=off               the kernels spell out every fma, so a row's
                                  operations are the same in every kernel variant.
  -fno-gpu-flush-denormals-to-zero  fp16 subnormal scales must survive.
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                  no packed fp32 instructions are generated.
  -mllvm -amdgpu-mfma-vgpr-form   (GEMM source only) the matrix-core results go to
                                  ordinary VGPRs, which the per-block scale fma reads
                                  directly, instead of accumulation registers that
                                  need one v_accvgpr_read per value.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqgemv.so")
SOURCES = ["qgemv_kernels.hip", "qgemm_kernels.hip", "qgemv_api.hip"]
HEADERS = ["layout.h", "dequant.h", "qgemv_kernels.h", "qgemm_kernels.h"]
SOURCE_FLAGS = {"qgemm_kernels.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libqgemv)")


def flags() -> list[str]:
    return ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
            "-fno-gpu-flush-denormals-to-zero",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function",
            "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every HIP source into block_dequant_gemv_amd/libqgemv.so (always rebuilds)."""
    cc = hipcc()
    objs = []
    build_dir = os.path.join(PKG, "_build")
    os.makedirs(build_dir, exist_ok=True)
    procs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        cmd = [cc, *flags(), *SOURCE_FLAGS.get(src, []), *(extra or []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        procs.append((subprocess.Popen(cmd), src))
        objs.append(obj)
    for p, src in procs:
        if p.wait() != 0:
            raise RuntimeError(f"hipcc failed on {src}")
    tmp = LIB + ".tmp"
    link = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(link), file=sys.stderr)
    subprocess.check_call(link)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
