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

The quantised GEMV templates (csrc/qgemv_device.h) are instantiated by
csrc/qgemv_inst.hip, compiled once per (qtype, activation rows) pair with
-DQG_INST_QT / -DQG_INST_M, so that the instantiations build in parallel.
The host pass of hipcc does not know the packed-fp32 target feature and says so
once per compile; that one line is dropped from the compiler output, every other
diagnostic is shown.
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
SOURCES = ["qgemv_kernels.hip", "qgemm_kernels.hip", "qgemv_api.hip", "probe_kernels.hip"]
HEADERS = ["layout.h", "dequant.h", "qgemv_kernels.h", "qgemv_device.h", "qgemm_kernels.h"]
INST_SOURCE = "qgemv_inst.hip"
# (qtype code of layout.h, activation rows): 1 = Q8_0, 2 = Q4_0, 3 = Q4_K, 4 = Q6_K
INSTANCES = [(qt, m) for qt in (1, 2, 3, 4) for m in range(1, 7)]
HOST_FEATURE_NOTE = "'-packed-fp32-ops' is not a recognized feature for this target"
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


def compile_jobs(cc: str, build_dir: str, extra: list[str]) -> list[tuple[list[str], str, str]]:
    """(command, object, label) of every translation unit."""
    jobs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        jobs.append(([cc, *flags(), *SOURCE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj],
                     obj, src))
    for qt, m in INSTANCES:
        obj = os.path.join(build_dir, f"qgemv_inst_t{qt}_m{m}.o")
        jobs.append(([cc, *flags(), f"-DQG_INST_QT={qt}", f"-DQG_INST_M={m}", *extra, "-c",
                      os.path.join(CSRC, INST_SOURCE), "-o", obj], obj, f"{INST_SOURCE} (qtype {qt}, M={m})"))
    return jobs


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every HIP source into block_dequant_gemv_amd/libqgemv.so (always rebuilds)."""
    cc = hipcc()
    build_dir = os.path.join(PKG, "_build")
    os.makedirs(build_dir, exist_ok=True)
    jobs = compile_jobs(cc, build_dir, list(extra or []))
    width = max(1, min(len(jobs), os.cpu_count() or 1, 16))
    pending, running, failed = list(jobs), [], []
    while pending or running:
        while pending and len(running) < width:
            cmd, obj, label = pending.pop(0)
            if verbose:
                print(" ".join(cmd), file=sys.stderr)
            running.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True),
                            label))
        proc, label = running.pop(0)
        out, _ = proc.communicate()
        lines = [ln for ln in out.splitlines() if HOST_FEATURE_NOTE not in ln]
        if lines:
            print("\n".join(lines), file=sys.stderr)
        if proc.returncode != 0:
            failed.append(label)
    if failed:
        raise RuntimeError(f"hipcc failed on {', '.join(failed)}")
    objs = [obj for _, obj, _ in jobs]
    tmp = LIB + ".tmp"
    link = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(link), file=sys.stderr)
    subprocess.check_call(link)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
