"""Build the HIP library ``w4_dequant_gemm_amd/libw4.so`` for gfx950 with hipcc.

Every kernel source is compiled for gfx950 only, with packed fp32 ops disabled
and IEEE-correct fp32 division; the quantizer and the row quantizer are also
built without FMA contraction so that their results are bit-reproducible.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
OUT = os.path.join(HERE, "libw4.so")
# measurement-only streaming-read kernel (bench.py), a library of its own
PROBE_SRC = "probe_read.hip"
PROBE_OUT = os.path.join(HERE, "libw4probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

KERNELS = ["quantize.hip", "prepack.hip", "rowquant.hip", "skinny.hip", "gemm.hip", "nf4.hip", "noalloc.hip", "gemm_f8.hip"]
NO_CONTRACT = {"quantize.hip", "rowquant.hip", "nf4.hip"}
# kernels whose MFMA results take VALU work: results in VGPRs, not AGPRs
MFMA_VGPR = {"gemm_f8.hip"}
HOST_SOURCES = ["api.cpp", "portable.cpp"]   # host C++ (argument checks, file I/O)

HIP_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
             "-fhip-fp32-correctly-rounded-divide-sqrt",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function",
             "-fvisibility=hidden"]   # kernels and launchers stay internal; the C ABI is in api.cpp / portable.cpp


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}):\n{' '.join(cmd)}\n{r.stdout}")
    # hipcc's host pass warns that it does not know the packed-fp32 feature; drop that noise
    lines = [l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if verbose and lines:
        print("\n".join(lines), flush=True)


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs_list = []
    for src in KERNELS:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        flags = list(HIP_FLAGS)
        if src in NO_CONTRACT:
            flags.append("-ffp-contract=off")
        if src in MFMA_VGPR:
            flags += ["-mllvm", "-amdgpu-mfma-vgpr-form"]
        jobs_list.append([HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
    for host_src in HOST_SOURCES:
        obj = os.path.join(BUILD, host_src.replace(".cpp", ".o"))
        jobs_list.append([HIPCC, "-x", "c++", "-O2", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__",
                          "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", "-c",
                          os.path.join(CSRC, host_src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_run, cmd, verbose) for cmd in jobs_list]:
            f.result()
    objs = [cmd[-1] for cmd in jobs_list]
    tmp = OUT + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, OUT)
    ptmp = PROBE_OUT + ".tmp"
    _run([HIPCC, *HIP_FLAGS, "-shared", os.path.join(CSRC, PROBE_SRC), "-o", ptmp], verbose)
    os.replace(ptmp, PROBE_OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
