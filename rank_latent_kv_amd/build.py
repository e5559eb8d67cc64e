"""Build libpalu.so in-tree with hipcc for gfx950.

Flags that matter for the results:
  -ffp-contract=off                 no implicit fusing of a*b + c; the kernels
                                    write every fused multiply-add they mean
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE fp32 division (the
                                    quantiser's (l - min) / scale)
  -Xclang -target-feature -Xclang -packed-fp32-ops   no packed fp32 ALU ops
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpalu.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall",
          "-ffp-contract=off", f"-I{INCLUDE}", f"-I{CSRC}"]
DEVICE = [f"--offload-arch={ARCH}", "-fhip-fp32-correctly-rounded-divide-sqrt",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
HOST_SOURCES = ["palu_host.cpp", "palu_eigen.cpp"]
DEVICE_SOURCES = ["palu_kernels.hip", "palu_decode.hip", "palu_prefill.hip"]
# Per-source extras.  No kernel handles NaN inputs (the quantiser's and the
# softmax's max / min need no quieting); the attention kernels' MFMA
# accumulators stay in ordinary VGPRs (no AGPR copies around the softmax).
SOURCE_FLAGS = {"palu_kernels.hip": ["-fno-honor-nans"],
                "palu_prefill.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form=1"],
                "palu_decode.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in p.stderr.splitlines() if noise not in l)
    if p.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err)


def build(verbose: bool = False) -> str:
    """Compiles every source (in parallel) and links libpalu.so."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs = []
    for src in DEVICE_SOURCES:
        obj = os.path.join(objdir, src + ".o")
        jobs.append(([HIPCC, *COMMON, *DEVICE, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj],
                     obj))
    for src in HOST_SOURCES:
        obj = os.path.join(objdir, src + ".o")
        jobs.append(([HIPCC, *COMMON, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-c",
                      os.path.join(CSRC, src), "-o", obj], obj))
    with ThreadPoolExecutor(max_workers=min(4, len(jobs))) as pool:
        list(pool.map(lambda j: _run(j[0], verbose), jobs))
    objs = [obj for _, obj in jobs]
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
