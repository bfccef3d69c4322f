"""Build libfwmoe.so (hipcc, gfx950) in-tree: every .hip source is compiled to
an object under _build/ and linked into sparse_moe_block_amd/libfwmoe.so."""

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfwmoe.so")
# the peak microbenchmarks (fp16 MFMA, HBM streaming): a library of their own
PEAK_SOURCE = "peak.hip"
PEAK_LIB = os.path.join(PKG, "libfwpeak.so")
SOURCES = ["abi.hip", "route.hip", "permute.hip", "forward.hip", "gemv.hip", "gemm.hip",
           "gemm_mx.hip", "gemm_i8.hip", "layer.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-Wall",
         "-Wno-unused-result", "-I" + os.path.join(ROOT, "include"),
         # no packed fp32 arithmetic anywhere (v_pk_{add,mul,fma}_f32)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # MFMA accumulators in ordinary VGPRs: the unified register file holds
         # them, and the AGPR form made the allocator copy accumulators between
         # register classes inside the K loops
         "-mllvm", "-amdgpu-mfma-vgpr-form"]


def _compile(src):
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    return obj, msg


def build(jobs=None, verbose=False):
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, SOURCES + [PEAK_SOURCE]))
    peak_obj, _ = results.pop()
    for _, msg in results:
        if verbose and msg.strip():
            print(msg, file=sys.stderr)
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp]
                          + [o for o, _ in results])
    os.replace(tmp, LIB)
    tmp = PEAK_LIB + ".tmp"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp,
                           peak_obj])
    os.replace(tmp, PEAK_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
