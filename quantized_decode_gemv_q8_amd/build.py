"""Builds libq8gemv.so in-tree with hipcc for gfx950 (no GPU needed).

    python -m quantized_decode_gemv_q8_amd.build
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libq8gemv.so")

# The matvec instances are split by VEC so that they compile in parallel.
SOURCES = ["q8_gemv_v16.hip", "q8_gemv_v8.hip", "q8_gemv_v4.hip", "q8_gemv_v2.hip", "q8_gemv_v1.hip",
           "q8_gemv.hip", "q8_gemm.hip", "dense_f32.hip", "dot_t.hip", "q8_api.hip"]

ARCH = "gfx950"
# No fast-math or flush-to-zero flags.  Packed fp32 instructions are disabled
# (the compiler would otherwise form v_pk_fma_f32 from scalar code).
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-source additions.  The matrix-core product keeps its MFMA results in
# ordinary VGPRs (the scale FMAs read every result; with accumulation
# registers each read would need an extra copy instruction).
EXTRA_FLAGS = {"q8_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _hipcc():
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return cand


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *HIP_FLAGS, *EXTRA_FLAGS.get(src, []), "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src),
           "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose=False):
    """Compiles every HIP source and links libq8gemv.so next to this file."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
