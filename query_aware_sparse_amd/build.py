"""Build libqas.so in-tree with hipcc for gfx950.

    python -m query_aware_sparse_amd.build [-v]

Each translation unit under csrc/ is compiled separately (in parallel) into
_build/, then linked into query_aware_sparse_amd/libqas.so.  hipcc
cross-compiles for gfx950 without a GPU.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libqas.so")
MICRO_LIB = os.path.join(HERE, "libqas_micro.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed fp32 instructions are left to the compiler's discretion nowhere:
# the feature is switched off for all device code.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]

SOURCES = ["qas_api.cpp", "append.hip", "append_fp8.hip", "score.hip", "topk.hip", "decode.hip", "decode_f32.hip",
           "decode_f16.hip", "decode_bf16.hip", "union.hip", "regroup.hip", "topr.hip"]
# measurement kernels of bench.py --micro, in a library of their own
MICRO_SOURCES = ["microbench.hip"]


def _compile(src, verbose):
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src.rsplit(".", 1)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    if verbose and res.stderr.strip():
        print(res.stderr, file=sys.stderr)
    return obj


def _link(objs, out, verbose):
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)


def build(verbose=False):
    """Compile every HIP source, link libqas.so and the measurement library
    libqas_micro.so (bench.py --micro); returns the libqas.so path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + MICRO_SOURCES
    jobs = min(len(srcs), max(1, (os.cpu_count() or 2)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs[:len(SOURCES)], LIB, verbose)
    _link(objs[len(SOURCES):], MICRO_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
