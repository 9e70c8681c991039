"""Build libmt.so in-tree: HIP kernels for gfx950 plus the host runtime.

Run ``python -m layer_streaming_amd.build`` (or ``__graft_entry__.build()``).
Every HIP source is compiled with ``--offload-arch=gfx950`` and packed FP32
instructions disabled; host C++ sources are compiled by the same clang with
the HIP runtime headers.  Objects are built in parallel and linked into
``layer_streaming_amd/libmt.so``.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmt.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

HIP_SOURCES = ["gemm.hip", "gemm_nt.hip", "attention.hip", "elementwise.hip"]
CXX_SOURCES = ["host.cpp", "shard.cpp", "engine.cpp", "abi.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]
HIP_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# host code: no FMA contraction, so the scalar and vector forms of the host
# Adam round identically
CXX_FLAGS = ["-x", "c++", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", "-march=x86-64-v3",
             "-ffp-contract=off", "-pthread"]


def _compile(src, flags):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(s, HIP_FLAGS) for s in HIP_SOURCES] + [(s, CXX_FLAGS) for s in CXX_SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs + \
        ["-pthread", f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
