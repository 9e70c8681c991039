"""Host-side sanitizer builds of libmt.so, run under the CPU tests.

``python -m layer_streaming_amd.sanitize thread|address [pytest arguments]``

builds a copy of the library whose host C++ sources (the runtime, the thread
pool, the host Adam and accumulation, the seeded init, the shard files and
the ABI) are compiled with clang's ThreadSanitizer or AddressSanitizer and
linked with the ordinary gfx950 kernel objects, then runs pytest on the CPU
tests (``tests/test_host.py`` unless other arguments are given) in a child
process that preloads the sanitizer runtime and loads that copy through the
``MT_LIBRARY`` variable.  The GPU kernels are not instrumented, and without a
GPU only the host paths the CPU tests reach run: argument validation, layout
and workspace sizing, the thread pool under the host Adam, accumulation and
init.  The exit status is pytest's; a sanitizer report makes it non-zero.

The sanitized host objects are compiled by clang++ itself, not by the HIP
compiler driver, so the instrumentation reaches host code only.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

from . import build as B

CLANGXX = os.path.join(B.ROCM, "llvm", "bin", "clang++")
KINDS = ("thread", "address")


def _runtime(kind):
    d = os.path.join(B.ROCM, "llvm", "lib", "clang")
    for ver in sorted(os.listdir(d), reverse=True):
        p = os.path.join(d, ver, "lib", "linux", f"libclang_rt.{'tsan' if kind == 'thread' else 'asan'}-x86_64.so")
        if os.path.exists(p):
            return p
    raise FileNotFoundError(f"no {kind} sanitizer runtime under {d}")


def build_sanitized(kind, verbose=True):
    """Compile the host sources with the sanitizer, reuse (or build) the kernel
    objects, and link ``_build/san_<kind>/libmt.so``.  Returns its path."""
    if kind not in KINDS:
        raise ValueError(f"sanitizer must be one of {KINDS}")
    out_dir = os.path.join(B.BUILD, f"san_{kind}")
    os.makedirs(out_dir, exist_ok=True)
    san = [f"-fsanitize={kind}", "-fno-omit-frame-pointer", "-g", "-O1"]
    host_flags = [f for f in B.CXX_FLAGS if f != "-x" and f != "c++"]

    def compile_host(src):
        obj = os.path.join(out_dir, src + ".o")
        cmd = [CLANGXX, "-x", "c++", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
               "-Wno-unused-variable"] + host_flags + san + ["-c", os.path.join(B.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        return obj

    def kernel_obj(src):
        # the product build's object when it is newer than every source and header
        obj = os.path.join(B.BUILD, src + ".o")
        newest = max(os.path.getmtime(os.path.join(B.CSRC, f)) for f in os.listdir(B.CSRC))
        if os.path.exists(obj) and os.path.getmtime(obj) >= newest:
            return obj
        return B._compile(src, B.HIP_FLAGS)

    os.makedirs(B.BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        host_objs = list(ex.map(compile_host, B.CXX_SOURCES))
        kern_objs = list(ex.map(kernel_obj, B.HIP_SOURCES))
    lib = os.path.join(out_dir, "libmt.so")
    cmd = [CLANGXX, "-shared", "-fPIC", f"-fsanitize={kind}", "-o", lib] + kern_objs + host_objs + \
        ["-pthread", f"-L{B.ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{B.ROCM}/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {lib}", flush=True)
    return lib


def run_tests(kind, pytest_args=None, lib=None):
    """Run pytest on the CPU tests against the sanitized library; returns
    (exit status, combined output)."""
    lib = lib or build_sanitized(kind)
    root = os.path.dirname(B.HERE)
    env = dict(os.environ)
    env["MT_LIBRARY"] = lib
    env["LD_PRELOAD"] = _runtime(kind)
    if kind == "thread":
        env["TSAN_OPTIONS"] = "halt_on_error=0 exitcode=66 second_deadlock_stack=1"
    else:
        # the interpreter itself keeps memory to exit; leaks are not what this run is for
        env["ASAN_OPTIONS"] = "detect_leaks=0 halt_on_error=1 exitcode=67"
    args = pytest_args or [os.path.join(root, "tests", "test_host.py")]
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu"] + list(args)
    r = subprocess.run(cmd, cwd=root, env=env, capture_output=True, text=True)
    out = r.stdout + r.stderr
    status = r.returncode
    if status == 0 and ("ThreadSanitizer" in out or "AddressSanitizer" in out):
        status = 1
    return status, out


def main(argv):
    if not argv or argv[0] not in KINDS:
        print(f"usage: python -m layer_streaming_amd.sanitize {{{'|'.join(KINDS)}}} [pytest arguments]")
        return 2
    status, out = run_tests(argv[0], argv[1:])
    sys.stdout.write(out)
    return status


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
