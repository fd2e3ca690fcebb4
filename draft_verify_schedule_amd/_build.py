"""Build libdspark.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIBNAME = "libdspark.so"
SOURCES = ["draft.hip", "schedule.hip", "verify.hip", "confidence.hip", "rnn.hip", "rng.hip", "api.cpp"]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 arithmetic.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-ffp-contract=fast",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics", "-Wno-unused-command-line-argument"]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: cannot build libdspark")
    return exe


def lib_path():
    return os.path.join(LIBDIR, LIBNAME)


def build_library(verbose=False):
    os.makedirs(LIBDIR, exist_ok=True)
    objdir = os.path.join(LIBDIR, "obj")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(objdir, src.rsplit(".", 1)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc] + HIP_FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("compile failed: %s\n%s%s" % (" ".join(cmd), res.stdout, res.stderr))
        if verbose and res.stderr.strip():
            print(res.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as pool:
        objs = list(pool.map(compile_one, SOURCES))
    tmp = lib_path() + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed: %s\n%s%s" % (" ".join(cmd), res.stdout, res.stderr))
    os.replace(tmp, lib_path())
    return lib_path()


if __name__ == "__main__":
    print(build_library(verbose=True))
