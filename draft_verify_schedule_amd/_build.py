"""Build libdspark.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

The library carries the hash of the sources it was built from
(dspark_build_id()); source_hash() computes the same hash from the tree, so
a loader can tell a library built from other sources from the current one.
"""
import hashlib
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
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


def source_files():
    """Every file the library is built from: csrc/* and include/*, sorted."""
    files = []
    for d in (CSRC, INCLUDE):
        for name in sorted(os.listdir(d)):
            p = os.path.join(d, name)
            if os.path.isfile(p) and name.endswith((".hip", ".cpp", ".hpp", ".h")):
                files.append(p)
    return files


def source_hash():
    """16 hex digits of SHA-256 over the sources (names and contents) and the flags."""
    h = hashlib.sha256()
    for p in source_files():
        h.update(os.path.relpath(p, ROOT).encode())
        h.update(b"\0")
        with open(p, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    h.update(" ".join(HIP_FLAGS).encode())
    return h.hexdigest()[:16]


def build_library(verbose=False):
    os.makedirs(LIBDIR, exist_ok=True)
    objdir = os.path.join(LIBDIR, "obj")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    build_id = source_hash()

    def compile_one(src):
        obj = os.path.join(objdir, src.rsplit(".", 1)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        defs = ['-DDSPARK_BUILD_ID="%s"' % build_id] if src == "api.cpp" else []
        cmd = [cc] + HIP_FLAGS + defs + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("compile failed: %s\n%s%s" % (" ".join(cmd), res.stdout, res.stderr))
        if verbose and res.stderr.strip():
            print(res.stderr)
        return obj

    # the largest translation units first, so the pool finishes together
    order = sorted(SOURCES, key=lambda s: -os.path.getsize(os.path.join(CSRC, s)))
    with ThreadPoolExecutor(max_workers=min(6, len(SOURCES))) as pool:
        objs = dict(zip(order, pool.map(compile_one, order)))
    tmp = lib_path() + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [objs[s] for s in SOURCES]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed: %s\n%s%s" % (" ".join(cmd), res.stdout, res.stderr))
    os.replace(tmp, lib_path())
    return lib_path()


def built_id(path=None):
    """The build id a library file carries (read from its bytes, without
    loading it), or None when the file is absent or carries none."""
    path = path or lib_path()
    if not os.path.exists(path):
        return None
    marker = b"dspark-build-id:"
    with open(path, "rb") as f:
        data = f.read()
    i = data.find(marker)
    if i < 0:
        return None
    return data[i + len(marker):i + len(marker) + 16].decode("ascii", "replace")


def is_current(path=None):
    """True when the library exists and was built from the current sources."""
    return built_id(path) == source_hash()


if __name__ == "__main__":
    print(build_library(verbose=True))
