"""Build libddtree.so (HIP, gfx950) in place: one object per source, then link.

    python -m tree_verification_ddtree_amd.build [--jobs N]
"""
import argparse
import concurrent.futures as cf
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libddtree.so")
SOURCES = ["plan.hip", "conv.hip", "gdn.hip", "attn.hip", "walk.hip", "commit.hip", "draft.hip", "fused.hip", "sample.hip",
           "host.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")
# the host-only part of the library (plain C++, no HIP)
CXXFLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-I" + os.path.join(ROOT, "include")]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"),
    # packed fp32 math off (v_pk_*_f32): only plain fp32 VALU ops are emitted
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the first 16 argument dwords of a kernel (scalars and pointers only)
    # arrive preloaded in scalar registers instead of being fetched
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]


def source_files():
    """The files a build reads: the C header and every file of csrc/, in name order."""
    files = [os.path.join(ROOT, "include", "ddtree.h")]
    files += [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC))]
    return files


def source_hash():
    """sha256 of the sources, as "<path relative to the repository>\\0<bytes>"
    records in name order; the library reports the value it was built with
    (ddt_source_hash), so a caller can tell which sources a binary came from."""
    h = hashlib.sha256()
    for f in source_files():
        h.update(os.path.relpath(f, ROOT).replace(os.sep, "/").encode() + b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _compile(src, src_hash):
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    if src.endswith(".cpp"):
        cmd = [CXX, *CXXFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    else:
        cmd = [HIPCC, *FLAGS, f'-DDDT_SOURCE_HASH="{src_hash}"', "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    return obj, msgs


def build(jobs=None, verbose=False):
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 16)
    h = source_hash()
    with cf.ThreadPoolExecutor(jobs) as ex:
        res = list(ex.map(lambda f: _compile(f, h), SOURCES))
    for _, m in res:
        if m.strip() and verbose:
            print(m)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in res]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose))
    sys.exit(0)
