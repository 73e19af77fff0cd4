"""Build libwringer.so (gfx950) from the HIP sources in this directory.

Each source is compiled to an object under ``_build/`` in parallel, then linked
into ``post_bit_weight_amd/libwringer.so``.  Always recompiles.
"""
import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
OUT = os.path.join(PKG, "libwringer.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]


def _compile(src, obj):
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l and "(ignoring feature)" not in l)
    return r.returncode, " ".join(cmd), err


def build(verbose=True):
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(HERE, "*.hip")))
    objs = [os.path.join(bdir, os.path.basename(s) + ".o") for s in srcs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs, objs))
    failed = False
    for (rc, cmd, err), src in zip(results, srcs):
        if err.strip() and verbose:
            print(f"[{os.path.basename(src)}]\n{err}", file=sys.stderr)
        if rc != 0:
            failed = True
            print(f"compile failed: {cmd}", file=sys.stderr)
    if failed:
        raise RuntimeError("HIP compilation failed")
    tmp = OUT + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
