"""Build libpkv.so in-tree for gfx950 with hipcc (no GPU needed to compile)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpkv.so")
SOURCES = [os.path.join(CSRC, f) for f in ("pkv_host.cpp", "pkv_decode.hip", "pkv_decode_mfma.hip",
                                           "pkv_decode_group.hip", "pkv_noalloc.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed-FP32 VALU ops stay off (see the design notes)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    """Compile every HIP/C++ source of the library (in parallel) and link
    paged_kv_split_amd/libpkv.so."""
    from concurrent.futures import ThreadPoolExecutor
    tag = "%d" % os.getpid()
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = [os.path.join(CSRC, os.path.basename(s) + ".%s.o" % tag) for s in SOURCES]
    cflags = [f for f in FLAGS if f != "-shared"]
    try:
        with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
            list(ex.map(lambda so: _run([HIPCC, *cflags, *inc, "-c", so[0], "-o", so[1]], verbose),
                        zip(SOURCES, objs)))
        tmp = LIB + ".tmp" + tag
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
