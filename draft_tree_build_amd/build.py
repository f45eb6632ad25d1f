"""Build libddtree.so (HIP, gfx950) in-tree with hipcc.

    python -m draft_tree_build_amd.build

Every source is compiled for gfx950 with FMA contraction off (the draft-tree
arithmetic is specified operation by operation) and packed-fp32 instructions
disabled; the objects are linked into draft_tree_build_amd/libddtree.so.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libddtree.so")
SOURCES = ["abi.hip", "k_build.hip", "k_tree.hip", "k_attn.hip", "k_accept.hip", "k_commit.hip",
           "k_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


# The row kernels keep a whole row in registers and visit it in fully
# unrolled loops; their bodies exceed LLVM's default size limit for a forced
# unroll, and a loop left rolled would index the register copy dynamically
# (moving it to scratch memory).
EXTRA = {"k_build.hip": ["-mllvm", "-pragma-unroll-threshold=200000"]}


def _compile(src: str, obj: str) -> None:
    cmd = [HIPCC] + FLAGS + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on %s" % src)


def build(verbose: bool = False) -> str:
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(6, len(SOURCES))) as ex:
        list(ex.map(lambda so: _compile(*so), zip(SOURCES, objs)))
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libddtree.so failed")
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
