"""Build libhca.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m decode_attention_compressed_amd.build [--jobs N]

Each .hip source is compiled to an object with hipcc, in parallel, then linked
into decode_attention_compressed_amd/libhca.so.
"""

import argparse
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libhca.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


# per-source extra flags: the indexer and the attention keep MFMA results in
# VGPRs.  The indexer's accumulators are small, and this saves AGPR-to-VGPR
# copies on every tile.  The attention's output accumulator is rescaled by
# VALU code and carried around the tile loop; in AGPRs it was copied out and
# back on every tile.
EXTRA = {"indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "compress.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout)
        raise RuntimeError("hipcc failed")
    return r.stdout


def build(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        outs = list(ex.map(lambda so: _run([HIPCC, *FLAGS, *EXTRA.get(os.path.basename(so[0]), []), "-c", so[0], "-o", so[1]]),
                           zip(srcs, objs)))
    if verbose:
        for o in outs:
            if o.strip():
                sys.stdout.write(o)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args()
    print(build(args.jobs, args.verbose))
