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
DEBUG_LIB = os.path.join(PKG, "libhca_debug.so")  # the same kernels with the index checks (-DHCA_DEBUG)
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


def build(jobs: int = 8, verbose: bool = False, debug: bool = False) -> str:
    """Build libhca.so, or with debug the same kernels with the index checks (-DHCA_DEBUG) as libhca_debug.so."""
    out_dir = os.path.join(BUILD, "debug") if debug else BUILD
    lib = DEBUG_LIB if debug else LIB
    flags = FLAGS + (["-DHCA_DEBUG"] if debug else [])
    os.makedirs(out_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(out_dir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        outs = list(ex.map(lambda so: _run([HIPCC, *flags, *EXTRA.get(os.path.basename(so[0]), []), "-c", so[0], "-o", so[1]]),
                           zip(srcs, objs)))
    if verbose:
        for o in outs:
            if o.strip():
                sys.stdout.write(o)
    tmp = lib + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--debug", action="store_true", help="also build libhca_debug.so (the index-checked kernels)")
    args = ap.parse_args()
    print(build(args.jobs, args.verbose))
    if args.debug:
        print(build(args.jobs, args.verbose, debug=True))
