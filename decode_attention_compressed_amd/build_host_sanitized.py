"""Build libhca with AddressSanitizer and UndefinedBehaviorSanitizer on its
host code (validation, planning, the page pool, the host encoders) and run the
CPU tests against it.  The device code is compiled as usual: the sanitizers
instrument the host pass only.

    python -m decode_attention_compressed_amd.build_host_sanitized [--no-test]

The library goes to _build/host_sanitized/libhca.so; the tests load it through
HCA_LIB with the ASan runtime preloaded into the interpreter (which is not
itself instrumented, so leak checking is off).
"""

import argparse
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

from decode_attention_compressed_amd import build as B

OUT = os.path.join(B.ROOT, "_build", "host_sanitized")
LIB = os.path.join(OUT, "libhca.so")
SAN = ["-Xarch_host -fsanitize=address", "-Xarch_host -fsanitize=undefined",
       "-Xarch_host -fno-sanitize-recover=undefined", "-Xarch_host -fno-omit-frame-pointer", "-Xarch_host -g"]
SAN_FLAGS = [f for pair in SAN for f in pair.split(" ")]
TESTS = ["tests/test_abi_cpu.py", "tests/test_pool_cpu.py"]


def asan_runtime() -> str:
    r = subprocess.run([os.path.join(os.path.dirname(B.HIPCC), "..", "lib", "llvm", "bin", "clang"),
                        "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the ASan runtime of the ROCm clang was not found")
    return path


def build(jobs: int) -> str:
    os.makedirs(OUT, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(B.CSRC, "*.hip")))
    objs = [os.path.join(OUT, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        list(ex.map(lambda so: B._run([B.HIPCC, *B.FLAGS, *SAN_FLAGS, *B.EXTRA.get(os.path.basename(so[0]), []),
                                       "-c", so[0], "-o", so[1]]), zip(srcs, objs)))
    B._run([B.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN_FLAGS, "-o", LIB, *objs])
    return LIB


def run_tests() -> int:
    env = dict(os.environ, HCA_LIB=LIB, LD_PRELOAD=asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *TESTS],
                          cwd=B.ROOT, env=env).returncode


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--no-test", action="store_true")
    args = ap.parse_args()
    print(build(args.jobs))
    if not args.no_test:
        sys.exit(run_tests())
