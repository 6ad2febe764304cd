"""CPU hygiene: the host half of libiqnn.so and the CPU oracle built with
AddressSanitizer and UndefinedBehaviorSanitizer, and the CPU test suite
(pytest -m "not gpu") run against them.

Host code only: on every hipcc line each sanitizer flag follows -Xarch_host, so no
GPU code is built with a sanitizer; the device code is the same as in libiqnn.so.
The oracle is built with clang (one sanitizer runtime for both libraries), without
OpenMP.  The libraries go to _build_san/ and oracle/_build_san/; the test run
preloads clang's ASan runtime and points the loaders at them through IQNN_LIB and
IQO_LIB.  A CPU-only tool: it is never run on a GPU.

    python -m integer_quantized_nn_amd.build_sanitized          # build + run the suite
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

from integer_quantized_nn_amd import build as B

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
BUILD = os.path.join(B.HERE, "_build_san")
LIB = os.path.join(BUILD, "libiqnn_san.so")
ORACLE_DIR = os.path.join(B.ROOT, "oracle")
ORACLE_LIB = os.path.join(ORACLE_DIR, "_build_san", "libiqo_san.so")
CLANG = "/opt/rocm/llvm/bin/clang"


def _host_only(flags):
    out = []
    for f in flags:
        out += ["-Xarch_host", f]
    return out


def asan_runtime():
    libs = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not libs:
        raise RuntimeError("clang's ASan runtime (libclang_rt.asan-x86_64.so) not found under /opt/rocm/llvm")
    return libs[-1]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [B.HIPCC, *B.FLAGS, *_host_only(SAN), "-x", "hip", "-c", os.path.join(B.CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stdout + r.stderr))
    return obj


def build():
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(B.SOURCES)) as ex:
        objs = list(ex.map(_compile, B.SOURCES))
    # the sanitizer runtime is not linked in: the preloaded one resolves its symbols
    subprocess.run([B.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB], check=True)
    os.makedirs(os.path.dirname(ORACLE_LIB), exist_ok=True)
    subprocess.run([CLANG, "-std=c11", "-O1", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
                    "-frounding-math", *SAN, os.path.join(ORACLE_DIR, "iqo.c"), "-o", ORACLE_LIB, "-lm"], check=True)
    return LIB, ORACLE_LIB


def run_tests(extra=()):
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan_runtime()
    # Python and torch are not instrumented: their allocations are not leaks of ours
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["IQNN_LIB"] = LIB
    env["IQO_LIB"] = ORACLE_LIB
    cmd = [sys.executable, "-m", "pytest", os.path.join(B.ROOT, "tests"), "-q", "-x", "-m", "not gpu",
           "-p", "no:cacheprovider", *extra]
    return subprocess.run(cmd, env=env, cwd=B.ROOT).returncode


if __name__ == "__main__":
    build()
    sys.exit(run_tests(sys.argv[1:]))
