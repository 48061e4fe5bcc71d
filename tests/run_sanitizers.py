"""Host-code sanitizer run: AddressSanitizer + UndefinedBehaviorSanitizer
builds of the CPU oracle (gcc) and of libaq's host code (hipcc, the flags
given to the host pass only), then the CPU tests against them.

    python tests/run_sanitizers.py

The two libraries use different sanitizer runtimes (gcc's and clang's), so
the oracle's tests and the C-ABI tests run in two pytest processes, each
with its runtime preloaded into the (uninstrumented) Python interpreter.
Device code is built as usual; sanitizers are not available for it.  Exit
status: 0 when both runs pass.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def build_oracle() -> str:
    lib = os.path.join(OUT, "liboracle.so")
    subprocess.check_call(
        ["gcc", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-Wall",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
         "-fno-omit-frame-pointer", "-shared", "-fPIC", os.path.join(ROOT, "oracle", "aq_oracle.c"),
         "-o", lib, "-lm"])
    return lib


def build_libaq() -> str:
    sys.path.insert(0, ROOT)
    from group_wise_affine_aq_amd import build as aqbuild
    objs = []
    for src in aqbuild.SOURCES:
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *aqbuild.CFLAGS, *SAN_HOST, "-x", "hip", "-c",
               os.path.join(aqbuild.CSRC, src), "-o", obj]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        objs.append(obj)
    lib = os.path.join(OUT, "libaq.so")
    subprocess.check_call([HIPCC, f"--offload-arch={aqbuild.ARCH}", "-shared", "-fPIC", *SAN_HOST,
                           *objs, "-o", lib])
    return lib


def run(tests, env_extra) -> int:
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
           *tests]
    print("+", " ".join(f"{k}={v}" for k, v in env_extra.items()), " ".join(cmd), flush=True)
    return subprocess.call(cmd, cwd=ROOT, env=env)


def main() -> int:
    os.makedirs(OUT, exist_ok=True)
    oracle_lib = build_oracle()
    aq_lib = build_libaq()
    gcc_asan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    gcc_ubsan = subprocess.check_output(["gcc", "-print-file-name=libubsan.so"], text=True).strip()
    clang_rt = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/"
                                "libclang_rt.asan-x86_64.so"))
    if not clang_rt:
        print("clang's AddressSanitizer runtime not found", file=sys.stderr)
        return 1
    oracle_tests = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    rc1 = run(oracle_tests, {"AQ_ORACLE_LIB": oracle_lib,
                             "LD_PRELOAD": f"{gcc_asan}:{gcc_ubsan}"})
    rc2 = run([os.path.join(ROOT, "tests", "test_abi.py")],
              {"AQ_LIB": aq_lib, "LD_PRELOAD": clang_rt[-1]})
    print(f"sanitized runs: oracle tests rc={rc1}, C-ABI tests rc={rc2}")
    return 0 if rc1 == 0 and rc2 == 0 else 1


if __name__ == "__main__":
    sys.exit(main())
