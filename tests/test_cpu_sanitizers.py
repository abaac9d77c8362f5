"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Builds a copy of libchs.so whose host code (argument checks, workspace sizing, launch set-up) is
instrumented with ASan and UBSan (the device code is compiled as usual and never runs here), and a
copy of the oracle (oracle.c) instrumented the same way, then runs the C-ABI contract tests and the
oracle pins against those copies in a child process with the sanitizer runtime preloaded. Any
sanitizer report fails the test: UBSan is set to stop at the first error, ASan stops by default.
Leak checking is off (the Python interpreter itself is not instrumented and keeps memory to exit).
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
RUNTIME = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
# Each sanitizer flag of a hipcc line applies to the host pass only.
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-shared-libsan", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(not (shutil.which(HIPCC) or os.path.exists(HIPCC)) or not os.path.exists(CLANG) or not RUNTIME,
                    reason="the ROCm toolchain or its sanitizer runtime is missing")
def test_contract_and_oracle_pins_run_clean_under_asan_ubsan(tmp_path):
    srcs = sorted(glob.glob(os.path.join(ROOT, "compressed_hybrid_sparse_amd", "csrc", "*.hip")))
    procs, objs = [], []
    for src in srcs:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
               "-Xclang", "-packed-fp32-ops", *HOST_SAN, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
        procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True), cmd))
        objs.append(obj)
    for p, cmd in procs:
        out, err = p.communicate()
        assert p.returncode == 0, f"{' '.join(cmd)}\n{err[-4000:]}"
    lib = str(tmp_path / "libchs_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SAN, *objs, "-o", lib])
    olib = str(tmp_path / "liboracle_san.so")
    _run([CLANG, "-std=c11", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
          "-fsanitize=address,undefined", "-shared-libsan", "-fno-omit-frame-pointer",
          os.path.join(ROOT, "oracle", "oracle.c"), "-o", olib, "-lm"])

    env = dict(os.environ)
    env.update(LD_PRELOAD=RUNTIME[-1], ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", CHS_LIB=lib, CHS_ORACLE_LIB=olib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_api_contract.py"),
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=str(tmp_path), env=env, capture_output=True, text=True, timeout=900)
    text = r.stdout + r.stderr
    assert r.returncode == 0, text[-6000:]
    for marker in ("runtime error", "AddressSanitizer", "UndefinedBehaviorSanitizer"):
        assert marker not in text, text[-6000:]
    assert " passed" in text
