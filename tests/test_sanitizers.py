"""Host-side sanitizer runs (CPU only): the C ABI's argument checks and the
fp64 oracle, each built with AddressSanitizer and UndefinedBehaviorSanitizer
(-fno-sanitize-recover, so any report fails), exercised by the existing CPU
tests in a subprocess that loads the sanitized builds.

* lam_api.cpp (validation, planning, workspace checks) is compiled with
  clang++ -fsanitize=address,undefined and linked with the regular objects of
  the kernel sources (whose host parts only size and launch); the subprocess
  runs tests/test_abi.py against it (LAM_LIBRARY), with clang's ASan runtime
  preloaded.  No call in those tests reaches a kernel launch.
* oracle/lam_oracle.c is compiled with gcc -fsanitize=address,undefined in
  both precisions; the subprocess runs the oracle pins and the golden
  fixtures against it (LAM_ORACLE_LIB, LAM_ORACLE_LIB_F32), with gcc's ASan
  runtime preloaded.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, env=None):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, cwd=ROOT)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def _clang_asan_runtime():
    hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return hits[0] if hits else None


def test_abi_checks_under_asan_ubsan():
    rt = _clang_asan_runtime()
    if not (os.path.exists(CLANG) and rt):
        pytest.skip("clang++ with its ASan runtime not installed")
    from gated_linear_attention_chunked_amd import build

    build.build()  # the regular kernel objects under _build/lam
    os.makedirs(OUT, exist_ok=True)
    csrc = os.path.join(ROOT, "gated_linear_attention_chunked_amd", "csrc")
    obj = os.path.join(OUT, "lam_api.o")
    _run([CLANG, "-std=c++17", "-O1", "-g", "-fPIC", *SAN, "-D__HIP_PLATFORM_AMD__",
          "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", csrc,
          "-c", os.path.join(csrc, "lam_api.cpp"), "-o", obj])
    kernels = [o for o in glob.glob(os.path.join(build.BUILD, "*.o")) if not o.endswith("lam_api.o")]
    lib = os.path.join(OUT, "liblam_asan.so")
    _run([CLANG, "-shared", "-fPIC", *SAN, "-shared-libsan", obj, *kernels, "-L", "/opt/rocm/lib",
          "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", lib])
    env = dict(os.environ, LD_PRELOAD=rt, LAM_LIBRARY=lib, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = _run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider", "tests/test_abi.py",
              "-k", "not binding_fails_loudly"], env=env)
    assert " passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]


def test_oracle_pins_under_asan_ubsan():
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not installed")
    rt = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(rt):
        pytest.skip("gcc's ASan runtime not installed")
    os.makedirs(OUT, exist_ok=True)
    src = os.path.join(ROOT, "oracle", "lam_oracle.c")
    libs = {}
    for prec, real in (("f64", "double"), ("f32", "float")):
        libs[prec] = os.path.join(OUT, f"liblam_oracle_{prec}_asan.so")
        _run([gcc, "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", *SAN,
              f"-DLAM_ORACLE_REAL={real}", src, "-o", libs[prec], "-lm"])
    env = dict(os.environ, LD_PRELOAD=rt, LAM_ORACLE_LIB=libs["f64"], LAM_ORACLE_LIB_F32=libs["f32"],
               ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               OMP_NUM_THREADS="4")
    r = _run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider", "tests/test_oracle_pins.py",
              "tests/test_golden.py", "tests/test_oracle_vla_ratio.py"], env=env)
    assert " passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]
