"""CPU sanitizer runs: AddressSanitizer + UndefinedBehaviorSanitizer over the host code.

* The C ABI's host validation (osc_api.hip) is rebuilt with the sanitizers on its host pass only
  (each -fsanitize= behind -Xarch_host: the GPU code is the ordinary build) and linked with the
  library's other objects; tests/test_abi.py then runs against it in a child process with the
  compiler's ASan runtime preloaded.  No kernel is launched: every call there is rejected by
  validation.
* The oracle (osc_oracle.c) is rebuilt with gcc's sanitizers and the oracle pin suites run against
  it the same way.

Any report aborts the child (halt_on_error / abort_on_error), so a clean exit is a clean run."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG_BUILD = os.path.join(ROOT, "w4a4_outlier_split_amd", "_build")
CSRC = os.path.join(ROOT, "w4a4_outlier_split_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def run_child(tests, preload, extra_env, tmp_path):
    env = dict(os.environ, **SAN_ENV, **extra_env, LD_PRELOAD=preload)
    log = tmp_path / "child.log"
    with open(log, "w") as f:
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu",
                            *tests], cwd=ROOT, env=env, stdout=f, stderr=subprocess.STDOUT, timeout=900)
    text = log.read_text()
    assert r.returncode == 0, f"sanitized run failed (exit {r.returncode}):\n{text[-6000:]}"
    assert "runtime error" not in text and "AddressSanitizer" not in text, text[-6000:]


def test_host_validation_under_sanitizers(tmp_path):
    objs = [os.path.join(PKG_BUILD, f) for f in ("osc_quant.o", "osc_gemm.o", "osc_gemm_mx4.o", "osc_gemm_dec.o")]
    if not os.path.exists(HIPCC) or not all(os.path.exists(o) for o in objs):
        pytest.skip("needs hipcc and the library's objects (python w4a4_outlier_split_amd/build.py)")
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rt:
        pytest.skip("no clang ASan runtime")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    api = str(tmp_path / "osc_api_san.o")
    lib = str(tmp_path / "libosc_san.so")
    subprocess.run([HIPCC, "-std=c++17", "-O1", "-g", "-fPIC", "--offload-arch=gfx950",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, "osc_api.hip"),
                    "-o", api], check=True, capture_output=True)
    subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", api, *objs, "-o", lib], check=True,
                   capture_output=True)
    run_child(["tests/test_abi.py"], rt[0], {"OSC_LIBRARY": lib}, tmp_path)


def test_oracle_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("no gcc ASan runtime")
    lib = str(tmp_path / "liboscoracle_san.so")
    subprocess.run([gcc, "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    os.path.join(ROOT, "oracle", "osc_oracle.c"), "-o", lib, "-lm"], check=True, capture_output=True)
    tests = sorted(os.path.relpath(p, ROOT) for p in glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    run_child(tests, asan, {"OSC_ORACLE_LIBRARY": lib}, tmp_path)
