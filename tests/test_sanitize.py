"""Host-side sanitizer runs (CPU only).

- The oracle (oracle/dsa_oracle.c) is built with AddressSanitizer and
  UndefinedBehaviorSanitizer together with tests/sanitize/oracle_driver.c,
  which calls every oracle entry point on small ragged inputs with several
  threads: an out-of-bounds access, a leak or undefined behaviour aborts it.
- The C ABI's host code (argument validation, workspace arithmetic, the
  batch-descriptor checks) is built with the same sanitizers on its host
  side (device code as usual) and tests/test_abi.py runs against that
  build, with the sanitizer runtime preloaded into the test interpreter.
  A grid of extreme sizes goes through every workspace-size function.
"""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from long_context_sparse_dsa_amd import build as B  # noqa: E402

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV_SAN = {"ASAN_OPTIONS": "detect_leaks=0:detect_odr_violation=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.fixture(scope="module")
def work(tmp_path_factory):
    return str(tmp_path_factory.mktemp("sanitize"))


def test_oracle_under_address_and_ub_sanitizers(work):
    exe = os.path.join(work, "oracle_driver")
    cmd = ["gcc", "-O1", "-g", *SAN, "-fno-omit-frame-pointer", "-ffp-contract=off", "-pthread",
           os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
           os.path.join(ROOT, "oracle", "dsa_oracle.c"), "-o", exe, "-lm"]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS=ENV_SAN["UBSAN_OPTIONS"])
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "oracle driver ok" in r.stdout
    assert "runtime error" not in r.stderr


def _compile_sanitized(args):
    src, obj = args
    # sanitizers on the host side only; the device code is built as usual
    cmd = [B.HIPCC, "-x", "hip", f"--offload-arch={B.ARCH}", "-O1", "-std=c++17", "-fPIC",
           "-I", B.INCLUDE, "-I", B.CSRC, "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-Xarch_host", SAN[0], "-Xarch_host", SAN[1],
           "-Xarch_host", "-fno-omit-frame-pointer", "-c", os.path.join(B.CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-3000:]}")
    return obj


def test_abi_host_code_under_address_and_ub_sanitizers(work):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime in this ROCm install")
    jobs = [(s, os.path.join(work, os.path.splitext(s)[0] + ".o")) for s in B.SOURCES]
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(_compile_sanitized, jobs))
    lib = os.path.join(work, "libdsa_sanitized.so")
    cmd = [B.HIPCC, "-shared", "-fPIC", f"--offload-arch={B.ARCH}", "-Xarch_host", SAN[0],
           "-Xarch_host", "-shared-libsan", *objs, "-o", lib]
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, DSA_LIBRARY=lib, LD_PRELOAD=rt, **ENV_SAN)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "runtime error" not in r.stderr
