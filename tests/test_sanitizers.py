"""Host-side AddressSanitizer and UndefinedBehaviorSanitizer runs, CPU only.

1. The oracle (oracle/nm_oracle.c: 320-bit limb arithmetic for the exact pattern scores,
   3-bit metadata fields that straddle words) is built with gcc -fsanitize=address,undefined
   and the oracle's pin suites run against that build in a child process, with gcc's
   sanitizer runtimes preloaded into the interpreter.
2. The C ABI's host code (nm_api.hip: argument checks, pointer-overlap arithmetic, the
   metadata check) is compiled with the same sanitizers on its host side only (its device
   code is unchanged), linked with the library's other objects, and the ABI host tests run
   against that build in a child process with clang's ASan runtime preloaded.

Every report stops the child (halt_on_error / abort_on_error), which fails the test.  No GPU
is used: on a host without one the ABI calls stop at the device check.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "nm_oracle.c")
ORACLE_PINS = ["tests/test_oracle_pins.py", "tests/test_srste_oracle.py",
               "tests/test_tmask_oracle.py", "tests/test_i8_oracle.py",
               "tests/test_perm_oracle.py", "tests/test_fp8_oracle.py"]
ABI_TESTS = ["tests/test_abi_host.py", "tests/test_check_meta.py"]
SAN_ENV = {
    "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
    "UBSAN_OPTIONS": "halt_on_error=1:abort_on_error=1:print_stacktrace=1",
}


def child_env(extra):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(extra)
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    return env


def run_pytest(files, env, timeout):
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
           *files]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "ERROR: AddressSanitizer" not in tail, tail
    assert "runtime error:" not in tail, tail
    return res.stdout


def gcc_runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan, ubsan = gcc_runtime("libasan.so"), gcc_runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = str(tmp_path / "libnm_oracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c99", "-ffp-contract=off", "-fPIC", "-shared",
                           "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", ORACLE_SRC, "-o", lib, "-lm"])
    out = run_pytest(ORACLE_PINS, child_env({"NM_ORACLE_LIB": lib,
                                             "LD_PRELOAD": asan + ":" + ubsan}), timeout=900)
    print(out.splitlines()[-1])


def clang_asan_runtime():
    import glob

    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not available")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    from masking_sparse_gemm_amd import build as b

    rt = clang_asan_runtime()
    if rt is None:
        pytest.skip("clang ASan runtime not installed")
    # the library's other objects, as the normal build leaves them under _build/
    b.build(incremental=True)
    objs = [os.path.join(b.OBJ, os.path.splitext(s)[0] + ".o") for s in b.SOURCES
            if s != "nm_api.hip"]
    api_obj = str(tmp_path / "nm_api_san.o")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                "-Xarch_host", "-g"]
    res = subprocess.run([b.hipcc(), *b.flags(), *host_san, "-c",
                          os.path.join(b.CSRC, "nm_api.hip"), "-o", api_obj],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    lib = str(tmp_path / "libnm_san.so")
    link = ["/opt/rocm/llvm/bin/clang++", "-shared", "-fPIC", "-shared-libsan",
            "-fsanitize=address,undefined", api_obj, *objs, "-L/opt/rocm/lib", "-lamdhip64",
            "-Wl,-rpath,/opt/rocm/lib", "-o", lib]
    res = subprocess.run(link, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    out = run_pytest(ABI_TESTS, child_env({"NM_LIB_PATH": lib, "LD_PRELOAD": rt}), timeout=900)
    print(out.splitlines()[-1])
