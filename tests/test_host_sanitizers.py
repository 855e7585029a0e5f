"""The C ABI's validation and sizing (api.cpp, workspace.cpp) and the host
block manager (block_manager.cpp) built with AddressSanitizer and
UndefinedBehaviorSanitizer, with the kernel launchers replaced by host stubs
(tests/sanitize/launch_stubs.cpp), and the CPU tests of both run against that
build: any out-of-bounds access, use after free or undefined arithmetic in
the host code aborts the run.  CPU only (g++ and its sanitizer runtimes)."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_431_amd", "csrc")
OUT_DIR = os.path.join(ROOT, "_build", "sanitize")
LIB = os.path.join(OUT_DIR, "libpkv_sanitized.so")
SOURCES = [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "block_manager.cpp"),
           os.path.join(CSRC, "workspace.cpp"), os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp")]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _runtime(name):
    path = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitized_lib():
    if shutil.which("g++") is None or _runtime("libasan.so") is None or _runtime("libubsan.so") is None:
        pytest.skip("g++ with AddressSanitizer and UndefinedBehaviorSanitizer runtimes is needed")
    os.makedirs(OUT_DIR, exist_ok=True)
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", *SAN, "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-I/opt/rocm/include", *SOURCES,
           "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", LIB]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, f"sanitized build failed:\n{' '.join(cmd)}\n{res.stderr}"
    return LIB


def test_abi_and_block_manager_under_sanitizers(sanitized_lib):
    env = dict(os.environ)
    env["LD_PRELOAD"] = " ".join([_runtime("libasan.so"), _runtime("libubsan.so")] +
                                 ([env["LD_PRELOAD"]] if env.get("LD_PRELOAD") else []))
    # the interpreter itself is not instrumented and keeps memory until exit
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    # load the sanitized library in place of the product one, then run the
    # two CPU test files against it
    code = ("import sys, pytest; sys.path.insert(0, %r); sys.path.insert(0, %r); "
            "import paged_kv_cache_431_amd as pkv; pkv.LIB_PATH = %r; "
            "rc = pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu', %r, %r]); "
            "assert pkv.lib()._name == %r; sys.exit(rc)") % (
        ROOT, os.path.join(ROOT, "tests"), sanitized_lib, os.path.join(ROOT, "tests", "test_block_manager.py"),
        os.path.join(ROOT, "tests", "test_abi.py"), sanitized_lib)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT,
                         timeout=600)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
