"""The C-ABI front end under AddressSanitizer and UndefinedBehaviorSanitizer, on
the CPU.  exact_attention_64_amd/csrc/attn_api.cpp (argument validation, the
split heuristic, parameter marshalling) is compiled with g++ together with a
host-only stub of the device layer (tests/hostsan/stub_device.cpp) into a
sanitizer-instrumented libattn.so stand-in; tests/test_abi.py (its cases that
need no GPU-free device answer) and tests/hostsan/stub_checks.py then run
against it in a child process with the ASan runtime preloaded.  Any invalid
memory access, signed overflow or other undefined behaviour aborts the child
with a sanitizer report."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gxx():
    return shutil.which("g++")


@pytest.mark.skipif(_gxx() is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_front_end_under_asan_and_ubsan(tmp_path):
    lib = tmp_path / "libattn_hostsan.so"
    cmd = [_gxx(), "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-shared", "-fPIC",
           os.path.join(ROOT, "exact_attention_64_amd", "csrc", "attn_api.cpp"),
           os.path.join(ROOT, "tests", "hostsan", "stub_device.cpp"), "-o", str(lib)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    asan = subprocess.run([_gxx(), "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    plugin = tmp_path / "hostsan_plugin.py"
    plugin.write_text("import os\n\n\ndef pytest_configure(config):\n"
                      "    from exact_attention_64_amd import _lib\n"
                      "    _lib.LIB_PATH = os.environ['HOSTSAN_LIB']\n")
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan, HOSTSAN_LIB=str(lib),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:new_delete_type_mismatch=0:alloc_dealloc_mismatch=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               PYTHONPATH=os.pathsep.join([str(tmp_path), ROOT, env.get("PYTHONPATH", "")]))
    # test_abi.py cases that expect "no device" (-8) assume a GPU-free host; the
    # stub answers as a gfx950 device, so those run in stub_checks.py instead.
    # -s: a sanitizer report is written to fd 2 just before the child exits, and
    # pytest's own capture would swallow it
    args = [sys.executable, "-m", "pytest", "-q", "-s", "-p", "hostsan_plugin", "-p", "no:cacheprovider",
            os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "hostsan", "stub_checks.py"),
            "-k", "not no_device and not ignored_delta and not probe"]
    r = subprocess.run(args, capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
    assert " passed" in out
