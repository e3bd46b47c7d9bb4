"""The host C++ of libtq.so (C ABI, dispatch and plans, codec builder) built
with AddressSanitizer and UndefinedBehaviorSanitizer and driven on the CPU.

The kernel launchers are replaced by stubs (tests/sanitize/launch_stubs.cpp);
the driver (tests/sanitize/host_checks.cpp) builds every codec the library
accepts, exports and checks its tables, and runs every argument check with
placeholder pointers.  Any sanitizer report, failed check or launch reached
fails the test.  g++ builds the host files only; nothing here runs on a GPU.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_decode_attention_04_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
HOST_SOURCES = [os.path.join(CSRC, f) for f in ("capi.cpp", "dispatch.cpp", "codec_host.cpp")] + [
    os.path.join(HERE, f) for f in ("launch_stubs.cpp", "host_checks.cpp")]


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "host_checks")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *HOST_SOURCES, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    supp = tmp_path / "lsan.supp"
    # the HIP runtime keeps allocations of its own until exit
    supp.write_text("leak:libamdhip64\nleak:libhsa-runtime64\n")
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:detect_leaks=1",
               LSAN_OPTIONS=f"suppressions={supp}", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               HIP_VISIBLE_DEVICES="")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "host checks passed" in run.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
