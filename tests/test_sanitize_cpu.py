"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer: the plan
builders and the C interface's argument checks (csrc/plan.cpp, csrc/api.cpp)
are compiled with g++ -fsanitize=address,undefined (no device code; the
kernel launchers are replaced by stubs that abort if a malformed call ever
got past the checks) and driven by tests/sanitize/abi_fuzz.cpp with random
valid and malformed inputs.  Any sanitizer report, leak or wrong status
fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "adapter_lora_segments_amd", "csrc")
HIP_INC = "/opt/rocm/include"
HIP_LIB = "/opt/rocm/lib"


@pytest.fixture(scope="module")
def fuzz_binary(tmp_path_factory):
    if shutil.which("g++") is None or not os.path.isdir(HIP_INC):
        pytest.skip("needs g++ and the HIP headers")
    out = str(tmp_path_factory.mktemp("san") / "abi_fuzz")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", HIP_INC,
           os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "api.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "abi_fuzz.cpp"),
           "-L", HIP_LIB, "-lamdhip64", f"-Wl,-rpath,{HIP_LIB}", "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    return out


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_plan_and_abi_checks_under_sanitizers(fuzz_binary, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([fuzz_binary, "20000", str(seed)], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-4000:]
    built = int(r.stdout.split("plans built")[0].split(":")[-1])
    assert built > 1000, r.stdout


def test_hip_error_surfaces_as_status():
    """A HIP runtime failure comes back as MLORA_ERR_HIP with the runtime's
    error name in the message.  Without a device, the device check's
    hipGetDevice fails for real; with an MI355X it succeeds."""
    from adapter_lora_segments_amd import _lib
    L = _lib.lib()
    s = L.mlora_device_check()
    if s == 0:
        pytest.skip("a gfx950 device is present: the device check succeeds")
    msg = L.mlora_last_error().decode()
    if s == -2:
        assert "gfx950" in msg
        return
    assert s == -3 and L.mlora_status_string(s).decode() == "MLORA_ERR_HIP", (s, msg)
    assert msg.startswith("hipGetDevice: hipError"), msg
