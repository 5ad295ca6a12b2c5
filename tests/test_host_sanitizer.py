"""The C-ABI layer (argument validation, chunk tables, workspace plans, launch
sequences of the ring sweeps) built for the host alone with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer, the kernel launchers replaced by
stand-ins that record each launch and check that every device range it would touch
lies inside the caller's buffers (tests/host_check/).  The driver runs every entry
point through its refusal paths and its launch plans on fake device addresses; a
sanitizer report, a launch before a refusal, an out-of-buffer range or a wrong
status fails it.  No GPU and no HIP runtime are involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HC = os.path.join(ROOT, "tests", "host_check")
OUT = os.path.join(ROOT, "_build", "abi_check")


@pytest.fixture(scope="module")
def abi_check_binary():
    if shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include/hip"):
        pytest.skip("needs g++ and the HIP headers")
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROOT}/include", "-I/opt/rocm/include", f"-I{ROOT}/context_attention_lse_kv_amd/csrc", f"-I{HC}",
           f"{ROOT}/context_attention_lse_kv_amd/csrc/ra_abi.cpp", f"{HC}/launch_stubs.cpp", f"{HC}/abi_check.cpp",
           "-o", OUT]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return OUT


def test_abi_layer_clean_under_asan_ubsan(abi_check_binary):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([abi_check_binary], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0, r.stderr[-4000:]
    assert "0 failed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
