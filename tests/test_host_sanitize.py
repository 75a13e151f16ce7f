"""AddressSanitizer + UBSan build of the C-ABI layer on the CPU.

h3k_api.cpp (validation, the lifetime planner, the launch sequence, the
profiler) is compiled with g++ for the host only, linked with stand-ins for the
kernel launchers and the HIP runtime calls (tests/host_sanitize/), and driven
with exactly sized host buffers, including the full 864x480x56-frame block
and its int8 variant with aliasing off.  Each launcher stand-in touches the
ends of every row its kernel would read or write, so any planner offset or
validation gap that would send a kernel outside a buffer is an ASan report;
it also checks the launch preconditions the kernels rely on.  No GPU code is
built or run."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = [os.path.join(ROOT, "video_diffusion_transformer_adaln_amd", "csrc", "h3k_api.cpp"),
       os.path.join(HERE, "host_sanitize", "launch_stubs.cpp"),
       os.path.join(HERE, "host_sanitize", "driver.cpp")]
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the ROCm headers")
def test_c_abi_layer_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "h3k_host_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "video_diffusion_transformer_adaln_amd", "csrc")] + SRC + ["-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, "full"], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "host sanitize OK" in r.stdout
