"""The C ABI's host-side validation under AddressSanitizer and UndefinedBehaviorSanitizer.

kda_api.hip is compiled for gfx950 with the sanitizers on its host pass only, together with
tests/sanitize/abi_host_driver.cpp, which stubs the kernel launchers and drives every
entry point through valid and invalid arguments. Any out-of-bounds access, use of freed
memory, overflow or other undefined behaviour in the validation aborts the driver; a
wrong status or a launch after a rejected call fails its own checks. Runs on the CPU.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_host_validation_is_clean_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_host_check")
    # sanitizers apply to the host pass only (-Xarch_host); the device pass builds the
    # library's scratch array and nothing else
    cmd = [HIPCC, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "--offload-arch=gfx950",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-x", "hip",
           os.path.join(ROOT, "gated_delta_rule_channel_amd", "csrc", "kda_api.hip"),
           os.path.join(ROOT, "tests", "sanitize", "abi_host_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    # a preloaded library ahead of the ASan runtime is tolerated, not removed
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
