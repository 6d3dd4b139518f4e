"""The library's threaded host code under sanitizers, on the CPU (no GPU, no HIP): the hybrid
backend's worker pool and expert kernel (host_ffn.cpp) and the bounce ring's copy team
(copy_team.cpp), driven by tests/native/host_stress.cpp, built with g++ once with AddressSanitizer
+ UndefinedBehaviorSanitizer and once with ThreadSanitizer.  Any sanitizer report or failed check
fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_expert_offload_amd", "csrc")
SRCS = [os.path.join(CSRC, "host_ffn.cpp"), os.path.join(CSRC, "copy_team.cpp"),
        os.path.join(ROOT, "tests", "native", "host_stress.cpp")]

SANITIZERS = {
    "asan_ubsan": (["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"],
                   {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
                    "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}),
    "tsan": (["-fsanitize=thread"], {"TSAN_OPTIONS": "halt_on_error=1:second_deadlock_stack=1"}),
}


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
@pytest.mark.parametrize("kind", sorted(SANITIZERS))
def test_threaded_host_code_under_sanitizer(kind, tmp_path):
    flags, env = SANITIZERS[kind]
    exe = str(tmp_path / ("host_stress_" + kind))
    cmd = ["g++", "-O1", "-g", "-std=c++17", *flags, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *SRCS,
           "-o", exe, "-lpthread"]
    subprocess.check_call(cmd)
    run_env = dict(os.environ)
    run_env.update(env)
    r = subprocess.run([exe], env=run_env, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host stress ok" in r.stdout
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
