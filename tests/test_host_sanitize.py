"""The engine's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

tests/host/sanitize_driver.cpp drives every path of the C ABI that needs no GPU (validation,
the item-trie build, workspace sizing, calls before a workspace is bound, scheduler and top-K
argument checks); it is compiled with g++ together with the engine's host source, the device
launchers stubbed, and must finish with no sanitizer report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(os.path.join(ROCM, "include")),
                    reason="needs g++ and the ROCm headers")
def test_host_code_is_clean_under_sanitizers(tmp_path):
    exe = tmp_path / "sanitize_driver"
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    cmd = ["g++", "-std=c++17", "-O1", "-g", *san, "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "semantic_id_beam_amd", "csrc"),
           "-I", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "host", "sanitize_driver.cpp"),
           os.path.join(ROOT, "semantic_id_beam_amd", "csrc", "gr_engine.cpp"),
           "-L", os.path.join(ROCM, "lib"), f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-lamdhip64",
           "-o", str(exe)]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert res.returncode == 0, res.stdout[-4000:]
    # verify_asan_link_order=0: the environment may preload a library ahead of the ASan runtime
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env,
                         timeout=300)
    assert run.returncode == 0, run.stdout[-4000:]
    assert "host paths clean" in run.stdout
    assert "runtime error" not in run.stdout and "Sanitizer" not in run.stdout
