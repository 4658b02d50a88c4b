"""The library's host code (planner, validation, pool sizing, every entry
point's error paths) built with AddressSanitizer and UndefinedBehaviorSanitizer
on the host side only, and driven by tests/host_sanitize_main.cpp. CPU only:
no call reaches a kernel launch."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_host_code_under_address_and_undefined_sanitizers(tmp_path):
    exe = tmp_path / "host_sanitize"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
           # sanitizers on the host pass only; the device code is built as usual
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(ROOT, "tests", "host_sanitize_main.cpp"),
           os.path.join(ROOT, "long_context_attention_upipe_amd", "csrc", "upipe_attn.hip"),
           "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-4000:]
    blob = exe.read_bytes()
    assert b"__asan_init" in blob and b"__ubsan_handle" in blob, "sanitizer runtimes not linked in"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "host checks: 0 failures" in out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    shutil.rmtree(tmp_path, ignore_errors=True)
