"""The library's host argument checks under AddressSanitizer and UBSan (CPU only).

tests/sanitize/build_sanitized.py compiles csrc/api.hip with both sanitizers for the host (device
code unchanged) and links tests/sanitize/abi_calls.c, which calls every entry point of
include/dflash.h with arguments the host checks must refuse (and, on a machine without
a GPU, fully valid calls that must come back as DFLASH_EHIP from their first HIP call).
The program must exit 0 with no sanitizer report.
"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return True


@pytest.mark.slow
def test_abi_checks_under_address_and_ub_sanitizers(tmp_path):
    from block_diffusion_draft_amd import build
    from tests.sanitize.build_sanitized import build_sanitized
    if not os.path.exists(os.path.join(build.BUILD, "q4k_stream.o")):
        build.build()
    exe = build_sanitized(str(tmp_path), os.path.join(HERE, "sanitize", "abi_calls.c"))
    assert "__asan_init" in subprocess.run(["nm", exe], capture_output=True, text=True).stdout
    args = [exe] + ([] if _gpu_visible() else ["no-gpu"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=99",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=98")
    r = subprocess.run(args, capture_output=True, text=True, timeout=120, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "0 failed checks" in r.stdout
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out
