"""Sanitizer build of the library's host code, for tests/test_abi_sanitized.py.

csrc/api.hip (the C ABI: argument checks, workspace plan, launch sequence) is compiled
with AddressSanitizer and UndefinedBehaviorSanitizer for the host only (each
-fsanitize= follows -Xarch_host; the device code is unchanged) and linked with a C
driver and the other objects of build.build() into one executable.
"""
import os
import subprocess

from block_diffusion_draft_amd import build

SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined " \
      "-Xarch_host -fno-sanitize-recover=undefined".split()


def build_sanitized(out_dir, driver):
    """Returns the path of the executable out_dir/abi_sanitized."""
    os.makedirs(out_dir, exist_ok=True)
    api_o = os.path.join(out_dir, "api_san.o")
    cmd = [build.HIPCC, *build.FLAGS, "-g", *SAN, "-c", os.path.join(build.CSRC, "api.hip"),
           "-o", api_o]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized api.hip failed:\n{r.stderr}")
    drv_o = os.path.join(out_dir, "driver.o")
    inc = os.path.join(os.path.dirname(build.HERE), "include")
    subprocess.check_call(["gcc", "-c", "-g", "-std=c11", "-I", inc, driver, "-o", drv_o])
    objs = [os.path.join(build.BUILD, s.replace(".hip", ".o")) for s in build.SOURCES
            if s != "api.hip"]
    exe = os.path.join(out_dir, "abi_sanitized")
    cmd = [build.HIPCC, "--offload-arch=gfx950", "-g", *SAN, drv_o, api_o, *objs, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr}")
    return exe
