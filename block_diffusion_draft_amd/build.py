"""Build the gfx950 library libdflash.so in-tree with hipcc (and the host data helper).

Every HIP source is compiled for gfx950 only, with packed-fp32 instructions
disabled, then linked into one shared library next to this file.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdflash.so")
SOURCES = ["api.hip", "q4k_dequant.hip", "q4k_tiled.hip", "q4k_stream.hip", "q8_0.hip", "fp8.hip", "gemm_bf16.hip", "gemm_big.hip", "layer_ops.hip", "attention.hip",
           "topk.hip", "verify.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result"]


# per-file extras: MFMA results in VGPRs (no accumulator-register round trips)
EXTRA = {"q4k_stream.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src):
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    workers = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    from . import synth
    synth.build_synth(force=True)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    sys.path.insert(0, os.path.dirname(HERE))
    from block_diffusion_draft_amd import build as b
    b.build(verbose=True)
