"""Q4_K (or Q8_0) GEMM microbenchmark at the drafter's matrix shapes, M = 8 rows (one block).

    python -m block_diffusion_draft_amd.gemm_bench [--iters N] [--min-bytes B] [--fmt q8_0]

Each shape (fc 25600->5120; q 5120->4096; k, v 5120->1024; o 4096->5120; gate, up
5120->17408; down 17408->5120; FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2", spec table
"Draft" row) runs through the library's q4k_gemm_tiled entry point (product + split-K
reduction to bf16) on bf16 N(0,1) activations and N(0, 0.02) weights packed to Q4_K
(seed 1), regrouped on the device into the tiled layout.  Calls rotate over enough
copies of the weight matrix to span at least --min-bytes, so no call is served from
the last-level cache.  Prints one JSON line per shape: microseconds per call and the
Q4_K weight bytes per second.  --fmt q8_0 runs the same shapes through q8_0_gemm_tiled with
the weights packed to Q8_0 (Mindket kit page "Qwen3.8-27B-DFlash2-GGUF by z-lab",
draft-file table).
"""
import argparse
import json
import sys

import numpy as np


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--iters", type=int, default=40)
    ap.add_argument("--min-bytes", type=int, default=1 << 30)
    ap.add_argument("--rows", type=int, default=8)
    ap.add_argument("--fmt", choices=("q4k", "q8_0"), default="q4k")
    args = ap.parse_args()

    import torch
    from . import binding, synth

    M = args.rows
    q8 = args.fmt == "q8_0"
    pack = synth.q8_0_normal if q8 else synth.q4k_normal
    to_tiled = binding.q8_0_to_tiled if q8 else binding.q4k_to_tiled
    gemm = binding.q8_0_gemm_tiled if q8 else binding.q4k_gemm_tiled
    ws_bytes = (binding.q8_0_gemm_tiled_workspace_bytes if q8
                else binding.q4k_gemm_tiled_workspace_bytes)
    for name, N, K in synth.GEMM_SHAPES:
        w_host = pack(synth.GEMM_SEED, f"gemm.{name}", N, K, 0.02)
        wbytes = w_host.size
        copies = max(1, -(-args.min_bytes // wbytes))
        w_rows = torch.from_numpy(w_host).cuda()
        w0 = torch.empty_like(w_rows)
        to_tiled(w_rows, w0, N, K)                    # the library's device layout
        del w_rows
        ws = [w0] + [w0.clone() for _ in range(copies - 1)]
        x = torch.from_numpy(synth.normal_bf16(synth.GEMM_SEED, f"gemm.{name}.x", (M, K), 1.0)
                             .view(np.int16)).cuda()
        y = torch.empty((M, N), dtype=torch.int16, device="cuda")
        work = torch.empty(ws_bytes(M, N, K), dtype=torch.uint8, device="cuda")
        for i in range(2 * copies):
            gemm(ws[i % copies], x, y, work)
        torch.cuda.synchronize()
        e0, e1 = binding.HipEvent(), binding.HipEvent()
        e0.record()
        for i in range(args.iters):
            gemm(ws[i % copies], x, y, work)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_ms(e1) * 1e3 / args.iters
        print(json.dumps({"matrix": name, "fmt": args.fmt, "M": M, "N": N, "K": K, "weight_bytes": int(wbytes),
                          "us_per_call": round(us, 2), "weight_GBps": round(wbytes / us / 1e3, 1),
                          "copies": copies}), flush=True)
        del ws, w0, work
        torch.cuda.empty_cache()


if __name__ == "__main__":
    sys.exit(main())
