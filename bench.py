"""Throughput of the DFlash 2 block-draft step on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic inputs
resident in HBM: dflash_draft_step (tap fusion, 5 drafter layers, shared output
head with top-16, Viterbi selector) followed by dflash_verify_prefix.  The
workload is the pages' 27B-draft shape at batch 1 with a 4096-row context.

--workload full_b16 / full_b64_bf16 measure the pages' batched draft steps instead (16
sequences with 32768-row contexts and Q4_K weights; 64 with 8192 and bf16 weights); the
default stays the batch-1 workload.  With --weights q8_0 (or fp8) the drafter's matrices
are Q8_0 (or FP8 E4M3 with a scale per row) instead of Q4_K (same shapes, same seed
recipe).  With --accept sampled the acceptance is dflash_verify_sampled instead (rejection
sampling against synthetic fp32 target logits [1][8][248320] resident in HBM, at the
pages' sampler settings).

Prints one JSON line: draft blocks/s from the median of the K step times (each step
timed by its own pair of HIP events, steps back to back), with p10 / p90 / mean; the
roofline of the dominant kernel (the 248320 x 5120 bf16 output head), timed with HIP
events that the library records on the step's stream immediately around the head's
launch, over K eager steps run right after the timed graph replays (HIP does not
time events recorded inside a captured graph); and the float64 CPU reference timed
on this host on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("gemm_bf16.hip", "common.h"):
        h.update(open(os.path.join(ROOT, "block_diffusion_draft_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per output-head launch from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, copy-calibrated), if it was taken on the
    current kernel source."""
    p = os.path.join(ROOT, "profiles", "lm_head_counters.txt")
    if not os.path.exists(p):
        return None
    kv = {}
    for line in open(p):
        parts = line.split()
        if len(parts) >= 2 and not line.startswith("#"):
            kv[parts[0]] = parts[1]
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return float(kv["hbm_bytes_per_launch"])


def first_sequence(inp):
    """The inputs of sequence 0 only (sequences are independent)."""
    from block_diffusion_draft_amd import synth
    out = {k: inp[k][:1] for k in ("taps", "last_token", "ctx_len")}
    for c in ("k_cache", "v_cache"):
        v = inp[c]
        out[c] = v[:, :1] if isinstance(v, np.ndarray) else \
            synth.WindowCache(v.rows[:1], v.lo[:1], v.shape)
    return out


def cpu_baseline(wl, bufs, min_s=10.0):
    """The oracle as it stands, on this host: whole float64 draft steps of the same
    workload (tap fusion, every layer, the full output head with top-K, the
    selector), repeated until at least min_s seconds of CPU work have run.  For a
    batch of several sequences the sample is sequence 0 alone (one block per step)."""
    from oracle import draft as od
    from oracle import select as osel
    from oracle.bf16 import bf16_to_f64
    s = wl.shape
    W = bufs.host_W
    inp = bufs.inputs if wl.batch == 1 else first_sequence(bufs.inputs)
    nseq = 1
    # numpy's BLAS runs on OMP_NUM_THREADS threads (all available cores when unset)
    avail = len(os.sched_getaffinity(0))
    threads = min(avail, int(os.environ.get("OMP_NUM_THREADS") or avail))
    A, B = bf16_to_f64(W["code_a"]), bf16_to_f64(W["code_b"])
    cfg = dict(s.as_dict())
    n = 0
    t0 = time.perf_counter()
    while True:
        out = od.draft_step(cfg, W, inp["taps"], inp["last_token"], inp["ctx_len"],
                            inp["k_cache"], inp["v_cache"], want_logits=False)
        for b in range(nseq):
            T = osel.pair_scores(out["cand_ids"][b], A, B, s.pair_scale)
            osel.viterbi(out["cand_logp"][b], T)
        n += 1
        el = time.perf_counter() - t0
        if el >= min_s:
            break
    what = (f"{n} whole {wl.name} steps" if wl.batch == 1 else
            f"{n} steps of sequence 0 of {wl.name}")
    return {"value": nseq * n / el, "unit": "draft blocks/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"{what} (batch 1: tap fusion, {s.n_layers} layers, full "
                       f"{s.vocab}-row output head with top-{s.top_k}, selector) in {el:.1f} s")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", type=int, default=1, help="replay the step as a HIP graph")
    ap.add_argument("--weights", choices=("q4k", "q8_0", "fp8"), default="q4k",
                    help="drafter weight format: Q4_K (the default), Q8_0 or FP8")
    ap.add_argument("--workload", choices=("full_b1", "full_b16", "full_b64_bf16"),
                    default="full_b1",
                    help="the 27B-draft workload: 1 sequence with a 4096-row context (the "
                         "default), 16 sequences with 32768 (Q4_K), 64 with 8192 (bf16)")
    ap.add_argument("--accept", choices=("greedy", "sampled"), default="greedy",
                    help="acceptance after the draft: greedy prefix (the default), or "
                         "rejection sampling against fp32 target logits [B][8][V] at "
                         "temperature 1.0, top-k 20, top-p 0.95")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after timing, run 3 plain device copies of this size (the "
                         "reference kernel that calibrates rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; the batch-1 draft step is "
                          "measured on one MI355X (multi-GPU sharding is design-only)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    from block_diffusion_draft_amd import binding, runner, synth

    key = args.workload
    if args.weights != "q4k":
        if key != "full_b1":
            sys.exit(f"--weights {args.weights} is measured on the batch-1 workload")
        key = "full_b1_" + args.weights
    wl = synth.WORKLOADS[key]
    s = wl.shape
    print(f"[bench] preparing {wl.name}", file=sys.stderr, flush=True)
    bufs = runner.StepBuffers(wl, dbg=False)
    # target tokens agreeing with the draft on a 4-token prefix
    bufs.step(dbg=False)
    torch.cuda.synchronize()
    d = bufs.draft.cpu().numpy()
    tgt = np.zeros((wl.batch, s.block), dtype=np.int32)
    tgt[:, :4] = d[:, :4]
    tgt[:, 4] = (d[:, 4] + 1) % s.vocab
    tgt[:, 5:] = synth.randint(wl.seed, "target_tail", (wl.batch, s.block - 5), 0, s.vocab)
    target = torch.from_numpy(tgt).cuda()
    sampled = args.accept == "sampled"
    if sampled:
        P = s.block - 1
        z = synth.target_logits(wl.seed, "bench.target_logits", d, s.vocab)
        u = synth.uniform(wl.seed, "bench.uniforms", (wl.batch, P + 1, 2))
        tlog = torch.from_numpy(z).cuda()
        unif = torch.from_numpy(u).cuda()
        sws = torch.empty(binding.verify_sampled_workspace_bytes(wl.batch, P, s.vocab),
                          dtype=torch.uint8, device="cuda")
        del z

    K, Wm = args.steps, args.warmup
    ev = [(binding.HipEvent(), binding.HipEvent()) for _ in range(K)]
    probes = [binding.make_probe(binding.PROBE_LM_HEAD, a, b) for a, b in ev]

    def one_step(probe=None):
        bufs.step(dbg=False, probe=probe)
        if sampled:
            binding.verify_sampled(bufs.draft, tlog, unif, 1.0, 20, 0.95, sws, bufs.accept_len,
                                   bufs.out_tokens)
        else:
            bufs.verify(target)

    for _ in range(Wm):
        one_step()
    torch.cuda.synchronize()
    graph = None
    if args.graph:
        # graphs replay the exact launches; the head's probe events are taken
        # from an eager pass over the same steps
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            one_step()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                one_step()
        torch.cuda.synchronize()
        for _ in range(Wm):
            graph.replay()
        torch.cuda.synchronize()

    # timed region: K steps back to back, an event pair around each (no host sync
    # in between), plus one pair around the whole run
    t_start, t_stop = binding.HipEvent(), binding.HipEvent()
    step_ev = [binding.HipEvent() for _ in range(K + 1)]
    torch.cuda.synchronize()
    t_start.record()
    for i in range(K):
        step_ev[i].record()
        if graph is not None:
            graph.replay()
        else:
            one_step(probes[i])
    step_ev[K].record()
    t_stop.record()
    torch.cuda.synchronize()
    ms_mean = t_start.elapsed_ms(t_stop) / K
    step_ms = np.array([step_ev[i].elapsed_ms(step_ev[i + 1]) for i in range(K)])
    ms = float(np.median(step_ms))

    # live timing of the dominant kernel (eager pass with probes)
    for i in range(K):
        one_step(probes[i])
    torch.cuda.synchronize()
    head_ms = float(np.mean([a.elapsed_ms(b) for a, b in ev]))
    R = wl.batch * (s.block - 1)
    # the head's algorithmic bytes: its bf16 weights and input rows once, fp32 logits out;
    # at many rows its 2 R V H flops take longer than those bytes at the peaks: then it is
    # an MFMA-bound kernel and is reported in TFLOP/s
    alg = s.vocab * s.hidden * 2 + R * s.hidden * 2 + R * s.vocab * 4
    flops = 2.0 * R * s.vocab * s.hidden
    mfma_bound = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > alg / (HBM_PEAK_GBS * 1e9)
    achieved = alg / (head_ms * 1e-3) / 1e9
    traffic = load_traffic() if wl.batch == 1 else None

    res = {
        "metric": "draft blocks/s (8 tok) at 27B-draft shape, 1 GPU; % of HBM roofline",
        "value": wl.batch / (ms * 1e-3),
        "unit": "draft blocks/s",
        "n_gpus": 1, "steps": K, "warmup": Wm, "ms_per_step": ms,
        "step_ms": {"median": ms, "p10": float(np.percentile(step_ms, 10)),
                    "p90": float(np.percentile(step_ms, 90)), "mean": ms_mean},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "ctx_len": wl.ctx_len,
                   "t_new": wl.t_new, "layers": s.n_layers, "hidden": s.hidden,
                   "vocab": s.vocab, "top_k": s.top_k, "weights": s.weight_fmt,
                   "step": ("draft_step + verify_sampled (T 1.0, top-k 20, top-p 0.95)"
                            if sampled else "draft_step + verify_prefix"),
                   "hip_graph": bool(graph)},
        "roofline": ({"kernel": "output head k_head_stream (bf16 MFMA, 248320 x 5120, 7 rows)",
                      "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                      "launch_ms": head_ms, "algorithmic_bytes": alg} if wl.batch == 1 else
                     {"kernel": f"output head (bf16 MFMA, {s.vocab} x {s.hidden}, {R} rows)",
                      "bound": "mfma" if mfma_bound else "hbm",
                      "achieved": (flops / (head_ms * 1e-3) / 1e12) if mfma_bound else achieved,
                      "peak": MFMA_BF16_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBS,
                      "unit": "TFLOP/s" if mfma_bound else "GB/s",
                      "frac": (flops / (head_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS) if mfma_bound
                      else achieved / HBM_PEAK_GBS,
                      "traffic": traffic, "launch_ms": head_ms, "algorithmic_bytes": alg,
                      "algorithmic_flops": flops}),
        "step_hbm_frac": None,
    }
    step_bytes = step_algorithmic_bytes(wl)
    if sampled:      # the target's logits and the uniforms, read once
        step_bytes += wl.batch * s.block * (s.vocab + 2) * 4
    res["step_hbm_frac"] = step_bytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9)
    if args.copy_bytes > 0:
        n = args.copy_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU reference", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(wl, bufs)
    print(json.dumps(res))


def step_algorithmic_bytes(wl):
    """Bytes the step must move at least once: every weight byte, the output
    head, the KV window of each sequence and layer, the appended rows, the taps,
    the codebook rows the selector gathers and the outputs."""
    s = wl.shape
    B = wl.batch
    qd, kd = s.n_q * s.head_dim, s.n_kv * s.head_dim
    lin = s.n_taps * s.hidden * s.hidden + s.n_layers * (
        qd * s.hidden + 2 * kd * s.hidden + s.hidden * qd + 3 * s.ffn * s.hidden)
    rows = s.hidden + s.n_layers * (qd + 2 * kd + s.hidden + 2 * s.ffn + s.hidden)
    wbytes = {"q4k": lin * 144 // 256, "q8_0": lin * 34 // 32,
              "fp8": lin + 4 * rows}.get(s.weight_fmt, lin * 2)
    small = s.n_layers * (2 * s.hidden + 2 * s.head_dim + 2 * s.n_q * qd) * 2 + 3 * s.hidden * 2
    head = s.vocab * s.hidden * 2
    win = min(s.window, wl.ctx_len + wl.t_new)
    kv = B * s.n_layers * 2 * (win * kd * 2)
    taps = B * wl.t_new * s.n_taps * s.hidden * 2
    codes = B * (s.block - 2) * 2 * s.top_k * s.sel_rank * 2
    outs = B * (s.block - 1) * (1 + 2 * s.top_k) * 4
    return wbytes + small + head + kv + taps + codes + outs


if __name__ == "__main__":
    main()
