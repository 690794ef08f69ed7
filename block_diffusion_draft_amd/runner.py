"""Device-side buffers for one draft-step workload (marshalling only).

Uploads the seeded host inputs of a workload to device memory, allocates the
outputs and the workspace the library asks for, and enqueues the step.  Rows of
the KV cache that the step can never read (outside the attention window) are
filled with a bf16 NaN pattern, so any stray read would surface in the outputs.
"""
import ctypes

import numpy as np
import torch

from . import binding, synth

BF16_NAN = 0x7FC0


def _i16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16))


class StepBuffers:
    def __init__(self, wl, weights=None, inputs=None, device="cuda", dbg=True,
                 poison_outside_window=True):
        self.wl = wl
        s = wl.shape
        self.cfg = binding.make_config(s)
        self.host_W = weights if weights is not None else synth.make_weights(s, wl.seed)
        self.dw = binding.DeviceWeights(s, self.host_W, device)
        self.inputs = inputs if inputs is not None else synth.make_step_inputs(wl)
        inp = self.inputs
        B, T, P, K = wl.batch, s.block, s.block - 1, s.top_k
        self.taps = _i16(inp["taps"]).to(device)
        self.last = torch.from_numpy(inp["last_token"]).to(device)
        self.ctx_len = torch.from_numpy(inp["ctx_len"]).to(device)
        cap = wl.cache_cap
        shape = (s.n_layers, B, s.n_kv, cap, s.head_dim)
        self.k_cache = self._cache(inp["k_cache"], shape, device, poison_outside_window)
        self.v_cache = self._cache(inp["v_cache"], shape, device, poison_outside_window)
        self.draft = torch.empty((B, P), dtype=torch.int32, device=device)
        self.cand_ids = torch.empty((B, P, K), dtype=torch.int32, device=device)
        self.cand_logp = torch.empty((B, P, K), dtype=torch.float32, device=device)
        self.dbg_hidden = torch.empty((s.n_layers + 1, B, T, s.hidden), dtype=torch.float32,
                                      device=device) if dbg else None
        self.dbg_logits = torch.empty((B, P, s.vocab), dtype=torch.float32,
                                      device=device) if dbg else None
        nbytes = binding.workspace_bytes(self.cfg, B, wl.t_new)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.accept_len = torch.empty(B, dtype=torch.int32, device=device)
        self.out_tokens = torch.empty((B, P + 1), dtype=torch.int32, device=device)

    def _cache(self, host, shape, device, poison):
        if isinstance(host, np.ndarray):
            return _i16(host).to(device)
        fill = BF16_NAN if poison else 0
        c = torch.full(shape, np.int16(np.uint16(fill).view(np.int16)), dtype=torch.int16,
                       device=device)
        for b, (rows, lo) in enumerate(zip(host.rows, host.lo)):
            S = rows.shape[2]
            if S:
                c[:, b, :, lo:lo + S, :] = _i16(rows).to(device)
        return c

    def step(self, dbg=True, probe=None):
        binding.draft_step(self.cfg, self.dw, self.taps, self.last, self.ctx_len, self.k_cache,
                           self.v_cache, self.draft, self.cand_ids, self.cand_logp, self.workspace,
                           self.dbg_hidden if dbg else None, self.dbg_logits if dbg else None,
                           probe)

    def verify(self, target):
        binding.verify_prefix(self.draft, target, self.accept_len, self.out_tokens)

    def new_rows(self, which="k"):
        """The cache rows this step writes: [L, B, n_kv, t_new, d] as uint16 numpy."""
        c = self.k_cache if which == "k" else self.v_cache
        n = self.inputs["ctx_len"]
        out = []
        for b in range(self.wl.batch):
            out.append(c[:, b, :, int(n[b]):int(n[b]) + self.wl.t_new, :].cpu().numpy())
        return np.stack(out, axis=1).view(np.uint16)
