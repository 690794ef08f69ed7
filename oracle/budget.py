"""Parameter budget of the drafter shapes (test infrastructure only).

Sources: FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2", spec table "Draft" row
(5 layers, hidden 5120, FFN 17408, 32 query / 8 KV heads of 128, selector top 16
rank 256; about 2 B parameters) and "Weights" row (fc, q/k/v/o and MLP in Q4_K;
norms, dynamic-convolution tensors, selector projection and two 248320 x 256
codebooks in BF16); aiqre page "Qwen3.8-27B-DFlash2", section "Specification"
(1,924,404,480 parameters, vocabulary 248,320) and section "Memory" (bf16 3.6
GiB, fp8 1.8 GiB, int4 0.9 GiB; KV cache 20 KiB per token at 16 bit).
"""

STATED_PARAMS = 1_924_404_480


def parts(L=5, H=5120, F=17408, n_q=32, n_kv=8, d=128, V=248_320, r=256, n_taps=5):
    """Named parameter groups of the drafter (embedding / output head are the
    target's and are not counted: the draft shares them)."""
    per_layer = {
        "q": n_q * d * H, "k": n_kv * d * H, "v": n_kv * d * H, "o": H * n_q * d,
        "gate": F * H, "up": F * H, "down": H * F,
    }
    return {
        "fc": n_taps * H * H,
        "layers": L * sum(per_layer.values()),
        "per_layer": per_layer,
        "codebooks": 2 * V * r,
        "projection": H * r,
        "norms": L * (2 * H + 2 * d) + H + H,   # in/post norms, q/k norms; final; fused-tap norm
        "qk_norms": L * 2 * d,
        "dyn_conv": L * 2 * n_q * n_q * d,      # W_c [2 n_q, n_q d] per layer
    }


def named_sum(p):
    return p["fc"] + p["layers"] + p["codebooks"] + p["projection"] + p["norms"]


def kv_bytes_per_token(L=5, n_kv=8, d=128, bytes_per=2):
    return L * 2 * n_kv * d * bytes_per
