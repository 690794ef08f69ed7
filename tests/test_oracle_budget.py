"""The drafter shapes against the parameter count and memory figures the pages print."""
from oracle import budget


def test_named_parts():
    p = budget.parts()
    assert p["fc"] == 131_072_000
    assert sum(p["per_layer"].values()) == 319_815_680
    assert p["layers"] == 1_599_078_400
    assert p["codebooks"] == 127_139_840
    assert p["projection"] == 1_310_720
    assert p["norms"] == 62_720
    assert budget.named_sum(p) == 1_858_663_680


def test_stated_count_remainder_pins_qk_norms():
    """aiqre "Specification": 1,924,404,480 parameters.  Everything but the
    per-head q/k norms is a multiple of the hidden size 5120; the stated count
    leaves exactly 5 layers x 2 norms x 128 over a multiple of 5120."""
    assert budget.STATED_PARAMS % 5120 == budget.parts()["qk_norms"] == 1280
    residual = budget.STATED_PARAMS - budget.named_sum(budget.parts())
    assert residual == 65_740_800 and residual % 5120 == 0
    # the dynamic-convolution tensors read as W_c [64, 4096] per layer fit inside it
    assert budget.parts()["dyn_conv"] < residual


def test_memory_table_and_kv_bytes():
    """aiqre "Memory": bf16 3.6 GiB, fp8 1.8 GiB, int4 0.9 GiB; KV 20 KiB per
    token at 16 bit, about 5.0 GiB for 262,144 tokens."""
    gib = 2 ** 30
    n = budget.STATED_PARAMS
    assert round(n * 2 / gib, 1) == 3.6
    assert round(n * 1 / gib, 1) == 1.8
    assert round(n * 0.5 / gib, 1) == 0.9
    assert budget.kv_bytes_per_token() == 20 * 1024
    assert round(budget.kv_bytes_per_token() * 262_144 / gib, 1) == 5.0


def test_q4k_matrix_bytes_fit_weight_file():
    """FastFlowLM "Weights" row: dflash_weight.q4nx is 1.39 GB, Q4_K matrices plus
    BF16 norms, conv tensors, projection and codebooks.  The Q4_K matrices
    (4.5 bits/weight) and the named BF16 tensors must stay under that size."""
    p = budget.parts()
    q4 = (p["fc"] + p["layers"]) * 144 // 256
    assert q4 == 973_209_600
    bf16 = 2 * (p["codebooks"] + p["projection"] + p["norms"] + p["dyn_conv"])
    assert q4 + bf16 < 1.39e9
