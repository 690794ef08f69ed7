"""Reference oracle for the DFlash 2 block-draft step and greedy prefix acceptance.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously-correct CPU
implementation (NumPy, float64) of what the GPU library computes.  Only the test
suite, the smoke check and the CPU-baseline leg of the benchmark may import it.
The product path (the C-ABI library and its Python binding) never imports, links
or calls anything in here, and this package shares no code with that path: it
reads the same input bytes (Q4_K blocks, bf16 tensors) and nothing else.

Sources (the pages this follows):
  * FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2": the spec table ("Draft",
    "Weights" and "Taps" rows) and the section "How it is used".
  * aiqre model page "Qwen3.8-27B-DFlash2": the "Specification" and "Memory"
    sections (parameter count, vocabulary, KV bytes per token).
  * Mindket kit page "Qwen3.8-27B-DFlash2-GGUF by z-lab": section "For
    newcomers and experts" (block drafting, candidates, selector, convolutions).
  * JetBrains card "Qwen3.8-3.6-27B-blend DFlash2": "Model details" and the
    SGLang/vLLM note in "Quick start" (block of 8 = anchor + 7 proposals).

Modules:
  bf16     - bf16 <-> float64 conversion (the storage format of the inputs)
  q4k      - Q4_K super-block decode
  q8_0     - Q8_0 block decode
  fp8      - FP8 (E4M3, one scale per row) decode
  draft    - the draft forward: tap fusion, layers, LM head, top-K
  select   - Viterbi path through the candidates, and brute force
  verify   - greedy accept-longest-prefix
  sample   - sampled acceptance (exact rejection sampling against the target's
             temperature / top-k / top-p distribution)
  budget   - parameter budget of the drafter shapes

Every function here is pinned by a test in tests/test_oracle_*.py against values
that do not come from this package (closed forms, hand-built blocks, brute
force, library routines, figures printed on the pages), except the composed
forward, whose composition has no worked example on the pages: "parity
unpinned" beyond its pinned components.
"""
