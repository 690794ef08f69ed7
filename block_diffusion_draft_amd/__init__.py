"""MI355X (gfx950) DFlash 2 block-draft step: the C-ABI library libdflash.so (built
in-tree by build.py from csrc/), its ctypes binding (binding.py), device buffers for
seeded workloads (runner.py), the seeded input generator (synth.py), and the
measurement helpers (gemm_bench.py, rocprof_summary.py)."""
