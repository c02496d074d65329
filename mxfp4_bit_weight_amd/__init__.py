"""Block-scaled 4-bit weights (NVFP4, MXFP4) and the dequant-fused W4A16 linear
on AMD Instinct MI355X (gfx950).

The GPU library is ``libfp4w.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/fp4w.h``); ``mxfp4_bit_weight_amd.fp4w`` is its thin
Python binding.  ``workloads`` builds seeded synthetic inputs.
"""
