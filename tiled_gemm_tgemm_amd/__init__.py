"""tiled_gemm_tgemm_amd: fp32 C = A·B for one MI355X (gfx950), hand-written HIP.

The compute lives in the C-ABI library libtgemm.so (sources in csrc/,
declarations in include/tgemm.h); this package only marshals arguments.
"""
