"""MI355X-native weight-streaming skinny GEMM for speculative-decoding verify passes.

Y[N, M] = X[N, K] . W^T for N = 1-8 columns, W stored as NVFP4 or as
row-scaled FP8-E4M3, X in BF16, Y in FP32, computed by hand-written HIP
kernels for gfx950 behind the C ABI declared in include/wq.h.

Submodules:
  wq      ctypes binding of libwq.so (same names as the C ABI)
  inputs  seeded synthetic inputs (no product arithmetic)
"""
