"""quantized_gemv_amd — batch-1 greedy decode of a Qwen3-style decoder as one
persistent HIP kernel per token on AMD MI355X (gfx950), with bf16, FP8
(E4M3, per-row scales) and NVFP4-mix weights dequantized in registers.

The product is the C-ABI library libmk.so (include/mk.h); `native` is its
ctypes binding.  Import `quantized_gemv_amd.native` to use it.
"""
__all__ = ["native", "build"]
