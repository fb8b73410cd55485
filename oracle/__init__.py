"""CPU oracle for batch-1 decode of a Qwen3-0.6B-shaped decoder.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow reference the HIP
path is checked against.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import it; the product path never does, and it shares no
code with the HIP kernels or the C-ABI library.

It is written from the monolith project page (projects.dotslasha.me/p/monolith):
  * "Upstream facts": the model (pre-norm decoder, QK-norm, RoPE, GQA, SwiGLU,
    tied embedding / LM head) and the greedy decode it runs.
  * "Design decisions", FP8 format: E4M3 weights, one fp32 scale per output
    row, symmetric, round to nearest; activations bf16, fp32 accumulation.
  * "Design decisions", NVFP4 format: E2M1 values, one E4M3 scale per 16
    weights, one fp32 scale per tensor, round to nearest, and a per-block
    scale search that minimizes the squared error.
and the e2m1 value grid printed on the TSCT super-kernel note
(sehaxe.github.io/dormouse, section 3b, execution path 2).

Numerics: numpy float32 by default (the accumulation precision both pages
fix), with optional float64 and no-rounding modes used only to bound the
oracle's own arithmetic error.

Modules:
  codecs  bf16, e4m3 (OCP E4M3FN) and e2m1 encode / decode
  quant   FP8 per-row and NVFP4 per-16-block quantizers (canonical packed form)
  model   one decode step, prefill, greedy generation
  quality quantization error and logit divergence on synthetic weights
"""
