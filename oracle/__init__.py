"""CPU oracle for the block-quantized decode GEMV, fused FFN and MoE layer.

TEST INFRASTRUCTURE ONLY. This package is imported by `tests/`, by the smoke
check in `__graft_entry__.py` and by the CPU-baseline leg of `bench.py`. The
library's product path (the HIP kernels behind the C ABI and the Python
binding in `block_quant_gemv_amd`) never imports, calls or links it, and the
oracle imports nothing from the product path. The two share no code; the only
common input source is the seeded generator package `synth`, which holds no
part of the method's arithmetic.

What it computes, in plain numpy, in fp64 wherever the method does not fix a
precision:

* `quant.quantize_q8`: the on-device activation quantizer (32-element int8
  blocks with an fp32 scale), whose decisions are taken in fp32 as the method
  states them.
* `quant.quantize_s16`: its 16-bit variant (int16 codes, scale absmax/32767),
  used by the 16-bit GEMV and MoE paths.
* `formats`: the seven block layouts (five from the decode workloads, plus
  Q5_K and IQ4_XS), byte-level decode and encode.
* `gemv`: the GEMV y = W_hat . x_hat in two independent forms -- the
  dequantize-then-accumulate form (fp64 matmul of decoded weights) and the
  integer block-dot form -- plus the exact per-block integer dot products.
* `ffn`: SwiGLU, re-quantization and the fused FFN chain, stage by stage.
* `moe`: the fp32 router GEMV, softmax / top-k / renormalisation, expert
  chains and the weighted combine with the shared expert.
* `attention`: decode attention of one token over an fp16 KV cache
  (grouped-query heads), the definition that the two-stage chunked
  reduction rearranges.

Sources: the method is described on three web pages -- "Why expert caching
can't save dense models: running a 27B dense model in 16 GB VRAM" (xhh.club
summary, sections on in-place quantized compute and its Q&A), "Understanding
Qwen3.6-35B-A3B in llama.cpp" (cnblogs, section 1.1 on MoE and its shape
list) and "01 · Phase overview: from 2B to 8B to MoE" (icman.com.cn, stage
three on device MoE kernels and the CPU reference matvec). Where the pages are
silent (byte order inside blocks, tie-breaking, the zero block), each module
states the reading it takes.
"""
from . import formats, quant, gemv, ffn, moe, attention  # noqa: F401
