"""Reference oracle for the quantized speculative-verify MLP block.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It is a plain, slow, obviously correct CPU
implementation (numpy, fp64 accumulation) of what the GPU path computes, and
it shares no code, tables or helpers with the HIP library.

Sources it follows (the post "OCRia 推理栈：单卡 B200 提速近 10 倍" and its
German/French/Spanish/Japanese re-writes):

* "Reducing the data moved: workload-aware quantization" -- weights stored as
  FP8 (one byte instead of two) or NVFP4, with precision chosen per layer and
  sensitive layers kept at higher precision (BF16).
* German page "Wie es funktioniert" (and the French "Comment cela
  fonctionne", Spanish "Cómo funciona", Japanese "仕組み") -- SiLU activation
  fused with the quantization that follows it.
* "Generate more tokens per target pass: speculative decoding" -- the weights
  are read on every step and the verify pass covers 1 + draft tokens per
  request, so a block sees M = requests x (1 + drafts) rows at once.

The pages fix no bit formats, scale rule or rounding; the formats are the
public OCP FP8 E4M3 ("OCP 8-bit Floating Point Specification") and OCP FP4
E2M1 ("OCP Microscaling Formats (MX) v1.0", element type E2M1) definitions,
and the NVFP4 two-level scaling is the public NVFP4 description (E2M1 elements,
one E4M3 scale per 16 consecutive elements, one fp32 per-tensor scale).

Functions:
  formats  -- code tables, nearest-value encoders, bf16 rounding
  mlp      -- weight packing (quantization) and the block forward
"""

from . import formats, mlp  # noqa: F401
