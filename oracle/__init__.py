"""CPU oracle for the routed-expert MoE layer with a GPU slot cache.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously-correct
reference: NumPy fp64 arithmetic and pure-Python control logic, written from
the FreeToken pages ("Making Large MoE Models Practical on a Single Machine",
"The Expert Cache That Follows the Router", the METAL MEDIA and hyper.ai
summaries of arXiv 2608.16157, and the txtmix long-form article).  Only the
tests, the smoke check and the benchmark's CPU-baseline leg may import it; the
product library never does, and this package imports nothing from it.

Modules
  formats  decoding of layer-expert records (bf16, e4m3 + 128x128 fp32 block
           scales, e2m1 + e8m0 per 32)
  route    top-k softmax routing with fp64 logits
  qstar    the bandwidth-adaptive fill count q
  cache    the slot-cache simulator: dedupe, hit/miss, q, LRU victims,
           route rewrite, full-layer buffer invalidation, resize
  moe      the SwiGLU expert FFN and the weighted top-k combine

Pinning status: every function is pinned by the `-m "not gpu"` tests in
tests/test_oracle_*.py against page examples, closed forms, textbook or library
special cases and brute force.  Float outputs of the layer are not printed on
the pages; they are pinned by one-hot closed forms, linearity and brute force,
not by page values.
"""
