"""CPU oracle for the latent-MoE layer forward (test infrastructure only).

A plain, slow, FP64 numpy implementation of what the layer computes, plus a
pure-Python brute-force version for tiny shapes. Only the tests, the smoke
check and the benchmark's CPU-baseline leg use it; the product path never
imports anything from here, and nothing here imports the product.

Sources followed (web pages on Muse Spark Open):
  [lmsys] "SGLang and Miles Add Day-0 Support for Muse Spark Open" (lmsys.org),
          sections "MoE with Pooler, Unpooler and Per-Expert Normalization",
          "The Fused Post-per-expert Norm", "Trainable Muse Spark Open Backend",
          "NVFP4 as a third MMA kind", "AMD Support / Day-0 Enablement".
  [vllm]  "vLLM 对 Muse Spark Open 的 Day 0 支持" (vLLM Day 0 support post),
          sections "潜空间 MoE" (latent MoE), "三明治归一化" (sandwich norm),
          "硬件后端" (hardware backends: FP32 router GEMM).

Parity status: every function here is pinned by tests/test_oracle_*.py against
brute force, closed forms, invariants and library special cases. The numeric
values of the full layer at real shapes have no printed example on the pages;
they are pinned only through those properties.
"""
