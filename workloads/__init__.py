"""Seeded synthetic inputs for the expert-layer workloads.

This module only draws random numbers and lays them out; it holds none of the
quantization or matmul arithmetic. Both the HIP path (tests, bench) and the
CPU oracle consume what it returns.

Every tensor has its own numpy Generator seeded with SeedSequence([cfg, tid]):
tid 0 = X, 1 = W (or W1), 2 = W2, 3 = dY (or dOut), 4 = H, 5 = routing,
6/7 = outlier masks of X/W, 8 = routing-weight scores. bfloat16 tensors are
returned as uint16 bit patterns made from float32 draws by
round-to-nearest-even, so both sides see identical values.

Workloads (shapes from the expert layer of Inkling 2 Small: 8 of 384 experts
per token, 48 experts per GPU at 8-way expert parallelism):

1. single expert: X fp32 [64, 256] ~ N(0,1), W fp32 [256, 512] ~ N(0,1), both
   with 0.1% of entries multiplied by 50; dY fp32 [64, 512] ~ N(0,1).
2. small MoE: X bf16 [4096, 1024] ~ N(0,1), 8 experts, W bf16 [8, 2048, 1024]
   ~ N(0, 0.02^2) stored [expert, out, in], top-2 uniform routing.
3. one GPU's expert share: 32768 tokens routed top-8 over 384 experts with
   Zipf(1.1) popularity, experts 144..191 local; X bf16 [32768, 4096],
   W1 [48, 1536, 4096], W2 [48, 4096, 1536] ~ N(0, 0.02^2); H bf16 [M, 1536].
4. backward at the workload-2 shapes: dY bf16 [8192, 2048] ~ N(0, sd 1e-3).
5. decode: 512 tokens top-8 uniform over 384, experts 144..191 local,
   d_model 4096, FFN 1536; streaming: X bf16 [262144, 2048] ~ N(0,1).
"""

from .gen import *  # noqa: F401,F403
