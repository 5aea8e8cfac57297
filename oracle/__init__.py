"""Plain CPU oracle of one masked-diffusion denoising iteration and its run loop.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this package; the library's product
path never does, and this package imports nothing from the library.  It shares
no code with the HIP implementation: the only common module is `synth`, which
draws the seeded inputs and computes nothing of the method.

What it computes, and where each step is stated (page titles; sections):
  [A] "dInfer: An Efficient Inference Framework for Diffusion Language Models"
      (abstract): four components -- model, diffusion iteration manager,
      decoding strategy, KV-cache manager; MoE model.
  [N] "dInfer框架发布：蚂蚁集团重塑LLM推理，速度狂飙10倍" (aigc.bar article):
      section "扩散模型的“理论翅膀”与“现实枷锁”" (bidirectional attention makes
      every token's KV change each iteration; classic decoding keeps only the
      most confident token), section "削减计算成本：邻近KV缓存刷新" (vicinity
      KV refresh), section "解码的艺术" (hierarchical decoding, credit
      decoding, iteration smoothing).
  [S] "Sangam: Efficiently Serving Diffusion LLMs with the AR Stack" (abstract):
      a masked response is denoised; several positions commit per invocation;
      cached KV is refreshed and reused across decodes; decodes are block-sized;
      a deficit token budget admits whole refreshes (sched.py).
  [T] "TIDE: Efficient and Lossless MoE Diffusion LLM Inference with I/O-aware
      Expert Offload" (abstract): block-level decoding; expert activations are
      stable within a block.

Precision: the model arithmetic is fp64.  Decisions that turn floats into
integers are taken in fp32, the precision of the GPU kernels: argmax and top-k
order on fp32-rounded biased logits, the confidence threshold, credit
(fl32(fl32(gamma*c) + fl32(lambda*p)), no fused multiply-add) and the fallback.

Parity pins live in tests/test_oracle_*.py.  Parts with no pin beyond the
invariants there are marked "parity unpinned" in their docstrings.
"""
from .model import OracleModel, rmsnorm, rope, attention, swiglu, moe_ffn  # noqa: F401
from .decode import (vocab_stats, credit_update, candidates, select_commits,  # noqa: F401
                     smoothing_state, soft_embedding, run_midpoints)
from .run import OracleRun, run_request  # noqa: F401
