"""Workload presets: model shape, decode parameters and request mix.

These are the five synthetic workloads the library is measured and checked on.
The model family is the bidirectional (non-causal) transformer of a masked
diffusion LM (dInfer abstract, "model" component; dInfer news article, section
on the "reality shackles" of diffusion models: bidirectional attention).  The
decode parameters drive the parallel-decode strategy of the dInfer news
article, section "解码的艺术" (the art of decoding).

Nothing here computes anything of the method; the values are plain data shared
by the oracle (tests) and the HIP library (bench, tests).

Readings taken where the workload text is silent (each one is listed in the
design notes):
  * MASK id is vocab-1 for every preset (the tiny preset states 4095 of 4096).
  * RMSNorm eps 1e-5, RoPE theta 10000, norm gains 1.
  * Credit weight lambda = 1 (the workload text gives only decay and kappa).
  * Planting for the MoE and long-context presets is not stated; they carry
    the dense 8B preset's +8 bias with probability 0.75.
  * The MoE preset mentions no smoothing, so smoothing is off there (alpha 0).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class ModelCfg:
    n_layers: int
    d_model: int
    n_heads: int
    head_dim: int
    ffn_dim: int            # dense SwiGLU hidden size (0 for MoE layers)
    vocab: int
    mask_id: int
    n_experts: int = 0      # 0 => dense FFN
    top_k: int = 0
    expert_ffn: int = 0
    shared_ffn: int = 0
    rope_theta: float = 10000.0
    rms_eps: float = 1e-5
    dtype: str = "bf16"     # "f32" or "bf16": storage type of weights, KV and activations

    @property
    def is_moe(self) -> bool:
        return self.n_experts > 0


@dataclass(frozen=True)
class DecodeCfg:
    block_len: int
    vicinity_w: int
    tau: float = 0.9
    credit_weight: float = 1.0      # lambda; 0 disables credit
    credit_decay: float = 0.7       # gamma
    credit_kappa: float = 1.5       # kappa
    smooth_alpha: float = 0.3       # 0 disables iteration smoothing
    smooth_topk: int = 8
    hierarchical: bool = False
    min_commit: int = 1
    eos_id: int = -1                # -1: no end-of-sequence token (early stop off)


@dataclass(frozen=True)
class WorkloadCfg:
    name: str
    model: ModelCfg
    decode: DecodeCfg
    batch: int
    prompt_len: tuple          # (lo, hi) inclusive range of prompt lengths
    gen_len: int
    plant_bias: float
    plant_prob: tuple          # (lo, hi): per-request planting probability drawn uniform
    router_pref_bias: float = 0.0   # MoE: per-(layer, block) preferred-expert bias
    router_pref_count: int = 8
    seed: int = 0
    extra: dict = field(default_factory=dict)

    def with_model(self, **kw) -> "WorkloadCfg":
        return replace(self, model=replace(self.model, **kw))

    def with_decode(self, **kw) -> "WorkloadCfg":
        return replace(self, decode=replace(self.decode, **kw))

    def with_(self, **kw) -> "WorkloadCfg":
        return replace(self, **kw)

    @property
    def max_len(self) -> int:
        return self.prompt_len[1] + self.gen_len


_DENSE_8B = dict(n_layers=32, d_model=4096, n_heads=32, head_dim=128, ffn_dim=12288,
                 vocab=126464, mask_id=126463, dtype="bf16")

PRESETS = {
    # Tiny dLLM, fp32, batch 1; the oracle finishes a whole run in seconds.
    "tiny_f32": WorkloadCfg(
        name="tiny_f32",
        model=ModelCfg(n_layers=2, d_model=256, n_heads=4, head_dim=64, ffn_dim=768,
                       vocab=4096, mask_id=4095, dtype="f32"),
        decode=DecodeCfg(block_len=32, vicinity_w=8, tau=0.9, smooth_alpha=0.3),
        batch=1, prompt_len=(64, 64), gen_len=64, plant_bias=6.0, plant_prob=(0.7, 0.7),
        seed=0),
    # Dense 8B shape, bf16, batch 1.
    "dense8b_b1": WorkloadCfg(
        name="dense8b_b1",
        model=ModelCfg(**_DENSE_8B),
        decode=DecodeCfg(block_len=32, vicinity_w=16, tau=0.9, smooth_alpha=0.3),
        batch=1, prompt_len=(512, 512), gen_len=256, plant_bias=8.0, plant_prob=(0.75, 0.75),
        seed=1),
    # Dense 8B shape, bf16, batch 16 with step-level batching.
    "dense8b_b16": WorkloadCfg(
        name="dense8b_b16",
        model=ModelCfg(**_DENSE_8B),
        decode=DecodeCfg(block_len=32, vicinity_w=16, tau=0.9, smooth_alpha=0.3),
        batch=16, prompt_len=(128, 1024), gen_len=256, plant_bias=8.0, plant_prob=(0.5, 0.9),
        seed=2),
    # MoE dLLM, bf16, batch 1.
    "moe_b1": WorkloadCfg(
        name="moe_b1",
        model=ModelCfg(n_layers=20, d_model=2048, n_heads=16, head_dim=128, ffn_dim=0,
                       vocab=157184, mask_id=157183, n_experts=64, top_k=8,
                       expert_ffn=1024, shared_ffn=2048, dtype="bf16"),
        decode=DecodeCfg(block_len=64, vicinity_w=32, tau=0.9, smooth_alpha=0.0),
        batch=1, prompt_len=(1024, 1024), gen_len=1024, plant_bias=8.0, plant_prob=(0.75, 0.75),
        router_pref_bias=2.0, router_pref_count=8, seed=3),
    # Long-context dense 8B shape, bf16, batch 4, hierarchical order.
    "dense8b_long_b4": WorkloadCfg(
        name="dense8b_long_b4",
        model=ModelCfg(**_DENSE_8B),
        decode=DecodeCfg(block_len=64, vicinity_w=32, tau=0.85, smooth_alpha=0.3,
                         hierarchical=True),
        batch=4, prompt_len=(8192, 8192), gen_len=1024, plant_bias=8.0, plant_prob=(0.75, 0.75),
        seed=4),
}

PRESET_ORDER = ["tiny_f32", "dense8b_b1", "dense8b_b16", "moe_b1", "dense8b_long_b4"]


def preset(name_or_index) -> WorkloadCfg:
    if isinstance(name_or_index, int):
        return PRESETS[PRESET_ORDER[name_or_index]]
    return PRESETS[name_or_index]
