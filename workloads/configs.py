"""Drafter shapes and workloads used by the tests and the benchmark.

Pure data: no arithmetic of the method lives here.  The five workloads are the
shapes the DFlash pages talk about (a 5-layer drafter for Qwen3-8B and
LLaMA-3.1-8B targets, gpt-oss-120b for the long-context case, block size 16
from the "-b16" checkpoint name on the DFlash wiki page, "Usage") plus a tiny
fp32 model that the oracle finishes in seconds.

Readings for values the pages leave open (stated once here, used everywhere):
  * the mask token is the last vocabulary id;
  * RMSNorm epsilon is 1e-6;
  * the LLaMA-3.1-8B-shaped drafter fuses 5 target layers of width 4096;
  * the gpt-oss-120b-shaped drafter uses RoPE theta 1.5e5.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

BLOCK = 16      # anchor + 15 masked slots ("b16" drafters)
PAGE = 16       # tokens per KV-cache page


@dataclass(frozen=True)
class DrafterConfig:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    n_feat_layers: int          # number of target layers whose hidden states are fused
    target_hidden: int          # width of one target layer's hidden state
    rope_theta: float
    dtype: str                  # "f32" or "bf16": storage and MFMA operand type
    rms_eps: float = 1e-6
    block_size: int = BLOCK
    page_size: int = PAGE
    mask_token_id: Optional[int] = None

    @property
    def feat_dim(self) -> int:
        return self.n_feat_layers * self.target_hidden

    @property
    def mask_id(self) -> int:
        return self.vocab - 1 if self.mask_token_id is None else self.mask_token_id

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def weight_shapes(self) -> dict:
        """Logical nn.Linear shapes [out, in] of every tensor of the drafter."""
        H, F, V, I = self.hidden, self.feat_dim, self.vocab, self.intermediate
        s = {
            "w_fuse": (H, F),
            "embed": (V, H),
            "lm_head": (V, H),
            "final_norm": (H,),
        }
        for l in range(self.n_layers):
            s[f"attn_norm.{l}"] = (H,)
            s[f"wq.{l}"] = (self.q_dim, H)
            s[f"wk.{l}"] = (self.kv_dim, H)
            s[f"wv.{l}"] = (self.kv_dim, H)
            s[f"wo.{l}"] = (H, self.q_dim)
            s[f"mlp_norm.{l}"] = (H,)
            s[f"w_gate.{l}"] = (I, H)
            s[f"w_up.{l}"] = (I, H)
            s[f"w_down.{l}"] = (H, I)
        return s

    def n_params(self, include_embed: bool = True) -> int:
        tot = 0
        for k, shp in self.weight_shapes().items():
            if k == "embed" and not include_embed:
                continue
            n = 1
            for x in shp:
                n *= x
            tot += n
        return tot


@dataclass(frozen=True)
class Workload:
    name: str
    cfg: DrafterConfig
    batch: int
    ctx: Tuple[int, int]        # context length range [lo, hi], inclusive; lo == hi for fixed
    verify: str = "greedy"      # "greedy" or "sampled"
    logit_std: float = 2.0      # sampled verify: std of the synthetic draft/target logits
    seed: int = 0
    notes: str = ""

    @property
    def fixed_ctx(self) -> bool:
        return self.ctx[0] == self.ctx[1]

    @property
    def max_ctx(self) -> int:
        return self.ctx[1]


TINY = DrafterConfig(
    name="tiny-f32", n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
    intermediate=768, vocab=4096, n_feat_layers=3, target_hidden=256, rope_theta=1e4,
    dtype="f32")

QWEN3_8B = DrafterConfig(
    name="qwen3-8b-shaped", n_layers=5, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
    intermediate=12288, vocab=151936, n_feat_layers=5, target_hidden=4096, rope_theta=1e6,
    dtype="bf16")

LLAMA31_8B = DrafterConfig(
    name="llama3.1-8b-shaped", n_layers=5, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
    intermediate=14336, vocab=128256, n_feat_layers=5, target_hidden=4096, rope_theta=5e5,
    dtype="bf16")

GPT_OSS_120B = DrafterConfig(
    name="gpt-oss-120b-shaped", n_layers=5, hidden=2880, n_q_heads=64, n_kv_heads=8, head_dim=64,
    intermediate=8192, vocab=201088, n_feat_layers=3, target_hidden=2880, rope_theta=1.5e5,
    dtype="bf16")

WORKLOADS = {
    "tiny": Workload("tiny-f32-b1-ctx128", TINY, batch=1, ctx=(128, 128)),
    "qwen3_b1": Workload("qwen3-8b-shaped-b16-drafter-batch1-ctx2048", QWEN3_8B, batch=1,
                         ctx=(2048, 2048)),
    "qwen3_b32": Workload("qwen3-8b-shaped-b16-drafter-batch32-ctx512..8192-paged", QWEN3_8B,
                          batch=32, ctx=(512, 8192)),
    "llama_b64": Workload("llama3.1-8b-shaped-b16-drafter-batch64-ctx4096-temp1", LLAMA31_8B,
                          batch=64, ctx=(4096, 4096), verify="sampled"),
    "gptoss_b128": Workload("gpt-oss-120b-shaped-b16-drafter-batch128-ctx32768", GPT_OSS_120B,
                            batch=128, ctx=(32768, 32768)),
}


def scaled(cfg: DrafterConfig, **kw) -> DrafterConfig:
    """A copy of `cfg` with some fields replaced (used for small test variants)."""
    return replace(cfg, **kw)
