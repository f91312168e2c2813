"""Workload configurations for the DeepSeekMoE layer forward.

Notation follows the DeepSeekMoE reading notes (heloowird.com): N' routed
experts, K' active routed experts per token, K_s shared experts; fine-grained
segmentation splits each of N coarse experts into m experts of width d_ff/m
("core design 1").  Model shapes are the pages' own: the 2B validation model
(1 shared + 63 routed, 1 + 7 active), the 16B model (2 shared + 64 routed,
2 + 6 active, hidden 2048), DeepSeek-V3 (256 routed top-8 + 1 shared, sigmoid
with renormalisation; V4 book ch. 02 sec. 1) and DeepSeek-V4 (384 routed,
top-9, sqrt-softplus scores; V4 book ch. 02 secs. 1-2, hash routing sec. 5).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

SCORINGS = ("softmax", "sigmoid", "sqrt_softplus", "hash")


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int                 # tokens in the batch
    d_model: int           # hidden size d
    n_routed: int          # N'  (= m N)
    top_k: int             # K'  (= m K - K_s)
    n_shared: int          # K_s
    d_ff: int              # routed expert width (coarse width / m)
    d_ff_shared: int       # shared expert width
    scoring: str           # softmax | sigmoid | sqrt_softplus | hash
    renorm: bool           # g = s / sum_selected s
    dtype: str             # "bf16" (fp32 accumulation) | "f32"
    bias: bool = False     # selection bias b_i ~ U(-0.05, 0.05)
    zipf_s: float = 0.0    # Zipf exponent of a per-expert logit offset (0: none)
    alpha1: float = 0.01   # expert-level balance factor
    seed: int = 0
    family: str = ""       # configs sharing a family share their weights
    m: int = 1             # segmentation factor (documentation only)
    n_groups: int = 0      # node-limited routing: expert groups (0: no limit)
    topk_groups: int = 0   # M: groups one token may draw its experts from

    @property
    def weight_family(self) -> str:
        return self.family or self.name

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


CONFIGS = {
    # 16 coarse experts split m=4 -> 64 routed of width 128; 1 shared; top-7.
    "toy_fp32": LayerConfig("toy_fp32", T=512, d_model=256, n_routed=64, top_k=7,
                            n_shared=1, d_ff=128, d_ff_shared=128,
                            scoring="softmax", renorm=False, dtype="f32", m=4),
    # 16B-like: 64 routed top-6 + 2 shared, hidden 2048.
    "mid": LayerConfig("mid", T=4096, d_model=2048, n_routed=64, top_k=6,
                       n_shared=2, d_ff=1408, d_ff_shared=1408,
                       scoring="softmax", renorm=False, dtype="bf16"),
    # DeepSeek-V3-shaped prefill.
    "v3_prefill": LayerConfig("v3_prefill", T=8192, d_model=7168, n_routed=256, top_k=8,
                              n_shared=1, d_ff=2048, d_ff_shared=2048,
                              scoring="sigmoid", renorm=True, dtype="bf16", bias=True,
                              family="v3"),
    # Same layer, decode regime (first 64 tokens of the prefill batch).
    "v3_decode": LayerConfig("v3_decode", T=64, d_model=7168, n_routed=256, top_k=8,
                             n_shared=1, d_ff=2048, d_ff_shared=2048,
                             scoring="sigmoid", renorm=True, dtype="bf16", bias=True,
                             family="v3"),
    # DeepSeek-V4-shaped with a Zipf-skewed logit offset.
    "v4_skew": LayerConfig("v4_skew", T=8192, d_model=7168, n_routed=384, top_k=9,
                           n_shared=1, d_ff=2048, d_ff_shared=2048,
                           scoring="sqrt_softplus", renorm=True, dtype="bf16",
                           zipf_s=1.1, family="v4"),
    # V4 hash-routed variant: expert = fmix32(token_id) mod 384, K' = 1, g = 1.
    "v4_hash": LayerConfig("v4_hash", T=8192, d_model=7168, n_routed=384, top_k=1,
                           n_shared=1, d_ff=2048, d_ff_shared=2048,
                           scoring="hash", renorm=False, dtype="bf16", family="v4"),
}

# The benchmark's headline workload: the V3-shaped prefill layer, T = 8192.
HEADLINE = "v3_prefill"


def scaled(cfg: LayerConfig, T: int, d_model: int | None = None, d_ff: int | None = None,
           name: str | None = None) -> LayerConfig:
    """A smaller copy of a workload (same routing structure), for parity tests
    the oracle finishes in seconds."""
    d = d_model or cfg.d_model
    f = d_ff or cfg.d_ff
    return cfg.with_(name=name or f"{cfg.name}_T{T}_d{d}_f{f}", T=T, d_model=d, d_ff=f,
                     d_ff_shared=f, family="")
