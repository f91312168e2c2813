"""Parameter, FLOP and byte accounting for one MoE layer forward.

* Parameters: an FFN of width f on hidden size d holds ``matrices * d * f``
  weights (2 for the classic up/down pair used in the parameter-accounting
  exercise of the MoE tutorial at ai.clawlihai.cn, 3 for SwiGLU).
* FLOPs: two per multiply-accumulate, i.e. two per active weight per token
  (the FLOPs comparison in sec. 7 of the freedeepseekapi.com MoE blog).
  Fine-grained segmentation keeps the count: K' = mK experts of width f/m
  cost what K experts of width f cost (airsota.com card, sec. 3).
* Algorithmic bytes: what the method must move at least once -- the weights
  of every expert that receives a token, the shared experts, W_g, the input
  x and the output h.  Re-reads, permutation buffers and workspace are
  implementation overhead and are not counted.
"""
from __future__ import annotations

from .configs import LayerConfig


def ffn_params(d_model: int, d_ff: int, matrices: int = 3) -> int:
    return matrices * d_model * d_ff


def moe_params(d_model: int, d_ff: int, n_experts: int, top_k: int,
               n_shared: int = 0, d_ff_shared: int = 0, matrices: int = 3):
    """(total, active) expert parameters of one MoE layer (router excluded)."""
    e = ffn_params(d_model, d_ff, matrices)
    s = ffn_params(d_model, d_ff_shared, matrices) if n_shared else 0
    return n_experts * e + n_shared * s, top_k * e + n_shared * s


def elem_bytes(cfg: LayerConfig) -> int:
    return 2 if cfg.dtype == "bf16" else 4


def layer_flops(cfg: LayerConfig) -> dict:
    T, d = cfg.T, cfg.d_model
    router = 0 if cfg.scoring == "hash" else 2 * T * d * cfg.n_routed
    routed = 6 * d * cfg.d_ff * T * cfg.top_k
    shared = 6 * d * cfg.d_ff_shared * T * cfg.n_shared
    return {"router": router, "routed": routed, "shared": shared,
            "total": router + routed + shared}


def expert_gemm_flops(cfg: LayerConfig) -> dict:
    """FLOPs of the two expert contractions (gate/up, then down), routed and
    shared together."""
    T, d = cfg.T, cfg.d_model
    rows_f = T * cfg.top_k * cfg.d_ff + T * cfg.n_shared * cfg.d_ff_shared
    return {"gate_up": 2 * d * 2 * rows_f, "down": 2 * d * rows_f}


def layer_bytes(cfg: LayerConfig, experts_touched: int) -> dict:
    """Algorithmic HBM bytes given how many routed experts received a token."""
    eb = elem_bytes(cfg)
    d = cfg.d_model
    routed_w = experts_touched * 3 * d * cfg.d_ff * eb
    shared_w = cfg.n_shared * 3 * d * cfg.d_ff_shared * eb
    router_w = 0 if cfg.scoring == "hash" else cfg.n_routed * d * eb
    act = 2 * cfg.T * d * eb
    return {"routed_weights": routed_w, "shared_weights": shared_w,
            "router_weights": router_w, "activations": act,
            "total": routed_w + shared_w + router_w + act}


def gemm_bytes(cfg: LayerConfig, experts_touched: int) -> dict:
    """Algorithmic bytes of each expert contraction: its weights once, its
    activation operand once and its output once."""
    eb = elem_bytes(cfg)
    d, T = cfg.d_model, cfg.T
    rows = T * cfg.top_k
    w13 = (experts_touched * 2 * cfg.d_ff + cfg.n_shared * 2 * cfg.d_ff_shared) * d * eb
    w2 = (experts_touched * cfg.d_ff + cfg.n_shared * cfg.d_ff_shared) * d * eb
    z = (rows * cfg.d_ff + T * cfg.n_shared * cfg.d_ff_shared) * eb
    return {"gate_up": w13 + T * d * eb + z, "down": w2 + z + (rows + T) * d * eb}
