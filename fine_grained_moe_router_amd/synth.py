"""Seeded synthetic inputs for the MoE layer (shared by the HIP path's tests,
the oracle's tests and the benchmark).

This module draws random numbers and nothing else: it holds none of the
layer's arithmetic.  Every tensor is built from blocks, each drawn from its
own torch generator whose seed is a hash of (config seed, weight family,
tensor name, block index), so that
  * a single expert's weights can be regenerated without the rest,
  * the decode workload reuses the prefill weights and its first 64 tokens,
  * the same call on the same device type returns the same bytes.
CPU and GPU generators produce different (but each reproducible) streams; a
test always hands the very same bytes to both sides.

Distributions (variance 1/fan_in for expert weights; 0.02 is the router's
standard deviation):
  x ~ N(0, 1); W1, W3 ~ N(0, 1/d); W2 ~ N(0, 1/d_ff); W_g ~ N(0, 0.02^2);
  b ~ U(-0.05, 0.05) (fp32); token ids ~ U{0, ..., 129279} (u32);
  Zipf offset: o_i = -s ln(r_i) for a seeded random permutation r of the ranks
  1..N', centred to mean zero (the log of a Zipf(s) weight, as a logit offset).
bf16 tensors are fp32 draws rounded to nearest-even.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass
from typing import Optional

import torch

from .configs import LayerConfig

TOKEN_BLOCK = 64          # tokens per x / token-id block
VOCAB = 129280            # token-id range of the hash-routed workload


def _seed(*parts) -> int:
    h = hashlib.blake2b(repr(parts).encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def _torch_dtype(cfg: LayerConfig):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def _normal(shape, std, gen, device, dtype):
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


@dataclass
class LayerInputs:
    cfg: LayerConfig
    x: torch.Tensor                 # [T][d]
    w_gate: Optional[torch.Tensor]  # [N'][d] (None under hash routing)
    w13: torch.Tensor               # [N'][2f][d]
    w2: torch.Tensor                # [N'][d][f]
    w13s: torch.Tensor              # [K_s][2fs][d]
    w2s: torch.Tensor               # [K_s][d][fs]
    bias: Optional[torch.Tensor]    # [N'] fp32
    offset: Optional[torch.Tensor]  # [N'] fp32
    token_ids: Optional[torch.Tensor]  # [T] int32 holding u32 values


def make_x(cfg: LayerConfig, device="cpu", T: Optional[int] = None) -> torch.Tensor:
    T = cfg.T if T is None else T
    dt = _torch_dtype(cfg)
    out = torch.empty((T, cfg.d_model), dtype=dt, device=device)
    dev = torch.device(device).type
    for b0 in range(0, T, TOKEN_BLOCK):
        n = min(TOKEN_BLOCK, T - b0)
        g = _gen(device, cfg.seed, cfg.weight_family, "x", dev, b0 // TOKEN_BLOCK)
        blk = _normal((TOKEN_BLOCK, cfg.d_model), 1.0, g, device, dt)
        out[b0:b0 + n] = blk[:n]
    return out


def make_token_ids(cfg: LayerConfig, device="cpu") -> torch.Tensor:
    out = torch.empty(cfg.T, dtype=torch.int64, device=device)
    dev = torch.device(device).type
    for b0 in range(0, cfg.T, TOKEN_BLOCK):
        n = min(TOKEN_BLOCK, cfg.T - b0)
        g = _gen(device, cfg.seed, cfg.weight_family, "token_ids", dev, b0 // TOKEN_BLOCK)
        blk = torch.randint(0, VOCAB, (TOKEN_BLOCK,), generator=g, device=device)
        out[b0:b0 + n] = blk[:n]
    return out.to(torch.int32)


def make_expert(cfg: LayerConfig, e: int, device="cpu", shared: bool = False):
    """(w13 [2f][d], w2 [d][f]) of routed expert e, or of shared expert e."""
    dt = _torch_dtype(cfg)
    d = cfg.d_model
    f = cfg.d_ff_shared if shared else cfg.d_ff
    kind = "shared" if shared else "routed"
    dev = torch.device(device).type
    g = _gen(device, cfg.seed, cfg.weight_family, kind, dev, d, f, e)
    w13 = _normal((2 * f, d), d ** -0.5, g, device, dt)
    w2 = _normal((d, f), f ** -0.5, g, device, dt)
    return w13, w2


def make_inputs(cfg: LayerConfig, device="cpu", experts: bool = True) -> LayerInputs:
    """All inputs of one layer forward on ``device``.  experts=False skips the
    expert weights (routing-only callers)."""
    dt = _torch_dtype(cfg)
    dev = torch.device(device).type
    d, N = cfg.d_model, cfg.n_routed
    x = make_x(cfg, device)
    w_gate = None
    if cfg.scoring != "hash":
        g = _gen(device, cfg.seed, cfg.weight_family, "w_gate", dev, d, N)
        w_gate = _normal((N, d), 0.02, g, device, dt)
    f, fs = cfg.d_ff, cfg.d_ff_shared
    if experts:
        w13 = torch.empty((N, 2 * f, d), dtype=dt, device=device)
        w2 = torch.empty((N, d, f), dtype=dt, device=device)
        for e in range(N):
            w13[e], w2[e] = make_expert(cfg, e, device)
        w13s = torch.empty((cfg.n_shared, 2 * fs, d), dtype=dt, device=device)
        w2s = torch.empty((cfg.n_shared, d, fs), dtype=dt, device=device)
        for j in range(cfg.n_shared):
            w13s[j], w2s[j] = make_expert(cfg, j, device, shared=True)
    else:
        w13 = w2 = w13s = w2s = None
    bias = None
    if cfg.bias:
        g = _gen(device, cfg.seed, cfg.weight_family, "bias", dev, N)
        bias = (torch.rand(N, generator=g, device=device) * 0.1 - 0.05).float()
    offset = None
    if cfg.zipf_s:
        g = _gen("cpu", cfg.seed, cfg.weight_family, "zipf_perm", N)
        ranks = torch.randperm(N, generator=g).double() + 1.0
        o = -cfg.zipf_s * torch.log(ranks)
        offset = (o - o.mean()).float().to(device)
    token_ids = make_token_ids(cfg, device) if cfg.scoring == "hash" else None
    return LayerInputs(cfg, x, w_gate, w13, w2, w13s, w2s, bias, offset, token_ids)


def to_numpy(t: Optional[torch.Tensor]):
    """Host numpy view of a tensor: bf16 becomes its uint16 bit pattern."""
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()


def make_share_routing(rows: int, n_local: int, top_k: int, seed: int = 0):
    """A seeded caller routing of the shape one GPU receives under expert
    parallelism (host tensors): row r names c_r distinct experts of the
    n_local resident ones, c_r uniform in 1..top_k, in random slots; the
    other slots hold -1 (no expert); gates uniform in [0, 1)."""
    g = _gen("cpu", seed, "share_routing", rows, n_local, top_k)
    n = torch.randint(1, top_k + 1, (rows,), generator=g)
    experts = torch.argsort(torch.rand((rows, n_local), generator=g), dim=1)[:, :top_k]
    slots = torch.argsort(torch.rand((rows, top_k), generator=g), dim=1)
    keep = torch.arange(top_k).unsqueeze(0) < n.unsqueeze(1)
    idx = torch.full((rows, top_k), -1, dtype=torch.int32)
    idx.scatter_(1, slots, torch.where(keep, experts, -1).to(torch.int32))
    gate = torch.rand((rows, top_k), generator=g).float()
    return idx, gate

