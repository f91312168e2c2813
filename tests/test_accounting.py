"""Accounting helper against the numbers the pages print."""
import json
import os

from fine_grained_moe_router_amd import accounting as acc
from fine_grained_moe_router_amd.configs import CONFIGS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_parameter_ledger_matches_printed_output():
    g = json.load(open(os.path.join(GOLDEN, "param_accounting.json")))
    d, mats = g["d_model"], g["matrices"]
    dense = acc.ffn_params(d, g["dense_d_ff"], mats)
    total, active = acc.moe_params(d, g["expert_d_ff"], g["experts"], g["top_k"], matrices=mats)
    idle = total - active
    p = g["printed_millions"]
    assert f"{dense / 1e6:.2f}" == p["dense"]
    assert f"{total / 1e6:.2f}" == p["moe_total"]
    assert f"{active / 1e6:.2f}" == p["active"]
    assert f"{idle / 1e6:.2f}" == p["idle_if_collapsed_to_2"]
    assert f"{total / dense:.1f}" == g["printed_ratios"]["params"]
    assert f"{active / dense:.1f}" == g["printed_ratios"]["compute"]


def test_segmentation_keeps_flops():
    """k' 2d d_ffn/m = k 2d d_ffn with k' = m k (airsota.com card, sec. 3)."""
    base = CONFIGS["toy_fp32"]
    for m in (1, 2, 4, 8):
        c = base.with_(n_routed=16 * m, top_k=2 * m, d_ff=512 // m, n_shared=0)
        assert acc.layer_flops(c)["routed"] == acc.layer_flops(base.with_(
            n_routed=16, top_k=2, d_ff=512, n_shared=0))["routed"]


def test_v3_flops_are_two_per_active_weight():
    """FLOPs per token = 2 x active parameters (freedeepseekapi.com blog sec. 7)."""
    c = CONFIGS["v3_prefill"]
    _, active = acc.moe_params(c.d_model, c.d_ff, c.n_routed, c.top_k, c.n_shared, c.d_ff_shared)
    fl = acc.layer_flops(c)
    assert fl["routed"] + fl["shared"] == 2 * active * c.T
    assert fl["router"] == 2 * c.d_model * c.n_routed * c.T
    assert abs(fl["total"] / 1e12 - 6.524) < 1e-3
