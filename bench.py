#!/usr/bin/env python3
"""Throughput of one DeepSeekMoE layer forward on one MI355X.

A step is one pass of the whole hot path over one batch: moe_route (router
GEMM, scores, selection bias, top-K', gates, counts), moe_forward
(permutation, grouped gate/up GEMM + SwiGLU, grouped down GEMM with the shared
experts folded in, combine + residual) and moe_balance_stats (f_i, P_i,
L_ExpBal).  Inputs are seeded synthetic tensors already resident in HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  `roofline` describes the dominant kernel, timed with
HIP events recorded by the library around each stage during the timed steps;
`cpu_baseline` is the CPU oracle timed on a bounded sample of the same
workload.  Other modes:
    --pmc-summary DIR   turn two `rocprofv3 --pmc` runs (FETCH_SIZE, then
                        WRITE_SIZE; their output folders DIR/fetch, DIR/write)
                        of `bench.py --pmc-run` into a traffic record under
                        profiles/.
    --extras            one JSON line timing node-limited routing, the
                        in-sequence and device-level statistics and the
                        bias update on the workload's inputs.
    --calibrate         one JSON line timing bf16 GEMMs of the layer's
                        expert-GEMM FLOP counts through the vendor library
                        (torch.matmul / torch.bmm), the attainable-rate
                        reference of the GPU the layer runs on.
    --ep-share G        one JSON line timing one GPU's share of the layer
                        under expert parallelism over G GPUs: the router on
                        its own T tokens, its N'/G resident experts on the
                        pairs that G T tokens send it, the shared expert on
                        its own tokens (the exchange itself is not run).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
COPY_BYTES = 1 << 30           # calibration copy: reads COPY_BYTES/2, writes COPY_BYTES/2

# Dominant kernel per stage name, with the symbol rocprofv3 reports for it.
KERNEL_OF_STAGE = {"gate_up": "k_gate_up_bf16", "down": "k_down_bf16"}

# Which roof binds each workload's expert GEMMs, from its arithmetic
# intensity against MI355X's ridge (2.5 PF / 8 TB/s = 312 FLOP per byte):
# about 384 rows per expert weight (mid) and 256 (V3 prefill, at the ridge)
# are compute-bound, 192 rows (V4 skew, Zipf-hot and -cold experts), 21 rows
# (V4 hash, K' = 1) and 2 rows (V3 decode) are bound by streaming weights.
BOUND = {"mid": "mfma", "v3_prefill": "mfma", "v3_decode": "hbm", "v4_skew": "hbm",
         "v4_hash": "hbm"}


# Sources that decide what the grouped GEMM kernels do (their code, their
# work lists and their launch arguments): a traffic record is valid for the
# kernel only while these are unchanged.
GEMM_SOURCES = ("common.h", "mfma_pipe.h", "expert_gemm.hip", "permute.hip", "api.hip")


def _code_only(text: str) -> str:
    """The source without comments and blank space: what decides the kernels
    (string literals in these sources hold no comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest() -> str:
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "fine_grained_moe_router_amd", "csrc", name), encoding="utf-8") as fh:
            h.update(name.encode())
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def traffic_record_path(workload: str, stage: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{KERNEL_OF_STAGE.get(stage, stage)}_{workload}.json")


def read_traffic(workload: str, stage: str):
    """HBM bytes per launch of the stage's kernel from the committed PMC
    record, or None if absent or taken on different GEMM sources."""
    p = traffic_record_path(workload, stage)
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        rec = json.load(fh)
    if rec.get("source_digest") != source_digest():
        return None
    return rec.get("traffic_bytes_per_launch")


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="v3_prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replayed timing of the same step")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the CPU-oracle sample")
    ap.add_argument("--pmc-run", action="store_true",
                    help="short run for rocprofv3 --pmc: a calibration copy plus a few steps")
    ap.add_argument("--pmc-summary", default=None)
    ap.add_argument("--clock-summary", default=None,
                    help="directory of a rocprofv3 --pmc GRBM_GUI_ACTIVE run of the layer step: "
                         "write the effective clock of its long kernels to profiles/")
    ap.add_argument("--extras", action="store_true",
                    help="time the entry points beyond the layer step (node-limited routing, "
                         "in-sequence and device-level statistics, bias update) instead")
    ap.add_argument("--ep-share", type=int, default=0, metavar="G",
                    help="time one GPU's share of the layer under expert parallelism over G GPUs")
    ap.add_argument("--calibrate", action="store_true",
                    help="time dense and batched bf16 GEMMs of the layer's expert-GEMM FLOP "
                         "counts through torch.matmul / torch.bmm (hipBLASLt), as the "
                         "attainable-rate reference of this GPU")
    return ap.parse_args(argv)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class Layer:
    """Inputs, outputs and workspaces of one workload, allocated once."""

    def __init__(self, cfg, device="cuda"):
        import torch
        from fine_grained_moe_router_amd import binding as B
        from fine_grained_moe_router_amd.synth import make_inputs

        self.B, self.cfg = B, cfg
        self.inp = make_inputs(cfg, device)
        T, N, K = cfg.T, cfg.n_routed, cfg.top_k
        hashed = cfg.scoring == "hash"
        c0 = B.make_config(cfg)
        self.route_out = {
            "idx": torch.empty((T, K), dtype=torch.int32, device=device),
            "w": torch.empty((T, K), dtype=torch.float32, device=device),
            "counts": torch.empty(N, dtype=torch.int32, device=device),
            "pstat": None if hashed else torch.empty(B.workspace_bytes(c0, B.WS_PSTAT), dtype=torch.uint8, device=device),
        }
        self.ws_route = B.alloc_workspace(c0, B.WS_ROUTE, device)
        self.ws_fwd = B.alloc_workspace(c0, B.WS_FORWARD, device)
        self.h = torch.empty_like(self.inp.x)
        self.stats_out = {"f": torch.empty(N, dtype=torch.float32, device=device),
                          "P": torch.empty(N, dtype=torch.float32, device=device),
                          "loss": torch.empty(2, dtype=torch.float32, device=device)}

    def step(self):
        B, cfg, inp = self.B, self.cfg, self.inp
        hashed = cfg.scoring == "hash"
        r = B.route(cfg, x=inp.x, w_gate=inp.w_gate, offset=inp.offset, bias=inp.bias,
                    token_ids=inp.token_ids, want_pstat=not hashed, out=self.route_out,
                    workspace=self.ws_route)
        B.forward(cfg, inp.x, r["idx"], r["w"], inp.w13, inp.w2, inp.w13s, inp.w2s, h=self.h,
                  workspace=self.ws_fwd)
        B.balance_stats(cfg, r["counts"], r["pstat"], want_P=not hashed, want_loss=not hashed,
                        out=self.stats_out)
        return r


def graph_step_ms(layer, steps: int) -> float:
    """The same step captured once in a HIP graph and replayed: ms per
    replay over `steps` replays (no launch overhead between the kernels).
    Reported beside the eagerly launched step, which `value` is."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.step()
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1000.0 / steps


def cold_step_ms(layer, steps: int) -> float:
    """Median ms of one step timed alone with HIP events on torch's stream
    (where the binding launches), each after writing a 512 MiB buffer, so
    that neither L2 nor the 256 MB Infinity Cache still holds the previous
    step's inputs or weights.  Reported beside the back-to-back step."""
    import statistics
    import torch
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for i in range(steps):
        flush.fill_(i & 0xFF)
        e0.record()
        layer.step()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del flush
    return statistics.median(times)


def cpu_baseline(layer, target_s: float):
    """The CPU oracle (as it stands) on the first S tokens of the same
    workload: router logits, routing and the layer output, double precision."""
    import numpy as np
    from oracle import oracle as O
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import host, host_experts

    cfg, inp = layer.cfg, layer.inp
    x_h = host(inp.x)
    wg_h = host(inp.w_gate)
    off_h, b_h = host(inp.offset), host(inp.bias)
    tid_h = None if inp.token_ids is None else host(inp.token_ids).view(np.uint32)
    w13s, w2s = host(inp.w13s), host(inp.w2s)

    def run(n):
        """Oracle wall time for tokens 0..n-1 (expert copies to the host are
        not timed)."""
        tokens = np.arange(n)
        t0 = time.perf_counter()
        if cfg.scoring == "hash":
            idx, gate, _, _ = O.route(None, cfg.n_routed, 1, "hash", False, token_ids=tid_h[:n])
        else:
            lg = O.router_logits(x_h, wg_h, tokens=tokens)
            idx, gate, _, _ = O.route(lg, cfg.n_routed, cfg.top_k, cfg.scoring, cfg.renorm,
                                      offset=off_h, bias=b_h)
        t_route = time.perf_counter() - t0
        need = np.unique(idx)
        w13 = host_experts(inp.w13, need)
        w2 = host_experts(inp.w2, need)
        idx_full = np.zeros((cfg.T, cfg.top_k), np.int32)
        gate_full = np.zeros((cfg.T, cfg.top_k), np.float32)
        idx_full[:n], gate_full[:n] = idx, gate
        t1 = time.perf_counter()
        O.forward(x_h, idx_full, gate_full, w13, w2, w13s, w2s, tokens=tokens)
        return t_route + time.perf_counter() - t1

    probe = max(4, O.threads()) if cfg.d_model >= 4096 else 64
    dt = run(probe)
    n = int(max(probe, min(cfg.T, probe * target_s / max(dt, 1e-3))))
    dt2 = run(n) if n > probe else dt
    return {"value": n / dt2, "unit": "tokens/s", "cores": O.threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"router logits, routing and layer output of the first {n} of {cfg.T} "
                      f"tokens ({cfg.name}), double-precision C oracle, {dt2:.1f} s wall"}


def pmc_summary(out_dir: str, workload: str, stage: str = "gate_up"):
    """Combine FETCH_SIZE / WRITE_SIZE counter runs into a traffic record."""
    from fine_grained_moe_router_amd.configs import CONFIGS
    kernel = KERNEL_OF_STAGE[stage]

    def load(sub, counter):
        rows = []
        for p in glob.glob(os.path.join(out_dir, sub, "**", "*counter_collection.csv"), recursive=True):
            with open(p) as fh:
                rows += [r for r in csv.DictReader(fh) if r.get("Counter_Name") == counter]
        if not rows:
            raise SystemExit(f"no {counter} rows under {out_dir}/{sub}")
        by = {}
        for r in rows:
            key = (r["Kernel_Name"], r.get("Dispatch_Id", r.get("Correlation_Id")))
            by[key] = by.get(key, 0.0) + float(r["Counter_Value"])
        return by

    res = {}
    for sub, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        by = load(sub, counter)
        copy = [v for (k, _), v in by.items() if "copy" in k.lower() or "elementwise" in k.lower()]
        kern = [v for (k, _), v in by.items() if kernel in k]
        if not copy or not kern:
            raise SystemExit(f"{counter}: copy or {kernel} dispatches missing")
        copy_kib = max(copy)
        factor = (COPY_BYTES / 2 / 1024.0) / copy_kib    # true KiB per counted KiB
        res[counter] = {"kernel_kib_per_launch": sum(kern) / len(kern), "copy_kib": copy_kib,
                        "scale": factor, "launches": len(kern)}
    traffic = sum(res[c]["kernel_kib_per_launch"] * res[c]["scale"] * 1024.0 for c in res)
    rec = {"kernel": kernel, "workload": workload, "config": CONFIGS[workload].__dict__,
           "counters": res, "traffic_bytes_per_launch": traffic,
           "copy_bytes": COPY_BYTES, "source_digest": source_digest(),
           "commands": [
               f"rocprofv3 --pmc FETCH_SIZE -d {out_dir}/fetch -o run --output-format csv -- python3 bench.py --pmc-run --workload {workload}",
               f"rocprofv3 --pmc WRITE_SIZE -d {out_dir}/write -o run --output-format csv -- python3 bench.py --pmc-run --workload {workload}",
               f"python3 bench.py --pmc-summary {out_dir} --workload {workload}"]}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(traffic_record_path(workload, stage), "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps({"traffic_bytes_per_launch": traffic, "record": traffic_record_path(workload, stage)}))


def clock_summary(out_dir: str, workload: str, min_ms: float = 0.5, path: str | None = None):
    """Effective clock of the kernels of a rocprofv3 --pmc GRBM_GUI_ACTIVE run:
    GPU-active cycles (summed over the XCDs, so divided by their count) over
    the dispatch's duration.  Only dispatches of at least min_ms count: the
    counter window is wider than the kernel, which inflates short ones."""
    rows, n_xcc = [], None
    for p in glob.glob(os.path.join(out_dir, "**", "*agent_info.csv"), recursive=True):
        with open(p) as fh:
            for r in csv.DictReader(fh):
                if r.get("Agent_Type") == "GPU" and r.get("Num_Xcc"):
                    n_xcc = int(r["Num_Xcc"])
    for p in glob.glob(os.path.join(out_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(p) as fh:
            rows += [r for r in csv.DictReader(fh) if r.get("Counter_Name") == "GRBM_GUI_ACTIVE"]
    if not rows or not n_xcc:
        raise SystemExit(f"no GRBM_GUI_ACTIVE rows or GPU agent under {out_dir}")
    by = {}
    for r in rows:
        ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        if ns >= min_ms * 1e6:
            name = r["Kernel_Name"].split("(")[0].replace("void ", "")
            by.setdefault(name, []).append((float(r["Counter_Value"]) / n_xcc / ns, ns / 1e6))
    out = {}
    for name, v in sorted(by.items()):
        ghz = sorted(g for g, _ in v)
        out[name] = {"dispatches": len(v), "ghz_median": round(ghz[len(ghz) // 2], 3),
                     "ghz_min": round(ghz[0], 3), "ghz_max": round(ghz[-1], 3),
                     "ms_median": round(sorted(m for _, m in v)[len(v) // 2], 3)}
    rec = {"workload": workload, "xcds": n_xcc, "kernels": out,
           "commands": [f"rocprofv3 --pmc GRBM_GUI_ACTIVE -d {out_dir} -o run --output-format csv -- "
                        f"python3 bench.py --workload {workload} --no-cpu-baseline",
                        f"python3 bench.py --clock-summary {out_dir} --workload {workload}"]}
    path = path or os.path.join(ROOT, "profiles", f"clock_{workload}.json")
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps({"record": path, "kernels": out}))


def time_calls(fn, reps=50):
    """Average ms of fn() over reps calls, HIP events on torch's current
    stream (the binding launches on that stream)."""
    import torch
    for _ in range(3):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def extras(cfg):
    """One JSON line timing the entry points beyond the layer step on the
    workload's own inputs: node-limited routing (8 groups, M = 4) against
    plain routing, moe_seq_balance_stats over 8 equal segments,
    moe_device_balance_stats over 8 devices, moe_bias_update."""
    import torch
    from fine_grained_moe_router_amd import binding as B
    from fine_grained_moe_router_amd.synth import make_inputs

    inp = make_inputs(cfg, "cuda", experts=False)
    T, N, K = cfg.T, cfg.n_routed, cfg.top_k
    grouped = cfg.with_(n_groups=8, topk_groups=4)
    res = {}
    for name, c in (("route_plain", cfg), ("route_node_limited", grouped)):
        ws = B.alloc_workspace(B.make_config(c), B.WS_ROUTE, "cuda")
        out = {"idx": torch.empty((T, K), dtype=torch.int32, device="cuda"),
               "w": torch.empty((T, K), dtype=torch.float32, device="cuda"),
               "counts": torch.empty(N, dtype=torch.int32, device="cuda"),
               "pstat": torch.empty(B.workspace_bytes(B.make_config(c), B.WS_PSTAT),
                                    dtype=torch.uint8, device="cuda")}

        def call(c=c, ws=ws, out=out):
            B.route(c, x=inp.x, w_gate=inp.w_gate, offset=inp.offset, bias=inp.bias, out=out,
                    workspace=ws)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        B.profile_enable(400)
        n = 50
        for _ in range(n):
            call()
        torch.cuda.synchronize()
        st = B.profile_collect()
        res[name] = {"select_us": st["select"]["ms"] / n * 1e3,
                     "router_gemm_us": st["router_gemm"]["ms"] / n * 1e3}
    sel = res["route_node_limited"]["select_us"]
    # the select stage reads the logits and writes K' (index, gate) pairs per token
    sel_bytes = T * N * 4 + T * K * 8
    res["route_node_limited"].update(bound="latency", bytes=sel_bytes,
                                     gbs=sel_bytes / (sel * 1e-6) / 1e9)

    r = B.route(cfg, x=inp.x, w_gate=inp.w_gate, offset=inp.offset, bias=inp.bias,
                logits_out=True)
    S = 8
    segs = torch.tensor([i * T // S for i in range(S + 1)], dtype=torch.int32, device="cuda")
    ws = B.alloc_workspace(B.make_config(cfg), B.WS_SEQSTAT, "cuda")
    outs = {"f_seq": torch.empty((S, N), device="cuda"), "p_seq": torch.empty((S, N), device="cuda"),
            "loss": torch.empty(S, device="cuda")}
    ms = time_calls(lambda: B.seq_balance_stats(cfg, r["logits"], r["idx"], segs, 1e-4,
                                                offset=inp.offset, out=outs, workspace=ws))
    alg = T * N * 4 + T * K * 4 + 2 * S * N * 4 + S * 4      # logits, idx in; f, p, loss out
    res["seq_balance_stats"] = {"segments": S, "us": ms * 1e3, "bound": "hbm",
                                "algorithmic_bytes": alg, "gbs": alg / (ms * 1e-3) / 1e9,
                                "frac": alg / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                "implementation_bytes": alg + 2 * T * N * 4}
    f, P, _ = B.balance_stats(cfg, r["counts"], r["pstat"])
    ms = time_calls(lambda: B.device_balance_stats(cfg, f, P, 8, 0.05))
    res["device_balance_stats"] = {"devices": 8, "us": ms * 1e3, "bound": "latency"}
    bias = inp.bias.clone() if inp.bias is not None else torch.zeros(N, device="cuda")
    ms = time_calls(lambda: B.bias_update(cfg, r["counts"], T, 1e-3, bias))
    res["bias_update"] = {"us": ms * 1e3, "bound": "latency"}
    print(json.dumps({"mode": "extras", "workload": cfg.name, "T": T, "n_routed": N,
                      "top_k": K, "entries": res}))
    return 0


def ep_share(cfg, gpus: int, steps: int, warmup: int):
    """One JSON line: one GPU's share of the layer under expert parallelism
    over `gpus` GPUs, at its real shape, with the kernels of the layer step.

    Routed experts are split evenly and contiguously over the GPUs (GPU g
    holds experts [g N'/G, (g+1) N'/G)); the router and the shared experts
    are replicated; each GPU routes its own T tokens.  G T tokens (the
    workload's seeded inputs, T per GPU) are routed once, untimed, to find
    what each GPU receives: one row per (token, GPU) pair with at least one
    of the GPU's experts among its K', that row's other slots out of range.
    The GPU that receives the most pairs, the one that sets an expert-
    parallel step's time, is measured.  Its step: moe_route over its own T
    tokens; moe_forward on the received rows with its N'/G experts and no
    shared expert; moe_forward of the shared expert over its own T tokens
    (one group, gate 1: the same work as the shared group inside the
    layer); moe_balance_stats.  The two all-to-all exchanges, and the final
    add of the returned rows, are not run (one GPU).  The routed forward
    also adds the received x row as a residual, which the returned
    contribution would not carry: one row read and one add per row."""
    import torch
    from fine_grained_moe_router_amd import binding as B
    from fine_grained_moe_router_amd.synth import make_inputs

    T, N, K, d = cfg.T, cfg.n_routed, cfg.top_k, cfg.d_model
    assert cfg.n_shared == 1 and cfg.scoring != "hash" and N % gpus == 0
    n_loc = N // gpus
    print(f"[ep-share] {cfg.name}: generating inputs for {gpus} x {T} tokens",
          file=sys.stderr, flush=True)
    all_cfg = cfg.with_(T=gpus * T)
    inp = make_inputs(all_cfg, "cuda")
    r = B.route(all_cfg, x=inp.x, w_gate=inp.w_gate, offset=inp.offset, bias=inp.bias,
                want_pstat=False)
    owner = r["idx"].long() // n_loc                          # [G T][K] destination GPU
    pairs = torch.stack([(owner == g).sum() for g in range(gpus)]).cpu()
    g = int(pairs.argmax())
    local = owner == g
    rows = local.any(dim=1).nonzero().squeeze(1)
    R = int(rows.numel())
    x_recv = inp.x[rows].contiguous()
    idx_recv = torch.where(local[rows], r["idx"][rows] - g * n_loc,
                           torch.full_like(r["idx"][rows], -1)).contiguous()
    w_recv = r["w"][rows].contiguous()
    counts = torch.bincount(idx_recv[idx_recv >= 0].long(), minlength=n_loc)
    w13 = inp.w13[g * n_loc:(g + 1) * n_loc].contiguous()
    w2 = inp.w2[g * n_loc:(g + 1) * n_loc].contiguous()
    x_own = inp.x[g * T:(g + 1) * T].contiguous()
    inp.w13 = inp.w2 = None
    torch.cuda.empty_cache()

    routed_cfg = cfg.with_(name=f"{cfg.name}_ep{gpus}_routed", T=R, n_routed=n_loc, n_shared=0)
    shared_cfg = cfg.with_(name=f"{cfg.name}_ep{gpus}_shared", n_routed=1, top_k=1, n_shared=0,
                           d_ff=cfg.d_ff_shared, bias=False, zipf_s=0.0)
    idx_sh = torch.zeros((T, 1), dtype=torch.int32, device="cuda")
    w_sh = torch.ones((T, 1), dtype=torch.float32, device="cuda")
    ws_route = B.alloc_workspace(B.make_config(cfg), B.WS_ROUTE, "cuda")
    ws_rt = B.alloc_workspace(B.make_config(routed_cfg), B.WS_FORWARD, "cuda")
    ws_sh = B.alloc_workspace(B.make_config(shared_cfg), B.WS_FORWARD, "cuda")
    route_out = {"idx": torch.empty((T, K), dtype=torch.int32, device="cuda"),
                 "w": torch.empty((T, K), dtype=torch.float32, device="cuda"),
                 "counts": torch.empty(N, dtype=torch.int32, device="cuda"),
                 "pstat": torch.empty(B.workspace_bytes(B.make_config(cfg), B.WS_PSTAT),
                                      dtype=torch.uint8, device="cuda")}
    h_recv = torch.empty_like(x_recv)
    h_own = torch.empty_like(x_own)
    stats_out = {"f": torch.empty(N, dtype=torch.float32, device="cuda"),
                 "P": torch.empty(N, dtype=torch.float32, device="cuda"),
                 "loss": torch.empty(2, dtype=torch.float32, device="cuda")}

    def route():
        return B.route(cfg, x=x_own, w_gate=inp.w_gate, offset=inp.offset, bias=inp.bias,
                       out=route_out, workspace=ws_route)

    def routed():
        B.forward(routed_cfg, x_recv, idx_recv, w_recv, w13, w2, h=h_recv, workspace=ws_rt)

    def shared():
        B.forward(shared_cfg, x_own, idx_sh, w_sh, inp.w13s, inp.w2s, h=h_own, workspace=ws_sh)

    def step():
        rr = route()
        routed()
        shared()
        B.balance_stats(cfg, rr["counts"], rr["pstat"], out=stats_out)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    print(f"[ep-share] GPU {g}: {R} rows, {int(pairs[g])} pairs; timing {steps} steps",
          file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / steps

    # per-call stage times: each call alone, the library's HIP events
    parts = {}
    for name, fn in (("route", route), ("routed_forward", routed), ("shared_forward", shared)):
        B.profile_enable(16 * steps)
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        st = B.profile_collect()
        parts[name] = {k: v["ms"] / v["launches"] for k, v in st.items() if v["launches"]}

    P = int(pairs[g])
    f = cfg.d_ff
    gemm = {}
    for stage, flop, wbytes in (("gate_up", 4 * d * f * P, n_loc * 2 * f * d * 2),
                                ("down", 2 * d * f * P, n_loc * d * f * 2)):
        t = parts["routed_forward"][stage] * 1e-3
        gemm[stage] = {"kernel": KERNEL_OF_STAGE[stage], "ms": t * 1e3,
                       "tflops": flop / t / 1e12, "mfma_frac": flop / t / 1e12 / PEAK_BF16_TFLOPS,
                       "weight_gbs": wbytes / t / 1e9}
    print(json.dumps({
        "mode": "ep_share", "workload": cfg.name, "gpus": gpus, "gpu": g,
        "tokens_per_gpu": T, "experts_per_gpu": n_loc,
        "pairs_per_gpu": [int(v) for v in pairs], "rows_received": R, "pairs_received": P,
        "rows_per_expert_mean": P / n_loc,
        "max_over_mean_load": float(counts.max()) / max(float(counts.float().mean()), 1e-9),
        "steps": steps, "warmup": warmup, "ms_per_step": ms,
        "tokens_per_s_per_gpu_exchange_excluded": T / (ms * 1e-3),
        "calls_ms": parts, "routed_gemms": gemm,
        "note": "the two all-to-all exchanges are not run; the routed forward adds a residual "
                "the returned rows would not carry"}))
    return 0


def calibrate(reps: int):
    """One JSON line: TFLOP/s of bf16 GEMMs through the vendor library
    (torch.matmul / torch.bmm -> hipBLASLt) on random normal operands, with
    the FLOP counts of the V3 prefill layer's two expert contractions
    (73,728 rows: 65,536 routed pairs and 8,192 shared rows; d = 7168,
    d_ff = 2048): dense, and batched as 256 experts of 288 rows each (the
    same rows spread evenly).  Every operand is contiguous, K-contiguous on
    the left, N-contiguous on the right."""
    import torch
    torch.manual_seed(0)
    rows, d, f, E = 73728, 7168, 2048, 256
    shapes = {"dense_gate_up": ((rows, d), (d, 2 * f)), "dense_down": ((rows, f), (f, d)),
              "grouped_gate_up": ((E, rows // E, d), (E, d, 2 * f)),
              "grouped_down": ((E, rows // E, f), (E, f, d))}
    res = {}
    for name, (sa, sb) in shapes.items():
        a = torch.randn(sa, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(sb, device="cuda", dtype=torch.bfloat16) * (sa[-1] ** -0.5)
        fn = (lambda: torch.matmul(a, b)) if len(sa) == 2 else (lambda: torch.bmm(a, b))
        ms = time_calls(fn, reps=max(reps, 10))
        flop = 2.0 * a.numel() * sb[-1]
        res[name] = {"a": list(sa), "b": list(sb), "ms": ms, "tflop": flop / 1e12,
                     "tflops": flop / (ms * 1e-3) / 1e12,
                     "mfma_frac": flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        print(f"[calibrate] {name}: {ms:.3f} ms, {res[name]['tflops']:.0f} TFLOP/s",
              file=sys.stderr, flush=True)
        del a, b
        torch.cuda.empty_cache()
    print(json.dumps({"mode": "calibrate", "library": "torch.matmul/torch.bmm (hipBLASLt)",
                      "dtype": "bf16", "reps": max(reps, 10), "gemms": res}))
    return 0


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the layer runs on one GPU's share); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        return 2
    if args.pmc_summary:
        pmc_summary(args.pmc_summary, args.workload)
        return 0
    if args.clock_summary:
        clock_summary(args.clock_summary, args.workload)
        return 0

    import torch
    from fine_grained_moe_router_amd import accounting as acc
    from fine_grained_moe_router_amd import binding as B
    from fine_grained_moe_router_amd.configs import CONFIGS

    cfg = CONFIGS[args.workload]
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.lib()   # fails loudly if the HIP library is not built
    if args.extras:
        return extras(cfg)
    if args.calibrate:
        return calibrate(args.steps)
    if args.ep_share:
        return ep_share(cfg, args.ep_share, args.steps, args.warmup)
    print(f"[bench] {cfg.name}: generating inputs", file=sys.stderr, flush=True)
    layer = Layer(cfg)
    torch.cuda.synchronize()

    if args.pmc_run:
        src = torch.empty(COPY_BYTES // 2, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)                    # the calibration copy: COPY_BYTES moved in total
        for _ in range(2):
            layer.step()
        torch.cuda.synchronize()
        print("[bench] pmc run done", file=sys.stderr, flush=True)
        return 0

    for _ in range(args.warmup):
        layer.step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done; timing {args.steps} steps", file=sys.stderr, flush=True)

    B.profile_enable(16 * args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        layer.step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stages = B.profile_collect()
    ms = (t1 - t0) * 1000.0 / args.steps
    graph_ms = None if args.no_graph else graph_step_ms(layer, args.steps)
    cold_ms = cold_step_ms(layer, args.steps)

    counts = layer.route_out["counts"].cpu()
    touched = int((counts > 0).sum())
    fl = acc.layer_flops(cfg)
    gf = acc.expert_gemm_flops(cfg)
    by = acc.layer_bytes(cfg, touched)
    stage_ms = {k: (v["ms"] / v["launches"] if v["launches"] else 0.0) for k, v in stages.items()}
    dominant = max(("gate_up", "down"), key=lambda s: stage_ms[s])
    dom_s = stage_ms[dominant] / 1000.0
    # both roofs for the dominant kernel: algorithmic FLOPs and algorithmic
    # bytes of one launch over its average launch time
    tflops = gf[dominant] / dom_s / 1e12
    gbs = acc.gemm_bytes(cfg, touched)[dominant] / dom_s / 1e9
    peak_fl = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    bound = BOUND.get(cfg.name, "mfma" if cfg.T >= 1024 else "hbm")
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": tflops, "peak": peak_fl, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = read_traffic(cfg.name, dominant)
    roof["kernel"] = KERNEL_OF_STAGE[dominant]
    roof["avg_launch_ms"] = stage_ms[dominant]
    roof["mfma_frac"] = tflops / peak_fl
    roof["hbm_frac"] = gbs / PEAK_HBM_GBS
    roof["layer_mfma_frac"] = fl["total"] / (ms / 1000.0) / 1e12 / peak_fl
    roof["layer_hbm_frac"] = by["total"] / (ms / 1000.0) / 1e9 / PEAK_HBM_GBS

    out = {
        "metric": "MoE-layer tokens/sec on 1 MI355X (V3 shape, T=8192); % MFMA / HBM roofline",
        "value": cfg.T / (ms / 1000.0),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "d_model": cfg.d_model,
                   "n_routed": cfg.n_routed, "top_k": cfg.top_k, "n_shared": cfg.n_shared,
                   "d_ff": cfg.d_ff, "d_ff_shared": cfg.d_ff_shared, "scoring": cfg.scoring,
                   "renorm": cfg.renorm, "selection_bias": cfg.bias, "zipf_offset": cfg.zipf_s,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "layer": {"algorithmic_tflop": fl["total"] / 1e12,
                  "tflops": fl["total"] / (ms / 1000.0) / 1e12,
                  "mfma_frac": fl["total"] / (ms / 1000.0) / 1e12 / PEAK_BF16_TFLOPS,
                  "algorithmic_gb": by["total"] / 1e9,
                  "gbs": by["total"] / (ms / 1000.0) / 1e9,
                  "experts_touched": touched,
                  "max_over_mean_load": float(counts.max()) / max(float(counts.float().mean()), 1e-9)},
        "stages_ms": stage_ms,
        "graph_ms_per_step": graph_ms,
        "cold_cache_ms_per_step": cold_ms,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(layer, args.cpu_seconds)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
