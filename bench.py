#!/usr/bin/env python3
"""Throughput of the routed MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the whole layer over one batch of synthetic input
resident in HBM: router + top-k, dispatch, grouped gate/up GEMM, grouped down
GEMM, weighted combine with the gated shared expert, as one moe_layer_forward
call on the current stream.  K steps are timed back to back between two device
synchronisations.  The same layer is then run K more times stage by stage,
each stage through its own C-ABI entry point with HIP events between them;
those events give the per-stage durations.

Prints one JSON line: tokens/s for the whole step, the roofline of the
dominant kernel (algorithmic bytes or FLOPs per launch over its event-timed
duration), and the fp64 CPU oracle timed on a bounded sample of the same
workload on this host's cores.  For bf16 workloads it also reports the
four-stream gated residual read and write around the layer at the same T and
H, and the expert-weight audit of the layer's gate tensor (event-timed, with
their own rooflines); they are not part of the step.  Every workload also
reports one GPU's share under expert parallelism over 8 GPUs: the grouped
FFN of each rank's E/8 experts on the rows the same routing sends them.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOADS = ["flash_prefill", "flash_decode", "max_prefill", "max_fp8", "toy_fp32"]
METRIC = "MoE layer tokens/s + % MFMA peak (prefill) / % HBM BW (decode), 1 MI355X"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="flash_prefill", choices=WORKLOADS)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--gemm-tile", default="auto", choices=["auto", "128", "256"],
                    help="pin the MFMA GEMM kernel (A/B runs); default picks by rows per expert")
    ap.add_argument("--path", default="auto", choices=["auto", "gemm", "stream"],
                    help="pin every expert to one path (A/B runs); default picks per expert by rows")
    ap.add_argument("--cpu-tokens", type=int, default=-1,
                    help="tokens of the same workload the CPU oracle runs on (0: skip; -1: grown from 64 "
                         "until one run takes 10 s or covers the batch)")
    ap.add_argument("--no-ep-share", action="store_true",
                    help="skip the expert-parallel share runs (they launch the layer's own FFN kernels, so "
                         "kernel traces and counter runs of the layer leave them out)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (scale factor for HBM byte counters)")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))


def kernel_source_sha():
    h = hashlib.sha256()
    for f in ("gemm.hip", "gemm_dma.hip", "stream.hip", "common.hpp"):
        h.update(open(os.path.join(ROOT, "sparse_moe_layer_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(workload, kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("source_sha") != kernel_source_sha():
        return None
    return d.get("bytes_per_launch")


def cpu_baseline(problem, n_tokens):
    """The fp64 oracle, as it stands, on the first n tokens of the workload.
    n_tokens < 0 sizes the sample by time: from 64 tokens, the sample grows
    (by the last run's rate, at least doubling) until one run takes 10 s or
    more or covers the whole batch; that run is reported.  (The oracle's time
    is not proportional to n: converting the touched experts' weights is a
    large fixed part, so one small probe underestimates the rate.)"""
    import types

    from threadpoolctl import threadpool_info

    from oracle import adapter

    def run(n):
        sub = types.SimpleNamespace(**{k: getattr(problem, k) for k in (
            "w_router", "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down", "sh_gate", "sh_up", "sh_down",
            "sh_gate_w")})
        sub.cfg = problem.cfg.with_(T=n)
        sub.x = problem.x[:n]
        sub.host_raw = problem.host_raw
        t0 = time.perf_counter()
        adapter.forward(sub)
        return time.perf_counter() - t0

    T = problem.cfg.T
    if n_tokens < 0:
        n = min(64, T)
        dt = run(n)
        while dt < 10.0 and n < T:
            n = min(T, max(2 * n, int(n * 15.0 / max(dt, 1e-3))))
            dt = run(n)
    else:
        n = min(n_tokens, T)
        dt = run(n)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {T} tokens of the same workload, full layer "
                      f"(route, dispatch, every routed and shared expert, combine) in fp64 NumPy; "
                      f"{dt:.1f} s wall"}


def gated_residual(lib, acc, args, cfg, dev, stream, comb):
    """The four-stream gated residual read and write around the layer at the
    workload's T and H (read bottleneck width 320), each entry point timed
    over --steps calls with HIP events on the launch stream, and the write
    fused into the layer's combine (comb: the layer's problem and the
    combine's inputs from the staged run).  Not part of the step: the layer
    is the step."""
    import torch
    from synthetic import make_gr_problem

    T, H, rank = cfg.T, cfg.H, 320
    g = make_gr_problem(T, H, rank, seed=args.seed, device=dev)
    P = lib.problem(T, H, cfg.E, cfg.k, cfg.I, cfg.I_shared, act="bf16", wdt=cfg.wdt)
    G = lib.gr_weights(g.norm_w, g.w_read, g.w_up, rank, g.eps)
    ws = lib.gr_workspace(P, rank)
    x = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    s = torch.empty((T, 4), dtype=torch.float32, device=dev)
    out = torch.empty_like(g.resid)
    for _ in range(max(1, args.warmup)):
        lib.moe_gr_read(P, G, g.resid, x, s, ws, stream)
        lib.moe_gr_write(P, g.resid, g.s, g.f, out, stream)
    PL, y, pos, tw, y_sh, sl = comb
    for _ in range(max(1, args.warmup)):
        lib.moe_combine_gr_write(PL, y, pos, tw, y_sh, sl, g.resid, g.s, None, out, stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record(stream)
    for _ in range(args.steps):
        lib.moe_gr_read(P, G, g.resid, x, s, ws, stream)
    ev[1].record(stream)
    for _ in range(args.steps):
        lib.moe_gr_write(P, g.resid, g.s, g.f, out, stream)
    ev[2].record(stream)
    for _ in range(args.steps):
        lib.moe_combine_gr_write(PL, y, pos, tw, y_sh, sl, g.resid, g.s, None, out, stream)
    ev[3].record(stream)
    torch.cuda.synchronize()
    t_read = ev[0].elapsed_time(ev[1]) / args.steps * 1e-3
    t_write = ev[1].elapsed_time(ev[2]) / args.steps * 1e-3
    t_cw = ev[2].elapsed_time(ev[3]) / args.steps * 1e-3
    fr, br = acc.gr_read_work(T, H, rank)
    fw, bw = acc.gr_write_work(T, H)
    fc, bc = acc.combine_gr_write_work(T, H, cfg.k, y_sh is not None)
    return {"rank": rank,
            "read_us": round(t_read * 1e6, 2), "read_roofline": acc.roofline(fr, br, t_read),
            "write_us": round(t_write * 1e6, 2), "write_roofline": acc.roofline(fw, bw, t_write),
            "combine_write_us": round(t_cw * 1e6, 2), "combine_write_roofline": acc.roofline(fc, bc, t_cw)}


def weight_audit(lib, acc, args, prob, stream):
    """The expert-weight audit (zero count and sigma_rob per expert and over
    the tensor) of the workload's own routed gate tensor [E, I, H], timed
    over --steps calls with HIP events on the launch stream; not part of the
    step."""
    import torch

    w = prob.w_gate
    E = w.shape[0]
    n = w[0].numel()
    stats = lib.audit_stats_buffer(E)
    ws = lib.audit_workspace(E)
    flat = w.reshape(-1)
    for _ in range(max(1, args.warmup)):
        lib.moe_weight_audit(flat, E, n, n, stats, ws, stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(args.steps):
        lib.moe_weight_audit(flat, E, n, n, stats, ws, stream)
    ev[1].record(stream)
    torch.cuda.synchronize()
    t = ev[0].elapsed_time(ev[1]) / args.steps * 1e-3
    whole = lib.audit_records(stats)[E]
    byts = acc.audit_work(E * n)
    return {"tensor": "w_gate", "slices": E, "values_per_slice": n, "us": round(t * 1e6, 2),
            "roofline": acc.roofline(0.0, byts, t),
            "whole": {"zero_frac": whole["n_zero"] / whole["n"], "median": whole["median"],
                      "sigma_rob": whole["sigma_rob"]}}


def ep_share(lib, acc, args, cfg, dev, stream, prob, offs, sa, ranks=8):
    """One GPU's share of the layer under expert parallelism over `ranks`
    GPUs (the Flash-Next MoE section, expert parallelism: each routed row
    travels to the GPU that owns its expert and its result travels back to
    the token's GPU for the combine).  Rank r owns
    the experts e = r (mod ranks) and runs the grouped FFN on every row that
    the whole batch's routing sends them, received as a compact [R_r, H]
    block: moe_expert_ffn with the owned experts addressed through expert
    strides.  Each rank's FFN is timed over --steps calls with HIP events on
    the launch stream, against its own roof max(F/P, B/BW) with
    F = 6 R_r H I and B = its touched experts' weights + the received rows
    + y.  The all-to-all exchanges, the shared expert (it runs at the token's
    home GPU) and the combine are not in it.  Not part of the step."""
    import torch

    E, k, H, I = cfg.E, cfg.k, cfg.H, cfg.I
    if E % ranks:
        return None
    Ep = E // ranks
    offs_h = offs.cpu().long()
    counts = torch.diff(offs_h)
    tok = sa.long() // k  # token of every dispatched row, in expert order
    fp8 = cfg.wdt == "fp8"
    a_b, w_b = acc.WBYTES[cfg.act], acc.WBYTES[cfg.wdt]
    res = {"ranks": ranks, "experts_per_rank": Ep, "rows": [], "touched": [], "ms": [], "roof_frac": []}
    for r in range(ranks):
        c = counts[r::ranks]
        Rr = int(c.sum())
        touched = int((c > 0).sum())
        res["rows"].append(Rr)
        res["touched"].append(touched)
        if Rr == 0:
            res["ms"].append(0.0)
            res["roof_frac"].append(None)
            continue
        idx = torch.cat([torch.arange(int(offs_h[e]), int(offs_h[e + 1])) for e in range(r, E, ranks)])
        xr = prob.x.index_select(0, tok[idx.to(dev)])  # the rows this rank receives
        offr = torch.zeros(Ep + 1, dtype=torch.int32)
        offr[1:] = torch.cumsum(c, 0)
        offr = offr.to(dev)
        sar = torch.arange(Rr, dtype=torch.int32, device=dev)
        P = lib.problem(Rr, H, Ep, 1, I, 0, cfg.act, cfg.wdt, cfg.scale_block, 0)
        sc = [t[r::ranks].contiguous() if fp8 else None for t in (prob.s_gate, prob.s_up, prob.s_down)]
        W = lib.weights(None, prob.w_gate[r], prob.w_up[r], prob.w_down[r], *sc,
                        stride_gate=ranks * I * H, stride_up=ranks * I * H, stride_down=ranks * H * I)
        ws = lib.workspace(P)
        y = torch.empty((Rr, H), dtype=prob.x.dtype, device=dev)
        for _ in range(max(1, args.warmup)):
            lib.moe_expert_ffn(P, W, xr, offr, sar, y, None, ws, stream)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(args.steps):
            lib.moe_expert_ffn(P, W, xr, offr, sar, y, None, ws, stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        t = ev[0].elapsed_time(ev[1]) / args.steps * 1e-3
        f = 6.0 * Rr * H * I
        b = touched * 3.0 * I * H * w_b + 2.0 * Rr * H * a_b
        if fp8:
            b += touched * 3.0 * (I // cfg.scale_block) * (H // cfg.scale_block) * 4
        t_roof = max(f / (acc.PEAK_BF16_TFLOPS * 1e12), b / (acc.PEAK_HBM_GBPS * 1e9))
        res["ms"].append(round(t * 1e3, 4))
        res["roof_frac"].append(round(t_roof / t, 4))
        del xr, y, ws
    res["max_ms"] = max(res["ms"])
    res["mean_ms"] = round(sum(res["ms"]) / ranks, 4)
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this layer is built and measured on a single MI355X; "
              "run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration()
        return

    import sparse_moe_layer_amd as lib
    from sparse_moe_layer_amd import accounting as acc
    from sparse_moe_layer_amd.tensors import structs
    from synthetic import CONFIGS, make_problem

    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    print(f"[bench] generating {cfg.name} on {torch.cuda.get_device_name(dev)}", file=sys.stderr, flush=True)
    prob = make_problem(cfg, args.seed, device=dev)
    T, H, E, k, I, Is = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.I_shared
    R = T * k
    adt = prob.x.dtype
    sh = Is > 0
    flags = {"auto": 0, "128": lib.MOE_FLAG_GEMM_TILE_128, "256": lib.MOE_FLAG_GEMM_TILE_256}[args.gemm_tile]
    flags |= {"auto": 0, "gemm": lib.MOE_FLAG_FORCE_GEMM, "stream": lib.MOE_FLAG_FORCE_STREAM}[args.path]
    P, W = structs(prob, flags)
    ws = lib.workspace(P)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, k), dtype=torch.float32, device=dev)
    sl = torch.empty(T, dtype=torch.float32, device=dev) if sh else None
    offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sa = torch.empty(R, dtype=torch.int32, device=dev)
    pos = torch.empty(R, dtype=torch.int32, device=dev)
    h = torch.empty((R, I), dtype=adt, device=dev)
    h_sh = torch.empty((T, Is), dtype=adt, device=dev) if sh else None
    y = torch.empty((R, H), dtype=adt, device=dev)
    y_sh = torch.empty((T, H), dtype=adt, device=dev) if sh else None
    out = torch.empty((T, H), dtype=adt, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev):
        ev[0].record(stream)
        lib.moe_route(P, prob.x, prob.w_router, prob.sh_gate_w, ids, tw, sl, ws, stream)
        ev[1].record(stream)
        lib.moe_dispatch(P, ids, offs, sa, pos, ws, stream)
        ev[2].record(stream)
        lib.moe_expert_gate_up(P, W, prob.x, offs, sa, h, h_sh, ws, stream)
        ev[3].record(stream)
        lib.moe_expert_down(P, W, offs, h, h_sh, y, y_sh, ws, stream)
        ev[4].record(stream)
        lib.moe_combine(P, y, pos, tw, y_sh, sl, out, stream)
        ev[5].record(stream)

    # the timed steps: the whole layer, one moe_layer_forward call per step
    for _ in range(args.warmup):
        lib.moe_layer_forward(P, W, prob.x, out, None, None, ws, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        lib.moe_layer_forward(P, W, prob.x, out, None, None, ws, stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # the same layer stage by stage, HIP events on the launch stream between the
    # entry points: per-stage durations for the roofline of the dominant kernel
    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for _ in range(max(1, args.warmup)):
        step(mk())
    torch.cuda.synchronize()
    evs = [mk() for _ in range(args.steps)]
    t2 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    staged_ms = (time.perf_counter() - t2) * 1e3 / args.steps
    names = ["route", "dispatch", "gate_up", "down", "combine"]
    stage_ms = {n: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps for j, n in enumerate(names)}

    counts = torch.diff(offs).cpu()
    touched = int((counts > 0).sum())
    work = acc.layer_work(T, H, E, k, I, Is, cfg.act, cfg.wdt, touched, cfg.scale_block)
    mfma_peak = acc.PEAK_BF16_TFLOPS  # every contraction runs on bf16 MFMA (fp8 weights are decoded to bf16)

    # dominant kernel: the longer grouped GEMM phase; its bound from its intensity vs the ridge
    dom = "gate_up" if stage_ms["gate_up"] >= stage_ms["down"] else "down"
    f_dom = work.flops_gate_up if dom == "gate_up" else work.flops_down
    b_dom = work.bytes_gate_up if dom == "gate_up" else work.bytes_down
    t_dom = stage_ms[dom] * 1e-3
    ridge = mfma_peak * 1e12 / (acc.PEAK_HBM_GBPS * 1e9)
    if f_dom / b_dom > ridge:
        ach, peak, unit, bound = f_dom / t_dom / 1e12, mfma_peak, "TFLOP/s", "mfma"
    else:
        ach, peak, unit, bound = b_dom / t_dom / 1e9, acc.PEAK_HBM_GBPS, "GB/s", "hbm"
    kname = "grouped_gemm_" + dom
    roof = {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit, "frac": round(ach / peak, 4),
            "traffic": load_traffic(args.workload, kname), "kernel": kname,
            "algorithmic": {"flops": f_dom, "bytes": b_dom}}

    gr = (gated_residual(lib, acc, args, cfg, dev, stream, (P, y, pos, tw, y_sh, sl))
          if cfg.act == "bf16" else None)
    audit = weight_audit(lib, acc, args, prob, stream) if cfg.wdt == "bf16" else None
    ep = None if args.no_ep_share else ep_share(lib, acc, args, cfg, dev, stream, prob, offs, sa)

    t_s = ms_step * 1e-3
    res = {
        "metric": METRIC,
        "value": round(T / t_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.act == "bf16" else "f32",
        "data": "synthetic (seeded counter-based generator, weights random-init at the pages' shapes)",
        "config": {"workload": cfg.name, "T": T, "H": H, "E": E, "k": k, "I": I, "I_shared": Is,
                   "act": cfg.act, "weights": cfg.wdt, "touched_experts": touched,
                   "max_tokens_per_expert": int(counts.max()), "gemm_tile": args.gemm_tile, "path": args.path},
        "layer": {"tflops": round(work.flops / t_s / 1e12, 2), "hbm_gbps": round(work.bytes / t_s / 1e9, 1),
                  "mfma_frac": round(work.flops / t_s / 1e12 / mfma_peak, 4),
                  "hbm_frac": round(work.bytes / t_s / 1e9 / acc.PEAK_HBM_GBPS, 4),
                  # the whole layer against its binding roof: t_roof = max(F/P, B/BW)
                  "bound": "mfma" if work.flops / (mfma_peak * 1e12) >= work.bytes / (acc.PEAK_HBM_GBPS * 1e9)
                           else "hbm",
                  "roof_frac": round(max(work.flops / (mfma_peak * 1e12), work.bytes / (acc.PEAK_HBM_GBPS * 1e9))
                                     / t_s, 4),
                  "staged_ms": round(staged_ms, 4)},
        "stages_ms": {n: round(v, 4) for n, v in stage_ms.items()},
        "roofline": roof,
        "gated_residual": gr,
        "weight_audit": audit,
        "ep_share": ep,
    }
    if args.cpu_tokens != 0:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(prob, args.cpu_tokens)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
