#!/usr/bin/env python3
"""Throughput of the routed MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--also NAMES]

One step is one pass of the whole layer over one batch of synthetic input
resident in HBM: router + top-k, dispatch, grouped gate/up GEMM, grouped down
GEMM, weighted combine with the gated shared expert, as one moe_layer_forward
call on the current stream.  The headline workload (default: the 2.4T-shape
prefill layer, 8192 tokens) is timed as K steps back to back between two
device synchronisations; `value` is its tokens/s.  K more steps are timed one
by one with HIP events after a 1 GiB read pass that evicts the caches
(`cold_ms`: median, p10, p90), and K more stage by stage through the five
entry points with HIP events between them (`stages_ms`).

Prints one JSON line: tokens/s for the whole step, the whole layer against
its binding roof, the roofline of the dominant kernel (algorithmic bytes or
FLOPs per launch over its event-timed duration), the fp64 CPU oracle timed on
a bounded sample of the same workload on this host's cores, and the same
layer-level numbers for the other workloads (`--also`; the decode layer's
repeated under `decode`; it is measured before the headline).  For bf16 workloads it also reports the four-stream
gated residual read and write around the layer at the same T and H, and the
expert-weight audit of the layer's gate tensor (event-timed, with their own
rooflines); they are not part of the step.
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
    ap.add_argument("--workload", default="max_prefill", choices=WORKLOADS,
                    help="the workload of the headline line (default: the 2.4T-shape 8192-token prefill layer)")
    ap.add_argument("--also", default="flash_decode,max_fp8,flash_prefill",
                    help="comma-separated workloads also measured in the same run (layer-level numbers; the "
                         "decode layer's are repeated under the line's 'decode' key); '' for none")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--gemm-tile", default="auto", choices=["auto", "128", "256"],
                    help="pin the MFMA GEMM kernel (A/B runs); default picks by rows per expert")
    ap.add_argument("--path", default="auto", choices=["auto", "gemm", "stream"],
                    help="pin every expert to one path (A/B runs); default picks per expert by rows")
    ap.add_argument("--cpu-tokens", type=int, default=-1,
                    help="tokens of the same workload the CPU oracle runs on (0: skip; -1: grown from 64 "
                         "until one run takes 10 s or covers the batch)")
    ap.add_argument("--ep-share", action="store_true",
                    help="also time one GPU's share under 8-way expert parallelism (off by default)")
    ap.add_argument("--no-ep-share", action="store_true", help="accepted for older commands (the default)")
    ap.add_argument("--layer-only", action="store_true",
                    help="skip the gated-residual and weight-audit rows (kernel traces of the layer alone)")
    ap.add_argument("--stream-ceiling", action="store_true",
                    help="only time moe_hbm_read_probe (one pass over 4 GiB, 16 B per lane) and print its rate")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only time moe_mfma_pipe_probe's variants, and the 256x256 tile kernel and hipBLASLt on "
                         "one dense 8192x4096x8192 gate/up product (zero and random operands), and print them")
    ap.add_argument("--mfma-launches", type=int, default=2000,
                    help="--mfma-ceiling: back-to-back launches of each dense run (fewer under a counter profiler)")
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


def stream_ceiling(lib, stream, nbytes=4 << 30, launches=20):
    """Practical HBM read ceiling: the rate of a kernel that only reads, with the
    streaming kernels' access shape, over a buffer far larger than the 256 MB
    last-level cache.  Timed with HIP events on the stream it is launched on."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(3)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    with torch.cuda.stream(stream):
        for _ in range(3):
            lib.moe_hbm_read_probe(src, sink, stream)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
        for a, b in evs:
            a.record(stream)
            lib.moe_hbm_read_probe(src, sink, stream)
            b.record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    del src
    torch.cuda.empty_cache()
    gbs = [nbytes / (m * 1e-3) / 1e9 for m in ms]
    return {"kernel": "hbm_read_probe_kernel", "bytes": nbytes, "launches": launches,
            "ms_median": round(pct(ms, 0.5), 4), "gbs_median": round(pct(gbs, 0.5), 1),
            "gbs_best": round(max(gbs), 1), "frac_of_8tbs": round(pct(gbs, 0.5) / 8000.0, 4)}


def mfma_ceiling(lib, stream, launches=2000):
    """What the tile kernel's pipeline costs the MFMA rate, and where it stands
    against the vendor GEMM on one dense product.

    - probe: moe_mfma_pipe_probe's variants (the tile kernel's per-step work
      taken apart, zero operands), each timed over 5 launches of 20000 steps
      with HIP events on the stream it is launched on;
    - dense: the gate/up product of one expert holding all 8192 rows (H 8192,
      I 2048: an 8192 x 4096 x 8192 GEMM) through moe_expert_gate_up with
      256-row tiles, and torch.matmul (hipBLASLt) on the same shape, each
      launched back to back for about a second so that the clock settles, with
      the shader clock sampled meanwhile (`launches` times each); once on zero operands (the clock stays
      near its maximum) and once on random ones (the chip's power limit lowers
      it)."""
    import torch
    res = {"probe": {}, "dense": {}}
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    src = torch.zeros(4 << 20, dtype=torch.uint8, device="cuda")  # 128 slots of 32 KB: stays in L2
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    steps = 20000
    names = ["mfma only", "+ fragment reads", "+ barrier per step", "+ direct loads", "direct loads, no barrier",
             "direct loads as global_load_lds"]
    for v, name in enumerate(names):
        with torch.cuda.stream(stream):
            lib.moe_mfma_pipe_probe(v, steps // 10, src, sink, stream)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(5):
                lib.moe_mfma_pipe_probe(v, steps, src, sink, stream)
            b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / 5
        tf = cus * 8 * steps * 16 * 32768 / (ms * 1e-3) / 1e12
        res["probe"][name] = {"variant": v, "ms": round(ms, 4), "tflops": round(tf, 1),
                              "frac_of_2500": round(tf / 2500.0, 4)}
    T, H, I = 8192, 8192, 2048
    flops = 4.0 * T * H * I
    for data in ("zeros", "random"):
        g = torch.Generator(device="cuda").manual_seed(0)
        x = torch.randn(T, H, device="cuda", generator=g).to(torch.bfloat16)
        wg = (torch.randn(1, I, H, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        wu = (torch.randn(1, I, H, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        wd = (torch.randn(1, H, I, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        if data == "zeros":
            for t in (x, wg, wu, wd):
                t.zero_()
        P = lib.problem(T, H, 1, 1, I, 0, "bf16", "bf16", 128, lib.MOE_FLAG_FORCE_GEMM | lib.MOE_FLAG_GEMM_TILE_256)
        W = lib.weights(None, wg, wu, wd, None, None, None)
        ws = lib.workspace(P)
        offs = torch.tensor([0, T], dtype=torch.int32, device="cuda")
        sa = torch.arange(T, dtype=torch.int32, device="cuda")
        h = torch.empty(T, I, dtype=torch.bfloat16, device="cuda")
        wgu = torch.cat([wg[0], wu[0]], 0).contiguous()
        runs = {"tile_kernel_gate_up": lambda: lib.moe_expert_gate_up(P, W, x, offs, sa, h, None, ws, stream),
                "hipblaslt_matmul": lambda: torch.matmul(x, wgu.T)}
        for name, fn in runs.items():
            with torch.cuda.stream(stream):
                for _ in range(5):
                    fn()
                torch.cuda.synchronize()
                n = launches
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                with ClockSampler(0.01) as clk:
                    a.record(stream)
                    for _ in range(n):
                        fn()
                    b.record(stream)
                    torch.cuda.synchronize()
            ms = a.elapsed_time(b) / n
            res["dense"][f"{name}_{data}"] = {"ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                                             "sclk": clk.summary()}
        del x, wg, wu, wd, h, wgu, ws
        torch.cuda.empty_cache()
    return res


def kernel_source_sha():
    h = hashlib.sha256()
    for f in ("gemm.hip", "gemm_dma.hip", "stream.hip", "stream_item.hpp", "common.hpp", "kernels.hpp"):
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
    model, blas = host_info()
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle", "cpu_model": model,
            "blas": blas,
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


def host_info():
    """CPU model and BLAS vendor of this host (for the CPU baseline)."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        libs = [f"{p.get('internal_api')} {p.get('version')}" for p in threadpool_info() if p.get("user_api") == "blas"]
        blas = ", ".join(libs) or None
    except Exception:
        pass
    return model, blas


def source_ids():
    """Git commit of the tree when .git is present (it is not on a copied tree),
    and a hash of the library and bench sources either way."""
    sha = None
    try:
        import subprocess
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "--short=12", "HEAD"], capture_output=True, text=True,
                           timeout=10)
        if r.returncode == 0:
            sha = r.stdout.strip()
    except Exception:
        pass
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_moe_layer_amd", "csrc")
    for f in sorted(os.listdir(csrc)) + ["../../include/moe_mi355x.h", "../../bench.py"]:
        path = os.path.join(csrc, f)
        if os.path.isfile(path):
            h.update(open(path, "rb").read())
    return sha, h.hexdigest()[:16]


class ClockSampler:
    """Samples the GPU shader clock level the driver reports (sysfs
    pp_dpm_sclk, the level marked '*') from a host thread while a timed region
    runs.  Reads a text file only; null where the file is not readable."""

    def __init__(self, period=0.02):
        import glob
        import threading
        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.period = period
        self.samples = []
        self._stop = threading.Event()
        self._th = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        for p in self.paths:
            try:
                for line in open(p):
                    if line.rstrip().endswith("*"):
                        return int(line.split(":")[1].strip().lower().split("mhz")[0])
            except (OSError, ValueError, IndexError):
                continue
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.paths:
            self._th.start()
        return self

    def __exit__(self, *a):
        self._stop.set()
        if self.paths:
            self._th.join()

    def summary(self):
        if not self.samples:
            return None
        v = sorted(self.samples)
        return {"median_mhz": v[len(v) // 2], "min_mhz": v[0], "max_mhz": v[-1], "samples": len(v)}


def pct(vals, q):
    v = sorted(vals)
    i = min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))
    return v[i]


def measure(lib, acc, cfg, args, dev, stream, flags, full):
    """One workload: the contract's timed region (K moe_layer_forward calls
    back to back between two device synchronisations), then K steps each
    timed alone with HIP events on the launch stream after a 1 GiB read pass
    that evicts the L2s and the 256 MB memory-side cache with clean lines
    (median, p10, p90), then K steps stage by stage with events between the
    entry points.
    full: also the roofline object and the widened rows."""
    import torch
    from sparse_moe_layer_amd.tensors import structs
    from synthetic import make_problem

    print(f"[bench] generating {cfg.name}", file=sys.stderr, flush=True)
    prob = make_problem(cfg, args.seed, device=dev)
    T, H, E, k, I, Is = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.I_shared
    R = T * k
    adt = prob.x.dtype
    sh = Is > 0
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
    # cache eviction between cold steps: one read pass over 1 GiB (twice the
    # 256 MB memory-side cache and every L2), by the library's read probe, so
    # the evicting lines are clean and leave no write-back behind them
    flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    flush_sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def layer():
        lib.moe_layer_forward(P, W, prob.x, out, None, None, ws, stream)

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

    # the contract's timed region: K whole-layer calls back to back
    for _ in range(args.warmup):
        layer()
    torch.cuda.synchronize()
    with ClockSampler() as clk:
        t0 = time.perf_counter()
        for _ in range(args.steps):
            layer()
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # each step alone after evicting the caches, HIP events around the call
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        lib.moe_hbm_read_probe(flush, flush_sink, stream)
        evs[i][0].record(stream)
        layer()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    cold = [a.elapsed_time(b) for a, b in evs]

    # stage by stage, events between the entry points
    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for _ in range(max(1, args.warmup)):
        step(mk())
    torch.cuda.synchronize()
    sevs = [mk() for _ in range(args.steps)]
    t2 = time.perf_counter()
    for i in range(args.steps):
        step(sevs[i])
    torch.cuda.synchronize()
    staged_ms = (time.perf_counter() - t2) * 1e3 / args.steps
    names = ["route", "dispatch", "gate_up", "down", "combine"]
    stage_ms = {n: sum(e[j].elapsed_time(e[j + 1]) for e in sevs) / args.steps for j, n in enumerate(names)}

    counts = torch.diff(offs).cpu()
    touched = int((counts > 0).sum())
    work = acc.layer_work(T, H, E, k, I, Is, cfg.act, cfg.wdt, touched, cfg.scale_block)
    mfma_peak = acc.PEAK_BF16_TFLOPS  # every contraction runs on bf16 MFMA (fp8 weights are decoded to bf16)
    t_roof = max(work.flops / (mfma_peak * 1e12), work.bytes / (acc.PEAK_HBM_GBPS * 1e9))
    t_s = ms_step * 1e-3
    res = {
        "ms_per_step": round(ms_step, 4),
        "tokens_per_s": round(T / t_s, 1),
        "cold_ms": {"median": round(pct(cold, 0.5), 4), "p10": round(pct(cold, 0.1), 4),
                    "p90": round(pct(cold, 0.9), 4)},
        "config": {"workload": cfg.name, "T": T, "H": H, "E": E, "k": k, "I": I, "I_shared": Is,
                   "act": cfg.act, "weights": cfg.wdt, "touched_experts": touched,
                   "max_tokens_per_expert": int(counts.max())},
        "layer": {"tflops": round(work.flops / t_s / 1e12, 2), "hbm_gbps": round(work.bytes / t_s / 1e9, 1),
                  "mfma_frac": round(work.flops / t_s / 1e12 / mfma_peak, 4),
                  "hbm_frac": round(work.bytes / t_s / 1e9 / acc.PEAK_HBM_GBPS, 4),
                  # the whole layer against its binding roof: t_roof = max(F/P, B/BW)
                  "bound": "mfma" if work.flops / (mfma_peak * 1e12) >= work.bytes / (acc.PEAK_HBM_GBPS * 1e9)
                           else "hbm",
                  "t_roof_ms": round(t_roof * 1e3, 4),
                  "roof_frac": round(t_roof / t_s, 4),
                  "roof_frac_cold_median": round(t_roof / (pct(cold, 0.5) * 1e-3), 4),
                  "staged_ms": round(staged_ms, 4)},
        "stages_ms": {n: round(v, 4) for n, v in stage_ms.items()},
        "sclk": clk.summary(),
    }
    if not full:
        del prob
        return res, None

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
    res["roofline"] = {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
                       "frac": round(ach / peak, 4), "traffic": load_traffic(cfg.name, kname), "kernel": kname,
                       "algorithmic": {"flops": f_dom, "bytes": b_dom}}
    if not args.layer_only:
        res["gated_residual"] = (gated_residual(lib, acc, args, cfg, dev, stream, (P, y, pos, tw, y_sh, sl))
                                 if cfg.act == "bf16" else None)
        res["weight_audit"] = weight_audit(lib, acc, args, prob, stream) if cfg.wdt == "bf16" else None
    if args.ep_share:
        res["ep_share"] = ep_share(lib, acc, args, cfg, dev, stream, prob, offs, sa)
    return res, prob


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
    from synthetic import CONFIGS

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    print(f"[bench] {torch.cuda.get_device_name(dev)}", file=sys.stderr, flush=True)
    if args.stream_ceiling:
        print(json.dumps({"stream_ceiling": stream_ceiling(lib, torch.cuda.current_stream())}), flush=True)
        return
    if args.mfma_ceiling:
        print(json.dumps({"mfma_ceiling": mfma_ceiling(lib, torch.cuda.current_stream(), args.mfma_launches)}),
              flush=True)
        return
    flags = {"auto": 0, "128": lib.MOE_FLAG_GEMM_TILE_128, "256": lib.MOE_FLAG_GEMM_TILE_256}[args.gemm_tile]
    flags |= {"auto": 0, "gemm": lib.MOE_FLAG_FORCE_GEMM, "stream": lib.MOE_FLAG_FORCE_STREAM}[args.path]
    stream = torch.cuda.current_stream()
    cfg = CONFIGS[args.workload]
    also = [w for w in args.also.split(",") if w and w != args.workload]
    # The decode layer goes first: after the 2.4T layers' runs its weight
    # streaming measured 3-4% slower in the same process (0.257 against 0.249
    # ms per step), at the same shader clock.
    others = {}
    for name in [w for w in also if w == "flash_decode"]:
        r, _ = measure(lib, acc, CONFIGS[name], args, dev, stream, flags, full=False)
        others[name] = r
        torch.cuda.empty_cache()
    main_res, prob = measure(lib, acc, cfg, args, dev, stream, flags, full=True)

    git_sha, src_sha = source_ids()
    res = {
        "metric": METRIC,
        "value": main_res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.act == "bf16" else "f32",
        "data": "synthetic (seeded counter-based generator, weights random-init at the pages' shapes)",
        "config": dict(main_res["config"], gemm_tile=args.gemm_tile, path=args.path),
        "cold_ms": main_res["cold_ms"],
        "layer": main_res["layer"],
        "stages_ms": main_res["stages_ms"],
        "roofline": main_res["roofline"],
        "sclk": main_res["sclk"],
        "git_sha": git_sha,
        "source_sha": src_sha,
    }
    for key in ("gated_residual", "weight_audit", "ep_share"):
        if key in main_res:
            res[key] = main_res[key]
    if args.cpu_tokens != 0:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(prob, args.cpu_tokens)
    else:
        res["cpu_baseline"] = None
    del prob
    torch.cuda.empty_cache()
    # the other workloads, each in the same run, with its own layer-level numbers
    for name in [w for w in also if w not in others]:
        r, _ = measure(lib, acc, CONFIGS[name], args, dev, stream, flags, full=False)
        others[name] = r
        torch.cuda.empty_cache()
    if "flash_decode" in others:
        d = others["flash_decode"]
        res["decode"] = {"workload": "flash_decode", "ms": d["ms_per_step"], "tokens_per_s": d["tokens_per_s"],
                         "cold_ms": d["cold_ms"], "hbm_frac": d["layer"]["hbm_frac"],
                         "hbm_frac_cold_median": d["layer"]["roof_frac_cold_median"],
                         "target_ms": round(d["layer"]["t_roof_ms"] / 0.7, 4), "stages_ms": d["stages_ms"]}
    if others:
        res["workloads"] = others
    res["stream_ceiling"] = stream_ceiling(lib, stream)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
