"""GPU parity of the gated residual read/write (moe_gr_read, moe_gr_write,
and the write fused into the combine, moe_combine_gr_write)
against the fp64 oracle (oracle/gr.py), Qwen3.8-Flash-Next study, section
"Gated residual: four streams, one sublayer input".

Tolerances, from the arithmetic the kernels do:
  * x (bf16 out): the bf16 bar of the layer, max|gpu - ref| <= 2e-2 max|ref|.
    The kernels round the normalised streams to bf16 (relative 2^-8) before
    both projections and the gated mean, and round x to bf16.
  * s (fp32 out): s = 2 sigmoid(p / 4) has slope <= 1/8 in the raw projection
    p = sum over 4H of Rhat_j w_j.  Rounding Rhat_j to bf16 moves it by
    ~2^-8 / sqrt(3) |Rhat_j| rms, so p moves by sqrt(4H) 0.02 2^-8 / sqrt(3)
    ~ 4.6e-3 rms at H = 2560 (weights ~ N(0, 0.02), Rhat ~ unit rms) and s by
    ~ 5.7e-4 rms; 4e-3 absolute is ~7 of those, enough for the maximum over
    thousands of gates.
  * resid_out (bf16 out) from the same fp32 s: one fp32 fma, then one
    round to bf16 (unit roundoff 2^-8), so every element within
    (2^-8 + 2^-23) |ref|.
"""
import numpy as np
import pytest
import torch

import sparse_moe_layer_amd as lib
from oracle import gr as ogr
from sparse_moe_layer_amd.tensors import structs
from synthetic import CONFIGS, make_gr_problem, make_problem

pytestmark = pytest.mark.gpu

RANK = 320  # read bottleneck width in the study


def _problem(T, H):
    # The layer's problem: the gated residual uses its T, H and activation dtype.
    return lib.problem(T, H, 512, 10, 640, 640, act="bf16", wdt="bf16")


def _read(g, T, H, rank):
    dev = g.resid.device
    P = _problem(T, H)
    G = lib.gr_weights(g.norm_w, g.w_read, g.w_up, rank, g.eps)
    ws = lib.gr_workspace(P, rank)
    x = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=dev)
    s = torch.full((T, 4), float("nan"), dtype=torch.float32, device=dev)
    lib.moe_gr_read(P, G, g.resid, x, s, ws)
    torch.cuda.synchronize()
    return x, s


def _check_read(g, x, s, rows):
    h = g.host
    ref_x, ref_s, _, _ = ogr.gr_read(h(g.resid)[rows], h(g.norm_w), h(g.w_read), h(g.w_up), g.eps)
    gx = x.float().cpu().numpy()[rows]
    gs = s.cpu().numpy()[rows]
    assert np.isfinite(gx).all() and np.isfinite(gs).all()
    ex = np.abs(gx - ref_x).max() / np.abs(ref_x).max()
    es = np.abs(gs - ref_s).max()
    print(f"[gr] read rows={len(rows)} x err {ex:.2e} (rel max), s err {es:.2e}", flush=True)
    assert ex <= 2e-2
    assert es <= 4e-3


@pytest.mark.parametrize("T,H,rank", [
    (16, 2560, RANK),    # Flash-Next decode batch, model width
    (1, 2560, RANK),
    (300, 96, 32),       # ragged token tiles (300 = 2 x 128 + 44), three column blocks
    (129, 2560, 16),     # one token past a tile, smallest bottleneck
    (3, 8224, 16),       # wider than the 2.4T model (H = 8192)
])
def test_gr_read_matches_oracle(T, H, rank):
    print(f"[gr] read T={T} H={H} rank={rank}", flush=True)
    g = make_gr_problem(T, H, rank, seed=3, device="cuda")
    x, s = _read(g, T, H, rank)
    _check_read(g, x, s, np.arange(T))


def test_gr_read_full_prefill_sampled():
    # Flash-Next prefill batch at model width; the oracle evaluates 256 sampled
    # tokens (every token is independent) including the first and last tiles.
    T, H = 4096, 2560
    print(f"[gr] read T={T} H={H} rank={RANK} sampled", flush=True)
    g = make_gr_problem(T, H, RANK, seed=5, device="cuda")
    x, s = _read(g, T, H, RANK)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, T - 1], rng.choice(T, 251, replace=False)]))
    _check_read(g, x, s, rows)


def test_gr_read_zero_stream():
    # A stream that is exactly zero normalises to zero (eps > 0); the others
    # are unaffected by it.
    T, H = 8, 256
    g = make_gr_problem(T, H, 32, seed=9, device="cuda")
    g.resid[2, 1].zero_()
    g.resid[5].zero_()
    x, s = _read(g, T, H, 32)
    _check_read(g, x, s, np.arange(T))
    assert torch.all(x[5] == 0)  # all four streams zero: the gated mean is 0


def test_gr_write_matches_oracle_and_may_alias():
    T, H = 300, 2560
    print(f"[gr] write T={T} H={H}", flush=True)
    g = make_gr_problem(T, H, 16, seed=11, device="cuda")
    P = _problem(T, H)
    out = torch.full_like(g.resid, float("nan"))
    lib.moe_gr_write(P, g.resid, g.s, g.f, out)
    torch.cuda.synchronize()
    ref = ogr.gr_write(g.host(g.resid), g.host(g.s), g.host(g.f))
    got = out.float().cpu().numpy()
    bad = np.abs(got - ref) > np.abs(ref) * (2.0 ** -8 + 2.0 ** -23)
    assert not bad.any(), f"{int(bad.sum())} elements off, first at {np.argwhere(bad)[0]}"
    # in place: resid_out == resid
    r = g.resid.clone()
    lib.moe_gr_write(P, r, g.s, g.f, r)
    torch.cuda.synchronize()
    assert torch.equal(r, out)


@pytest.mark.parametrize("shared", [640, 0])
def test_combine_with_fused_write_equals_combine_then_write(shared):
    # The fused pass must give moe_combine followed by moe_gr_write bit for
    # bit (both are checked against the oracle on their own), with and
    # without F(x) stored, and in place.
    cfg = CONFIGS["flash_prefill"].with_(name="combine_write", T=300, k=10, I_shared=shared)
    print(f"[gr] combine+write T={cfg.T} H={cfg.H} shared={shared}", flush=True)
    prob = make_problem(cfg, 21, device="cuda")
    T, H, E, k = cfg.T, cfg.H, cfg.E, cfg.k
    P, W = structs(prob)
    ws = lib.workspace(P)
    dev = prob.x.device
    sh = shared > 0
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    sl = torch.empty(T, dtype=torch.float32, device=dev) if sh else None
    offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sa = torch.empty(T * k, dtype=torch.int32, device=dev)
    pos = torch.empty(T * k, dtype=torch.int32, device=dev)
    y = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
    ysh = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if sh else None
    lib.moe_route(P, prob.x, prob.w_router, prob.sh_gate_w, ids, w, sl, ws)
    lib.moe_dispatch(P, ids, offs, sa, pos, ws)
    lib.moe_expert_ffn(P, W, prob.x, offs, sa, y, ysh, ws)
    g = make_gr_problem(T, H, 16, seed=22, device="cuda")
    f = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ref = torch.empty_like(g.resid)
    lib.moe_combine(P, y, pos, w, ysh, sl, f)
    lib.moe_gr_write(P, g.resid, g.s, f, ref)
    f2 = torch.full_like(f, float("nan"))
    out2 = torch.full_like(g.resid, float("nan"))
    lib.moe_combine_gr_write(P, y, pos, w, ysh, sl, g.resid, g.s, f2, out2)
    out3 = torch.full_like(g.resid, float("nan"))
    lib.moe_combine_gr_write(P, y, pos, w, ysh, sl, g.resid, g.s, None, out3)
    r = g.resid.clone()
    lib.moe_combine_gr_write(P, y, pos, w, ysh, sl, r, g.s, None, r)
    torch.cuda.synchronize()
    assert torch.equal(f2, f)
    assert torch.equal(out2, ref) and torch.equal(out3, ref) and torch.equal(r, ref)
    # and against the oracle's write of the stored F(x)
    want = ogr.gr_write(g.host(g.resid), g.host(g.s), f.float().cpu().numpy())
    got = out2.float().cpu().numpy()
    assert not (np.abs(got - want) > np.abs(want) * (2.0 ** -8 + 2.0 ** -23)).any()


def test_gr_empty_batch_is_a_no_op():
    P = _problem(0, 2560)
    dev = torch.device("cuda")
    g = make_gr_problem(1, 2560, RANK, seed=0, device="cuda")
    G = lib.gr_weights(g.norm_w, g.w_read, g.w_up, RANK, g.eps)
    e = torch.empty(0, device=dev)
    lib.moe_gr_read(P, G, e, e, e, torch.empty(256, dtype=torch.uint8, device=dev))
    lib.moe_gr_write(P, e, e, e, e)
    torch.cuda.synchronize()
