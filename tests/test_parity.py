"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Expert ids, the dispatch offsets and permutation must match bit-exact (inputs
are redrawn until every token's sorted fp32 logits have gaps >= 1e-3 between
consecutive ranks 1..k+1).  Float outputs must satisfy
max|gpu - ref| <= tol * max|ref| with tol 2e-2 (bf16), 6e-2 (fp8 weights),
1e-5 (fp32 layer); routing weights within 1e-5 absolute.

Full-size workloads are checked on every integer output and on sampled
tokens for the float outputs (the oracle evaluates those tokens one expert at
a time); small and edge-case layers are checked everywhere.
"""
import numpy as np
import pytest
import torch

import sparse_moe_layer_amd as lib
from oracle import adapter, moe
from sparse_moe_layer_amd.tensors import structs
from synthetic import CONFIGS, make_problem

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}


def tol(cfg):
    return TOL["fp8"] if cfg.wdt == "fp8" else TOL[cfg.act]


def gpu_problem(cfg, seed=0, page=False):
    print(f"[parity] generating {cfg.name} T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} I={cfg.I} "
          f"Is={cfg.I_shared} {cfg.act}/{cfg.wdt} seed={seed} page={page}", flush=True)
    p = make_problem(cfg, seed, device="cuda")
    adapter.ensure_margin(p, 1e-3, page=page)
    return p


def run_stages(p, flags=0):
    """Each stage through its own entry point, then the whole layer in one call."""
    c = p.cfg
    dev = p.x.device
    T, k, E, H = c.T, c.k, c.E, c.H
    P, W = structs(p, flags)
    ws = lib.workspace(P)
    sh = c.I_shared > 0
    ids = torch.full((T, k), -1, dtype=torch.int32, device=dev)
    w = torch.zeros((T, k), dtype=torch.float32, device=dev)
    sl = torch.zeros(T, dtype=torch.float32, device=dev) if sh else None
    lib.moe_route(P, p.x, p.w_router, p.sh_gate_w, ids, w, sl, ws)
    offs = torch.full((E + 1,), -1, dtype=torch.int32, device=dev)
    sa = torch.full((T * k,), -1, dtype=torch.int32, device=dev)
    pos = torch.full((T * k,), -1, dtype=torch.int32, device=dev)
    lib.moe_dispatch(P, ids, offs, sa, pos, ws)
    y = torch.zeros((T * k, H), dtype=p.x.dtype, device=dev)
    ysh = torch.zeros((T, H), dtype=p.x.dtype, device=dev) if sh else None
    lib.moe_expert_ffn(P, W, p.x, offs, sa, y, ysh, ws)
    # the two GEMM phases as separate calls must give the same bits
    hh = torch.zeros((T * k, c.I), dtype=p.x.dtype, device=dev)
    hh_sh = torch.zeros((T, c.I_shared), dtype=p.x.dtype, device=dev) if sh else None
    y2 = torch.zeros_like(y)
    y2_sh = torch.zeros_like(ysh) if sh else None
    lib.moe_expert_gate_up(P, W, p.x, offs, sa, hh, hh_sh, ws)
    lib.moe_expert_down(P, W, offs, hh, hh_sh, y2, y2_sh, ws)
    out = torch.zeros((T, H), dtype=p.x.dtype, device=dev)
    lib.moe_combine(P, y, pos, w, ysh, sl, out)
    out2 = torch.zeros((T, H), dtype=p.x.dtype, device=dev)
    ids2 = torch.full((T, k), -1, dtype=torch.int32, device=dev)
    w2 = torch.zeros((T, k), dtype=torch.float32, device=dev)
    lib.moe_layer_forward(P, W, p.x, out2, ids2, w2, ws)
    torch.cuda.synchronize()
    f = lambda t: None if t is None else t.detach().float().cpu().numpy() if t.is_floating_point() else t.cpu().numpy()
    assert torch.equal(y.view(torch.int16) if y.dtype == torch.bfloat16 else y,
                       y2.view(torch.int16) if y2.dtype == torch.bfloat16 else y2), "split GEMM phases differ"
    if sh:
        assert torch.equal(ysh.float(), y2_sh.float()), "split GEMM phases differ (shared)"
    # the one-call layer gives the same bits as the stage calls (a small
    # batch's top-k and dispatch run as one kernel there)
    assert torch.equal(ids2, ids) and torch.equal(w2, w), "layer call routing differs"
    assert torch.equal(out2.float(), out.float()), "layer call output differs"
    return dict(ids=f(ids), w=f(w), sl=f(sl), offsets=f(offs), sorted=f(sa), pos=f(pos), y=f(y), ysh=f(ysh),
                out=f(out), out_layer=f(out2), ids_layer=f(ids2), w_layer=f(w2))


def rel_err(a, ref):
    return np.abs(a - ref).max() / max(np.abs(ref).max(), 1e-30)


def check(p, g, tokens=None, page=False):
    c = p.cfg
    r = adapter.forward(p, tokens, page=page)
    tk = r["tokens"]
    # integer outputs: bit-exact
    assert np.array_equal(g["ids"], r["ids"]), "expert ids differ"
    assert np.array_equal(g["ids_layer"], r["ids"]), "expert ids (layer call) differ"
    assert np.array_equal(g["offsets"], r["offsets"]), "expert offsets differ"
    assert np.array_equal(g["sorted"], r["sorted_assign"]), "dispatch permutation differs"
    assert np.array_equal(g["pos"], r["assign_pos"]), "inverse permutation differs"
    # routing weights (bf16-rounded with the page's numerics: one bf16 step,
    # 2^-8 below 1, where fp32 and fp64 land on either side of a rounding boundary)
    wtol = 2.0 ** -8 if page and c.act == "bf16" else 1e-5
    assert np.abs(g["w"] - r["w"]).max() <= wtol
    assert np.abs(g["w_layer"] - r["w"]).max() <= wtol
    if c.I_shared > 0:
        assert np.abs(g["sl"] - r["shared_logit"]).max() <= 1e-4 * (1 + np.abs(r["shared_logit"]).max())
    # per-assignment expert outputs (permuted rows) and the shared expert
    k = c.k
    rows = g["pos"][(tk[:, None] * k + np.arange(k)[None, :]).reshape(-1)]
    y_gpu = g["y"][rows].reshape(len(tk), k, c.H)
    e_y = rel_err(y_gpu, r["y"])
    assert e_y <= tol(c), f"routed expert outputs rel err {e_y:.3e}"
    if c.I_shared > 0:
        e_sh = rel_err(g["ysh"][tk], r["y_shared"])
        assert e_sh <= tol(c), f"shared expert rel err {e_sh:.3e}"
    e_out = rel_err(g["out"][tk], r["out"])
    e_lay = rel_err(g["out_layer"][tk], r["out"])
    print(f"[parity] {c.name}: y {e_y:.2e} out {e_out:.2e} layer {e_lay:.2e} (tol {tol(c):.0e}) "
          f"tokens {len(tk)}", flush=True)
    assert e_out <= tol(c), f"combine output rel err {e_out:.3e}"
    assert e_lay <= tol(c), f"layer output rel err {e_lay:.3e}"
    return r


def sample_tokens(T, n, seed=0):
    if n >= T:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(T, n - 2, replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(pick))


# Rows per expert group at or below which a group streams its weights instead
# of taking GEMM tiles, and the two m-tile heights of the GEMM kernels.
STREAM_ROWS = 16
TILE_ROWS = (128, 256)


def tile_class_tokens(g, cfg, per_class=2):
    """Tokens whose rows land in every kind of tile the expert GEMMs form.

    From the (already bit-exact) expert offsets and permutation: per expert
    group of n rows, rows at the edges of full m-tiles of either height, the
    first and last rows of a ragged last m-tile (after full tiles, alone, and
    one row long), and rows of groups that stream (n <= STREAM_ROWS, one row
    long included).  Shared-expert rows are the tokens themselves, so token
    indices at m-tile edges cover its tiles.  Every sampled row is compared
    over all output columns, which covers every n-tile of both phases.
    Returns (tokens, {class: [(expert, row in group, token), ...]})."""
    offs, sa, k = g["offsets"], g["sorted"], cfg.k
    n = np.diff(offs)
    order = np.argsort(-n, kind="stable")          # hottest groups first
    classes = {}

    def add(cls, e, r):
        lst = classes.setdefault(cls, [])
        if len(lst) < per_class and r < n[e]:
            lst.append((int(e), int(r), int(sa[offs[e] + r]) // k))

    for e in order:
        ne = int(n[e])
        if ne == 0:
            continue
        if ne <= STREAM_ROWS:
            add("stream" if ne > 1 else "stream_1row", e, ne - 1)
            add("stream_first", e, 0)
            continue
        for bm in TILE_ROWS:
            full, rem = divmod(ne, bm)
            if full:
                add(f"full{bm}_edges", e, 0)
                add(f"full{bm}_edges", e, bm - 1)
                if full > 1:
                    add(f"full{bm}_inner", e, bm)
            if rem:
                where = "after_full" if full else "alone"
                add(f"ragged{bm}_{where}_first", e, full * bm)
                add(f"ragged{bm}_{where}_last", e, ne - 1)
                if rem == 1:
                    add(f"ragged{bm}_1row", e, ne - 1)
    toks = {0, cfg.T - 1}
    if cfg.I_shared > 0:
        for bm in TILE_ROWS:
            toks |= {t for t in (bm - 1, bm, cfg.T - (cfg.T % bm or bm)) if 0 <= t < cfg.T}
    for lst in classes.values():
        toks |= {t for _, _, t in lst}
    return np.array(sorted(toks)), classes


# ----------------------------------------------------------------------------
# The five workloads at full size
# ----------------------------------------------------------------------------
@pytest.mark.timeout(400)
@pytest.mark.parametrize("name,n_tok", [("toy_fp32", None), ("flash_decode", None), ("flash_prefill", 8),
                                        ("max_fp8", 4), ("max_prefill", 4)])
def test_workload_parity(name, n_tok):
    """Small workloads everywhere; full-size ones on tokens chosen to put a
    row in every tile class of both GEMM phases, plus a few drawn at random."""
    cfg = CONFIGS[name]
    p = gpu_problem(cfg)
    g = run_stages(p)
    if n_tok is None:
        check(p, g)
    else:
        toks, classes = tile_class_tokens(g, cfg, per_class=1)
        for cls, lst in sorted(classes.items()):
            print(f"[coverage] {name} {cls}: " + ", ".join(f"e{e} row {r} -> t{t}" for e, r, t in lst), flush=True)
        assert any(c.startswith("ragged") for c in classes), "no ragged m-tile sampled"
        if cfg.zipf_s:
            # the skewed batches hold full 256-row tiles, ragged tails and streamed groups
            assert any(c.startswith("full256") for c in classes), "no full 256-row tile sampled"
            assert any(c.startswith("stream") for c in classes), "no streamed group sampled"
        toks = np.union1d(toks, sample_tokens(cfg.T, n_tok))
        print(f"[coverage] {name}: {len(classes)} classes, {len(toks)} tokens", flush=True)
        check(p, g, toks)
    del p
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------
# Edge cases (small layers, every token checked)
# ----------------------------------------------------------------------------
RAGGED = CONFIGS["flash_prefill"].with_(name="ragged", T=37, H=136, E=12, k=3, I=72, I_shared=40)


@pytest.mark.parametrize("flags", [0, lib.MOE_FLAG_FORCE_GEMM, lib.MOE_FLAG_FORCE_STREAM])
def test_ragged_shapes_both_paths(flags):
    p = gpu_problem(RAGGED, 1)
    check(p, run_stages(p, flags))


@pytest.mark.parametrize("flags", [lib.MOE_FLAG_FORCE_GEMM, lib.MOE_FLAG_FORCE_STREAM])
def test_paths_multi_tile_groups(flags):
    # several m-tiles per expert and several n-tiles, both paths
    cfg = CONFIGS["flash_prefill"].with_(name="multitile", T=700, H=320, E=4, k=2, I=192, I_shared=96)
    p = gpu_problem(cfg, 2)
    check(p, run_stages(p, flags))


@pytest.mark.parametrize("tile", [lib.MOE_FLAG_GEMM_TILE_128, lib.MOE_FLAG_GEMM_TILE_256])
def test_gemm_tile_kernels(tile):
    # experts with several 256-row tiles plus ragged remainders (partial M-blocks)
    cfg = CONFIGS["flash_prefill"].with_(name="tiles", T=900, H=512, E=4, k=2, I=384, I_shared=128)
    p = gpu_problem(cfg, 12)
    check(p, run_stages(p, lib.MOE_FLAG_FORCE_GEMM | tile))


def test_256_row_tiles_with_128_row_remainders():
    # skewed load in 256-row tiling: every m-tile of a group, its ragged last
    # one included, runs in the persistent 256-row kernel; the streamed
    # groups run beside it on the library's second stream
    cfg = CONFIGS["max_prefill"].with_(name="two_lists", T=1536, H=256, E=16, k=2, I=128, I_shared=64,
                                       zipf_s=1.1)
    p = gpu_problem(cfg, 13)
    g = run_stages(p, lib.MOE_FLAG_GEMM_TILE_256)
    n = np.diff(g["offsets"])
    r = n % 256
    assert np.any((n > 0) & (n <= 16))                 # streamed
    assert np.any((n > 16) & (n <= 128))               # one 128-row tile only
    assert np.any((n > 256) & (r > 0) & (r <= 128))    # 256-row tiles + a 128-row remainder
    assert np.any((n > 128) & (r > 128))               # ends in a partial 256-row tile
    assert cfg.T % 256 == 0                            # the shared expert: whole 256-row tiles
    check(p, g)


@pytest.mark.parametrize("shared", [0, 128])
@pytest.mark.parametrize("force", [0, lib.MOE_FLAG_FORCE_GEMM])
def test_fp8_256_row_tiles(shared, force):
    # fp8 codes through the 256-row direct-load tiles: several K blocks of
    # scales (H = 384, I = 256), the last W_down row block of a tile past H
    # (its scales clamped), ragged remainders in the 128-row fp8 tiles, the
    # shared expert in bf16 tiles of both kernels
    cfg = CONFIGS["max_fp8"].with_(name="fp8_tiles", T=1536, H=384, E=8, k=2, I=256, I_shared=shared,
                                   zipf_s=1.1)
    p = gpu_problem(cfg, 14)
    g = run_stages(p, lib.MOE_FLAG_GEMM_TILE_256 | force)
    n = np.diff(g["offsets"])
    assert np.any(n >= 256) and np.any((n % 256 > 0) & (n % 256 <= 128))
    check(p, g)


def test_one_expert_takes_every_token():
    # a steep per-expert bias: the rank-1 expert wins every token (k = 1)
    cfg = CONFIGS["max_prefill"].with_(name="all_to_one", T=300, H=256, E=8, k=1, I=128, I_shared=64, zipf_s=8.0)
    p = gpu_problem(cfg, 3)
    g = run_stages(p)
    assert np.count_nonzero(np.diff(g["offsets"])) == 1
    check(p, g)


def test_k_equals_E_and_E1_k1():
    cfg = CONFIGS["flash_prefill"].with_(name="k_eq_E", T=40, H=128, E=8, k=8, I=64, I_shared=0)
    p = gpu_problem(cfg, 4)
    check(p, run_stages(p))
    cfg = CONFIGS["flash_prefill"].with_(name="E1k1", T=33, H=128, E=1, k=1, I=64, I_shared=64)
    p = gpu_problem(cfg, 5)
    g = run_stages(p)
    assert np.all(g["w"] == 1.0)
    check(p, g)


def test_single_token_and_many_empty_experts():
    cfg = CONFIGS["flash_decode"].with_(name="one_token", T=1, H=256, E=512, k=10, I=128, I_shared=128)
    p = gpu_problem(cfg, 6)
    g = run_stages(p)
    assert np.count_nonzero(np.diff(g["offsets"])) == 10
    check(p, g)


@pytest.mark.parametrize("shared", [0, 128])
def test_fp8_decode_batch(shared):
    # T <= 16: the streaming kernels list the groups themselves; fp8 routed
    # groups and the bf16 shared expert in their two launches
    cfg = CONFIGS["max_fp8"].with_(name="fp8_decode", T=12, H=512, E=64, k=4, I=256, I_shared=shared, zipf_s=0.0)
    p = gpu_problem(cfg, 15)
    check(p, run_stages(p))


def test_decode_batch_max_experts():
    # E = 1024, the most experts a layer may have: the groups are listed in
    # four 256-group chunks
    cfg = CONFIGS["flash_decode"].with_(name="e1024", T=16, H=256, E=1024, k=8, I=64, I_shared=64)
    p = gpu_problem(cfg, 16)
    g = run_stages(p)
    assert np.count_nonzero(np.diff(g["offsets"])[768:]) > 0  # touched groups in the last chunk
    check(p, g)


@pytest.mark.parametrize("T,E,k,H,Is", [(1, 40, 3, 256, 0), (7, 100, 10, 512, 64), (16, 64, 64, 128, 128),
                                         (16, 512, 10, 136, 64), (12, 1000, 8, 2560, 640)])
def test_small_batch_fused_route_and_dispatch(T, E, k, H, Is):
    # T <= 16, bf16: the layer call's dispatch is built by the gate/up
    # streaming launch from the top-k ids (k = 64 gives R = 1024 assignments,
    # the most it takes); same bits as the dispatch kernels of the stage calls
    # (offsets, sorted and pos feed the down launch and the combine)
    cfg = CONFIGS["flash_decode"].with_(name=f"small_T{T}_E{E}_k{k}", T=T, H=H, E=E, k=k, I=64, I_shared=Is)
    p = gpu_problem(cfg, 21 + T)
    g = run_stages(p)
    check(p, g)


@pytest.mark.parametrize("T,E,k,H,I,Is", [(16, 64, 8, 200, 8, 24), (3, 20, 2, 96, 16, 0), (9, 33, 33, 40, 24, 8),
                                           (16, 400, 24, 128, 32, 16)])
def test_small_batch_layer_edge_shapes(T, E, k, H, I, Is):
    # T <= 16, bf16 (the dispatch from the gate/up streaming launch): one
    # gate/up item per group (I = 8), a shared expert wider than the routed
    # ones, no shared expert, every expert touched (k = E), output columns
    # that end inside a down item (H % 32 != 0), 384 assignments over up to
    # 400 groups.  The layer call must give the stage calls' bits.
    cfg = CONFIGS["flash_decode"].with_(name=f"small_edge_T{T}_E{E}_k{k}", T=T, H=H, E=E, k=k, I=I, I_shared=Is)
    p = gpu_problem(cfg, 41 + T)
    check(p, run_stages(p))


@pytest.mark.parametrize("case", ["f32", "fp8", "gemm"])
def test_small_batch_dispatch_from_topk(case):
    # T <= 16 with fp32 activations, fp8 weights or the GEMM path forced: the
    # layer call's top-k workgroups also dispatch (the last one to finish)
    if case == "fp8":
        cfg = CONFIGS["max_fp8"].with_(name="small_fp8", T=16, H=256, E=96, k=6, I=128, I_shared=128, zipf_s=0.0)
    else:
        cfg = CONFIGS["flash_decode"].with_(name=f"small_{case}", T=13, H=192, E=80, k=7, I=96, I_shared=64,
                                            act="f32" if case == "f32" else "bf16",
                                            wdt="f32" if case == "f32" else "bf16")
    p = gpu_problem(cfg, 31)
    check(p, run_stages(p, lib.MOE_FLAG_FORCE_GEMM if case == "gemm" else 0))


@pytest.mark.timeout(400)
def test_per_assignment_outputs_beyond_2_31_elements():
    # R*H > 2^31: the rows of y past element 2^31 (64-bit offsets in the
    # GEMM epilogues and the combine) checked against the oracle
    cfg = CONFIGS["max_prefill"].with_(name="big_y", T=32800, H=8192, E=16, k=8, I=128, I_shared=128, zipf_s=0.0)
    T, H, E, k = cfg.T, cfg.H, cfg.E, cfg.k
    R = T * k
    assert R * H > 2 ** 31
    p = gpu_problem(cfg, 51)
    P, W = structs(p)
    ws = lib.workspace(P)
    dev = p.x.device
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    sl = torch.empty(T, dtype=torch.float32, device=dev)
    lib.moe_route(P, p.x, p.w_router, p.sh_gate_w, ids, w, sl, ws)
    offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sa = torch.empty(R, dtype=torch.int32, device=dev)
    pos = torch.empty(R, dtype=torch.int32, device=dev)
    lib.moe_dispatch(P, ids, offs, sa, pos, ws)
    y = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
    ysh = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    lib.moe_expert_ffn(P, W, p.x, offs, sa, y, ysh, ws)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    lib.moe_combine(P, y, pos, w, ysh, sl, out)
    out2 = torch.empty_like(out)
    lib.moe_layer_forward(P, W, p.x, out2, None, None, ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    # tokens with an assignment in y rows at or past element 2^31, and the ends
    first_far = 2 ** 31 // H
    far_tok = torch.unique(sa[first_far:].long() // k).cpu().numpy()
    rng = np.random.default_rng(5)
    toks = np.union1d(rng.choice(far_tok, min(8, len(far_tok)), replace=False), [0, T - 1])
    print(f"[parity] big_y: {len(far_tok)} tokens with rows past 2^31 elements; checking {len(toks)}", flush=True)
    r = adapter.forward(p, toks)
    assert np.array_equal(ids.cpu().numpy(), r["ids"])
    assert np.array_equal(offs.cpu().numpy(), r["offsets"])
    assert np.array_equal(sa.cpu().numpy(), r["sorted_assign"])
    assert np.array_equal(pos.cpu().numpy(), r["assign_pos"])
    rows = pos.cpu().numpy()[(toks[:, None] * k + np.arange(k)[None, :]).reshape(-1)]
    assert (rows >= first_far).any()
    y_s = y[torch.from_numpy(rows).long().to(dev)].float().cpu().numpy().reshape(len(toks), k, H)
    e_y = rel_err(y_s, r["y"])
    e_out = rel_err(out[torch.from_numpy(toks).long().to(dev)].float().cpu().numpy(), r["out"])
    print(f"[parity] big_y: y {e_y:.2e} out {e_out:.2e}", flush=True)
    assert e_y <= tol(cfg) and e_out <= tol(cfg)
    del y, ysh, out, out2, ws, p
    torch.cuda.empty_cache()


def test_decode_batch_forced_gemm():
    # T <= 16 with the GEMM path forced: the plan kernel runs, no group streams
    cfg = CONFIGS["flash_decode"].with_(name="decode_gemm", T=16, H=256, E=32, k=4, I=128, I_shared=64)
    p = gpu_problem(cfg, 17)
    check(p, run_stages(p, lib.MOE_FLAG_FORCE_GEMM))


def test_empty_batch_is_noop():
    cfg = CONFIGS["flash_prefill"].with_(name="empty", T=0, H=128, E=8, k=2, I=64, I_shared=64)
    p = make_problem(cfg, 0, device="cuda")
    P, W = structs(p)
    ws = lib.workspace(P)
    out = torch.full((1, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    lib.moe_layer_forward(P, W, p.x, out, None, None, ws)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


@pytest.mark.parametrize("T", [20, 300])
def test_dispatch_repeated_and_out_of_range_ids(T):
    # moe_dispatch takes caller ids (the router never repeats one within a
    # token): a repeated id still gets its own slot, in ascending flat index
    # like the oracle's stable sort, and ids outside [0, E) are clamped into
    # range, so the outputs stay a permutation and its inverse.  T = 20 runs
    # the one-workgroup dispatch, T = 300 the chunked one.
    E, k = 24, 6
    rng = np.random.default_rng(T)
    ids = rng.integers(0, 3, size=(T, k)).astype(np.int32)  # three experts: many repeats per token
    ids[::3] = rng.integers(0, E, size=ids[::3].shape)
    P = lib.problem(T, 64, E, k, 64, 0)
    ws = lib.workspace(P)
    for case in ("repeated", "clamped"):
        host = ids.copy()
        if case == "clamped":
            host[0, 0], host[1, 3], host[T - 1, k - 1] = -5, E + 7, -1
        print(f"[parity] dispatch T={T} {case}", flush=True)
        offs = torch.full((E + 1,), -1, dtype=torch.int32, device="cuda")
        sa = torch.full((T * k,), -1, dtype=torch.int32, device="cuda")
        pos = torch.full((T * k,), -1, dtype=torch.int32, device="cuda")
        lib.moe_dispatch(P, torch.from_numpy(host).cuda(), offs, sa, pos, ws)
        torch.cuda.synchronize()
        _, r_off, r_sa, r_pos = moe.dispatch(np.clip(host, 0, E - 1), E)
        assert np.array_equal(offs.cpu().numpy(), r_off)
        assert np.array_equal(sa.cpu().numpy(), r_sa)
        assert np.array_equal(pos.cpu().numpy(), r_pos)


@pytest.mark.parametrize("shared", [0, 128])
def test_fp8_small_with_and_without_shared(shared):
    cfg = CONFIGS["max_fp8"].with_(name="fp8_small", T=50, H=256, E=8, k=2, I=256, I_shared=shared)
    for flags in (lib.MOE_FLAG_FORCE_GEMM, lib.MOE_FLAG_FORCE_STREAM):
        p = gpu_problem(cfg, 7)
        check(p, run_stages(p, flags))


@pytest.mark.parametrize("flags", [0, lib.MOE_FLAG_FORCE_STREAM])
def test_fp8_streaming_several_batches(flags):
    # H = 1024: four 256-wide K batches and eight 128-wide scale blocks per
    # gate/up row; I = 384: the down rows end in half a batch
    cfg = CONFIGS["max_fp8"].with_(name="fp8_stream", T=24, H=1024, E=6, k=2, I=384, I_shared=128)
    p = gpu_problem(cfg, 10)
    check(p, run_stages(p, flags))


@pytest.mark.parametrize("name,n_tok,flags", [("flash_decode", None, 0), ("flash_prefill", 48, 0),
                                               ("ragged", None, lib.MOE_FLAG_FORCE_GEMM),
                                               ("ragged", None, lib.MOE_FLAG_FORCE_STREAM)])
def test_page_routing_numerics(name, n_tok, flags):
    # bf16-rounded logits for the top-k (ties to the lower id), bf16 mixing weights
    cfg = RAGGED if name == "ragged" else CONFIGS[name]
    p = gpu_problem(cfg, 21, page=True)
    r = check(p, run_stages(p, flags | lib.MOE_FLAG_PAGE_ROUTING), sample_tokens(cfg.T, n_tok or cfg.T),
              page=True)
    if name == "flash_prefill":
        # the rounding changes the selection or its order for some tokens
        fp32_ids = adapter.forward(p, np.array([0]))["ids"]
        assert not np.array_equal(fp32_ids, r["ids"])


def test_fused_gate_up_strides():
    cfg = CONFIGS["flash_prefill"].with_(name="fused", T=64, H=128, E=6, k=2, I=64, I_shared=0)
    p = gpu_problem(cfg, 8)
    ref = run_stages(p)
    fused = torch.cat([p.w_gate, p.w_up], dim=1).contiguous()  # [E, 2I, H], gate rows first
    P, _ = structs(p)
    W = lib.weights(p.w_router, fused, fused, p.w_down, stride_gate=2 * cfg.I * cfg.H,
                    stride_up=2 * cfg.I * cfg.H)
    W.w_up = fused.data_ptr() + cfg.I * cfg.H * fused.element_size()  # up rows follow the gate rows
    ws = lib.workspace(P)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")
    lib.moe_layer_forward(P, W, p.x, out, None, None, ws)
    torch.cuda.synchronize()
    assert np.array_equal(out.float().cpu().numpy(), ref["out_layer"])


@pytest.mark.parametrize("name,flags", [
    ("max_prefill", lib.MOE_FLAG_FORCE_GEMM | lib.MOE_FLAG_GEMM_TILE_128),
    ("max_prefill", lib.MOE_FLAG_FORCE_GEMM | lib.MOE_FLAG_GEMM_TILE_256),
    ("max_prefill", lib.MOE_FLAG_FORCE_STREAM),
    ("max_fp8", lib.MOE_FLAG_FORCE_GEMM | lib.MOE_FLAG_GEMM_TILE_256)])
def test_expert_parallel_share(name, flags):
    # one GPU's share under expert parallelism over 4 ranks: rank r owns the
    # experts e = r (mod 4), addressed through expert strides, and receives
    # the rows the routing sends them as a compact block; with the kernel
    # pinned, every row of its y has the bits of the whole layer's y row
    ranks = 4
    cfg = CONFIGS[name].with_(name="ep_" + name, T=384, H=256, E=16, k=4, I=128, I_shared=0)
    p = gpu_problem(cfg, 12)
    full = run_stages(p, flags)
    offs = full["offsets"].astype(np.int64)
    counts = np.diff(offs)
    tok = full["sorted"].astype(np.int64) // cfg.k
    fp8 = cfg.wdt == "fp8"
    for r in range(ranks):
        own = list(range(r, cfg.E, ranks))
        rows = np.concatenate([np.arange(offs[e], offs[e + 1]) for e in own])
        Rr = len(rows)
        print(f"[parity] ep share rank {r}: {Rr} rows", flush=True)
        if Rr == 0:
            continue
        xr = p.x.index_select(0, torch.from_numpy(tok[rows]).cuda())
        offr = torch.from_numpy(np.concatenate([[0], np.cumsum(counts[r::ranks])]).astype(np.int32)).cuda()
        sar = torch.arange(Rr, dtype=torch.int32, device="cuda")
        P = lib.problem(Rr, cfg.H, len(own), 1, cfg.I, 0, cfg.act, cfg.wdt, cfg.scale_block, flags)
        sc = [t[r::ranks].contiguous() if fp8 else None for t in (p.s_gate, p.s_up, p.s_down)]
        W = lib.weights(None, p.w_gate[r], p.w_up[r], p.w_down[r], *sc, stride_gate=ranks * cfg.I * cfg.H,
                        stride_up=ranks * cfg.I * cfg.H, stride_down=ranks * cfg.H * cfg.I)
        y = torch.zeros((Rr, cfg.H), dtype=p.x.dtype, device="cuda")
        lib.moe_expert_ffn(P, W, xr, offr, sar, y, None, lib.workspace(P))
        torch.cuda.synchronize()
        assert np.array_equal(y.float().cpu().numpy(), full["y"][rows]), f"rank {r}"


def test_run_to_run_bit_identical():
    cfg = CONFIGS["flash_prefill"].with_(name="determinism", T=512, H=512, E=64, k=6, I=128, I_shared=128)
    p = gpu_problem(cfg, 9)
    a = run_stages(p)
    b = run_stages(p)
    for key in ("ids", "w", "offsets", "sorted", "pos", "y", "out", "out_layer"):
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("name", ["flash_prefill", "max_fp8"])
def test_one_call_python_layer_forward(name):
    # the convenience wrapper infers the problem from the tensors and gives the
    # same bits as the stage-by-stage and struct-level calls
    cfg = CONFIGS[name].with_(name="conv_" + name, T=40, H=256, E=8, k=2, I=128,
                              I_shared=128 if name == "flash_prefill" else 0)
    p = gpu_problem(cfg, 10)
    ref = run_stages(p)
    out, ids, w = lib.layer_forward(p.x, cfg.k, p.w_router, p.w_gate, p.w_up, p.w_down, p.s_gate, p.s_up, p.s_down,
                                    p.sh_gate, p.sh_up, p.sh_down, p.sh_gate_w)
    torch.cuda.synchronize()
    assert np.array_equal(out.float().cpu().numpy(), ref["out_layer"])
    assert np.array_equal(ids.cpu().numpy(), ref["ids_layer"])
    assert np.array_equal(w.cpu().numpy(), ref["w_layer"])
