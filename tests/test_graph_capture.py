"""The whole-layer call inside a captured HIP graph.

A layer with both 256-row tiles and streamed groups forks its streaming
launches onto the library's second stream and joins them back; under capture
the fork and join become graph edges.  The graph is replayed several times,
with eager work (a fill, a reduction, an eager layer call) and
synchronisations between the replays, and every replay must give the eager
call's bits.
"""
import pytest
import torch

import sparse_moe_layer_amd as lib
from oracle import adapter
from sparse_moe_layer_amd.tensors import structs
from synthetic import CONFIGS, make_problem

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,flags", [("max_prefill", lib.MOE_FLAG_GEMM_TILE_256), ("max_fp8", 0),
                                        ("flash_decode", 0)])
def test_layer_call_replays_under_graph_capture(name, flags):
    base = CONFIGS[name]
    if name == "flash_decode":
        cfg = base.with_(name="graph_decode", T=16, H=256, E=64, k=8, I=128, I_shared=64)
    else:
        cfg = base.with_(name="graph_" + name, T=1536, H=256, E=16, k=2, I=128,
                         I_shared=64 if name == "max_prefill" else 0, zipf_s=1.1)
    print(f"[graph] {cfg.name} flags={flags}", flush=True)
    p = make_problem(cfg, 41, device="cuda")
    adapter.ensure_margin(p, 1e-3)
    P, W = structs(p, flags)
    ws = lib.workspace(P)
    ref = torch.empty((cfg.T, cfg.H), dtype=p.x.dtype, device="cuda")
    # eager first: creates the library's second stream outside the capture
    lib.moe_layer_forward(P, W, p.x, ref, None, None, ws)
    torch.cuda.synchronize()
    out = torch.zeros_like(ref)
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        lib.moe_layer_forward(P, W, p.x, out, None, None, ws, side)
    other = torch.empty_like(ref)
    for i in range(4):
        out.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()
        lib.moe_layer_forward(P, W, p.x, other, None, None, ws)  # eager use of the same workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {i} differs"
        assert torch.equal(other.view(torch.int16), ref.view(torch.int16))
        del junk
