"""Pins of the glue that turns a stored problem into the oracle's operands.

`oracle.adapter` decides which stored tensor is the gate, the up and the down
projection of each expert, which fp8 block scales belong to which codes, and
the order of the shared expert's triple.  These tests rebuild the layer from
the problem's *named* tensors with torch float64 CPU ops (a composition
written here from eq. expert(x) and eq. MoE(x) of the Qwen3.8-Flash-Next
study's MoE section, sharing nothing with the oracle's code), and check that
planting any of the plausible mix-ups in the glue changes its result.
"""
import numpy as np
import pytest
import torch

from oracle import adapter
from synthetic import CONFIGS, make_problem


def _small(wdt):
    base = CONFIGS["max_fp8" if wdt == "fp8" else "flash_prefill"]
    # every tensor of the layer distinct; a shared expert in both layouts
    return base.with_(name=f"adapter_{wdt}", T=12, H=256, E=6, k=3, I=128, I_shared=128, zipf_s=0.0)


def _dequant(codes: torch.Tensor, scales: torch.Tensor, b: int) -> torch.Tensor:
    vals = codes.view(torch.float8_e4m3fn).to(torch.float64)
    return vals * scales.to(torch.float64).repeat_interleave(b, 0).repeat_interleave(b, 1)


def _named(p, which: str, e: int) -> torch.Tensor:
    """Expert e's matrix `which` in fp64, read by name from the problem."""
    w = {"gate": p.w_gate, "up": p.w_up, "down": p.w_down}[which][e]
    if p.cfg.wdt == "fp8":
        s = {"gate": p.s_gate, "up": p.s_up, "down": p.s_down}[which][e]
        return _dequant(w, s, p.cfg.scale_block)
    return w.to(torch.float64)


def _torch_layer(p):
    """out[t] = sum_j w_tj expert_{e_tj}(x_t) + sigmoid(w_sg . x_t) shared(x_t)."""
    c = p.cfg
    x = p.x.to(torch.float64)
    # the section's softmax runs in fp32: logits formed exactly, then rounded to fp32
    logits = (x @ p.w_router.to(torch.float64).T).to(torch.float32).to(torch.float64)
    top = torch.topk(logits, c.k, dim=1)
    w = torch.softmax(top.values, dim=1)
    out = torch.zeros_like(x)
    for t in range(c.T):
        for j in range(c.k):
            e = int(top.indices[t, j])
            h = torch.nn.functional.silu(_named(p, "gate", e) @ x[t]) * (_named(p, "up", e) @ x[t])
            out[t] += w[t, j] * (_named(p, "down", e) @ h)
    if c.I_shared > 0:
        hs = torch.nn.functional.silu(x @ p.sh_gate.to(torch.float64).T) * (x @ p.sh_up.to(torch.float64).T)
        ys = hs @ p.sh_down.to(torch.float64).T
        gam = torch.sigmoid(x @ p.sh_gate_w.to(torch.float64).reshape(-1))
        out += gam[:, None] * ys
    return top.indices.numpy(), out.numpy()


@pytest.fixture(scope="module", params=["bf16", "fp8"])
def prob(request):
    p = make_problem(_small(request.param), 3)
    adapter.ensure_margin(p, 1e-3)
    return p


def test_adapter_forward_matches_named_composition(prob):
    ids, ref = _torch_layer(prob)
    got = adapter.forward(prob)
    assert np.array_equal(got["ids"], ids)
    assert np.abs(got["out"] - ref).max() <= 1e-12 * np.abs(ref).max()


class _Swapped:
    """The problem with some named tensors exchanged (a planted glue mistake)."""

    def __init__(self, p, **swap):
        self._p = p
        self._swap = swap

    def __getattr__(self, name):
        return getattr(self._p, self._swap.get(name, name))


@pytest.mark.parametrize("swap", [
    dict(w_gate="w_up", w_up="w_gate"),                       # (up, gate, down)
    dict(s_gate="s_up", s_up="s_gate"),                       # scales paired with the other codes
    dict(sh_gate="sh_up", sh_up="sh_gate"),                   # shared triple reordered
    dict(sh_gate_w="sh_gate_w_swapped"),                      # shared gate projection wrong
])
def test_planted_glue_mistakes_are_caught(prob, swap):
    if "s_gate" in swap and prob.cfg.wdt != "fp8":
        pytest.skip("bf16 layers carry no block scales")
    p = prob
    if "sh_gate_w" in swap:
        p.sh_gate_w_swapped = -p.sh_gate_w  # gamma -> 1 - gamma
    _, ref = _torch_layer(p)
    bad = adapter.forward(_Swapped(p, **swap))["out"]
    assert np.abs(bad - ref).max() > 1e-3 * np.abs(ref).max(), swap
