"""Bind a layer's torch tensors to the C structs (argument marshalling only).

`layer` is any object with the attributes
  cfg (T, H, E, k, I, I_shared, act, wdt, scale_block), x, w_router,
  w_gate, w_up, w_down, s_gate, s_up, s_down, sh_gate, sh_up, sh_down, sh_gate_w
holding contiguous device tensors (or None where absent).
"""
from __future__ import annotations

from . import problem, weights


def structs(layer, flags: int = 0, T: int = None):
    c = layer.cfg
    p = problem(c.T if T is None else T, c.H, c.E, c.k, c.I, c.I_shared, c.act, c.wdt, c.scale_block, flags)
    w = weights(layer.w_router, layer.w_gate, layer.w_up, layer.w_down, layer.s_gate, layer.s_up, layer.s_down,
                layer.sh_gate, layer.sh_up, layer.sh_down, layer.sh_gate_w)
    return p, w
