"""Glue between seeded problem objects and the fp64 oracle.

TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU baseline of the benchmark).
Duck-typed on the problem object (attributes cfg, x, w_router, sh_*, w_*, s_*
and host_raw()); it imports nothing from the generator or the library.
"""
from __future__ import annotations

import numpy as np

from . import moe


def _dec(problem, t, dt):
    return None if t is None else moe.decode(problem.host_raw(t), dt)


def dense_inputs(problem):
    """fp64 x, W_r, shared-expert triple (or None) and w_sg (or None)."""
    c = problem.cfg
    x = _dec(problem, problem.x, c.act)
    wr = _dec(problem, problem.w_router, c.act)
    shared = None
    sg = None
    if c.I_shared > 0:
        shared = (_dec(problem, problem.sh_gate, c.act), _dec(problem, problem.sh_up, c.act),
                  _dec(problem, problem.sh_down, c.act))
        sg = _dec(problem, problem.sh_gate_w, c.act).reshape(-1)
    return x, wr, shared, sg


def expert_weights_fn(problem):
    """e -> fp64 (W_gate[e], W_up[e], W_down[e]), decoded from storage."""
    c = problem.cfg

    def get(e):
        if c.wdt == "fp8":
            b = c.scale_block
            return tuple(moe.dequant_blocks(problem.host_raw(w[e]), problem.host_raw(s[e]), b)
                         for w, s in ((problem.w_gate, problem.s_gate), (problem.w_up, problem.s_up),
                                      (problem.w_down, problem.s_down)))
        return tuple(moe.decode(problem.host_raw(w[e]), c.wdt)
                     for w in (problem.w_gate, problem.w_up, problem.w_down))
    return get


def ensure_margin(problem, min_margin: float = 1e-3, adjacent: bool = True, max_attempts: int = 64,
                  page: bool = False, min_midpoint: float = 1e-4):
    """Redraw token rows of x until every token's routing is decided with room
    to spare against the GPU's own fp32 logit rounding (~1e-6):

    page=False: the sorted fp32 logits have gaps >= min_margin between
    consecutive ranks 1..k+1 (adjacent=True) or between ranks k and k+1;
    page=True : the fp32 logits of the experts that can decide the bf16-rounded
    top-k lie >= min_midpoint from every bf16 rounding boundary.

    Uses the oracle's router; returns the number of redraws."""
    c = problem.cfg
    wr = _dec(problem, problem.w_router, c.act)
    redraws = 0
    rows = np.arange(c.T)
    for _ in range(max_attempts + 1):
        x = moe.decode(problem.host_raw(problem.x[rows] if len(rows) < c.T else problem.x), c.act)
        l32 = moe.to_fp32(moe.router_logits(x, wr))
        if page:
            bad = rows[moe.bf16_midpoint_distance(l32, c.k) < min_midpoint]
        else:
            bad = rows[moe.margins(l32, c.k, adjacent) < min_margin]
        if bad.size == 0:
            return redraws
        attempts = [problem.x_attempts.get(int(t), 0) + 1 for t in bad]
        if max(attempts) > max_attempts:
            raise RuntimeError(f"margin not reached for tokens {bad[:8]}")
        problem.redraw_tokens([int(t) for t in bad], attempts)
        redraws += bad.size
        rows = bad
    raise RuntimeError("margin fix-up did not converge")


def forward(problem, tokens=None, page: bool = False):
    """Oracle forward pass of the problem; see moe.moe_forward.  page: the
    section's bf16 routing numerics (a no-op for fp32 layers, whose activation
    dtype is fp32)."""
    x, wr, shared, sg = dense_inputs(problem)
    return moe.moe_forward(x, wr, problem.cfg.k, expert_weights_fn(problem), problem.cfg.E,
                           shared, sg, tokens, page=page and problem.cfg.act == "bf16")
