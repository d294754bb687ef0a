"""Plain fp64 CPU oracle of the routed Mixture-of-Experts FFN layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline of the benchmark may import or run this module.  The library path
(HIP kernels behind the C ABI) never calls it, and it shares no code, table or
helper with that path.

What is computed, and where the pages define it
------------------------------------------------
Source: the Qwen3.8-Flash-Next study, section "MoE: 512 experts behind a
width-640 intermediate" (its pipeline figure and its two equations), unless a
function says otherwise.

  expert(x) = W_down ( SiLU(W_gate x) * (W_up x) )                 eq. expert(x)
  MoE(x)    = sum_{e in top-k} p_e expert_e(x) + sigmoid(w_shared x) shared(x)
                                                                    eq. MoE(x)
  pipeline  : Router [T, E] -> top-k + normalise -> dispatch R = kT assignments
              -> grouped expert GEMMs -> weighted combine + gated shared expert
                                                  (figure; "The model at a glance"
                                                   defines R as kT, no drops)

Readings where the pages leave a step open (each is listed in the design notes):
  * logits are formed exactly (fp64) from the stored inputs and then rounded
    to fp32, the precision the section gives for the softmax; the selection
    is decided on those fp32 values (no rounding to the activation dtype);
  * top-k order is descending logit, ties to the lower expert id;
  * the selected probabilities are renormalised to sum to one, and the
    mixing weights are kept in full precision (not cast to the activation
    dtype);
  * dropless dispatch, stable: assignments a = t*k + j sorted by (expert, a);
  * the shared expert's gate is a scalar per token, sigmoid(w_sg . x_t), no bias;
  * fp8 routed weights are OCP E4M3FN codes times one fp32 scale per
    128x128 block ("What FP8 actually quantizes" in the "Qwen3.8, weights in
    hand" article names FP8 for the routed experts only).

No intermediate is rounded (h, y, y_shared stay fp64); the output is returned
in fp64 and compared against the GPU's act-dtype output with a tolerance.
"""
from __future__ import annotations

from typing import Callable, Dict, Optional, Tuple

import numpy as np


# ----------------------------------------------------------------------------
# Storage decoding (exact)
# ----------------------------------------------------------------------------
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> fp64.  A bf16 value is the fp32 value
    whose upper 16 bits are the pattern and whose lower 16 bits are zero."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """OCP 8-bit floating point E4M3FN codes (uint8) -> fp64.

    Bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa.  Exponent 0
    is subnormal: m/8 * 2^-6.  Otherwise (1 + m/8) * 2^(exp-7).  The pattern
    S.1111.111 is NaN; there is no infinity (max finite 448)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = c & 0x7
    sub = man / 8.0 * 2.0 ** -6
    nrm = (1.0 + man / 8.0) * np.exp2(ex - 7.0)
    val = np.where(ex == 0, sub, nrm) * sign
    val = np.where((ex == 15) & (man == 7), np.nan, val)
    return val.astype(np.float64)


def dequant_blocks(codes: np.ndarray, scales: np.ndarray, block: int = 128) -> np.ndarray:
    """w[n, k] = decode(q[n, k]) * s[n // block, k // block] for one matrix."""
    w = decode_e4m3fn(codes)
    s = np.asarray(scales, dtype=np.float64)
    n_idx = np.arange(w.shape[0]) // block
    k_idx = np.arange(w.shape[1]) // block
    return w * s[n_idx][:, k_idx]


def decode(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Stored tensor (raw host array) -> fp64.  dtype: 'f32' | 'bf16'."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return decode_bf16(raw)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# Elementwise functions
# ----------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) (hidden_act "silu" on the atlas page's config)."""
    return z / (1.0 + np.exp(-z))


def sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


# ----------------------------------------------------------------------------
# Router: logits, softmax, top-k, renormalisation
# ----------------------------------------------------------------------------
def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """l[t, e] = sum_h x[t, h] W_r[e, h]  (Router [T, E] in the figure), fp64."""
    return np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T


def shared_gate_logit(x: np.ndarray, sh_gate_w: np.ndarray) -> np.ndarray:
    """s[t] = w_sg . x_t, the argument of the shared expert's sigmoid gate."""
    return np.asarray(x, np.float64) @ np.asarray(sh_gate_w, np.float64).reshape(-1)


def to_fp32(a: np.ndarray) -> np.ndarray:
    """Round to fp32 (the softmax precision the section gives), back in fp64."""
    return np.asarray(a, np.float64).astype(np.float32).astype(np.float64)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (the activation dtype), back in fp64: the value is
    first taken to fp32, then its low 16 bits are rounded away to nearest,
    ties to even (add 0x7FFF plus the lowest kept bit, truncate)."""
    u = np.asarray(a, np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def softmax(logits: np.ndarray) -> np.ndarray:
    """p[t, e] = exp(l[t,e] - max_e l) / sum_e exp(l[t,e] - max_e l) over all E."""
    m = logits.max(axis=1, keepdims=True)
    ex = np.exp(logits - m)
    return ex / ex.sum(axis=1, keepdims=True)


def topk_ids(logits: np.ndarray, k: int) -> np.ndarray:
    """Per token, the k experts with the largest logits, in descending logit
    order; equal logits are ordered by ascending expert id.  int32 [T, k]."""
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    eidx = np.arange(E)
    for t in range(T):
        order = np.lexsort((eidx, -logits[t]))  # primary: -logit, secondary: id
        ids[t] = order[:k]
    return ids


def renormalised_weights(probs: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """w[t, j] = p[t, ids[t,j]] / sum_j' p[t, ids[t,j']]  ("Selected router
    probabilities are normalized")."""
    sel = np.take_along_axis(probs, ids.astype(np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def route(x: np.ndarray, w_router: np.ndarray, k: int, page: bool = False):
    """Router -> top-k + normalise.  Returns (logits the selection used, ids, w).

    page=False: fp32 logits, full-precision mixing weights.
    page=True : the section's stated numerics for a bf16 model: the softmax
    runs on the logits rounded to the activation dtype, and the mixing
    weights are cast to the activation dtype.  Rounded logits tie often;
    ties go to the lower expert id."""
    l = to_fp32(router_logits(x, w_router))
    if page:
        l = round_bf16(l)
    ids = topk_ids(l, k)
    w = renormalised_weights(softmax(l), ids)
    if page:
        w = round_bf16(w)
    return l, ids, w


def margins(l32: np.ndarray, k: int, adjacent: bool = True) -> np.ndarray:
    """Per token, the smallest gap between consecutive ranks 1..k+1 of the
    sorted logits (adjacent=True) or only the rank-k / rank-(k+1) gap."""
    s = -np.sort(-l32, axis=1)
    kk = min(k + 1, l32.shape[1])
    gaps = s[:, : kk - 1] - s[:, 1:kk]
    if gaps.shape[1] == 0:
        return np.full(l32.shape[0], np.inf)
    if adjacent:
        return gaps.min(axis=1)
    return gaps[:, -1] if kk == k + 1 else np.full(l32.shape[0], np.inf)


def bf16_midpoint_distance(l32: np.ndarray, k: int) -> np.ndarray:
    """Per token, the smallest distance from an fp32 logit to a bf16 rounding
    boundary, over the experts that can decide the page-numerics top-k: every
    expert whose rounded logit is within 2^-7 (relative; at least one bf16
    step) of the (k+1)-th largest rounded logit, or above it.  Two fp32
    evaluations of a logit that differ by less than this distance round to
    the same bf16 value.  The boundaries around a bf16 value are the fp32
    numbers whose bit patterns are its own plus and minus 0x8000 (half a bf16
    step; this holds across binade edges too)."""
    T, E = l32.shape
    r = round_bf16(l32)
    out = np.full(T, np.inf)
    for t in range(T):
        v = -np.sort(-r[t])[min(k, E - 1)]
        crit = np.nonzero(r[t] >= v - max(abs(v), 2.0 ** -126) * 2.0 ** -7)[0]
        u = r[t, crit].astype(np.float32).view(np.uint32).astype(np.int64)
        mids = np.concatenate([(u + 0x8000), (u - 0x8000)]).astype(np.uint32).view(np.float32).astype(np.float64)
        vals = np.concatenate([l32[t, crit], l32[t, crit]])
        out[t] = np.abs(vals - mids).min()
    return out


# ----------------------------------------------------------------------------
# Dispatch ("Dispatch R tokens"): counting sort of the R = T*k assignments
# ----------------------------------------------------------------------------
def dispatch(ids: np.ndarray, E: int):
    """Histogram -> exclusive prefix sum -> stable scatter.

    counts[e]        = number of assignments to expert e
    offsets[e]       = sum of counts[0..e-1]; offsets[E] = R
    sorted_assign[p] = flat assignment a = t*k + j placed at p; within an
                       expert the assignments keep ascending a
    assign_pos[a]    = p, the inverse permutation
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    R = flat.size
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:E].copy()
    sorted_assign = np.empty(R, dtype=np.int64)
    assign_pos = np.empty(R, dtype=np.int64)
    for a in range(R):  # ascending a keeps each expert's segment stable
        e = flat[a]
        p = cursor[e]
        cursor[e] += 1
        sorted_assign[p] = a
        assign_pos[a] = p
    return (counts.astype(np.int32), offsets.astype(np.int32),
            sorted_assign.astype(np.int32), assign_pos.astype(np.int32))


# ----------------------------------------------------------------------------
# Experts
# ----------------------------------------------------------------------------
def swiglu(x: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """expert(x) = W_down (SiLU(W_gate x) * (W_up x)) for each row x of X [n, H].
    W_gate, W_up: [I, H]; W_down: [H, I] (PyTorch Linear out x in).  [n, H] fp64."""
    g = x @ w_gate.T
    u = x @ w_up.T
    return (silu(g) * u) @ w_down.T


ExpertFn = Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]]


def routed_outputs(x: np.ndarray, ids: np.ndarray, E: int, expert_weights: ExpertFn,
                   tokens: Optional[np.ndarray] = None) -> np.ndarray:
    """y[t, j] = expert_{ids[t,j]}(x_t), fp64 [T', k, H] for the rows `tokens`
    (all rows by default).  expert_weights(e) -> fp64 (W_gate, W_up, W_down)."""
    if tokens is None:
        tokens = np.arange(x.shape[0])
    tokens = np.asarray(tokens)
    k = ids.shape[1]
    sub_ids = ids[tokens]
    y = np.zeros((len(tokens), k, x.shape[1]), dtype=np.float64)
    for e in np.unique(sub_ids):
        rows, js = np.nonzero(sub_ids == e)
        wg, wu, wd = expert_weights(int(e))
        y[rows, js] = swiglu(x[tokens[rows]], wg, wu, wd)
    return y


def combine(y: np.ndarray, w: np.ndarray, y_shared: Optional[np.ndarray] = None,
            gamma: Optional[np.ndarray] = None) -> np.ndarray:
    """out_t = sum_j w[t,j] y[t,j] + gamma_t y_shared[t]  (eq. MoE(x))."""
    out = np.einsum("tj,tjh->th", w, y)
    if y_shared is not None:
        out = out + gamma[:, None] * y_shared
    return out


def moe_forward(x: np.ndarray, w_router: np.ndarray, k: int, expert_weights: ExpertFn,
                E: Optional[int] = None, shared: Optional[Tuple[np.ndarray, np.ndarray, np.ndarray]] = None,
                sh_gate_w: Optional[np.ndarray] = None, tokens: Optional[np.ndarray] = None,
                page: bool = False) -> Dict[str, np.ndarray]:
    """The whole layer on fp64 inputs.  Routing and dispatch cover all T tokens;
    the expert math and combine cover `tokens` (default: all).

    page: the routing numerics of `route(page=True)`.

    Returns logits (as the selection used them), ids, w, counts, offsets, sorted_assign,
    assign_pos, shared_logit, gamma, y (routed outputs [T',k,H]),
    y_shared [T',H] and out [T',H] for the rows in `tokens`."""
    x = np.asarray(x, np.float64)
    E = w_router.shape[0] if E is None else E
    l32, ids, w = route(x, w_router, k, page)
    counts, offsets, sorted_assign, assign_pos = dispatch(ids, E)
    if tokens is None:
        tokens = np.arange(x.shape[0])
    tokens = np.asarray(tokens)
    y = routed_outputs(x, ids, E, expert_weights, tokens)
    res = dict(logits=l32, ids=ids, w=w, counts=counts, offsets=offsets,
               sorted_assign=sorted_assign, assign_pos=assign_pos, y=y, tokens=tokens)
    if shared is not None:
        s = shared_gate_logit(x, sh_gate_w)
        gamma = sigmoid(s)
        y_sh = swiglu(x[tokens], *shared)
        res.update(shared_logit=s, gamma=gamma, y_shared=y_sh,
                   out=combine(y, w[tokens], y_sh, gamma[tokens]))
    else:
        res.update(out=combine(y, w[tokens]))
    return res
