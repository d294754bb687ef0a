"""Pins of the fp64 oracle against things other than itself.

Each test fixes part of the oracle against a hand-worked example, a closed
form, a brute-force enumeration, a documented format value or an independent
library routine (torch's float64 CPU ops, Python's sorted), chosen so that a
dropped term, a wrong sign/index or a transposed operand fails at least one.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import moe

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def s(z):
    return 1.0 / (1.0 + math.exp(-z))


def _closed(expr):
    return eval(expr, {"s": s})  # expressions in the golden file use only s() and numbers


# ----------------------------------------------------------------------------
# storage decoding
# ----------------------------------------------------------------------------
def test_decode_bf16_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = moe.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # documented patterns: 1.0 = 0x3F80, -2.0 = 0xC000, 2^-7 = 0x3C00
    assert moe.decode_bf16(np.array([0x3F80, 0xC000, 0x3C00], np.uint16)).tolist() == [1.0, -2.0, 2.0 ** -7]


def test_decode_e4m3fn_documented_values():
    g = json.load(open(os.path.join(GOLD, "e4m3fn_codes.json")))
    for code, val in g["codes"].items():
        got = moe.decode_e4m3fn(np.array([int(code, 16)], np.uint8))[0]
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code
    for code in g["nan_codes"]:
        assert np.isnan(moe.decode_e4m3fn(np.array([int(code, 16)], np.uint8))[0])


def test_decode_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = moe.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_dequant_blocks_is_kron_of_scales():
    # every code = 1.0 (0x38): the dequantised matrix is the scale grid blown up
    rng = np.random.default_rng(0)
    sc = rng.uniform(0.5, 2.0, size=(3, 2))
    q = np.full((3 * 128, 2 * 128), 0x38, np.uint8)
    assert np.array_equal(moe.dequant_blocks(q, sc, 128), np.kron(sc, np.ones((128, 128))))
    # a single nonzero code lands in its own block's scale
    q = np.zeros((256, 256), np.uint8)
    q[130, 5] = 0x40  # 2.0 in row-block 1, col-block 0
    sc = np.array([[1.0, 3.0], [5.0, 7.0]])
    d = moe.dequant_blocks(q, sc, 128)
    assert d[130, 5] == 10.0 and np.count_nonzero(d) == 1


# ----------------------------------------------------------------------------
# elementwise
# ----------------------------------------------------------------------------
def test_silu_and_sigmoid_closed_forms():
    z = np.array([0.0, 1.0, -1.0, 2.0, 40.0, -40.0])
    assert np.allclose(moe.silu(z), [0.0, s(1), -s(-1), 2 * s(2), 40.0, 0.0], rtol=1e-15, atol=1e-15)
    assert np.allclose(moe.sigmoid(np.array([0.0, math.log(3)])), [0.5, 0.75], rtol=1e-15)
    zz = np.linspace(-8, 8, 101)
    assert np.allclose(moe.silu(zz), F.silu(torch.from_numpy(zz)).numpy(), rtol=1e-14, atol=1e-15)


# ----------------------------------------------------------------------------
# router
# ----------------------------------------------------------------------------
def test_router_logits_identity_and_permutation():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 6))
    assert np.array_equal(moe.router_logits(x, np.eye(6)), x)
    perm = np.array([3, 0, 5, 1, 4, 2])
    assert np.array_equal(moe.router_logits(x, np.eye(6)[perm]), x[:, perm])
    # non-square: W_r [E=2, H=3]; a transposed operand cannot produce [T, E]
    w = np.array([[1.0, 0, 0], [0, 0, 2.0]])
    assert moe.router_logits(np.array([[1.0, 2.0, 3.0]]), w).tolist() == [[1.0, 6.0]]


def test_softmax_closed_form_and_rows():
    l = np.array([[0.0, math.log(3.0)], [5.0, 5.0]])
    p = moe.softmax(l)
    assert np.allclose(p, [[0.25, 0.75], [0.5, 0.5]], rtol=1e-15)
    rng = np.random.default_rng(2)
    l = rng.standard_normal((7, 9)) * 3
    assert np.allclose(moe.softmax(l), torch.softmax(torch.from_numpy(l), dim=1).numpy(), rtol=1e-13)


@pytest.mark.parametrize("E,k", [(4, 1), (5, 2), (6, 3), (8, 3), (7, 7)])
def test_topk_brute_force(E, k):
    rng = np.random.default_rng(E * 10 + k)
    l = rng.standard_normal((40, E))
    ids = moe.topk_ids(l, k)
    for t in range(l.shape[0]):
        best = max(itertools.combinations(range(E), k), key=lambda c: sum(l[t, list(c)]))
        assert set(ids[t].tolist()) == set(best)
        vals = l[t, ids[t]]
        assert np.all(np.diff(vals) < 0)  # strictly descending (no ties in draws)


def test_topk_tie_goes_to_lower_id():
    l = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]])
    assert moe.topk_ids(l, 2).tolist() == [[1, 2]]
    assert moe.topk_ids(l, 4).tolist() == [[1, 2, 4, 3]]


def test_renormalised_weights_closed_forms():
    # k = 2: w = (s(a-b), s(b-a)) for the two selected logits a > b
    l = np.array([[0.3, 2.0, -1.0, 1.2]])
    ids = moe.topk_ids(l, 2)
    w = moe.renormalised_weights(moe.softmax(l), ids)
    assert np.allclose(w, [[s(0.8), s(-0.8)]], rtol=1e-14)
    # k = 1: weight exactly 1; k = E: the full softmax in id order
    rng = np.random.default_rng(3)
    l = rng.standard_normal((6, 5))
    w1 = moe.renormalised_weights(moe.softmax(l), moe.topk_ids(l, 1))
    assert np.allclose(w1, 1.0, rtol=0, atol=1e-15)
    idsE = moe.topk_ids(l, 5)
    wE = moe.renormalised_weights(moe.softmax(l), idsE)
    full = torch.softmax(torch.from_numpy(l), 1).numpy()
    assert np.allclose(wE, np.take_along_axis(full, idsE.astype(np.int64), 1), rtol=1e-13)
    # invariants on a larger draw
    _, ids, w = moe.route(rng.standard_normal((50, 16)), rng.standard_normal((32, 16)), 6)
    assert np.allclose(w.sum(1), 1.0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_route_rounds_logits_to_fp32_before_selecting():
    # two logits equal in fp32 but not in fp64 -> fp32 tie -> lower id first
    x = np.array([[1.0]])
    wr = np.array([[1.0], [1.0 + 2.0 ** -30]])
    l32, ids, w = moe.route(x, wr, 1)
    assert l32[0, 0] == l32[0, 1] and ids.tolist() == [[0]]


def test_margins():
    l = np.array([[5.0, 4.0, 3.5, 3.4, 0.0]])
    assert np.isclose(moe.margins(l, 2, adjacent=True)[0], 0.5)
    assert np.isclose(moe.margins(l, 2, adjacent=False)[0], 0.5)
    assert np.isclose(moe.margins(l, 3, adjacent=True)[0], 0.1)
    assert np.isclose(moe.margins(l, 3, adjacent=False)[0], 0.1)
    assert np.isclose(moe.margins(l, 1, adjacent=True)[0], 1.0)


# ----------------------------------------------------------------------------
# dispatch
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("T,E,k", [(1, 4, 2), (13, 5, 3), (64, 16, 4), (37, 8, 8), (50, 1, 1)])
def test_dispatch_against_comparison_sort(T, E, k):
    rng = np.random.default_rng(T + E + k)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, sorted_assign, assign_pos = moe.dispatch(ids, E)
    flat = ids.reshape(-1)
    R = T * k
    ref = sorted(range(R), key=lambda a: (int(flat[a]), a))
    assert sorted_assign.tolist() == ref
    assert counts.sum() == R and offsets[0] == 0 and offsets[E] == R
    assert np.all(np.diff(offsets) == counts)
    assert np.array_equal(assign_pos[sorted_assign], np.arange(R))
    for e in range(E):
        seg = sorted_assign[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


def test_dispatch_all_to_one_expert_and_empty():
    ids = np.full((6, 1), 3, np.int32)
    counts, offsets, sa, pos = moe.dispatch(ids, 5)
    assert counts.tolist() == [0, 0, 0, 6, 0] and offsets.tolist() == [0, 0, 0, 0, 6, 6]
    assert sa.tolist() == list(range(6)) and pos.tolist() == list(range(6))
    counts, offsets, sa, pos = moe.dispatch(np.zeros((0, 2), np.int32), 3)
    assert offsets.tolist() == [0, 0, 0, 0] and sa.size == 0


# ----------------------------------------------------------------------------
# experts and the whole layer
# ----------------------------------------------------------------------------
def _torch_swiglu(x, wg, wu, wd):
    """Textbook dense SwiGLU from torch library ops (float64 CPU)."""
    X = torch.from_numpy(x)
    return F.linear(F.silu(F.linear(X, torch.from_numpy(wg))) * F.linear(X, torch.from_numpy(wu)),
                    torch.from_numpy(wd)).numpy()


def test_worked_layer_example():
    g = json.load(open(os.path.join(GOLD, "worked_layer.json")))
    A = {k: np.array(v, dtype=np.float64) for k, v in g.items()
         if k in ("x", "w_router", "w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down", "sh_gate_w")}
    res = moe.moe_forward(A["x"], A["w_router"], g["k"],
                          lambda e: (A["w_gate"][e], A["w_up"][e], A["w_down"][e]), g["E"],
                          (A["sh_gate"], A["sh_up"], A["sh_down"]), A["sh_gate_w"])
    ex = g["expected"]
    assert res["ids"].tolist() == ex["ids"]
    assert res["offsets"].tolist() == ex["offsets"]
    assert res["sorted_assign"].tolist() == ex["sorted_assign"]
    assert res["assign_pos"].tolist() == ex["assign_pos"]
    w_exp = np.array([[_closed(v) for v in row] for row in ex["w"]])
    assert np.allclose(res["w"], w_exp, rtol=1e-14)
    assert np.allclose(res["gamma"], [float(v) for v in ex["gamma"]], rtol=1e-14)
    out_exp = np.array([[_closed(v) for v in row] for row in ex["out"]])
    assert np.allclose(res["out"], out_exp, rtol=1e-14, atol=1e-15)


def _rand_layer(rng, T, H, E, I, k, shared=True):
    x = rng.standard_normal((T, H))
    wr = rng.standard_normal((E, H)) * 0.5
    Wg = rng.standard_normal((E, I, H)) * 0.2
    Wu = rng.standard_normal((E, I, H)) * 0.2
    Wd = rng.standard_normal((E, H, I)) * 0.2
    sh = (rng.standard_normal((I, H)) * 0.2, rng.standard_normal((I, H)) * 0.2,
          rng.standard_normal((H, I)) * 0.2) if shared else None
    sg = rng.standard_normal(H) * 0.2 if shared else None
    return x, wr, Wg, Wu, Wd, sh, sg


def test_E1_k1_reduces_to_dense_swiglu():
    rng = np.random.default_rng(5)
    x, wr, Wg, Wu, Wd, _, _ = _rand_layer(rng, 9, 6, 1, 4, 1, shared=False)
    res = moe.moe_forward(x, wr, 1, lambda e: (Wg[e], Wu[e], Wd[e]), 1)
    assert np.allclose(res["w"], 1.0)
    assert np.allclose(res["out"], _torch_swiglu(x, Wg[0], Wu[0], Wd[0]), rtol=1e-12, atol=1e-14)


def test_swiglu_matches_torch_and_separates_gate_from_up():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((7, 5))
    wg, wu, wd = rng.standard_normal((3, 5)), rng.standard_normal((3, 5)), rng.standard_normal((5, 3))
    assert np.allclose(moe.swiglu(x, wg, wu, wd), _torch_swiglu(x, wg, wu, wd), rtol=1e-12, atol=1e-14)
    # swapping gate and up changes the answer (the non-linearity sits on gate only)
    assert not np.allclose(moe.swiglu(x, wu, wg, wd), _torch_swiglu(x, wg, wu, wd))


def test_identical_experts_give_expert_output_for_any_routing():
    rng = np.random.default_rng(7)
    x, wr, Wg, Wu, Wd, _, _ = _rand_layer(rng, 11, 8, 6, 5, 3, shared=False)
    res = moe.moe_forward(x, wr, 3, lambda e: (Wg[0], Wu[0], Wd[0]), 6)
    assert np.allclose(res["out"], _torch_swiglu(x, Wg[0], Wu[0], Wd[0]), rtol=1e-11, atol=1e-13)


def test_shared_expert_gate_and_zero_routed():
    rng = np.random.default_rng(8)
    x, wr, Wg, Wu, Wd, sh, sg = _rand_layer(rng, 10, 8, 5, 4, 2)
    zeros = np.zeros_like(Wd[0])
    res = moe.moe_forward(x, wr, 2, lambda e: (Wg[e], Wu[e], zeros), 5, sh, np.zeros(8))
    assert np.allclose(res["gamma"], 0.5)
    assert np.allclose(res["out"], 0.5 * _torch_swiglu(x, *sh), rtol=1e-12, atol=1e-14)
    res = moe.moe_forward(x, wr, 2, lambda e: (Wg[e], Wu[e], zeros), 5, sh, sg)
    gam = torch.sigmoid(torch.from_numpy(x @ sg)).numpy()
    assert np.allclose(res["out"], gam[:, None] * _torch_swiglu(x, *sh), rtol=1e-12, atol=1e-14)


def test_layer_against_torch_reference_composition():
    """Whole layer vs a torch float64 composition (topk, softmax, F.linear)."""
    rng = np.random.default_rng(9)
    T, H, E, I, k = 23, 12, 7, 5, 3
    x, wr, Wg, Wu, Wd, sh, sg = _rand_layer(rng, T, H, E, I, k)
    res = moe.moe_forward(x, wr, k, lambda e: (Wg[e], Wu[e], Wd[e]), E, sh, sg)
    X = torch.from_numpy(x)
    logits = F.linear(X, torch.from_numpy(wr)).to(torch.float32).to(torch.float64)  # fp32 softmax input
    p = torch.softmax(logits, 1)
    top_p, top_i = torch.topk(p, k, dim=1)
    top_p = top_p / top_p.sum(1, keepdim=True)
    out = torch.zeros(T, H, dtype=torch.float64)
    for t in range(T):
        for j in range(k):
            e = int(top_i[t, j])
            out[t] += top_p[t, j] * torch.from_numpy(_torch_swiglu(x[t:t + 1], Wg[e], Wu[e], Wd[e]))[0]
    out += torch.sigmoid(X @ torch.from_numpy(sg))[:, None] * torch.from_numpy(_torch_swiglu(x, *sh))
    assert res["ids"].tolist() == top_i.tolist()
    assert np.allclose(res["w"], top_p.numpy(), rtol=1e-13)
    assert np.allclose(res["out"], out.numpy(), rtol=1e-12, atol=1e-15)


def test_linearity_in_down_and_up():
    rng = np.random.default_rng(10)
    x, wr, Wg, Wu, Wd, _, _ = _rand_layer(rng, 8, 6, 4, 3, 2, shared=False)
    base = moe.moe_forward(x, wr, 2, lambda e: (Wg[e], Wu[e], Wd[e]), 4)["out"]
    r2 = moe.moe_forward(x, wr, 2, lambda e: (Wg[e], Wu[e], 3.0 * Wd[e]), 4)["out"]
    r3 = moe.moe_forward(x, wr, 2, lambda e: (Wg[e], -2.0 * Wu[e], Wd[e]), 4)["out"]
    assert np.allclose(r2, 3.0 * base, rtol=1e-12, atol=1e-15)
    assert np.allclose(r3, -2.0 * base, rtol=1e-12, atol=1e-15)


def test_token_independence_and_relabelling():
    rng = np.random.default_rng(11)
    x, wr, Wg, Wu, Wd, sh, sg = _rand_layer(rng, 12, 8, 6, 4, 2)
    f = lambda e: (Wg[e], Wu[e], Wd[e])
    full = moe.moe_forward(x, wr, 2, f, 6, sh, sg)["out"]
    for t in (0, 5, 11):
        one = moe.moe_forward(x[t:t + 1], wr, 2, f, 6, sh, sg)["out"]
        assert np.allclose(one[0], full[t], rtol=1e-13, atol=1e-15)
    perm = rng.permutation(6)
    inv = np.argsort(perm)
    g = lambda e: (Wg[perm[e]], Wu[perm[e]], Wd[perm[e]])
    rel = moe.moe_forward(x, wr[perm], 2, g, 6, sh, sg)
    assert np.allclose(rel["out"], full, rtol=1e-13, atol=1e-15)
    assert np.array_equal(perm[rel["ids"]], moe.moe_forward(x, wr, 2, f, 6, sh, sg)["ids"])
    del inv


def test_zero_gate_row_zeroes_hidden_column():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((4, 6))
    wg, wu, wd = rng.standard_normal((3, 6)), rng.standard_normal((3, 6)), rng.standard_normal((6, 3))
    wg[1] = 0.0
    wd_masked = wd.copy()
    wd_masked[:, 1] = 123.0  # whatever column 1 of W_down holds cannot matter
    assert np.allclose(moe.swiglu(x, wg, wu, wd), moe.swiglu(x, wg, wu, wd_masked), rtol=1e-14)


# ----------------------------------------------------------------------------
# Page-exact routing numerics (Flash-Next MoE section: fp32 softmax on logits
# rounded to the activation dtype, mixing weights cast to the activation dtype)
# ----------------------------------------------------------------------------
def test_round_bf16_matches_torch_and_ties_to_even():
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.normal(size=100000) * 10.0 ** rng.integers(-8, 8, size=100000),
                        rng.standard_cauchy(size=100000)]).astype(np.float32).astype(np.float64)
    ref = torch.tensor(v, dtype=torch.float32).to(torch.bfloat16).double().numpy()
    assert np.array_equal(moe.round_bf16(v), ref)
    # halfway cases go to the even neighbour: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert moe.round_bf16(1 + 2.0 ** -8) == 1.0
    assert moe.round_bf16(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6
    assert moe.round_bf16(-(1 + 2.0 ** -8)) == -1.0


def test_page_routing_ties_and_rounded_weights():
    # W_r = identity, so the logits are x itself (4 experts, k = 2)
    x = np.array([[1.0, 1.0 + 2.0 ** -10, 0.25, -1.0]])
    wr = np.eye(4)
    _, ids, w = moe.route(x, wr, 2)
    assert ids.tolist() == [[1, 0]]            # fp32 logits: 1 + 2^-10 ranks first
    l, ids_p, w_p = moe.route(x, wr, 2, page=True)
    assert l[0, 1] == 1.0                       # 1 + 2^-10 rounds to 1 in bf16: a tie
    assert ids_p.tolist() == [[0, 1]]           # the tie goes to the lower id
    assert w_p.tolist() == [[0.5, 0.5]]
    # rounded logits one apart: weights sigmoid(1) and 1 - sigmoid(1), each
    # rounded to bf16 (8 significant bits: steps 2^-8 in [0.5, 1), 2^-9 in [0.25, 0.5))
    x2 = np.array([[2.0, 1.0, -3.0]])
    _, ids2, w2 = moe.route(x2, np.eye(3), 2, page=True)
    assert ids2.tolist() == [[0, 1]]
    s = 1.0 / (1.0 + np.exp(-1.0))
    assert w2[0, 0] == np.round(s / 2.0 ** -8) * 2.0 ** -8 == 0.73046875
    assert w2[0, 1] == np.round((1 - s) / 2.0 ** -9) * 2.0 ** -9 == 0.26953125


def test_bf16_midpoint_distance():
    # logit 1 + 2^-8 + 1e-5 sits 1e-5 above the boundary between 1 and 1 + 2^-7
    l = np.array([[1.0 + 2.0 ** -8 + 1e-5, -2.0, -3.0]])
    d = moe.bf16_midpoint_distance(moe.to_fp32(l), 1)
    assert abs(d[0] - 1e-5) < 1e-7
    # a bf16 value itself: half a step to either side; below 1 the step is
    # 2^-8, so the nearest boundary is 1 - 2^-9
    d2 = moe.bf16_midpoint_distance(np.array([[1.0, -2.0, -3.0]]), 1)
    assert d2[0] == 2.0 ** -9
