"""Seeded input generator: determinism, distributions, structure, margin fix-up."""
import math

import numpy as np
import pytest
import torch

from oracle import adapter, moe
from synthetic import CONFIGS, make_problem
from synthetic import gen


def _small(name, **kw):
    return CONFIGS[name].with_(**kw)


def test_seed_determinism_and_seed_sensitivity():
    c = _small("flash_prefill", T=16, H=128, E=8, I=64, I_shared=64)
    a = make_problem(c, 3)
    b = make_problem(c, 3)
    d = make_problem(c, 4)
    for name in ("x", "w_router", "w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down", "sh_gate_w"):
        assert torch.equal(getattr(a, name).view(torch.int16), getattr(b, name).view(torch.int16)), name
        assert not torch.equal(getattr(a, name).view(torch.int16), getattr(d, name).view(torch.int16)), name


def test_normal_draw_moments():
    z = gen.normals([gen.stream_key(0, 99, i) for i in range(4)], 1 << 18, "cpu").double()
    assert abs(z.mean().item()) < 3e-3
    assert abs(z.std().item() - 1.0) < 3e-3
    # fourth moment of a normal is 3
    assert abs(((z - z.mean()) ** 4).mean().item() / z.var().item() ** 2 - 3.0) < 0.05
    assert z.abs().max().item() < 5.0


def test_rows_are_independent_streams():
    c = _small("flash_prefill", T=8, H=64, E=4, I=32, I_shared=0)
    p = make_problem(c, 1)
    x0 = p.x.clone()
    p.redraw_tokens([3], [0])  # attempt 0 reproduces the original row
    assert torch.equal(p.x.view(torch.int16), x0.view(torch.int16))
    p.redraw_tokens([3], [1])
    changed = (p.x.view(torch.int16) != x0.view(torch.int16)).any(dim=1)
    assert changed.tolist() == [False, False, False, True, False, False, False, False]


def test_bf16_storage_is_round_to_nearest_even():
    v = torch.tensor([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)], dtype=torch.float32)
    got = gen.to_storage(v, "bf16").to(torch.float64).tolist()
    assert got == [1.0, 1.0 + 2 ** -6, -1.0]  # ties go to the even mantissa


def test_fp8_blocks_zero_mask_and_roundtrip():
    c = _small("max_fp8", T=8, H=256, E=3, I=256)
    p = make_problem(c, 2)
    # 71% of gate/up entries are exact zeros, down has no mask
    zf = (p.w_gate == 0).double().mean().item()
    assert abs(zf - 0.71) < 0.01
    assert (p.w_down == 0).double().mean().item() < 0.01
    for e in range(c.E):
        w32 = p.expert_fp32(e, "gate").double().numpy()
        deq = moe.dequant_blocks(p.host_raw(p.w_gate[e]), p.host_raw(p.s_gate[e]), 128)
        assert np.array_equal(deq == 0, w32 == 0)  # zeros stay exactly zero, nothing else flushes
        # e4m3 keeps 3 mantissa bits: relative error <= 2^-4 for normal codes
        s_full = np.kron(p.host_raw(p.s_gate[e]), np.ones((128, 128)))
        normal = np.abs(w32) >= s_full * 2 ** -6
        rel = np.abs(deq - w32)[normal] / np.abs(w32)[normal]
        assert rel.max() <= 2 ** -4 + 1e-7
        # block amax maps to code 448 exactly
        amax = np.abs(w32).reshape(2, 128, 2, 128).max(axis=(1, 3))
        assert np.allclose(np.abs(deq).reshape(2, 128, 2, 128).max(axis=(1, 3)), amax, rtol=2 ** -4)


def test_zipf_bias_channel():
    c = _small("max_prefill", T=32, H=128, E=16, I=64, I_shared=64)
    p = make_problem(c, 0)
    ranks = p.zipf_ranks()
    assert sorted(ranks.tolist()) == list(range(1, 17))
    assert torch.all(p.x[:, -1] == 1.0)
    b = p.w_router[:, -1].double().numpy()
    expect = torch.tensor(-1.1 * np.log(ranks), dtype=torch.float32).to(torch.bfloat16).double().numpy()
    assert np.array_equal(b, expect)


def test_router_logit_scale():
    c = _small("flash_prefill", T=256, H=2560, E=64, I=64, I_shared=0)
    p = make_problem(c, 0, materialize_experts=False)
    x, wr, _, _ = adapter.dense_inputs(p)
    l = moe.router_logits(x, wr)
    assert 0.9 < l.std() < 1.1  # "router logits std ~ 1"


@pytest.mark.parametrize("name", ["toy_fp32", "flash_decode"])
def test_margin_fixup(name):
    c = CONFIGS[name]
    if name == "flash_decode":
        c = c.with_(T=64)
    p = make_problem(c, 0, materialize_experts=False)
    n = adapter.ensure_margin(p, 1e-3)
    x, wr, _, _ = adapter.dense_inputs(p)
    l32 = moe.to_fp32(moe.router_logits(x, wr))
    assert moe.margins(l32, c.k, adjacent=True).min() >= 1e-3
    assert n >= 0
