"""Pins of the gated-residual oracle (Qwen3.8-Flash-Next study, "Gated
residual: four streams, one sublayer input") against closed forms, invariants
and an independent torch composition."""
import numpy as np
import torch

from oracle import gr


def _rand(T=3, H=16, rank=5, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.normal(size=(T, 4, H)), 1 + 0.1 * rng.normal(size=(4, H)),
            0.3 * rng.normal(size=(rank + 4, 4 * H)), 0.3 * rng.normal(size=(4 * H, rank)))


def test_group_rmsnorm_hand_example():
    # stream [3, 4]: rms = sqrt((9 + 16) / 2) = sqrt(12.5); stream [1, -1]: rms 1
    r = np.zeros((1, 4, 2))
    r[0, 1] = [3.0, 4.0]
    r[0, 0] = r[0, 2] = r[0, 3] = [1.0, -1.0]
    out = gr.group_rmsnorm(r, np.ones((4, 2)), 0.0)
    assert np.allclose(out[0, 1], [3 / np.sqrt(12.5), 4 / np.sqrt(12.5)], rtol=0, atol=1e-15)
    assert np.array_equal(out[0, 0], [1.0, -1.0])
    # a zero stream stays zero (eps keeps the division finite)
    rz = r.copy()
    rz[0, 0] = 0.0
    assert np.all(gr.group_rmsnorm(rz, np.ones((4, 2)), 1e-6)[0, 0] == 0.0)
    # the gain multiplies per channel
    g = np.array([[1, 1], [2, -1], [1, 1], [1, 1]], dtype=float)
    assert np.allclose(gr.group_rmsnorm(r, g, 0.0)[0, 1], [6 / np.sqrt(12.5), -4 / np.sqrt(12.5)])


def test_rmsnorm_is_scale_invariant_per_stream():
    r, g, _, _ = _rand()
    scale = np.array([1.0, 3.0, 0.5, 10.0])[None, :, None]
    assert np.allclose(gr.group_rmsnorm(r * scale, g, 0.0), gr.group_rmsnorm(r, g, 0.0), rtol=1e-12, atol=1e-12)


def test_zero_bottleneck_closed_form():
    # W_down = W_write = 0 and W_up = 0: G = sigmoid(0) = 1/2, s = 2 sigmoid(0) = 1
    r, g, wr, wu = _rand()
    x, s, rhat, G = gr.gr_read(r, g, np.zeros_like(wr), np.zeros_like(wu), 1e-6)
    assert np.all(G == 0.5) and np.all(s == 1.0)
    assert np.allclose(x, rhat.sum(axis=1) / 8.0, rtol=0, atol=1e-15)
    f = np.random.default_rng(1).normal(size=(r.shape[0], r.shape[2]))
    assert np.allclose(gr.gr_write(r, s, f), r + f[:, None, :])


def test_stream_permutation_equivariance():
    # relabelling the streams (with their gains, w_read column blocks, w_up row
    # blocks and write-gate rows) leaves x unchanged and permutes s
    r, g, wr, wu = _rand(seed=3)
    T, S, H = r.shape
    rank = wr.shape[0] - S
    perm = np.array([2, 0, 3, 1])
    cols = np.concatenate([np.arange(H) + H * i for i in perm])
    wr_p = wr[:, cols].copy()
    wr_p[rank:] = wr_p[rank:][perm]
    x, s, _, _ = gr.gr_read(r, g, wr, wu, 1e-6)
    xp, sp, _, _ = gr.gr_read(r[:, perm], g[perm], wr_p, wu[cols], 1e-6)
    assert np.allclose(xp, x, rtol=1e-12, atol=1e-12)
    assert np.allclose(sp, s[:, perm], rtol=1e-12, atol=1e-12)


def test_write_special_cases():
    r, _, _, _ = _rand(seed=4)
    f = np.random.default_rng(5).normal(size=(r.shape[0], r.shape[2]))
    assert np.array_equal(gr.gr_write(r, np.zeros((r.shape[0], 4)), f), r)
    assert np.array_equal(gr.gr_write(r, np.ones((r.shape[0], 4)), np.zeros_like(f)), r)
    s = np.random.default_rng(6).uniform(0, 2, size=(r.shape[0], 4))
    assert np.allclose(gr.gr_write(r, s, 2 * f) - r, 2 * (gr.gr_write(r, s, f) - r))


def test_against_torch_composition():
    r, g, wr, wu = _rand(T=5, H=32, rank=7, seed=7)
    x, s, _, G = gr.gr_read(r, g, wr, wu, 1e-6)
    R = torch.tensor(r)
    rhat = torch.nn.functional.rms_norm(R, (32,), eps=1e-6) * torch.tensor(g)
    v = rhat.reshape(5, 128) / 4
    proj = torch.nn.functional.linear(v, torch.tensor(wr))
    Gt = torch.sigmoid(torch.nn.functional.linear(torch.nn.functional.silu(proj[:, :7]), torch.tensor(wu)))
    xt = (Gt.reshape(5, 4, 32) * rhat).mean(dim=1)
    st = 2 * torch.sigmoid(proj[:, 7:])
    assert np.allclose(x, xt.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(s, st.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(G, Gt.reshape(5, 4, 32).numpy(), rtol=1e-12, atol=1e-12)
