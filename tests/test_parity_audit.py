"""GPU parity of the expert-weight audit (moe_weight_audit) against the fp64
oracle (oracle/audit.py): model-hub discussion "singular matrices in
Qwen3.8-2.4T-A95B", zero share and sigma_rob = 1.4826 * MAD.

The statistics are exact on both sides (bf16 values convert exactly to
fp64; the median, the distances |w - median| and the mean of two middle
values are the same fp64 operations), so every field must be equal: counts
bit-exact, median / mad / sigma_rob equal as fp64 (NaN where both are NaN;
the sign of a zero median is not compared)."""
import math

import numpy as np
import pytest
import torch

import sparse_moe_layer_amd as lib
from oracle import audit as oa
from synthetic import make_audit_tensor

pytestmark = pytest.mark.gpu


def run_audit(w2d: torch.Tensor, slices: int, n: int, stride: int, base=None):
    """Audit `slices` slices of n values, stride apart, starting at base (a
    flat bf16 tensor) or at w2d."""
    flat = base if base is not None else w2d.reshape(-1)
    stats = lib.audit_stats_buffer(slices)
    ws = lib.audit_workspace(slices)
    lib.moe_weight_audit(flat, slices, n, stride, stats, ws)
    torch.cuda.synchronize()
    return lib.audit_records(stats)


def same(a, b):
    return (math.isnan(a) and math.isnan(b)) or a == b


def check_record(got, ref, where):
    for f in ("n", "n_zero", "n_nan"):
        assert got[f] == ref[f], (where, f, got[f], ref[f])
    for f in ("median", "mad", "sigma_rob"):
        assert same(got[f], ref[f]), (where, f, got[f], ref[f])


def host_slices(flat: torch.Tensor, slices, n, stride):
    h = flat.float().cpu().double().numpy()
    return [h[s * stride: s * stride + n] for s in range(slices)]


@pytest.mark.parametrize("slices,n,zero_frac", [(3, 1000, 0.0), (5, 4099, 0.71), (1, 1, 0.0), (2, 7, 0.5),
                                                (16, 65536 * 3 + 5, 0.0)])
def test_audit_matches_oracle(slices, n, zero_frac):
    print(f"[audit] slices={slices} n={n} zero_frac={zero_frac}", flush=True)
    w = make_audit_tensor(slices, n, seed=1, zero_frac=zero_frac, device="cuda")
    recs = run_audit(w, slices, n, n)
    hs = host_slices(w.reshape(-1), slices, n, n)
    for s in range(slices):
        check_record(recs[s], oa.audit_values(hs[s]), f"slice {s}")
    check_record(recs[slices], oa.audit_values(np.concatenate(hs)), "whole")


def test_audit_special_values_and_layout():
    # NaN, +-inf, |w| >= 2 and normal |w| < 2^-63 (outside the LDS histogram,
    # with 2^-63 itself the least value inside it), subnormals, -0, an
    # unaligned first slice and gaps between slices (stride > n)
    slices, n, stride = 4, 3001, 3011
    print(f"[audit] special values slices={slices} n={n} stride={stride}", flush=True)
    flat = (torch.randn(1 + slices * stride, device="cuda") * 0.5).to(torch.bfloat16)
    base = flat[1:]  # 2-byte offset: the first slice starts off 16-byte alignment
    base[0 * stride + 10] = float("nan")
    base[1 * stride + 3] = float("inf")
    base[1 * stride + 4] = float("-inf")
    base[2 * stride: 2 * stride + 500] = torch.linspace(-300, 300, 500, device="cuda").to(torch.bfloat16)
    base[3 * stride: 3 * stride + 40] = torch.tensor([1e-39, -2e-39] * 20, device="cuda").to(torch.bfloat16)
    base[3 * stride + 40: 3 * stride + 1700] = -0.0
    tiny = [2.0 ** -63, -(2.0 ** -63), 2.0 ** -64, -(2.0 ** -64), 1e-25, -3e-30, 2.0 ** -126]
    base[3 * stride + 1700: 3 * stride + 1700 + 7 * 30] = torch.tensor(tiny * 30, device="cuda").to(torch.bfloat16)
    recs = run_audit(None, slices, n, stride, base=base)
    hs = host_slices(base, slices, n, stride)
    assert recs[0]["n_nan"] == 1 and math.isnan(recs[0]["sigma_rob"])
    for s in range(slices):
        check_record(recs[s], oa.audit_values(hs[s]), f"slice {s}")
    check_record(recs[slices], oa.audit_values(np.concatenate(hs)), "whole")
    # whole tensor without the NaN slice
    recs = run_audit(None, 3, n, stride, base=base[stride:])
    check_record(recs[3], oa.audit_values(np.concatenate(hs[1:])), "whole without NaN")


def test_audit_infinite_median_and_empty():
    t = torch.tensor([float("inf"), float("inf"), 1.0, float("-inf"), float("inf"), 2.0], device="cuda")
    t = t.to(torch.bfloat16)
    recs = run_audit(None, 2, 3, 3, base=t)  # slice 0: inf, inf, 1 -> median inf, MAD NaN
    hs = host_slices(t, 2, 3, 3)
    for s in range(2):
        check_record(recs[s], oa.audit_values(hs[s]), f"slice {s}")
    recs = run_audit(None, 3, 0, 0, base=t)  # empty slices
    for r in recs:
        assert r["n"] == 0 and math.isnan(r["median"]) and math.isnan(r["sigma_rob"])


def test_audit_repeat_call_reuses_workspace():
    # the workspace's histograms are cleared by the call itself
    w = make_audit_tensor(4, 5000, seed=2, zero_frac=0.3, device="cuda")
    stats = lib.audit_stats_buffer(4)
    ws = lib.audit_workspace(4)
    lib.moe_weight_audit(w.reshape(-1), 4, 5000, 5000, stats, ws)
    first = lib.audit_records(stats)
    lib.moe_weight_audit(w.reshape(-1), 4, 5000, 5000, stats, ws)
    assert lib.audit_records(stats) == first


def test_audit_full_size_2p4t_gate_sampled():
    # the 2.4T gate tensor's shape [512 experts, 2048, 8192] with the
    # discussion's 71% zeros: every slice's counts against properties, four
    # sampled experts against the oracle, the whole tensor's counts as sums
    E, N = 512, 2048 * 8192
    print(f"[audit] full size E={E} N={N}", flush=True)
    w = make_audit_tensor(E, N, seed=7, zero_frac=0.71, device="cuda")
    recs = run_audit(w, E, N, N)
    assert all(r["n"] == N and r["n_nan"] == 0 for r in recs[:E])
    whole = recs[E]
    assert whole["n"] == E * N and whole["n_zero"] == sum(r["n_zero"] for r in recs[:E])
    assert abs(whole["n_zero"] / whole["n"] - 0.71) < 1e-3
    # more than half zeros: median 0 and sigma_rob 0, the discussion's case
    assert whole["median"] == 0.0 and whole["sigma_rob"] == 0.0
    for e in (0, 137, 300, 511):
        ref = oa.audit_values(w[e].float().cpu().double().numpy())
        check_record(recs[e], ref, f"expert {e}")
    del w
    torch.cuda.empty_cache()


def test_audit_full_size_flash_gate_sampled():
    # the Flash-Next gate tensor's shape [512, 640, 2560], no zero mask:
    # sampled experts against the oracle
    E, N = 512, 640 * 2560
    w = make_audit_tensor(E, N, seed=8, device="cuda")
    recs = run_audit(w, E, N, N)
    for e in (0, 255, 511):
        check_record(recs[e], oa.audit_values(w[e].float().cpu().double().numpy()), f"expert {e}")
    assert recs[E]["n"] == E * N
    assert abs(recs[E]["sigma_rob"] / 0.02 - 1) < 0.01  # N(0, 0.02) draws
