"""Seeded synthetic inputs for the routed Mixture-of-Experts FFN layer.

Test and benchmark infrastructure.  Both the fp64 oracle's tests and the HIP
path's tests and benchmark take their inputs from here.  This module holds no
step of the layer's arithmetic (no logits, no selection, no expert math): it
only draws tensors and rounds them to their storage type.

Workload shapes follow the pages:
  * Qwen3.8-Flash-Next study, "The model at a glance" and "MoE: 512 experts
    behind a width-640 intermediate": hidden 2560, 512 routed experts,
    10 chosen per token, intermediate width 640, one gated shared expert.
  * Model-atlas page "Qwen3.8 2.4T A95B", raw config fields: hidden_size 8192,
    num_experts 512, num_experts_per_tok 10, moe_intermediate_size 2048,
    shared_expert_intermediate_size 2048, hidden_act silu.
  * "Qwen3.8, weights in hand", section "What FP8 actually quantizes": only
    the routed experts are FP8; router, shared expert and its gate stay bf16.
  * Hub discussion on singular matrices in Qwen3.8-2.4T-A95B, zero-fraction
    table: 71.0% of blk.0 gate/up expert entries are zero.

Random numbers
--------------
Every tensor is drawn from a counter-based generator: element n of a stream
with 64-bit key K gets the 32-bit hash  h = mix(mix(n ^ K_lo) ^ K_hi), with
mix = the "lowbias32" integer hash (xorshift-multiply, constants 0x7feb352d
and 0x846ca68b).  The top 16 bits of h pick a cell of a 65537-entry table of
standard-normal quantiles, the low 16 bits interpolate linearly inside it.
Keys come from splitmix64 over (seed, tensor id, row/expert index, attempt),
so any token row or any expert can be (re)drawn on its own, on any torch
device, with identical bits (integer ops, then IEEE fp32 mul/add done as
separate, correctly rounded operations).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np
import torch
from scipy.special import ndtri

M32 = 0xFFFFFFFF
M64 = 0xFFFFFFFFFFFFFFFF

# Stream tensor ids.
T_X, T_ROUTER, T_SHGATE_W, T_SH_G, T_SH_U, T_SH_D = 1, 2, 3, 4, 5, 6
T_EG, T_EU, T_ED, T_MASK_G, T_MASK_U, T_ZIPF = 7, 8, 9, 10, 11, 12


# ----------------------------------------------------------------------------
# Configurations (names say what they are; sizes as in the pages)
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    I_shared: int = 0          # 0: no shared expert
    act: str = "bf16"          # "f32" | "bf16"
    wdt: str = "bf16"          # "f32" | "bf16" | "fp8"
    x_std: float = 1.0
    w_std: float = 0.02
    router_std: Optional[float] = None  # None: 1/sqrt(H) (logit std ~1)
    zipf_s: float = 0.0        # >0: per-expert router bias -s*ln(rank)
    zero_frac: float = 0.0     # fraction of gate/up entries forced to 0 (fp8)
    scale_block: int = 128     # fp8 block edge

    @property
    def R(self) -> int:
        return self.T * self.k

    @property
    def rstd(self) -> float:
        return self.router_std if self.router_std is not None else 1.0 / math.sqrt(self.H)

    def with_(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[str, MoEConfig] = {
    # toy fp32 layer, small enough for brute force checks
    "toy_fp32": MoEConfig("toy_fp32", T=128, H=256, E=16, k=4, I=128, I_shared=0,
                          act="f32", wdt="f32", router_std=0.05),
    # Flash-Next shape prefill chunk: T=4096 tokens, near-uniform load
    "flash_prefill": MoEConfig("flash_prefill", T=4096, H=2560, E=512, k=10, I=640,
                               I_shared=640),
    # Flash-Next shape decode step: 16 tokens, weight streaming
    "flash_decode": MoEConfig("flash_decode", T=16, H=2560, E=512, k=10, I=640,
                              I_shared=640),
    # 2.4T shape prefill, Zipf-skewed load
    "max_prefill": MoEConfig("max_prefill", T=8192, H=8192, E=512, k=10, I=2048,
                             I_shared=2048, zipf_s=1.1),
    # 2.4T shape, fp8 e4m3fn routed experts with 128x128 block scales
    "max_fp8": MoEConfig("max_fp8", T=2048, H=8192, E=512, k=10, I=2048, I_shared=0,
                         wdt="fp8", zipf_s=1.1, zero_frac=0.71),
}
CONFIG_ORDER = ["toy_fp32", "flash_prefill", "flash_decode", "max_prefill", "max_fp8"]


# ----------------------------------------------------------------------------
# Counter-based generator
# ----------------------------------------------------------------------------
def _splitmix64(z: int) -> int:
    z = (z + 0x9E3779B97F4A7C15) & M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def stream_key(seed: int, tensor: int, index: int = 0, attempt: int = 0) -> int:
    z = _splitmix64(seed & M64)
    for v in (tensor, index, attempt):
        z = _splitmix64(z ^ ((v * 0xD1B54A32D192ED03) & M64))
    return z


def _mul32(a: torch.Tensor, c: int) -> torch.Tensor:
    """(a * c) mod 2^32 for int64 tensors holding values < 2^32, overflow-free."""
    lo = a * (c & 0xFFFF)
    hi = ((a * (c >> 16)) & 0xFFFF) << 16
    return (lo + hi) & M32


def _mix32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    return x ^ (x >> 16)


_TABLES: Dict[str, torch.Tensor] = {}


def _normal_table(device) -> torch.Tensor:
    key = str(device)
    if key not in _TABLES:
        q = (np.arange(65537, dtype=np.float64) + 0.5) / 65538.0
        _TABLES[key] = torch.from_numpy(ndtri(q).astype(np.float32)).to(device)
    return _TABLES[key]


def hash_stream(keys: torch.Tensor, n: int, device) -> torch.Tensor:
    """32-bit hashes (int64 tensor) of shape [len(keys), n]; keys: int64 [rows] of 64-bit keys
    stored as (lo, hi) pairs -> pass a [rows, 2] tensor."""
    ctr = torch.arange(n, dtype=torch.int64, device=device).unsqueeze(0)
    klo = keys[:, 0:1]
    khi = keys[:, 1:2]
    h = _mix32(ctr ^ klo)
    return _mix32(h ^ khi)


def _keys_tensor(keys, device) -> torch.Tensor:
    arr = [[k & M32, (k >> 32) & M32] for k in keys]
    return torch.tensor(arr, dtype=torch.int64, device=device).reshape(-1, 2)


def normals(keys, n: int, device) -> torch.Tensor:
    """Standard-normal fp32 draws, shape [len(keys), n], one stream per key."""
    h = hash_stream(_keys_tensor(keys, device), n, device)
    tab = _normal_table(device)
    i = h >> 16
    f = (h & 0xFFFF).to(torch.float32) * (1.0 / 65536.0)
    t0 = tab[i]
    t1 = tab[i + 1]
    d = t1 - t0
    return t0 + d * f


def uniforms_u32(keys, n: int, device) -> torch.Tensor:
    """Raw 32-bit hashes as int64, shape [len(keys), n]."""
    return hash_stream(_keys_tensor(keys, device), n, device)


# ----------------------------------------------------------------------------
# Storage rounding
# ----------------------------------------------------------------------------
def to_storage(t32: torch.Tensor, dt: str) -> torch.Tensor:
    if dt == "f32":
        return t32.contiguous()
    if dt == "bf16":
        return t32.to(torch.bfloat16)  # round to nearest even
    raise ValueError(dt)


def quantize_e4m3fn_blocks(w32: torch.Tensor, block: int):
    """Quantise one [N, K] fp32 matrix to OCP e4m3fn codes with one fp32 scale per
    block x block tile: s = amax(tile)/448 (an all-zero tile gets s = 1), code =
    round-to-nearest-even(w / s).  Returns (codes uint8 [N,K], scales fp32 [N/b, K/b])."""
    N, K = w32.shape
    assert N % block == 0 and K % block == 0
    tiles = w32.reshape(N // block, block, K // block, block)
    amax = tiles.abs().amax(dim=(1, 3))
    s = amax / 448.0
    s = torch.where(amax > 0, s, torch.ones_like(s))
    q = (tiles / s[:, None, :, None]).reshape(N, K)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), s.to(torch.float32).contiguous()


# ----------------------------------------------------------------------------
# Problem tensors
# ----------------------------------------------------------------------------
class Problem:
    """All input tensors of one layer invocation, on one torch device.

    x           [T, H]      act
    w_router    [E, H]      act   (bf16 when act is bf16, also in the fp8 layout)
    sh_gate_w   [1, H]      act   or None
    sh_gate/up  [I_s, H]    act   or None;  sh_down [H, I_s]
    w_gate/up   [E, I, H]   act or uint8 e4m3fn codes;  w_down [E, H, I]
    s_gate/up   [E, I/b, H/b] fp32 (fp8 only);  s_down [E, H/b, I/b]
    """

    def __init__(self, cfg: MoEConfig, seed: int, device="cpu", x_attempts=None,
                 materialize_experts: bool = True):
        self.cfg = cfg
        self.seed = seed
        self.device = torch.device(device)
        self.x_attempts = dict(x_attempts or {})
        c = cfg
        if c.wdt == "fp8":
            assert c.H % c.scale_block == 0 and c.I % c.scale_block == 0
        self.x = self._draw_x()
        self.w_router = self._draw_router()
        if c.I_shared > 0:
            self.sh_gate_w = to_storage(
                normals([stream_key(seed, T_SHGATE_W)], c.H, self.device) * c.w_std, c.act)
            self.sh_gate = self._dense(T_SH_G, c.I_shared, c.H)
            self.sh_up = self._dense(T_SH_U, c.I_shared, c.H)
            self.sh_down = self._dense(T_SH_D, c.H, c.I_shared)
        else:
            self.sh_gate_w = self.sh_gate = self.sh_up = self.sh_down = None
        self.w_gate = self.w_up = self.w_down = None
        self.s_gate = self.s_up = self.s_down = None
        if materialize_experts:
            self._draw_experts()

    # -- activations ---------------------------------------------------------
    def x_row_keys(self, rows):
        return [stream_key(self.seed, T_X, t, self.x_attempts.get(t, 0)) for t in rows]

    def _draw_x(self) -> torch.Tensor:
        c = self.cfg
        x32 = normals(self.x_row_keys(range(c.T)), c.H, self.device) * c.x_std
        if c.zipf_s > 0:
            x32[:, c.H - 1] = 1.0
        return to_storage(x32, c.act)

    def redraw_tokens(self, rows, attempts):
        """Redraw the given token rows with the given attempt numbers (margin fix-up)."""
        c = self.cfg
        rows = list(rows)
        for t, a in zip(rows, attempts):
            self.x_attempts[t] = a
        x32 = normals(self.x_row_keys(rows), c.H, self.device) * c.x_std
        if c.zipf_s > 0:
            x32[:, c.H - 1] = 1.0
        idx = torch.tensor(rows, dtype=torch.int64, device=self.device)
        self.x[idx] = to_storage(x32, c.act)

    # -- router --------------------------------------------------------------
    def zipf_ranks(self) -> np.ndarray:
        rng = np.random.Generator(np.random.PCG64(stream_key(self.seed, T_ZIPF)))
        return rng.permutation(self.cfg.E) + 1

    def _draw_router(self) -> torch.Tensor:
        c = self.cfg
        keys = [stream_key(self.seed, T_ROUTER, e) for e in range(c.E)]
        w32 = normals(keys, c.H, self.device) * c.rstd
        if c.zipf_s > 0:
            bias = (-c.zipf_s * np.log(self.zipf_ranks().astype(np.float64))).astype(np.float32)
            w32[:, c.H - 1] = torch.from_numpy(bias).to(self.device)
        return to_storage(w32, c.act)

    # -- weights -------------------------------------------------------------
    def _dense(self, tensor_id, n_rows, n_cols, index=0):
        w32 = normals([stream_key(self.seed, tensor_id, index)], n_rows * n_cols,
                      self.device).reshape(n_rows, n_cols) * self.cfg.w_std
        return to_storage(w32, self.cfg.act)

    def expert_fp32(self, e: int, which: str) -> torch.Tensor:
        """Unrounded fp32 draw of one expert matrix (gate/up masked when zero_frac>0)."""
        c = self.cfg
        tid, n_rows, n_cols, mid = {
            "gate": (T_EG, c.I, c.H, T_MASK_G),
            "up": (T_EU, c.I, c.H, T_MASK_U),
            "down": (T_ED, c.H, c.I, None),
        }[which]
        w32 = normals([stream_key(self.seed, tid, e)], n_rows * n_cols,
                      self.device).reshape(n_rows, n_cols) * c.w_std
        if c.zero_frac > 0 and mid is not None:
            h = uniforms_u32([stream_key(self.seed, mid, e)], n_rows * n_cols,
                             self.device).reshape(n_rows, n_cols)
            thresh = int(round(c.zero_frac * 2 ** 32))
            w32 = torch.where(h < thresh, torch.zeros_like(w32), w32)
        return w32

    def expert_storage(self, e: int, which: str):
        """(stored matrix, scales or None) of one expert matrix."""
        w32 = self.expert_fp32(e, which)
        if self.cfg.wdt == "fp8":
            return quantize_e4m3fn_blocks(w32, self.cfg.scale_block)
        return to_storage(w32, self.cfg.wdt), None

    def _draw_experts(self):
        c = self.cfg
        dev = self.device
        if c.wdt == "fp8":
            wdtype = torch.uint8
        else:
            wdtype = torch.bfloat16 if c.wdt == "bf16" else torch.float32
        self.w_gate = torch.empty((c.E, c.I, c.H), dtype=wdtype, device=dev)
        self.w_up = torch.empty((c.E, c.I, c.H), dtype=wdtype, device=dev)
        self.w_down = torch.empty((c.E, c.H, c.I), dtype=wdtype, device=dev)
        if c.wdt == "fp8":
            b = c.scale_block
            self.s_gate = torch.empty((c.E, c.I // b, c.H // b), dtype=torch.float32, device=dev)
            self.s_up = torch.empty((c.E, c.I // b, c.H // b), dtype=torch.float32, device=dev)
            self.s_down = torch.empty((c.E, c.H // b, c.I // b), dtype=torch.float32, device=dev)
        for e in range(c.E):
            for which, dst, sdst in (("gate", self.w_gate, self.s_gate),
                                     ("up", self.w_up, self.s_up),
                                     ("down", self.w_down, self.s_down)):
                w, s = self.expert_storage(e, which)
                dst[e].copy_(w)
                if s is not None:
                    sdst[e].copy_(s)

    # -- raw host views (what the oracle consumes) ---------------------------
    def host_raw(self, t: Optional[torch.Tensor]):
        """Host numpy view of a stored tensor's raw representation:
        fp32 -> float32, bf16 -> uint16 bit patterns, fp8 codes -> uint8."""
        if t is None:
            return None
        t = t.detach().to("cpu")
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        if t.dtype in (torch.float32, torch.uint8, torch.int32):
            return t.numpy()
        raise TypeError(t.dtype)


def make_problem(cfg, seed: int = 0, device="cpu", **kw) -> Problem:
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    return Problem(cfg, seed, device, **kw)


# ----------------------------------------------------------------------------
# Gated residual around a sublayer (Qwen3.8-Flash-Next study, "Gated residual:
# four streams, one sublayer input"): four residual streams of width H, a
# per-stream RMSNorm gain, a rank-r read-gate bottleneck and four write gates.
# ----------------------------------------------------------------------------
T_GR_R, T_GR_NW, T_GR_RD, T_GR_UP, T_GR_F, T_GR_S = 13, 14, 15, 16, 17, 18


class GRProblem:
    """resid  [T, 4, H] act   the four residual streams
    norm_w [4, H]     act   RMSNorm gain of each stream (1 + 0.1 N(0,1))
    w_read [r+4, 4H]  act   rows 0..r-1: the read bottleneck's down projection,
                            rows r..r+3: the four write-gate projections
    w_up   [4H, r]    act   the read bottleneck's up projection
    f      [T, H]     act   a sublayer output to write back
    s      [T, 4]     fp32  write gates for the write step alone (1 + 0.25 N(0,1))
    Weights ~ N(0, 0.02), streams and f ~ N(0, 1); eps is the model config's
    rms_norm_eps (1e-6, model-atlas page, raw config)."""

    def __init__(self, T: int, H: int, rank: int = 320, seed: int = 0, device="cpu", act: str = "bf16"):
        self.T, self.H, self.rank, self.seed, self.act = T, H, rank, seed, act
        self.eps = 1e-6
        self.device = torch.device(device)
        dev = self.device
        self.resid = to_storage(normals([stream_key(seed, T_GR_R, t) for t in range(T)], 4 * H, dev), act).reshape(T, 4, H)
        self.norm_w = to_storage(1.0 + 0.1 * normals([stream_key(seed, T_GR_NW)], 4 * H, dev).reshape(4, H), act)
        self.w_read = to_storage(normals([stream_key(seed, T_GR_RD)], (rank + 4) * 4 * H, dev).reshape(rank + 4, 4 * H)
                                 * 0.02, act)
        self.w_up = to_storage(normals([stream_key(seed, T_GR_UP)], 4 * H * rank, dev).reshape(4 * H, rank) * 0.02, act)
        self.f = to_storage(normals([stream_key(seed, T_GR_F, t) for t in range(T)], H, dev), act)
        self.s = 1.0 + 0.25 * normals([stream_key(seed, T_GR_S, t) for t in range(T)], 4, dev)

    def host(self, t: torch.Tensor) -> np.ndarray:
        """Host fp64 copy of a stored tensor (exact: bf16 and fp32 convert exactly)."""
        return t.detach().to("cpu").to(torch.float64).numpy()


def make_gr_problem(T: int, H: int, rank: int = 320, seed: int = 0, device="cpu", act: str = "bf16") -> GRProblem:
    return GRProblem(T, H, rank, seed, device, act)


T_AUD_W, T_AUD_M = 19, 20


def make_audit_tensor(S: int, N: int, seed: int = 0, zero_frac: float = 0.0, std: float = 0.02,
                      device="cpu") -> torch.Tensor:
    """bf16 [S, N] weight-like tensor for the expert-weight audit: slice s is
    drawn from its own stream, N(0, std), with entries set to exactly zero
    with probability zero_frac (the discussion's table has 71.0% and 84.3%
    zeros in early gate/up expert tensors)."""
    out = torch.empty((S, N), dtype=torch.bfloat16, device=device)
    thresh = int(round(zero_frac * 2 ** 32))
    for s in range(S):
        w32 = normals([stream_key(seed, T_AUD_W, s)], N, device).reshape(N) * std
        if zero_frac > 0:
            h = uniforms_u32([stream_key(seed, T_AUD_M, s)], N, device).reshape(N)
            w32 = torch.where(h < thresh, torch.zeros_like(w32), w32)
        out[s] = w32.to(torch.bfloat16)
    return out
