"""Algorithmic work of the routed MoE layer: FLOPs and HBM bytes that the
method must spend (no padding, no re-reads, no intermediates beyond the
stage boundaries).  Used to turn measured times into TFLOP/s, GB/s and
roofline fractions.

Weight counts follow the Qwen3.8-Flash-Next study's MoE section ("routed
bank = 48 x 512 x 3 x 2560 x 640"; ten experts per token select 2.359B
weights across layers) and the byte accounting of "Qwen3.8, weights in
hand", section "What FP8 actually quantizes" (routed parameters at one byte
in FP8, everything else at two).
"""
from __future__ import annotations

import dataclasses

# MI355X published peaks (dense): bf16 MFMA 2.5 PFLOP/s, fp8 5.0, HBM3E 8 TB/s
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBPS = 8000.0

WBYTES = {"f32": 4, "bf16": 2, "fp8": 1}


def routed_params_per_layer(E: int, H: int, I: int) -> int:
    """gate, up and down matrices of every routed expert: E * 3 * H * I."""
    return E * 3 * H * I


def selected_params_per_token(k: int, H: int, I: int) -> int:
    return k * 3 * H * I


@dataclasses.dataclass
class Work:
    flops: float          # whole layer
    bytes: float          # whole layer
    flops_gate_up: float
    bytes_gate_up: float
    flops_down: float
    bytes_down: float


def layer_work(T, H, E, k, I, I_shared, act="bf16", wdt="bf16", touched=None, scale_block=128) -> Work:
    """touched: number of experts with at least one token (default: min(E, T*k))."""
    R = T * k
    if touched is None:
        touched = min(E, R)
    a = WBYTES[act]
    wb = WBYTES[wdt]
    sh = I_shared > 0
    # FLOPs: router (E columns + the shared gate column), routed SwiGLU, shared SwiGLU
    f_router = 2.0 * T * H * (E + (1 if sh else 0))
    f_gu = 4.0 * R * H * I + (4.0 * T * H * I_shared if sh else 0.0)
    f_dn = 2.0 * R * H * I + (2.0 * T * H * I_shared if sh else 0.0)
    # bytes of weights read once per touched expert
    w_gu = touched * 2.0 * I * H * wb
    w_dn = touched * 1.0 * H * I * wb
    if wdt == "fp8":
        nb = (I // scale_block) * (H // scale_block) * 4.0
        w_gu += touched * 2 * nb
        w_dn += touched * nb
    sh_gu = 2.0 * I_shared * H * a if sh else 0.0
    sh_dn = 1.0 * H * I_shared * a if sh else 0.0
    x_b = 1.0 * T * H * a
    h_b = (1.0 * R * I + (T * I_shared if sh else 0)) * a
    y_b = (1.0 * R * H + (T * H if sh else 0)) * a
    b_gu = w_gu + sh_gu + x_b + h_b
    b_dn = w_dn + sh_dn + h_b + y_b
    b_layer = w_gu + w_dn + sh_gu + sh_dn + E * H * a + (H * a if sh else 0) + x_b + 1.0 * T * H * a
    return Work(flops=f_router + f_gu + f_dn, bytes=b_layer, flops_gate_up=f_gu, bytes_gate_up=b_gu,
                flops_down=f_dn, bytes_down=b_dn)


def gr_read_work(T: int, H: int, rank: int):
    """Gated residual read (Qwen3.8-Flash-Next study, "Gated residual: four
    streams, one sublayer input"): FLOPs of the two projections
    (vec(Rhat) [T, 4H] times [W_down; W_write]^T, then z [T, rank] times
    W_up^T) and the bytes that must cross HBM (the four bf16 streams, the
    gains, both weight matrices, x [T, H] bf16 and s [T, 4] fp32)."""
    flops = 2.0 * T * 4 * H * (rank + 4) + 2.0 * T * rank * 4 * H
    byts = 2.0 * (T * 4 * H + 4 * H + (rank + 4) * 4 * H + 4 * H * rank + T * H) + 4.0 * T * 4
    return flops, byts


def gr_write_work(T: int, H: int):
    """Gated residual write R'_i = R_i + s_i F(x): read the four bf16 streams,
    F(x) and s, write the four streams (the update has 2 FLOPs per element)."""
    return 2.0 * T * 4 * H, 2.0 * (2 * T * 4 * H + T * H) + 4.0 * T * 4


def combine_gr_write_work(T: int, H: int, k: int, shared: bool):
    """The combine with the gated-residual write in its epilogue: read the k
    routed output rows of every token (and its shared-expert row), the
    weights, positions and gate logit, and the four bf16 streams with their
    gates; write the four streams.  F(x) itself does not cross HBM.  FLOPs:
    the weighted sum (2 per term) and the update (2 per stream element)."""
    terms = k + (1 if shared else 0)
    flops = 2.0 * T * H * terms + 2.0 * T * 4 * H
    byts = 2.0 * T * H * terms + 8.0 * T * k + (4.0 * T if shared else 0.0) + 2.0 * 2 * T * 4 * H + 4.0 * T * 4
    return flops, byts


def audit_work(values: int) -> float:
    """Expert-weight audit: every bf16 value is read once (the histograms it
    writes are a few hundred KB per slice and are not counted)."""
    return 2.0 * values


def roofline(flops: float, byts: float, seconds: float, mfma_peak: float = PEAK_BF16_TFLOPS) -> dict:
    """Bound from the intensity against the ridge, then achieved / peak."""
    if flops / byts > mfma_peak * 1e12 / (PEAK_HBM_GBPS * 1e9):
        ach = flops / seconds / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": mfma_peak, "unit": "TFLOP/s",
                "frac": round(ach / mfma_peak, 4)}
    ach = byts / seconds / 1e9
    return {"bound": "hbm", "achieved": round(ach, 2), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBPS, 4)}
