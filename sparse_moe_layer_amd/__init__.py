"""Routed Mixture-of-Experts FFN layer for AMD Instinct MI355X (gfx950).

Python face of the C ABI in include/moe_mi355x.h: the functions below have
the C entry points' names and arguments, take torch tensors (device memory)
and pass their pointers plus the current HIP stream to the library.  No
computation happens here.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from ._lib import (LIB, MOE_BF16, MOE_F32, MOE_FLAG_FORCE_GEMM, MOE_FLAG_FORCE_STREAM,  # noqa: F401
                   MOE_FLAG_GEMM_TILE_128, MOE_FLAG_GEMM_TILE_256, MOE_FLAG_PAGE_ROUTING, MOE_FP8_E4M3FN,
                   MOE_NOALLOC_SCRATCH_BYTES, MOE_OK, EXPORTS, moe_audit_stats, moe_gr_weights, moe_problem,
                   moe_weights)

_DT = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3FN}


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {LIB.moe_status_str(status).decode()} (status {status})")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(st: int, where: str):
    if st != MOE_OK:
        raise MoEError(st, where)


def problem(T, H, E, k, I, I_shared=0, act="bf16", wdt="bf16", scale_block=128, flags=0) -> moe_problem:
    return moe_problem(T, H, E, k, I, I_shared, _DT[act], _DT[wdt], scale_block, flags)


def weights(w_router, w_gate, w_up, w_down, s_gate=None, s_up=None, s_down=None, sh_gate=None, sh_up=None,
            sh_down=None, sh_gate_w=None, stride_gate=0, stride_up=0, stride_down=0) -> moe_weights:
    return moe_weights(_ptr(w_router), _ptr(w_gate), _ptr(w_up), _ptr(w_down), stride_gate, stride_up,
                       stride_down, _ptr(s_gate), _ptr(s_up), _ptr(s_down), _ptr(sh_gate), _ptr(sh_up),
                       _ptr(sh_down), _ptr(sh_gate_w))


def moe_abi_version() -> int:
    return LIB.moe_abi_version()


def moe_validate(p: moe_problem) -> int:
    return LIB.moe_validate(ctypes.byref(p))


def moe_workspace_bytes(p: moe_problem) -> int:
    return LIB.moe_workspace_bytes(ctypes.byref(p))


def workspace(p: moe_problem, device="cuda") -> torch.Tensor:
    """A device buffer of moe_workspace_bytes(p) bytes (torch allocations are 256-byte aligned)."""
    n = moe_workspace_bytes(p)
    if n == 0:
        _check(moe_validate(p), "moe_workspace_bytes")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def moe_route(p, x, w_router, sh_gate_w, topk_ids, topk_w, shared_logit, ws, stream=None):
    _check(LIB.moe_route(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(sh_gate_w), _ptr(topk_ids), _ptr(topk_w),
                         _ptr(shared_logit), _ptr(ws), ws.numel(), _stream(stream)), "moe_route")


def moe_dispatch(p, topk_ids, expert_offsets, sorted_assign, assign_pos, ws, stream=None):
    _check(LIB.moe_dispatch(ctypes.byref(p), _ptr(topk_ids), _ptr(expert_offsets), _ptr(sorted_assign),
                            _ptr(assign_pos), _ptr(ws), ws.numel(), _stream(stream)), "moe_dispatch")


def moe_expert_ffn(p, w: moe_weights, x, expert_offsets, sorted_assign, y, y_shared, ws, stream=None):
    _check(LIB.moe_expert_ffn(ctypes.byref(p), ctypes.byref(w), _ptr(x), _ptr(expert_offsets), _ptr(sorted_assign),
                              _ptr(y), _ptr(y_shared), _ptr(ws), ws.numel(), _stream(stream)), "moe_expert_ffn")


def moe_expert_gate_up(p, w: moe_weights, x, expert_offsets, sorted_assign, h, h_shared, ws, stream=None):
    _check(LIB.moe_expert_gate_up(ctypes.byref(p), ctypes.byref(w), _ptr(x), _ptr(expert_offsets),
                                  _ptr(sorted_assign), _ptr(h), _ptr(h_shared), _ptr(ws), ws.numel(),
                                  _stream(stream)), "moe_expert_gate_up")


def moe_expert_down(p, w: moe_weights, expert_offsets, h, h_shared, y, y_shared, ws, stream=None):
    _check(LIB.moe_expert_down(ctypes.byref(p), ctypes.byref(w), _ptr(expert_offsets), _ptr(h), _ptr(h_shared),
                               _ptr(y), _ptr(y_shared), _ptr(ws), ws.numel(), _stream(stream)), "moe_expert_down")


def moe_combine(p, y, assign_pos, topk_w, y_shared, shared_logit, out, stream=None):
    _check(LIB.moe_combine(ctypes.byref(p), _ptr(y), _ptr(assign_pos), _ptr(topk_w), _ptr(y_shared),
                           _ptr(shared_logit), _ptr(out), _stream(stream)), "moe_combine")


def moe_layer_forward(p, w: moe_weights, x, out, topk_ids, topk_w, ws, stream=None):
    _check(LIB.moe_layer_forward(ctypes.byref(p), ctypes.byref(w), _ptr(x), _ptr(out), _ptr(topk_ids),
                                 _ptr(topk_w), _ptr(ws), ws.numel(), _stream(stream)), "moe_layer_forward")


def moe_hbm_read_probe(src, sink, stream=None):
    _check(LIB.moe_hbm_read_probe(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(stream)),
           "moe_hbm_read_probe")


def moe_mfma_pipe_probe(variant: int, steps: int, src, sink, stream=None):
    nbytes = 0 if src is None else src.numel() * src.element_size()
    _check(LIB.moe_mfma_pipe_probe(variant, steps, _ptr(src), nbytes, _ptr(sink), _stream(stream)),
           "moe_mfma_pipe_probe")


def moe_layer_forward_noalloc(p, w: moe_weights, x, out, topk_ids, topk_w, stream=None):
    _check(LIB.moe_layer_forward_noalloc(ctypes.byref(p), ctypes.byref(w), _ptr(x), _ptr(out), _ptr(topk_ids),
                                         _ptr(topk_w), _stream(stream)), "moe_layer_forward_noalloc")


def gr_weights(norm_w, w_read, w_up, rank: int, eps: float = 1e-6) -> moe_gr_weights:
    return moe_gr_weights(_ptr(norm_w), _ptr(w_read), _ptr(w_up), rank, eps)


def moe_gr_workspace_bytes(p: moe_problem, rank: int) -> int:
    return LIB.moe_gr_workspace_bytes(ctypes.byref(p), rank)


def gr_workspace(p: moe_problem, rank: int, device="cuda") -> torch.Tensor:
    """A device buffer of moe_gr_workspace_bytes(p, rank) bytes."""
    n = moe_gr_workspace_bytes(p, rank)
    if n == 0:
        st = LIB.moe_validate(ctypes.byref(p))
        raise MoEError(st if st != MOE_OK else 6, "moe_gr_workspace_bytes")  # 6: MOE_ERR_UNSUPPORTED
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_gr_read(p, g: moe_gr_weights, resid, x, s, ws, stream=None):
    _check(LIB.moe_gr_read(ctypes.byref(p), ctypes.byref(g), _ptr(resid), _ptr(x), _ptr(s), _ptr(ws), ws.numel(),
                           _stream(stream)), "moe_gr_read")


def moe_gr_write(p, resid, s, f, resid_out, stream=None):
    _check(LIB.moe_gr_write(ctypes.byref(p), _ptr(resid), _ptr(s), _ptr(f), _ptr(resid_out), _stream(stream)),
           "moe_gr_write")


def moe_combine_gr_write(p, y, assign_pos, topk_w, y_shared, shared_logit, resid, s, out, resid_out, stream=None):
    _check(LIB.moe_combine_gr_write(ctypes.byref(p), _ptr(y), _ptr(assign_pos), _ptr(topk_w), _ptr(y_shared),
                                    _ptr(shared_logit), _ptr(resid), _ptr(s), _ptr(out), _ptr(resid_out),
                                    _stream(stream)), "moe_combine_gr_write")


# numpy dtype of one moe_audit_stats record (int64 n, n_zero, n_nan; float64 median, mad, sigma_rob)
AUDIT_STATS_FIELDS = ("n", "n_zero", "n_nan", "median", "mad", "sigma_rob")


def moe_audit_workspace_bytes(slices: int) -> int:
    return LIB.moe_audit_workspace_bytes(slices)


def audit_workspace(slices: int, device="cuda") -> torch.Tensor:
    n = moe_audit_workspace_bytes(slices)
    if n == 0:
        raise MoEError(2, "moe_audit_workspace_bytes")  # 2: MOE_ERR_SHAPE
    return torch.empty(n, dtype=torch.uint8, device=device)


def audit_stats_buffer(slices: int, device="cuda") -> torch.Tensor:
    """Device buffer for slices + 1 records (48 bytes each, 8-byte aligned)."""
    return torch.empty((slices + 1, 6), dtype=torch.float64, device=device)


def moe_weight_audit(w, slices: int, n: int, slice_stride: int, stats, ws, stream=None):
    """w: bf16 device tensor; stats: audit_stats_buffer(slices)."""
    if w.dtype != torch.bfloat16:
        raise MoEError(6, "moe_weight_audit")  # 6: MOE_ERR_UNSUPPORTED
    _check(LIB.moe_weight_audit(_ptr(w), MOE_BF16, slices, n, slice_stride, _ptr(stats), _ptr(ws), ws.numel(),
                                _stream(stream)), "moe_weight_audit")


def audit_records(stats: torch.Tensor) -> list:
    """Host dicts of the records in an audit_stats_buffer (after the stream is synchronised)."""
    host = stats.detach().cpu().contiguous()
    ints = host.view(torch.int64)
    return [{"n": int(ints[i, 0]), "n_zero": int(ints[i, 1]), "n_nan": int(ints[i, 2]),
             "median": float(host[i, 3]), "mad": float(host[i, 4]), "sigma_rob": float(host[i, 5])}
            for i in range(host.shape[0])]


_DT_OF_TORCH = {torch.float32: "f32", torch.bfloat16: "bf16", torch.uint8: "fp8"}


def layer_forward(x, k: int, w_router, w_gate, w_up, w_down, s_gate=None, s_up=None, s_down=None, sh_gate=None,
                  sh_up=None, sh_down=None, sh_gate_w=None, flags: int = 0, stream=None):
    """The whole layer in one call: returns (out [T, H], ids [T, k] int32, w [T, k] fp32).

    Shapes come from the tensors: x [T, H] (bf16 or fp32), w_router [E, H], w_gate / w_up [E, I, H],
    w_down [E, H, I] (bf16, fp32, or uint8 e4m3fn codes with fp32 128 x 128 block scales s_*), and
    the optional shared expert sh_gate / sh_up [I_s, H], sh_down [H, I_s], sh_gate_w [1, H].
    Outputs and the workspace are allocated on x's device; every computation runs in the library.
    """
    T, H = x.shape
    E, I = w_gate.shape[0], w_gate.shape[1]
    Is = sh_gate.shape[0] if sh_gate is not None else 0
    wdt = _DT_OF_TORCH[w_gate.dtype]
    P = problem(T, H, E, k, I, Is, _DT_OF_TORCH[x.dtype], wdt, 128, flags)
    W = weights(w_router, w_gate, w_up, w_down, s_gate, s_up, s_down, sh_gate, sh_up, sh_down, sh_gate_w)
    ws = workspace(P, device=x.device)
    out = torch.empty((T, H), dtype=x.dtype, device=x.device)
    ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    tw = torch.empty((T, k), dtype=torch.float32, device=x.device)
    moe_layer_forward(P, W, x, out, ids, tw, ws, stream)
    return out, ids, tw
