"""MI355X (gfx950) sparse-MoE expert FFN: Python binding of libmoe_ffn.so.

Every step of the layer runs in the library's HIP kernels; this module only
checks tensor dtypes/devices, allocates outputs with torch on the input's
device and passes raw pointers and torch's current HIP stream. Names follow
the C ABI in include/moe_ffn.h:

    route, permute, grouped_gemm, grouped_gemm_wgrad, combine, combine_bwd,
    ffn_fwd, ffn_bwd

Tensors: bf16 activations/weights, fp32 router weights/logits/top-k weights,
int32 indices, all contiguous and on one CUDA (HIP) device.
"""
from __future__ import annotations

import ctypes as C

import torch

from . import _lib
from ._lib import (MOE_EPI_NONE, MOE_EPI_SWIGLU, MOE_EPI_SWIGLU_BWD, MOE_NN, MOE_NT, MoeError,  # noqa: F401
                   MoeGemmRows, MoeSaved, MoeShape)

__all__ = ["route", "permute", "grouped_gemm", "grouped_gemm_wgrad", "combine", "combine_bwd", "ffn_fwd", "ffn_bwd",
           "query_support", "workspace_bytes", "MoeError"]

_EPI = {"none": MOE_EPI_NONE, "swiglu": MOE_EPI_SWIGLU, "swiglu_bwd": MOE_EPI_SWIGLU_BWD}
_OP = {"nn": MOE_NN, "nt": MOE_NT}


def _ptr(t: torch.Tensor | None):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return C.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t, name, dtype, device=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def query_support(T: int, emb: int, mlp: int, E: int, k: int) -> None:
    """Raise MoeError if the layer kernels do not support this shape."""
    s = _lib.shape(T, emb, mlp, E, k)
    _lib.check(_lib.lib().moe_query_support(C.byref(s)), "moe_query_support")


def workspace_bytes(T: int, emb: int, mlp: int, E: int, k: int, backward: bool = False,
                    recompute_h: bool = False) -> int:
    s = _lib.shape(T, emb, mlp, E, k)
    return int(_lib.lib().moe_workspace_bytes(C.byref(s), (2 if recompute_h else 1) if backward else 0))


def route(k: int, x: torch.Tensor | None = None, wr: torch.Tensor | None = None, bias: torch.Tensor | None = None,
          logits: torch.Tensor | None = None):
    """(topk_idx [T,k] int32, topk_w [T,k] fp32). Either x [T,emb] bf16 + wr [emb,E] fp32 (+ bias [E]),
    or logits [T,E] fp32."""
    if logits is not None:
        _need(logits, "logits", torch.float32)
        dev = logits.device
        T, E = logits.shape
        emb = 64
    else:
        _need(x, "x", torch.bfloat16)
        dev = x.device
        _need(wr, "wr", torch.float32, dev)
        _need(bias, "bias", torch.float32, dev)
        T, emb = x.shape
        E = wr.shape[1]
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    s = _lib.shape(T, emb, 64, E, k)
    _lib.check(_lib.lib().moe_route(C.byref(s), _ptr(x), _ptr(wr), _ptr(bias), _ptr(logits), _ptr(idx), _ptr(w),
                                    _stream(dev)), "moe_route")
    return idx, w


def permute(x: torch.Tensor, topk_idx: torch.Tensor, E: int, rows: bool = True, noalloc: bool = False) -> dict:
    """Expert-sorted gather: dict of group_sizes [E], group_offsets [E+1], sorted_slot [S], slot_row [S]
    (int32) and xs [S, emb] bf16. rows=False builds the index only (no xs). noalloc=True calls
    moe_permute_noalloc, which takes no workspace (the library's fixed per-GPU scratch)."""
    _need(x, "x", torch.bfloat16)
    dev = x.device
    _need(topk_idx, "topk_idx", torch.int32, dev)
    T, emb = x.shape
    k = topk_idx.shape[1]
    S = T * k
    s = _lib.shape(T, emb, 64, E, k)
    out = dict(group_sizes=torch.empty(E, dtype=torch.int32, device=dev),
               group_offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
               sorted_slot=torch.empty(S, dtype=torch.int32, device=dev),
               slot_row=torch.empty(S, dtype=torch.int32, device=dev),
               xs=torch.empty((S, emb), dtype=torch.bfloat16, device=dev) if rows else None)
    if noalloc:
        _lib.check(_lib.lib().moe_permute_noalloc(C.byref(s), _ptr(x), _ptr(topk_idx), _ptr(out["group_sizes"]),
                                                  _ptr(out["group_offsets"]), _ptr(out["sorted_slot"]),
                                                  _ptr(out["slot_row"]), _ptr(out["xs"]), _stream(dev)),
                   "moe_permute_noalloc")
        return out
    ws_n = int(_lib.lib().moe_permute_workspace_bytes(C.byref(s)))
    ws = torch.empty(max(ws_n, 16), dtype=torch.uint8, device=dev)
    _lib.check(_lib.lib().moe_permute(C.byref(s), _ptr(x), _ptr(topk_idx), _ptr(out["group_sizes"]),
                                      _ptr(out["group_offsets"]), _ptr(out["sorted_slot"]), _ptr(out["slot_row"]),
                                      _ptr(out["xs"]), _ptr(ws), ws.numel(), _stream(dev)), "moe_permute")
    return out


def grouped_gemm(A: torch.Tensor, B: torch.Tensor, group_offsets: torch.Tensor, op: str = "nn",
                 epilogue: str = "none", aux_in: torch.Tensor | None = None, save_h: bool = False,
                 out: torch.Tensor | None = None, row_slot: torch.Tensor | None = None, slot_div: int = 1,
                 slot_scale: torch.Tensor | None = None, M: int | None = None, grid: int = 0):
    """Ragged grouped GEMM (see moe_grouped_gemm). Returns C, or (C, h) with save_h (SwiGLU, h in fp32).

    row_slot [M] int32 (optional): output row r reads A row row_slot[r] // slot_div (A is not permuted).
    slot_scale (optional, fp32): per-row scale, indexed by row_slot[r] (or r).
    grid: workgroups of the persistent grid (0 = one per compute unit; see moe_grouped_gemm_grid)."""
    _need(A, "A", torch.bfloat16)
    dev = A.device
    _need(B, "B", torch.bfloat16, dev)
    _need(group_offsets, "group_offsets", torch.int32, dev)
    _need(aux_in, "aux_in", torch.float32, dev)
    _need(row_slot, "row_slot", torch.int32, dev)
    _need(slot_scale, "slot_scale", torch.float32, dev)
    K = A.shape[1]
    if M is None:
        M = row_slot.numel() if row_slot is not None else A.shape[0]
    E = B.shape[0]
    N = B.shape[2] if op == "nn" else B.shape[1]
    epi = _EPI[epilogue]
    width = N if epi == MOE_EPI_NONE else (N // 2 if epi == MOE_EPI_SWIGLU else 2 * N)
    C_ = out if out is not None else torch.empty((M, width), dtype=torch.bfloat16, device=dev)
    _need(C_, "out", torch.bfloat16, dev)
    h = torch.empty((M, N), dtype=torch.float32, device=dev) if (save_h and epi == MOE_EPI_SWIGLU) else None
    rows = None
    if row_slot is not None or slot_scale is not None:
        n_slots = A.shape[0] * slot_div if row_slot is not None else 0
        rows = C.byref(MoeGemmRows(None if row_slot is None else row_slot.data_ptr(), n_slots, slot_div,
                                   None if slot_scale is None else slot_scale.data_ptr()))
    _lib.check(_lib.lib().moe_grouped_gemm_grid(_OP[op], epi, _ptr(A), _ptr(B), _ptr(aux_in), _ptr(h),
                                                _ptr(group_offsets), E, M, K, N, rows, _ptr(C_), grid, _stream(dev)),
               "moe_grouped_gemm")
    return (C_, h) if save_h else C_


def grouped_gemm_wgrad(A: torch.Tensor, D: torch.Tensor, group_offsets: torch.Tensor, E: int,
                       grid: int = 0) -> torch.Tensor:
    """C [E, P, Q] = per-group A^T D (grid as in grouped_gemm)."""
    _need(A, "A", torch.bfloat16)
    dev = A.device
    _need(D, "D", torch.bfloat16, dev)
    _need(group_offsets, "group_offsets", torch.int32, dev)
    M, P = A.shape
    Q = D.shape[1]
    C_ = torch.empty((E, P, Q), dtype=torch.bfloat16, device=dev)
    _lib.check(_lib.lib().moe_grouped_gemm_wgrad_grid(_ptr(A), _ptr(D), _ptr(group_offsets), E, M, P, Q, _ptr(C_),
                                                      grid, _stream(dev)), "moe_grouped_gemm_wgrad")
    return C_


_SCHED = {"gemm": _lib.MOE_SCHED_GEMM, "swiglu": _lib.MOE_SCHED_GEMM_SWIGLU, "wgrad": _lib.MOE_SCHED_WGRAD}


def tile_schedule(kind: str, group_offsets, M: int, N: int, grid: int, Q: int = 0):
    """Host-side tile list of a persistent grouped GEMM (moe_tile_schedule): int32 array [n, 7] of
    (workgroup, turn, expert, row0, row1, col0, col1). group_offsets: host integer array [E + 1]."""
    import numpy as np

    off = np.ascontiguousarray(group_offsets, dtype=np.int32)
    E = len(off) - 1
    count = C.c_int64(0)
    f = _lib.lib().moe_tile_schedule
    _lib.check(f(_SCHED[kind], off.ctypes.data, E, M, N, Q, grid, None, 0, C.byref(count)), "moe_tile_schedule")
    out = np.empty((count.value, 7), np.int32)
    _lib.check(f(_SCHED[kind], off.ctypes.data, E, M, N, Q, grid, out.ctypes.data if count.value else None,
                 count.value, C.byref(count)), "moe_tile_schedule")
    return out


def combine(ys: torch.Tensor, slot_row: torch.Tensor, topk_w: torch.Tensor | None, T: int, k: int) -> torch.Tensor:
    """y [T, emb] = sum_j topk_w[t,j] ys[slot_row[t*k+j]] (unit weights when topk_w is None)."""
    _need(ys, "ys", torch.bfloat16)
    dev = ys.device
    _need(slot_row, "slot_row", torch.int32, dev)
    _need(topk_w, "topk_w", torch.float32, dev)
    emb = ys.shape[1]
    y = torch.empty((T, emb), dtype=torch.bfloat16, device=dev)
    s = _lib.shape(T, emb, 64, max(k, 1), k)
    _lib.check(_lib.lib().moe_combine(C.byref(s), _ptr(ys), _ptr(slot_row), _ptr(topk_w), _ptr(y), _stream(dev)),
               "moe_combine")
    return y


def combine_bwd(dy: torch.Tensor, ys: torch.Tensor | None, slot_row: torch.Tensor, topk_w: torch.Tensor, k: int):
    """(dys [S, emb] bf16, dtopk_w [T, k] fp32 or None when ys is None)."""
    _need(dy, "dy", torch.bfloat16)
    dev = dy.device
    _need(ys, "ys", torch.bfloat16, dev)
    _need(slot_row, "slot_row", torch.int32, dev)
    _need(topk_w, "topk_w", torch.float32, dev)
    T, emb = dy.shape
    dys = torch.empty((T * k, emb), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((T, k), dtype=torch.float32, device=dev) if ys is not None else None
    s = _lib.shape(T, emb, 64, max(k, 1), k)
    _lib.check(_lib.lib().moe_combine_bwd(C.byref(s), _ptr(dy), _ptr(ys), _ptr(slot_row), _ptr(topk_w), _ptr(dys),
                                          _ptr(dw), _stream(dev)), "moe_combine_bwd")
    return dys, dw


_SAVED_NAMES = ("topk_idx", "topk_w", "group_sizes", "group_offsets", "sorted_slot", "slot_row", "xs", "h", "a", "o")


def alloc_saved(T: int, emb: int, mlp: int, E: int, k: int, device, keep_h: bool = True) -> dict:
    """Buffers of one forward pass for the backward; keep_h=False leaves h out (the backward recomputes it)."""
    S = T * k
    i32, f32, bf = torch.int32, torch.float32, torch.bfloat16
    return dict(topk_idx=torch.empty((T, k), dtype=i32, device=device),
                topk_w=torch.empty((T, k), dtype=f32, device=device),
                group_sizes=torch.empty(E, dtype=i32, device=device),
                group_offsets=torch.empty(E + 1, dtype=i32, device=device),
                sorted_slot=torch.empty(S, dtype=i32, device=device),
                slot_row=torch.empty(S, dtype=i32, device=device),
                xs=torch.empty((S, emb), dtype=bf, device=device),
                h=torch.empty((S, 2 * mlp), dtype=f32, device=device) if keep_h else None,
                a=torch.empty((S, mlp), dtype=bf, device=device),
                o=torch.empty((S, emb), dtype=bf, device=device))


def _saved_struct(saved: dict) -> MoeSaved:
    return MoeSaved(*[0 if saved[n] is None else saved[n].data_ptr() for n in _SAVED_NAMES])


def route_bwd(x: torch.Tensor, wr: torch.Tensor, topk_idx: torch.Tensor, topk_w: torch.Tensor,
              dtopk_w: torch.Tensor, sorted_slot: torch.Tensor, group_offsets: torch.Tensor,
              dx: torch.Tensor | None = None, want_dbias: bool = True) -> dict:
    """Router gradients with the picks held fixed (see moe_route_bwd): dict(dwr [emb, E] fp32, dbias [E] fp32
    or None). dx (bf16 [T, emb], optional) is updated in place: dx += dlogits . wr^T."""
    _need(x, "x", torch.bfloat16)
    dev = x.device
    for t, n, d in ((wr, "wr", torch.float32), (topk_idx, "topk_idx", torch.int32), (topk_w, "topk_w", torch.float32),
                    (dtopk_w, "dtopk_w", torch.float32), (sorted_slot, "sorted_slot", torch.int32),
                    (group_offsets, "group_offsets", torch.int32), (dx, "dx", torch.bfloat16)):
        _need(t, n, d, dev)
    T, emb = x.shape
    E = wr.shape[1]
    k = topk_idx.shape[1]
    s = _lib.shape(T, emb, 64, E, k)
    ws_n = int(_lib.lib().moe_route_bwd_workspace_bytes(C.byref(s)))
    if ws_n == 0:
        _lib.check(_lib.lib().moe_query_support(C.byref(s)), "route_bwd")
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    dwr = torch.empty((emb, E), dtype=torch.float32, device=dev)
    dbias = torch.empty(E, dtype=torch.float32, device=dev) if want_dbias else None
    _lib.check(_lib.lib().moe_route_bwd(C.byref(s), _ptr(x), _ptr(wr), _ptr(topk_idx), _ptr(topk_w), _ptr(dtopk_w),
                                        _ptr(sorted_slot), _ptr(group_offsets), _ptr(dwr), _ptr(dbias), _ptr(dx),
                                        _ptr(ws), ws.numel(), _stream(dev)), "moe_route_bwd")
    return dict(dwr=dwr, dbias=dbias)


def ffn_fwd(x: torch.Tensor, wi: torch.Tensor, wo: torch.Tensor, k: int, wr: torch.Tensor | None = None,
            bias: torch.Tensor | None = None, logits: torch.Tensor | None = None, save: bool = False,
            workspace: torch.Tensor | None = None, out: torch.Tensor | None = None, keep_h: bool = True):
    """MoE FFN forward. Returns (y [T, emb] bf16, saved dict or None). With save and keep_h=False the
    saved set has no h, and ffn_bwd recomputes it."""
    _need(x, "x", torch.bfloat16)
    dev = x.device
    for t, n, d in ((wi, "wi", torch.bfloat16), (wo, "wo", torch.bfloat16), (wr, "wr", torch.float32),
                    (bias, "bias", torch.float32), (logits, "logits", torch.float32)):
        _need(t, n, d, dev)
    T, emb = x.shape
    E, _, n2 = wi.shape
    mlp = n2 // 2
    s = _lib.shape(T, emb, mlp, E, k)
    ws_n = int(_lib.lib().moe_workspace_bytes(C.byref(s), 0))
    if ws_n == 0:
        _lib.check(_lib.lib().moe_query_support(C.byref(s)), "ffn_fwd")
    ws = workspace if workspace is not None and workspace.numel() >= ws_n else \
        torch.empty(ws_n, dtype=torch.uint8, device=dev)
    y = out if out is not None else torch.empty((T, emb), dtype=torch.bfloat16, device=dev)
    saved = alloc_saved(T, emb, mlp, E, k, dev, keep_h=keep_h) if save else None
    sv = C.byref(_saved_struct(saved)) if save else None
    _lib.check(_lib.lib().moe_ffn_fwd(C.byref(s), _ptr(x), _ptr(wr), _ptr(bias), _ptr(logits), _ptr(wi), _ptr(wo),
                                      _ptr(y), sv, _ptr(ws), ws.numel(), _stream(dev)), "moe_ffn_fwd")
    return y, saved


def ffn_bwd(dy: torch.Tensor, saved: dict, wi: torch.Tensor, wo: torch.Tensor, k: int,
            need=("dx", "dwi", "dwo", "dtopk_w"), workspace: torch.Tensor | None = None) -> dict:
    """MoE FFN backward with the routing held fixed; returns the requested gradients."""
    _need(dy, "dy", torch.bfloat16)
    dev = dy.device
    _need(wi, "wi", torch.bfloat16, dev)
    _need(wo, "wo", torch.bfloat16, dev)
    T, emb = dy.shape
    E, _, n2 = wi.shape
    mlp = n2 // 2
    s = _lib.shape(T, emb, mlp, E, k)
    ws_n = int(_lib.lib().moe_workspace_bytes(C.byref(s), 2 if saved.get("h") is None else 1))
    if ws_n == 0:
        _lib.check(_lib.lib().moe_query_support(C.byref(s)), "ffn_bwd")
    ws = workspace if workspace is not None and workspace.numel() >= ws_n else \
        torch.empty(ws_n, dtype=torch.uint8, device=dev)
    g = {}
    if "dx" in need:
        g["dx"] = torch.empty((T, emb), dtype=torch.bfloat16, device=dev)
    if "dwi" in need:
        g["dwi"] = torch.empty((E, emb, 2 * mlp), dtype=torch.bfloat16, device=dev)
    if "dwo" in need:
        g["dwo"] = torch.empty((E, mlp, emb), dtype=torch.bfloat16, device=dev)
    if "dtopk_w" in need:
        g["dtopk_w"] = torch.empty((T, k), dtype=torch.float32, device=dev)
    _lib.check(_lib.lib().moe_ffn_bwd(C.byref(s), _ptr(dy), C.byref(_saved_struct(saved)), _ptr(wi), _ptr(wo),
                                      _ptr(g.get("dx")), _ptr(g.get("dwi")), _ptr(g.get("dwo")),
                                      _ptr(g.get("dtopk_w")), _ptr(ws), ws.numel(), _stream(dev)), "moe_ffn_bwd")
    return g


def mx_quantize_rows(src: torch.Tensor, row_index: torch.Tensor | None = None, row_div: int = 1,
                     rows: int | None = None):
    """MXFP8 of rows of src [R, K] bf16 (see moe_mx_quantize_rows): (codes [M, K] uint8, scales [K/64, M, 4]
    uint8). With row_index, output row r is source row row_index[r] // row_div."""
    _need(src, "src", torch.bfloat16)
    dev = src.device
    _need(row_index, "row_index", torch.int32, dev)
    R, K = src.shape
    M = rows if rows is not None else (row_index.numel() if row_index is not None else R)
    codes = torch.empty((M, K), dtype=torch.uint8, device=dev)
    scales = torch.empty((K // 64, M, 4), dtype=torch.uint8, device=dev)
    _lib.check(_lib.lib().moe_mx_quantize_rows(_ptr(src), R, K, _ptr(row_index), row_div, M, _ptr(codes),
                                               _ptr(scales), _stream(dev)), "moe_mx_quantize_rows")
    return codes, scales


def mx_quantize_weight(w: torch.Tensor):
    """MXFP8 of expert weights w [E, K, N] bf16 along K, transposed (see moe_mx_quantize_weight):
    (codes [E, N, K] uint8, scales [E, K/64, N, 4] uint8)."""
    _need(w, "w", torch.bfloat16)
    E, K, N = w.shape
    codes = torch.empty((E, N, K), dtype=torch.uint8, device=w.device)
    scales = torch.empty((E, K // 64, N, 4), dtype=torch.uint8, device=w.device)
    _lib.check(_lib.lib().moe_mx_quantize_weight(_ptr(w), E, K, N, _ptr(codes), _ptr(scales), _stream(w.device)),
               "moe_mx_quantize_weight")
    return codes, scales


def grouped_gemm_mx(a_codes: torch.Tensor, a_scales: torch.Tensor, b_codes: torch.Tensor, b_scales: torch.Tensor,
                    group_offsets: torch.Tensor, epilogue: str = "none", out: torch.Tensor | None = None,
                    row_slot: torch.Tensor | None = None, slot_div: int = 1, rows: int | None = None,
                    mx_out: bool = False, bf16_out: bool = True):
    """Grouped GEMM on MXFP8 operands (see moe_grouped_gemm_mx): a_codes [a_rows, K] with a_scales
    [K/64, a_rows, 4] from mx_quantize_rows, b_codes [E, N, K] with b_scales [E, K/64, N, 4] from
    mx_quantize_weight. With row_slot, output row r reads A row row_slot[r] // slot_div (rows = number of
    output rows, default row_slot's length). Returns C [M, N] bf16, or [M, N/2] for epilogue "swiglu"; with
    mx_out (SwiGLU only) returns (C or None, codes [M, N/2], scales [N/128, M, 4]) of the MXFP8 output."""
    dev = a_codes.device
    for t, n in ((a_codes, "a_codes"), (a_scales, "a_scales"), (b_codes, "b_codes"), (b_scales, "b_scales")):
        _need(t, n, torch.uint8, dev)
    _need(group_offsets, "group_offsets", torch.int32, dev)
    _need(row_slot, "row_slot", torch.int32, dev)
    a_rows, K = a_codes.shape
    M = a_rows if row_slot is None else (rows if rows is not None else row_slot.numel())
    E, N, _ = b_codes.shape
    epi = {"none": 0, "swiglu": 1}[epilogue]
    width = N if epi == 0 else N // 2
    C_ = (out if out is not None else torch.empty((M, width), dtype=torch.bfloat16, device=dev)) if bf16_out \
        else None
    cq = torch.empty((M, width), dtype=torch.uint8, device=dev) if mx_out else None
    cqs = torch.zeros((width // 64, M, 4), dtype=torch.uint8, device=dev) if mx_out else None
    _lib.check(_lib.lib().moe_grouped_gemm_mx(epi, _ptr(a_codes), _ptr(a_scales), a_rows, _ptr(row_slot), slot_div,
                                              _ptr(b_codes), _ptr(b_scales), _ptr(group_offsets), E, M, K, N,
                                              _ptr(C_), _ptr(cq), _ptr(cqs), _stream(dev)),
               "moe_grouped_gemm_mx")
    return (C_, cq, cqs) if mx_out else C_


def mx_quantize_expert_weights(wi: torch.Tensor, wo: torch.Tensor) -> dict:
    """Weight preparation for ffn_fwd_mx: the MXFP8 codes and scales of wi and wo along their K."""
    wic, wis = mx_quantize_weight(wi)
    woc, wos = mx_quantize_weight(wo)
    return dict(wi_codes=wic, wi_scales=wis, wo_codes=woc, wo_scales=wos, mlp=wi.shape[2] // 2)


def ffn_fwd_mx(x: torch.Tensor, wq: dict, k: int, wr: torch.Tensor | None = None, bias: torch.Tensor | None = None,
               logits: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
               out: torch.Tensor | None = None) -> torch.Tensor:
    """MoE FFN forward with MXFP8 grouped GEMMs (see moe_ffn_fwd_mx); wq from mx_quantize_expert_weights."""
    _need(x, "x", torch.bfloat16)
    dev = x.device
    for t, n, d in ((wr, "wr", torch.float32), (bias, "bias", torch.float32), (logits, "logits", torch.float32)):
        _need(t, n, d, dev)
    T, emb = x.shape
    E = wq["wi_codes"].shape[0]
    mlp = wq["mlp"]
    s = _lib.shape(T, emb, mlp, E, k)
    ws_n = int(_lib.lib().moe_workspace_bytes_mx(C.byref(s)))
    if ws_n == 0:
        _lib.check(_lib.lib().moe_query_support(C.byref(s)), "ffn_fwd_mx")
        raise _lib.MoeError(_lib.MOE_ERR_UNSUPPORTED, "ffn_fwd_mx", "mlp must be a multiple of 64")
    ws = workspace if workspace is not None and workspace.numel() >= ws_n else \
        torch.empty(ws_n, dtype=torch.uint8, device=dev)
    y = out if out is not None else torch.empty((T, emb), dtype=torch.bfloat16, device=dev)
    _lib.check(_lib.lib().moe_ffn_fwd_mx(C.byref(s), _ptr(x), _ptr(wr), _ptr(bias), _ptr(logits),
                                         _ptr(wq["wi_codes"]), _ptr(wq["wi_scales"]), _ptr(wq["wo_codes"]),
                                         _ptr(wq["wo_scales"]), _ptr(y), _ptr(ws), ws.numel(), _stream(dev)),
               "moe_ffn_fwd_mx")
    return y
