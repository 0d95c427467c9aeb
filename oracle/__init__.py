"""CPU oracle of the sparse-MoE expert FFN (ctypes wrapper over moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product package never does.

Arrays are numpy: bf16 tensors travel as their raw uint16 bit patterns,
fp32 as float32, fp64 as float64. ``real`` picks the accumulation type of the
FFN arithmetic ("f32" or "f64"); the router is always fp32 (see moe_oracle.c).
Per-token functions split their token list over ``threads`` host threads;
each token is computed independently, so the result does not depend on the
thread count.
"""
from __future__ import annotations

import ctypes as C
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import build as _build

BF16, F32, F64 = 0, 1, 2
_ERR = {1: "invalid argument", 2: "NaN input", 3: "index out of range", 4: "expert picked twice by a token",
        5: "out of memory"}
_libs: dict[str, C.CDLL] = {}

_p = C.c_void_p
_i32, _i64 = C.c_int32, C.c_int64


def _lib(real: str) -> C.CDLL:
    if real not in _libs:
        path = _build.lib_path(real)
        if not os.path.exists(path):
            _build.build()
        lib = C.CDLL(path)
        sigs = {
            "orc_real_bytes": ([], C.c_int),
            "orc_router_logits": ([_i64, _i32, _i32, _p, C.c_int, _p, _p, _p], C.c_int),
            "orc_topk": ([_i64, _i32, _i32, _p, _p, _p], C.c_int),
            "orc_dispatch": ([_i64, _i32, _i32, _p, _p, _p, _p, _p], C.c_int),
            "orc_permute": ([_i64, _i32, _i32, _p, _p, _p], C.c_int),
            "orc_ffn_fwd_tokens": ([_i32, _i32, _i32, _i32, _p, C.c_int, _p, _p, _p, C.c_int, _p, C.c_int,
                                    _i64, _p, _p, _p, _p, _p], C.c_int),
            "orc_ffn_bwd_tokens": ([_i32, _i32, _i32, _i32, _p, C.c_int, _p, _p, _p, C.c_int, _p, C.c_int,
                                    _p, C.c_int, _i64, _p, _p, _p, _i32], C.c_int),
            "orc_ffn_wgrad_expert": ([_i32, _i32, _i32, _i32, _p, C.c_int, _p, _p, _p, C.c_int, _p, C.c_int,
                                      _p, C.c_int, _i32, _i64, _p, _p, _p, _i32], C.c_int),
            "orc_grouped_gemm": ([_i32, _i32, _p, C.c_int, _p, C.c_int, _p, C.c_int, _p, _i32, _i64, _i32, _i32,
                                  _i64, _i64, _p], C.c_int),
            "orc_grouped_wgrad": ([_p, C.c_int, _p, C.c_int, _p, _i32, _i64, _i32, _i32, _i32, _p], C.c_int),
            "orc_combine": ([_i64, _i32, _i32, _p, C.c_int, _p, _p, _p], C.c_int),
            "orc_combine_bwd": ([_i64, _i32, _i32, _p, C.c_int, _p, C.c_int, _p, _p, _p, _p], C.c_int),
            "orc_e4m3_value": ([C.c_uint8], C.c_double),
            "orc_mx_quantize": ([_i64, _i32, _p, _p, _p], C.c_int),
            "orc_router_bwd": ([_i64, _i32, _i32, _i32, _p, C.c_int, _p, _p, _p, _p, C.c_int, _p, _p, _p, _p],
                               C.c_int),
        }
        for name, (args, res) in sigs.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = res
        assert lib.orc_real_bytes() == (4 if real == "f32" else 8)
        _libs[real] = lib
    return _libs[real]


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise OracleError(f"{what}: {_ERR.get(rc, rc)}")


def _typed(a):
    """(pointer, dtype code) of a C-contiguous numpy array; None -> (None, F32)."""
    if a is None:
        return None, F32
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("oracle inputs must be C-contiguous")
    dt = {np.dtype(np.uint16): BF16, np.dtype(np.float32): F32, np.dtype(np.float64): F64}.get(a.dtype)
    if dt is None:
        raise TypeError(f"unsupported oracle dtype {a.dtype} (use uint16 bf16 bits, float32, float64)")
    return a.ctypes.data, dt


def _ptr(a):
    return None if a is None else a.ctypes.data


def _np_real(real: str):
    return np.float32 if real == "f32" else np.float64


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _split(n: int, threads: int):
    threads = max(1, min(threads, n))
    bounds = np.linspace(0, n, threads + 1).astype(np.int64)
    return [(int(bounds[i]), int(bounds[i + 1])) for i in range(threads) if bounds[i + 1] > bounds[i]]


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ----------------------------------------------------------------- routing

def router_logits(x, wr, bias=None, threads: int | None = None) -> np.ndarray:
    """fp32 logits [T, E] by the fixed fma chain over emb, plus bias."""
    x = np.ascontiguousarray(x)
    wr = _c(wr, np.float32)
    bias = None if bias is None else _c(bias, np.float32)
    T, emb = x.shape
    E = wr.shape[1]
    out = np.empty((T, E), np.float32)
    lib = _lib("f32")

    def run(lo_hi):
        lo, hi = lo_hi
        xp, xdt = _typed(x[lo:hi])
        _check(lib.orc_router_logits(hi - lo, emb, E, xp, xdt, _ptr(wr), _ptr(bias), out[lo:hi].ctypes.data),
               "router_logits")

    chunks = _split(T, threads or default_threads())
    with ThreadPoolExecutor(len(chunks) or 1) as ex:
        list(ex.map(run, chunks))
    return out


def topk(logits, k: int):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _check(_lib("f32").orc_topk(T, E, k, _ptr(logits), _ptr(idx), _ptr(w)), "topk")
    return idx, w


def route(x, wr, bias, k: int, logits_in=None, threads: int | None = None):
    """(topk_idx [T,k] int32, topk_w [T,k] float32, logits [T,E] float32)."""
    logits = _c(logits_in, np.float32) if logits_in is not None else router_logits(x, wr, bias, threads)
    idx, w = topk(logits, k)
    return idx, w, logits


def dispatch(topk_idx, E: int):
    """(group_sizes [E], group_offsets [E+1], sorted_slot [S], slot_row [S]), all int32."""
    topk_idx = _c(topk_idx, np.int32)
    T, k = topk_idx.shape
    gs = np.empty(E, np.int32)
    go = np.empty(E + 1, np.int32)
    ss = np.empty(T * k, np.int32)
    sr = np.empty(T * k, np.int32)
    _check(_lib("f32").orc_dispatch(T, E, k, _ptr(topk_idx), _ptr(gs), _ptr(go), _ptr(ss), _ptr(sr)), "dispatch")
    return gs, go, ss, sr


def permute(x_bits, sorted_slot, k: int) -> np.ndarray:
    x_bits = _c(x_bits, np.uint16)
    sorted_slot = _c(sorted_slot, np.int32)
    T, emb = x_bits.shape
    xs = np.empty((T * k, emb), np.uint16)
    _check(_lib("f32").orc_permute(T, emb, k, _ptr(x_bits), _ptr(sorted_slot), _ptr(xs)), "permute")
    return xs


# ----------------------------------------------------------------- full layer

def ffn_fwd_tokens(x, topk_idx, topk_w, wi, wo, tokens=None, real: str = "f32", want_intermediates=False,
                   threads: int | None = None):
    """y [n, emb] for the listed tokens (all tokens when None).

    With want_intermediates, also returns h [n,k,2mlp], a [n,k,mlp], o [n,k,emb]."""
    x = np.ascontiguousarray(x)
    wi = np.ascontiguousarray(wi)
    wo = np.ascontiguousarray(wo)
    topk_idx = _c(topk_idx, np.int32)
    topk_w = _c(topk_w, np.float32)
    T, emb = x.shape
    E, _, n2 = wi.shape
    mlp = n2 // 2
    k = topk_idx.shape[1]
    tokens = np.arange(T, dtype=np.int64) if tokens is None else _c(tokens, np.int64)
    n = len(tokens)
    rt = _np_real(real)
    y = np.empty((n, emb), rt)
    h = np.empty((n, k, n2), rt) if want_intermediates else None
    a = np.empty((n, k, mlp), rt) if want_intermediates else None
    o = np.empty((n, k, emb), rt) if want_intermediates else None
    lib = _lib(real)
    xp, xdt = _typed(x)
    wip, widt = _typed(wi)
    wop, wodt = _typed(wo)

    def run(lo_hi):
        lo, hi = lo_hi
        sl = lambda arr: None if arr is None else arr[lo:hi].ctypes.data  # noqa: E731
        _check(lib.orc_ffn_fwd_tokens(emb, mlp, E, k, xp, xdt, _ptr(topk_idx), _ptr(topk_w), wip, widt, wop, wodt,
                                      hi - lo, tokens[lo:hi].ctypes.data, sl(y), sl(h), sl(a), sl(o)),
               "ffn_fwd_tokens")

    chunks = _split(n, threads or default_threads())
    with ThreadPoolExecutor(len(chunks) or 1) as ex:
        list(ex.map(run, chunks))
    return (y, h, a, o) if want_intermediates else y


def ffn_bwd_tokens(x, topk_idx, topk_w, wi, wo, dy, tokens=None, real: str = "f32", threads: int | None = None,
                   stored_bf16: bool = False):
    """(dx [n, emb], dtopk_w [n, k]) for the listed tokens, routing held fixed. With stored_bf16, a, o, dh
    and dxs are rounded to bf16 where the layer stores them (moe_oracle.c, R9)."""
    x = np.ascontiguousarray(x)
    dy = np.ascontiguousarray(dy)
    wi = np.ascontiguousarray(wi)
    wo = np.ascontiguousarray(wo)
    topk_idx = _c(topk_idx, np.int32)
    topk_w = _c(topk_w, np.float32)
    T, emb = x.shape
    E, _, n2 = wi.shape
    mlp = n2 // 2
    k = topk_idx.shape[1]
    tokens = np.arange(T, dtype=np.int64) if tokens is None else _c(tokens, np.int64)
    n = len(tokens)
    rt = _np_real(real)
    dx = np.empty((n, emb), rt)
    dw = np.empty((n, k), rt)
    lib = _lib(real)
    xp, xdt = _typed(x)
    dyp, dydt = _typed(dy)
    wip, widt = _typed(wi)
    wop, wodt = _typed(wo)

    def run(lo_hi):
        lo, hi = lo_hi
        _check(lib.orc_ffn_bwd_tokens(emb, mlp, E, k, xp, xdt, _ptr(topk_idx), _ptr(topk_w), wip, widt, wop, wodt,
                                      dyp, dydt, hi - lo, tokens[lo:hi].ctypes.data, dx[lo:hi].ctypes.data,
                                      dw[lo:hi].ctypes.data, int(bool(stored_bf16))), "ffn_bwd_tokens")

    chunks = _split(n, threads or default_threads())
    with ThreadPoolExecutor(len(chunks) or 1) as ex:
        list(ex.map(run, chunks))
    return dx, dw


def ffn_wgrad_experts(x, topk_idx, topk_w, wi, wo, dy, experts, real: str = "f32", threads: int | None = None,
                      stored_bf16: bool = False):
    """{e: (dwi_e [emb, 2mlp], dwo_e [mlp, emb])} for the listed experts, routing held fixed.

    Each expert's slots are taken in expert-sorted order (token ascending). With stored_bf16, the factors
    a, do and dh are rounded to bf16 before the products, as the layer stores them (moe_oracle.c, R9)."""
    x = np.ascontiguousarray(x)
    dy = np.ascontiguousarray(dy)
    wi = np.ascontiguousarray(wi)
    wo = np.ascontiguousarray(wo)
    topk_idx = _c(topk_idx, np.int32)
    topk_w = _c(topk_w, np.float32)
    T, emb = x.shape
    E, _, n2 = wi.shape
    mlp = n2 // 2
    k = topk_idx.shape[1]
    rt = _np_real(real)
    lib = _lib(real)
    xp, xdt = _typed(x)
    dyp, dydt = _typed(dy)
    wip, widt = _typed(wi)
    wop, wodt = _typed(wo)
    flat = topk_idx.reshape(-1)

    def run(e):
        slots = np.nonzero(flat == e)[0].astype(np.int64)  # slot = t*k + j, ascending t
        dwi = np.empty((emb, n2), rt)
        dwo = np.empty((mlp, emb), rt)
        _check(lib.orc_ffn_wgrad_expert(emb, mlp, E, k, xp, xdt, _ptr(topk_idx), _ptr(topk_w), wip, widt, wop, wodt,
                                        dyp, dydt, int(e), len(slots), _ptr(slots), _ptr(dwi), _ptr(dwo),
                                        int(bool(stored_bf16))),
               "ffn_wgrad_expert")
        return dwi, dwo

    experts = list(experts)
    with ThreadPoolExecutor(max(1, min(len(experts), threads or default_threads()))) as ex:
        res = list(ex.map(run, experts))
    return dict(zip(experts, res))


# ----------------------------------------------------------------- single stages

def grouped_gemm(op: int, epi: int, A, B, group_offsets, aux=None, rows=None, real: str = "f32",
                 threads: int | None = None):
    """Rows [r0, r1) of a grouped GEMM (see orc_grouped_gemm). op 0 = NN, 1 = NT; epi 0 none, 1 SwiGLU,
    2 SwiGLU backward (aux = saved h)."""
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    aux = None if aux is None else np.ascontiguousarray(aux)
    off = _c(group_offsets, np.int32)
    M, K = A.shape
    E = B.shape[0]
    N = B.shape[2] if op == 0 else B.shape[1]
    width = N if epi == 0 else (N // 2 if epi == 1 else 2 * N)
    r0, r1 = (0, M) if rows is None else rows
    C_ = np.zeros((r1 - r0, width), _np_real(real))
    lib = _lib(real)
    ap, adt = _typed(A)
    bp, bdt = _typed(B)
    xp, xdt = _typed(aux)

    def run(lo_hi):
        lo, hi = lo_hi
        _check(lib.orc_grouped_gemm(op, epi, ap, adt, bp, bdt, xp, xdt, _ptr(off), E, M, K, N, r0 + lo, r0 + hi,
                                    C_[lo:hi].ctypes.data), "grouped_gemm")

    chunks = _split(r1 - r0, threads or default_threads())
    with ThreadPoolExecutor(len(chunks) or 1) as ex:
        list(ex.map(run, chunks))
    return C_


def grouped_wgrad(A, D, group_offsets, e: int, real: str = "f32") -> np.ndarray:
    A = np.ascontiguousarray(A)
    D = np.ascontiguousarray(D)
    off = _c(group_offsets, np.int32)
    M, P = A.shape
    Q = D.shape[1]
    E = len(off) - 1
    out = np.empty((P, Q), _np_real(real))
    ap, adt = _typed(A)
    dp, ddt = _typed(D)
    _check(_lib(real).orc_grouped_wgrad(ap, adt, dp, ddt, _ptr(off), E, M, P, Q, e, _ptr(out)), "grouped_wgrad")
    return out


def combine(ys, slot_row, topk_w, T: int, k: int, real: str = "f32") -> np.ndarray:
    ys = np.ascontiguousarray(ys)
    slot_row = _c(slot_row, np.int32)
    w = None if topk_w is None else _c(topk_w, np.float32)
    emb = ys.shape[1]
    y = np.empty((T, emb), _np_real(real))
    p, dt = _typed(ys)
    _check(_lib(real).orc_combine(T, emb, k, p, dt, _ptr(slot_row), _ptr(w), _ptr(y)), "combine")
    return y


def combine_bwd(dy, ys, slot_row, topk_w, k: int, real: str = "f32"):
    """(dys [S, emb], dtopk_w [T, k] or None)."""
    dy = np.ascontiguousarray(dy)
    ys = None if ys is None else np.ascontiguousarray(ys)
    slot_row = _c(slot_row, np.int32)
    w = _c(topk_w, np.float32)
    T, emb = dy.shape
    rt = _np_real(real)
    dys = np.empty((T * k, emb), rt)
    dw = np.empty((T, k), rt) if ys is not None else None
    p, dt = _typed(dy)
    yp, ydt = _typed(ys)
    _check(_lib(real).orc_combine_bwd(T, emb, k, p, dt, yp, ydt, _ptr(slot_row), _ptr(w), _ptr(dys), _ptr(dw)),
           "combine_bwd")
    return dys, dw


def router_bwd(x, wr, topk_idx, topk_w, dtopk_w, real: str = "f64", want_dx: bool = True):
    """Router backward with the picks held fixed: (dlogits [T, E], dwr [emb, E], dbias [E], dx [T, emb] or None)."""
    x = np.ascontiguousarray(x)
    wr = _c(wr, np.float32)
    idx = _c(topk_idx, np.int32)
    w = _c(topk_w, np.float32)
    g = np.ascontiguousarray(dtopk_w)
    T, emb = x.shape
    E = wr.shape[1]
    k = idx.shape[1]
    rt = _np_real(real)
    dl = np.empty((T, E), rt)
    dwr = np.empty((emb, E), rt)
    db = np.empty(E, rt)
    dx = np.empty((T, emb), rt) if want_dx else None
    xp, xdt = _typed(x)
    gp, gdt = _typed(g)
    _check(_lib(real).orc_router_bwd(T, emb, E, k, xp, xdt, _ptr(wr), _ptr(idx), _ptr(w), gp, gdt, _ptr(dl),
                                     _ptr(dwr), _ptr(db), _ptr(dx)), "router_bwd")
    return dl, dwr, db, dx


# ---------------------------------------------------------------- MXFP8

def e4m3_value(code: int) -> float:
    """Value of one FP8 E4M3 ("FN") code (NaN for 0x7f / 0xff)."""
    return float(_lib("f32").orc_e4m3_value(int(code) & 0xFF))


def mx_quantize(x_bits):
    """MXFP8 of x [M, K] (bf16 bits) in blocks of 32 along K: (codes [M, K] uint8 E4M3, scales [M, K/32] uint8
    E8M0). See moe_oracle.c, reading R8."""
    x_bits = _c(x_bits, np.uint16)
    M, K = x_bits.shape
    codes = np.empty((M, K), np.uint8)
    scales = np.empty((M, K // 32), np.uint8)
    _check(_lib("f32").orc_mx_quantize(M, K, _ptr(x_bits), _ptr(codes), _ptr(scales)), "mx_quantize")
    return codes, scales


_E4M3_TABLE = None


def mx_dequantize(codes, scales) -> np.ndarray:
    """float64 values code * 2^(scale - 127) of an MXFP8 tensor [..., K] with scales [..., K/32]."""
    global _E4M3_TABLE
    if _E4M3_TABLE is None:
        _E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], np.float64)
    codes = np.asarray(codes, np.uint8)
    scales = np.asarray(scales, np.uint8)
    v = _E4M3_TABLE[codes]
    f = np.ldexp(1.0, scales.astype(np.int64) - 127)
    return v * np.repeat(f, 32, axis=-1)


def mx_grouped_gemm_nt(a_codes, a_scales, b_codes, b_scales, group_offsets, epi: int = 0) -> np.ndarray:
    """Grouped GEMM on MXFP8 operands, in float64 on the dequantized values: rows of group e of
    A [M, K] times B[e] [N, K] transposed; epi 0 none, 1 SwiGLU (gate = columns [0, N/2), up = [N/2, N)).
    The contraction runs over the exact products, so the only error of a device result against this is
    its own summation."""
    A = mx_dequantize(a_codes, a_scales)
    B = mx_dequantize(b_codes, b_scales)
    off = np.asarray(group_offsets, np.int64)
    M = A.shape[0]
    N = B.shape[1]
    C_ = np.zeros((M, N), np.float64)
    for e in range(B.shape[0]):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            C_[lo:hi] = A[lo:hi] @ B[e].T
    if epi == 1:
        g, u = C_[:, : N // 2], C_[:, N // 2:]
        return g / (1.0 + np.exp(-g)) * u
    return C_
