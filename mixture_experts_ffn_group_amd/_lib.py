"""ctypes loader for libmoe_ffn.so (the C ABI of include/moe_ffn.h).

torch is imported first on purpose: the library's NEEDED libamdhip64.so.7
then binds to the HIP runtime copy torch already loaded, so torch's streams
and device pointers are valid inside the library.
"""
from __future__ import annotations

import ctypes as C
import os

import torch  # noqa: F401  (must precede loading the library)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_ffn.so")

MOE_OK = 0
MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP, MOE_ERR_ALIGN = 1, 2, 3, 4, 5, 6
MOE_NN, MOE_NT = 0, 1
MOE_EPI_NONE, MOE_EPI_SWIGLU, MOE_EPI_SWIGLU_BWD = 0, 1, 2
MOE_SCHED_GEMM, MOE_SCHED_GEMM_SWIGLU, MOE_SCHED_WGRAD = 0, 1, 2

# Every function the header declares, with its ctypes signature.
_p = C.c_void_p
_i32, _i64, _sz = C.c_int32, C.c_int64, C.c_size_t


class MoeShape(C.Structure):
    _fields_ = [("T", C.c_int64), ("emb", C.c_int32), ("mlp", C.c_int32), ("E", C.c_int32), ("k", C.c_int32)]


class MoeSaved(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("topk_idx", "topk_w", "group_sizes", "group_offsets", "sorted_slot",
                                           "slot_row", "xs", "h", "a", "o")]


class MoeGemmRows(C.Structure):
    _fields_ = [("row_slot", C.c_void_p), ("n_slots", C.c_int32), ("slot_div", C.c_int32),
                ("slot_scale", C.c_void_p)]


_SHP = C.POINTER(MoeShape)
SIGNATURES = {
    "moe_status_str": ([C.c_int], C.c_char_p),
    "moe_last_error_detail": ([], C.c_char_p),
    "moe_version": ([], C.c_char_p),
    "moe_query_support": ([_SHP], C.c_int),
    "moe_permute_workspace_bytes": ([_SHP], _sz),
    "moe_workspace_bytes": ([_SHP, C.c_int], _sz),
    "moe_route_bwd_workspace_bytes": ([_SHP], _sz),
    "moe_route": ([_SHP, _p, _p, _p, _p, _p, _p, _p], C.c_int),
    "moe_permute": ([_SHP, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p], C.c_int),
    "moe_permute_noalloc": ([_SHP, _p, _p, _p, _p, _p, _p, _p, _p], C.c_int),
    "moe_grouped_gemm": ([C.c_int, C.c_int, _p, _p, _p, _p, _p, _i32, _i64, _i32, _i32, C.POINTER(MoeGemmRows), _p,
                          _p], C.c_int),
    "moe_grouped_gemm_wgrad": ([_p, _p, _p, _i32, _i64, _i32, _i32, _p, _p], C.c_int),
    "moe_grouped_gemm_grid": ([C.c_int, C.c_int, _p, _p, _p, _p, _p, _i32, _i64, _i32, _i32, C.POINTER(MoeGemmRows),
                               _p, _i32, _p], C.c_int),
    "moe_grouped_gemm_wgrad_grid": ([_p, _p, _p, _i32, _i64, _i32, _i32, _p, _i32, _p], C.c_int),
    "moe_tile_schedule": ([_i32, _p, _i32, _i64, _i32, _i32, _i32, _p, _i64, C.POINTER(_i64)], C.c_int),
    "moe_combine": ([_SHP, _p, _p, _p, _p, _p], C.c_int),
    "moe_combine_bwd": ([_SHP, _p, _p, _p, _p, _p, _p, _p], C.c_int),
    "moe_ffn_fwd": ([_SHP, _p, _p, _p, _p, _p, _p, _p, C.POINTER(MoeSaved), _p, _sz, _p], C.c_int),
    "moe_ffn_bwd": ([_SHP, _p, C.POINTER(MoeSaved), _p, _p, _p, _p, _p, _p, _p, _sz, _p], C.c_int),
    "moe_workspace_bytes_mx": ([_SHP], _sz),
    "moe_ffn_fwd_mx": ([_SHP, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p], C.c_int),
    "moe_grouped_gemm_mx": ([_i32, _p, _p, _i64, _p, _i32, _p, _p, _p, _i32, _i64, _i32, _i32, _p, _p, _p, _p],
                            C.c_int),
    "moe_mx_quantize_rows": ([_p, _i64, _i32, _p, _i32, _i64, _p, _p, _p], C.c_int),
    "moe_mx_quantize_weight": ([_p, _i32, _i32, _i32, _p, _p, _p], C.c_int),
    "moe_route_bwd": ([_SHP, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p], C.c_int),
}


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status}){': ' + detail if detail else ''}")


_lib: C.CDLL | None = None


def lib() -> C.CDLL:
    """The loaded library. Raises if it has not been built: there is no fallback path."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m mixture_experts_ffn_group_amd.build` "
                              "(the MoE FFN has no CPU or PyTorch fallback)")
        h = C.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            f = getattr(h, name)
            f.argtypes = args
            f.restype = res
        _lib = h
    return _lib


def status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where, lib().moe_last_error_detail().decode())


def shape(T: int, emb: int, mlp: int, E: int, k: int) -> MoeShape:
    return MoeShape(T, emb, mlp, E, k)
