"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and host-side validation rejects bad arguments before any
HIP call is made."""
import ctypes as C
import os
import re

import pytest

from mixture_experts_ffn_group_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ffn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from mixture_experts_ffn_group_amd import build
        build.build()
    return _lib.lib()


def test_header_declares_the_hot_path_entry_points():
    names = _declared()
    for n in ("moe_route", "moe_permute", "moe_grouped_gemm", "moe_grouped_gemm_wgrad", "moe_combine",
              "moe_combine_bwd", "moe_ffn_fwd", "moe_ffn_bwd"):
        assert n in names


def test_every_declared_symbol_is_exported_and_bound(lib):
    for n in _declared():
        assert hasattr(lib, n), f"{n} not exported"
        assert n in _lib.SIGNATURES, f"{n} has no ctypes signature"
    assert set(_lib.SIGNATURES) == set(_declared())


def test_status_strings(lib):
    for s in range(7):
        assert _lib.status_str(s)
    assert lib.moe_version().decode().endswith("gfx950")


def _shape(T=64, emb=128, mlp=256, E=8, k=2):
    return _lib.shape(T, emb, mlp, E, k)


@pytest.mark.parametrize("kw,status", [
    (dict(), _lib.MOE_OK),
    (dict(T=0), _lib.MOE_OK),
    (dict(T=-1), _lib.MOE_ERR_SHAPE),
    (dict(k=9), _lib.MOE_ERR_SHAPE),
    (dict(E=300, k=8), _lib.MOE_ERR_UNSUPPORTED),
    (dict(E=100, k=65), _lib.MOE_ERR_UNSUPPORTED),
    (dict(emb=96), _lib.MOE_ERR_UNSUPPORTED),
    (dict(mlp=100), _lib.MOE_ERR_UNSUPPORTED),
    (dict(T=1 << 30, k=4, E=8), _lib.MOE_ERR_UNSUPPORTED),
    (dict(T=1 << 20, emb=2048, k=1, E=8), _lib.MOE_ERR_UNSUPPORTED),  # T*emb = 2^31
    (dict(T=32768, emb=2048, mlp=768, E=128, k=8), _lib.MOE_OK),
    (dict(T=8192, emb=7168, mlp=2048, E=256, k=8), _lib.MOE_OK),
])
def test_query_support(lib, kw, status):
    s = _shape(**kw)
    assert lib.moe_query_support(C.byref(s)) == status
    if status != _lib.MOE_OK:
        assert lib.moe_last_error_detail().decode()


def test_workspace_sizes(lib):
    s = _shape(T=32768, emb=2048, mlp=768, E=128, k=8)
    fwd = lib.moe_workspace_bytes(C.byref(s), 0)
    bwd = lib.moe_workspace_bytes(C.byref(s), 1)
    S = 32768 * 8
    assert fwd >= S * 2048 * 2 * 2 + S * 768 * 2  # xs, o, a
    assert bwd >= S * 2048 * 2 * 2 + S * 1536 * 2  # do, dxs, dh
    assert lib.moe_permute_workspace_bytes(C.byref(s)) >= 512 * 128 * 12
    bad = _shape(k=20)
    assert lib.moe_workspace_bytes(C.byref(bad), 0) == 0


def test_validation_precedes_any_launch(lib):
    """Every one of these fails in host validation, so it runs without a GPU."""
    s = _shape()
    fake = C.c_void_p(0x1000)          # aligned, never dereferenced
    odd = C.c_void_p(0x1001)           # misaligned
    nul = None
    assert lib.moe_route(C.byref(s), nul, fake, nul, nul, fake, fake, nul) == _lib.MOE_ERR_NULL
    assert lib.moe_route(C.byref(s), odd, fake, nul, nul, fake, fake, nul) == _lib.MOE_ERR_ALIGN
    assert lib.moe_route(C.byref(s), fake, fake, nul, fake, fake, fake, nul) == _lib.MOE_ERR_SHAPE  # x with logits
    assert lib.moe_permute(C.byref(s), fake, fake, fake, fake, fake, fake, fake, fake, 0, nul) == \
        _lib.MOE_ERR_WORKSPACE
    assert lib.moe_permute(C.byref(s), fake, fake, fake, fake, fake, fake, fake, nul, 1 << 20, nul) == \
        _lib.MOE_ERR_NULL
    # index-only permute: xs and x may be NULL, the index outputs may not
    assert lib.moe_permute(C.byref(s), nul, fake, fake, fake, nul, fake, nul, fake, 0, nul) == _lib.MOE_ERR_NULL
    assert lib.moe_permute(C.byref(s), nul, fake, fake, fake, fake, fake, nul, fake, 0, nul) == \
        _lib.MOE_ERR_WORKSPACE
    # grouped GEMM: bad op, wrong epilogue/op pairs, K not a multiple of 64, N not a multiple of 8
    assert lib.moe_grouped_gemm(7, 0, fake, fake, nul, nul, fake, 4, 128, 64, 64, None, fake, nul) == _lib.MOE_ERR_SHAPE
    assert lib.moe_grouped_gemm(1, 1, fake, fake, nul, nul, fake, 4, 128, 64, 64, None, fake, nul) == \
        _lib.MOE_ERR_UNSUPPORTED
    assert lib.moe_grouped_gemm(0, 2, fake, fake, fake, nul, fake, 4, 128, 64, 64, None, fake, nul) == \
        _lib.MOE_ERR_UNSUPPORTED
    assert lib.moe_grouped_gemm(0, 0, fake, fake, nul, nul, fake, 4, 128, 96, 64, None, fake, nul) == \
        _lib.MOE_ERR_UNSUPPORTED
    assert lib.moe_grouped_gemm(0, 0, fake, fake, nul, nul, fake, 4, 128, 64, 60, None, fake, nul) == \
        _lib.MOE_ERR_UNSUPPORTED
    assert lib.moe_grouped_gemm(1, 2, fake, fake, nul, nul, fake, 4, 128, 64, 64, None, fake, nul) == _lib.MOE_ERR_NULL
    assert lib.moe_grouped_gemm(0, 0, fake, fake, nul, nul, fake, 300, 128, 64, 64, None, fake, nul) == \
        _lib.MOE_ERR_UNSUPPORTED
    assert lib.moe_grouped_gemm_wgrad(fake, fake, fake, 4, 128, 12, 64, fake, nul) == _lib.MOE_ERR_UNSUPPORTED
    assert lib.moe_grouped_gemm_wgrad(fake, fake, nul, 4, 128, 64, 64, fake, nul) == _lib.MOE_ERR_NULL
    assert lib.moe_combine(C.byref(s), fake, fake, odd, fake, nul) == _lib.MOE_ERR_ALIGN
    assert lib.moe_combine_bwd(C.byref(s), fake, nul, fake, nul, fake, nul, nul) == _lib.MOE_ERR_NULL
    # router backward: dwr required, dtopk_w required with tokens, workspace size checked
    assert lib.moe_route_bwd(C.byref(s), fake, fake, fake, fake, fake, fake, fake, nul, nul, nul, fake, 1 << 20,
                             nul) == _lib.MOE_ERR_NULL
    assert lib.moe_route_bwd(C.byref(s), fake, fake, fake, fake, nul, fake, fake, fake, nul, nul, fake, 1 << 20,
                             nul) == _lib.MOE_ERR_NULL
    assert lib.moe_route_bwd(C.byref(s), fake, fake, fake, fake, fake, fake, fake, fake, nul, nul, fake, 16,
                             nul) == _lib.MOE_ERR_WORKSPACE
    assert lib.moe_route_bwd_workspace_bytes(C.byref(s)) >= 3 * 64 * 2 * 4 + 2 * 8 * 128 * 4
    # layer calls: workspace too small, missing saved set
    assert lib.moe_ffn_fwd(C.byref(s), fake, fake, nul, nul, fake, fake, fake, None, fake, 16, nul) == \
        _lib.MOE_ERR_WORKSPACE
    assert lib.moe_ffn_bwd(C.byref(s), fake, None, fake, fake, fake, fake, fake, fake, fake, 1 << 30, nul) == \
        _lib.MOE_ERR_NULL
    partial = _lib.MoeSaved(*([0x1000] * 9 + [0]))
    assert lib.moe_ffn_fwd(C.byref(s), fake, fake, nul, nul, fake, fake, fake, C.byref(partial), fake, 1 << 40,
                           nul) == _lib.MOE_ERR_NULL
    # MXFP8 quantizers: K must be a multiple of 64, pointers present, gather divisor positive
    assert lib.moe_mx_quantize_rows(fake, 8, 96, nul, 1, 8, fake, fake, nul) == _lib.MOE_ERR_UNSUPPORTED
    assert lib.moe_mx_quantize_rows(nul, 8, 128, nul, 1, 8, fake, fake, nul) == _lib.MOE_ERR_NULL
    assert lib.moe_mx_quantize_rows(fake, 8, 128, fake, 0, 8, fake, fake, nul) == _lib.MOE_ERR_SHAPE
    assert lib.moe_mx_quantize_rows(fake, 8, 128, nul, 1, 0, nul, nul, nul) == _lib.MOE_OK  # no rows: no-op
    assert lib.moe_mx_quantize_weight(fake, 2, 96, 64, fake, fake, nul) == _lib.MOE_ERR_UNSUPPORTED
    assert lib.moe_mx_quantize_weight(fake, 2, 128, 64, nul, fake, nul) == _lib.MOE_ERR_NULL
    # MXFP8 layer forward: workspace query, NULL inputs, small workspace
    assert lib.moe_workspace_bytes_mx(C.byref(s)) > 0
    assert lib.moe_ffn_fwd_mx(C.byref(s), nul, fake, nul, nul, fake, fake, fake, fake, fake, fake, 1 << 40,
                              nul) == _lib.MOE_ERR_NULL
    assert lib.moe_ffn_fwd_mx(C.byref(s), fake, fake, nul, nul, fake, fake, fake, fake, fake, fake, 16,
                              nul) == _lib.MOE_ERR_WORKSPACE
    # a saved set without h: the backward recomputes it and needs the larger workspace
    ws1, ws2 = lib.moe_workspace_bytes(C.byref(s), 1), lib.moe_workspace_bytes(C.byref(s), 2)
    assert ws2 >= ws1 + s.T * s.k * 2 * s.mlp * 4
    no_h = _lib.MoeSaved(*([0x1000] * 7 + [0] + [0x1000] * 2))
    assert lib.moe_ffn_bwd(C.byref(s), fake, C.byref(no_h), fake, fake, fake, fake, fake, fake, fake, ws1,
                           nul) == _lib.MOE_ERR_WORKSPACE


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError, match="no CPU or PyTorch fallback"):
        _lib.lib()
