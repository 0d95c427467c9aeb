"""Helpers shared by the GPU parity tests (comparison metrics, conversions)."""
import numpy as np
import torch

import workloads

# Tolerance for bf16 outputs against the oracle: relative Frobenius error and
# max absolute error, per output tensor.
REL_FROB = 1e-2
MAX_ABS = 2e-2
# fp32 top-k weights against the oracle's double-evaluated softmax.
W_ABS = 1e-6


def bits(t: torch.Tensor) -> np.ndarray:
    return workloads.bf16_bits(t)


def bf16_values(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return bf16_values(bits(t))
    return t.detach().cpu().numpy()


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    diff = got - ref
    denom = np.linalg.norm(ref)
    rel = np.linalg.norm(diff) / denom if denom > 0 else np.linalg.norm(diff)
    return float(rel), float(np.abs(diff).max() if diff.size else 0.0), float(np.abs(ref).max() if ref.size else 0.0)


def assert_close(got, ref, name: str, rel: float = REL_FROB, abs_: float = MAX_ABS):
    r, a, m = errors(got, ref)
    assert np.isfinite(np.asarray(got, np.float64)).all(), f"{name}: non-finite values"
    assert r <= rel and a <= abs_, f"{name}: rel_frob={r:.3e} (<= {rel}) max_abs={a:.3e} (<= {abs_}) max|ref|={m:.3g}"
    return r, a


def bf16_ulp(v):
    """Unit in the last place of bf16 at |v| (8 significand bits): 2^(floor(log2|v|) - 7); the smallest
    normal's for |v| below it."""
    a = np.maximum(np.abs(np.asarray(v, np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(np.int64) - 7)


def assert_close_bf16_out(got, ref, name: str):
    """A bf16 output against a reference with the same bf16-stored inputs: relF <= 1e-2, and per element
    |G - O| <= max(2e-2, ulp_bf16(O)). Two fp32 accumulations of the same terms in different orders can
    round to adjacent bf16 values, one ulp apart; from |O| >= 4 that ulp (2^-5 and up) is larger than
    2e-2, so no bf16 result could meet the fixed bound there. Below 4 the bound is the fixed 2e-2."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    r, a, m = errors(got, ref)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    bound = np.maximum(MAX_ABS, bf16_ulp(ref))
    worst = float(np.max(np.abs(got - ref) / bound)) if got.size else 0.0
    assert r <= REL_FROB and worst <= 1.0, (f"{name}: rel_frob={r:.3e} (<= {REL_FROB}) max_abs={a:.3e} "
                                            f"worst |G-O|/max(2e-2, ulp(O))={worst:.3f} max|ref|={m:.3g}")
    return r, a


def bf16_ulp_diff(a_bits: np.ndarray, b_bits: np.ndarray) -> int:
    """Largest distance in bf16 units in the last place between two bf16 arrays (same sign assumed near 0)."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7fff), 0x8000 + x)
    return int(np.abs(ordered(a_bits) - ordered(b_bits)).max()) if a_bits.size else 0
