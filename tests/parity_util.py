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


def bf16_ulp_diff(a_bits: np.ndarray, b_bits: np.ndarray) -> int:
    """Largest distance in bf16 units in the last place between two bf16 arrays (same sign assumed near 0)."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7fff), 0x8000 + x)
    return int(np.abs(ordered(a_bits) - ordered(b_bits)).max()) if a_bits.size else 0
