"""MXFP8 quantizers and grouped GEMM on the GPU against the oracle (reading R8 of the oracle).

Quantization decides integers (codes and scales) from exact operations (a maximum, a power-of-two
rescaling, a rounding), so the device and the oracle must agree bit for bit."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_group_amd as moe
import oracle
from parity_util import bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16)


def _oracle_scales_to_device_layout(sc):
    """oracle scales [M, K/32] -> device layout [K/64, M, 4] (bytes 2, 3 zero)."""
    M, nb = sc.shape
    out = np.zeros((nb // 2, M, 4), np.uint8)
    out[:, :, 0] = sc[:, 0::2].T
    out[:, :, 1] = sc[:, 1::2].T
    return out


def _rows_case(M, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)) * np.exp(rng.uniform(-20, 20, (M, 1)))
    x[0, :32] = 0.0
    x[0, 40] = -0.0
    x[1, :] = np.where(rng.random(K) < 0.5, 1e-30, -3e30)  # far-apart magnitudes in one row
    x[2, 64:128] = 448.0 * 2.0 ** 5                          # exactly representable, saturating boundary
    x[3, :] = rng.choice([-1.0, 1.0], K) * 2.0 ** rng.integers(-20, 20, K)
    return _bf16(x)


@pytest.mark.parametrize("M,K,seed", [(5, 64, 0), (37, 192, 1), (300, 2048, 2), (129, 7168, 3)])
def test_mx_quantize_rows_bit_exact(M, K, seed):
    x = _rows_case(M, K, seed)
    codes, scales = moe.mx_quantize_rows(x.to(DEV))
    rc, rs = oracle.mx_quantize(bits(x))
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy(), _oracle_scales_to_device_layout(rs))


def test_mx_quantize_rows_gather_through_sorted_slot():
    T, K, k = 200, 256, 4
    rng = np.random.default_rng(7)
    x = _bf16(rng.standard_normal((T, K)))
    slots = rng.permutation(T * k).astype(np.int32)  # row r comes from token slots[r] // k
    codes, scales = moe.mx_quantize_rows(x.to(DEV), torch.from_numpy(slots).to(DEV), k)
    rc, rs = oracle.mx_quantize(bits(x)[slots // k])
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy(), _oracle_scales_to_device_layout(rs))


@pytest.mark.parametrize("E,K,N,seed", [(3, 64, 40, 0), (4, 192, 72, 1), (2, 2048, 256, 2)])
def test_mx_quantize_weight_bit_exact(E, K, N, seed):
    rng = np.random.default_rng(seed)
    w = _bf16(rng.standard_normal((E, K, N)) * np.exp(rng.uniform(-10, 10, (E, 1, N))))
    codes, scales = moe.mx_quantize_weight(w.to(DEV))
    wt = np.ascontiguousarray(np.transpose(bits(w), (0, 2, 1)))  # [E, N, K]
    for e in range(E):
        rc, rs = oracle.mx_quantize(wt[e])
        assert np.array_equal(codes[e].cpu().numpy(), rc)
        assert np.array_equal(scales[e].cpu().numpy(), _oracle_scales_to_device_layout(rs))
