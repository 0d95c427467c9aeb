"""Seeded synthetic inputs for the sparse-MoE expert-FFN workloads.

This module only draws random tensors with the shapes, distributions and
routing structure of the workloads. It does no MoE arithmetic. The HIP path
and the CPU oracle both take their inputs from here, so they see the same
bits.

Workloads (shapes from the pages' model settings, sizes per device):

* ``tiny``: T=64, emb=128, mlp=256, E=8, top-2. Every stage finishes on the
  oracle in well under a second.
* ``mid_skewed``: T=4096, emb=1024, mlp=512, E=32, top-4. Router bias +2.0
  on experts 0..3 gives a skewed load. Bias -inf on the last expert keeps it
  empty, which exercises zero-size groups.
* ``gemma4_class``: T=32768 (seq 16384 x batch 2), emb=2048, mlp=768,
  E=128, top-8. This is one device's share of the Gemma4-26B-A4B step in
  "MoE: fused TensorCore Pallas permute/combine kernels and split-expert wi
  layout for TPU v6e" (Context), which uses 128 experts, top-8, seq 16k and
  per-device batch 2.
* ``sweep_zipf_T{1024,2048,4096,8192}``: E=128, top-8, emb=2048, mlp=768.
  The router logits are given directly as log p_e + Gumbel noise, with
  p_e proportional to (e+1)^-1.1. Gumbel-top-k then samples k distinct
  experts from the Zipf(1.1) law, so the expert load follows it up to the
  cap of one pick per token. The token counts mirror the m sweep in
  "Fused MoE Kernel integration and optimization - #3388" (Description).
* ``deepseek_v3_shape``: T=8192, emb=7168, mlp=2048, E=256, top-8,
  weights ~ N(0, 0.006), plus an upstream gradient dy ~ N(0, 1) for the
  backward.

Distributions: x ~ N(0,1) rounded to bf16 (round-to-nearest-even, as torch
does); router weight Wr ~ N(0, 0.02) fp32; wi [E, emb, 2*mlp] and
wo [E, mlp, emb] ~ N(0, sigma) rounded to bf16. sigma is a standard
deviation.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

SWEEP_T = (1024, 2048, 4096, 8192)


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    emb: int
    mlp: int
    E: int
    k: int
    sigma_w: float = 0.02
    seed: int = 0
    hot_experts: int = 0          # experts 0..hot-1 get +hot_bias on the router logits
    hot_bias: float = 0.0
    empty_last: bool = False      # last expert gets -inf router bias (never chosen)
    zipf_s: float = 0.0           # > 0: logits are given as Gumbel-Zipf draws, no router matmul
    backward: bool = False
    extra: dict = field(default_factory=dict)

    @property
    def S(self) -> int:
        return self.T * self.k


def _workloads() -> dict[str, Workload]:
    w = {
        "tiny": Workload("tiny", 64, 128, 256, 8, 2, seed=1000),
        "mid_skewed": Workload("mid_skewed", 4096, 1024, 512, 32, 4, seed=2000,
                               hot_experts=4, hot_bias=2.0, empty_last=True),
        "gemma4_class": Workload("gemma4_class", 32768, 2048, 768, 128, 8, seed=3000),
        "deepseek_v3_shape": Workload("deepseek_v3_shape", 8192, 7168, 2048, 256, 8,
                                      sigma_w=0.006, seed=5000, backward=True),
    }
    for i, t in enumerate(SWEEP_T):
        n = f"sweep_zipf_T{t}"
        w[n] = Workload(n, t, 2048, 768, 128, 8, seed=4000 + 100 * i, zipf_s=1.1)
    return w


WORKLOADS = _workloads()


def custom(T: int, emb: int, mlp: int, E: int, k: int, seed: int, sigma_w: float = 0.02,
           **kw) -> Workload:
    """A workload of arbitrary shape (tests use these for edge cases)."""
    return Workload(f"custom_T{T}_emb{emb}_mlp{mlp}_E{E}_k{k}", T, emb, mlp, E, k,
                    sigma_w=sigma_w, seed=seed, **kw)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal_bf16(shape, sigma: float, device, seed: int, chunk_dim0: bool = False) -> torch.Tensor:
    """N(0, sigma) rounded to bf16. With chunk_dim0, draw one leading slice at a
    time so the fp32 temporary stays one slice big."""
    g = _gen(device, seed)
    if not chunk_dim0:
        return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * sigma).to(torch.bfloat16)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    for i in range(shape[0]):
        out[i] = (torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32) * sigma).to(torch.bfloat16)
    return out


def make_inputs(wl: Workload | str, device: str | torch.device = "cpu", with_weights: bool = True) -> dict:
    """Draw the workload's inputs on ``device``.

    Returns a dict with
      x [T, emb] bf16, wr [emb, E] fp32 or None, bias [E] fp32 or None,
      logits_in [T, E] fp32 or None, wi [E, emb, 2mlp] bf16, wo [E, mlp, emb] bf16,
      dy [T, emb] bf16 (backward workloads only, else None).
    Seeds: workload seed + {x: 1, wr: 2, wi: 3, wo: 4, dy: 5, gumbel: 6}.
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    dev = torch.device(device)
    s = wl.seed
    out: dict = {"workload": wl}
    out["x"] = _normal_bf16((wl.T, wl.emb), 1.0, dev, s + 1)
    if wl.zipf_s > 0:
        g = _gen(dev, s + 6)
        u = torch.rand((wl.T, wl.E), generator=g, device=dev, dtype=torch.float64)
        u = u.clamp_(min=1e-300)
        gumbel = -torch.log(-torch.log(u))
        logp = -wl.zipf_s * torch.log(torch.arange(1, wl.E + 1, device=dev, dtype=torch.float64))
        out["logits_in"] = (logp[None, :] + gumbel).to(torch.float32)
        out["wr"] = None
        out["bias"] = None
    else:
        g = _gen(dev, s + 2)
        out["wr"] = torch.randn((wl.emb, wl.E), generator=g, device=dev, dtype=torch.float32) * 0.02
        out["logits_in"] = None
        if wl.hot_experts or wl.empty_last:
            b = torch.zeros(wl.E, dtype=torch.float32, device=dev)
            b[: wl.hot_experts] = wl.hot_bias
            if wl.empty_last:
                b[wl.E - 1] = -math.inf
            out["bias"] = b
        else:
            out["bias"] = None
    if with_weights:
        big = wl.E * wl.emb * wl.mlp > (1 << 28)
        out["wi"] = _normal_bf16((wl.E, wl.emb, 2 * wl.mlp), wl.sigma_w, dev, s + 3, chunk_dim0=big)
        out["wo"] = _normal_bf16((wl.E, wl.mlp, wl.emb), wl.sigma_w, dev, s + 4, chunk_dim0=big)
    out["dy"] = _normal_bf16((wl.T, wl.emb), 1.0, dev, s + 5) if wl.backward else None
    return out


def bf16_bits(t: torch.Tensor):
    """Host numpy view of a bf16 tensor's raw 16-bit patterns (uint16)."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")
