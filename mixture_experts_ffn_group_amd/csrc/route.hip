// Router: logits, top-k and renormalised weights, one workgroup per 64 tokens.
//
// Gate and top-k routing come first in the MoE block ("[DRAFT][JAX] Optimize
// MoE block", Flowchart), and the top-k weights are computed on the main
// compute units ("Gemma4 26B MoE on TPU v6e: MaxText layer/model
// optimizations", Commits table, commit 6).
//
// Logit contract (an integer decision hangs on it, so it is fixed exactly):
// logits[t, e] = fp32 fma chain over i = 0..emb-1 of x[t, i] * wr[i, e],
// starting from +0, then one fp32 add of bias[e]. Each (t, e) chain is one
// lane's register; lanes run experts, the wave runs 16 tokens, so x values are
// LDS broadcasts and wr values are conflict-free LDS reads. The chain is on
// the fp32 vector ALU: its bound is 2*T*emb*E flop at the non-packed fp32 rate.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kWaves = 4;
constexpr int kBK = 32;  // emb slice staged in LDS per step

// Order-preserving key of a logit: larger logit -> larger key. -0 maps like +0;
// NaN maps to 0, below every number.
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f != f) return 0u;
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    uint32_t lo = __shfl_xor((unsigned int)(uint32_t)v, s);
    uint32_t hi = __shfl_xor((unsigned int)(uint32_t)(v >> 32), s);
    uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s);
  return v;
}

// EQ = experts per lane: lane L holds experts L, L + 64, ..., L + 64 (EQ - 1).
// kTPW = tokens per wave: 16 up to 128 experts; 8 beyond, which halves the
// registers of the chains and doubles the number of workgroups.
template <int EQ, int kTPW>
__global__ __launch_bounds__(256) void route_kernel(int64_t T, int emb, int E, int k, const uint16_t* __restrict__ x,
                                                    const float* __restrict__ wr, const float* __restrict__ bias,
                                                    const float* __restrict__ logits_in, int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ topk_w) {
  constexpr int kTB = kTPW * kWaves;  // tokens per workgroup
  static_assert(kTB <= 2 * kBK, "the two w buffers must hold the logits of a workgroup's tokens");
  __shared__ __attribute__((aligned(16))) float s_x[2][kBK][kTB];
  __shared__ __attribute__((aligned(16))) float s_w[2][kBK][64 * EQ];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kTB;
  const int64_t tw = t0 + wave * kTPW;

  float acc[kTPW][EQ];
  if (logits_in) {
#pragma unroll
    for (int tt = 0; tt < kTPW; ++tt)
#pragma unroll
      for (int q = 0; q < EQ; ++q) {
        const int e = lane + 64 * q;
        const int64_t t = tw + tt;
        acc[tt][q] = (t < T && e < E) ? logits_in[t * E + e] : 0.0f;
      }
  } else {
#pragma unroll
    for (int tt = 0; tt < kTPW; ++tt)
#pragma unroll
      for (int q = 0; q < EQ; ++q) acc[tt][q] = 0.0f;
    // Slices of kBK emb values are double-buffered: the next slice is loaded
    // into registers while the current one feeds the FMA chains, then written
    // to the other LDS buffer; one barrier per slice.
    constexpr int kXV = kTB * kBK / 256;  // x values per thread per slice: 8 or 4
    const int tk = tid / (kBK / kXV), seg = tid % (kBK / kXV);  // x: token tk of the block, kXV values at seg*kXV
    const int64_t tx = t0 + tk;
    const bool vec_w = (E & 3) == 0;
    constexpr int kW4 = kBK * 64 * EQ / 4 / 256;  // float4 of the w slice per thread
    u32x4_t xr;
    f32x4_t wr4[kW4];
    auto load = [&](int i0) {
      if (kXV == 8) {
        xr = tx < T ? ld16(x + tx * emb + i0 + seg * 8) : u32x4_t{0u, 0u, 0u, 0u};
      } else {
        const u32x2_t v = tx < T ? *reinterpret_cast<const u32x2_t*>(x + tx * emb + i0 + seg * 4) : u32x2_t{0u, 0u};
        xr = u32x4_t{v[0], v[1], 0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < kW4; ++j) {
        const int idx = (tid + 256 * j) * 4, ii = idx / (64 * EQ), e = idx % (64 * EQ);
        const float* src = wr + (int64_t)(i0 + ii) * E + e;
        if (vec_w && e + 3 < E) {
          wr4[j] = *reinterpret_cast<const f32x4_t*>(src);
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) wr4[j][u] = e + u < E ? src[u] : 0.0f;
        }
      }
    };
    auto store = [&](int b) {
#pragma unroll
      for (int u = 0; u < kXV / 2; ++u) {
        s_x[b][seg * kXV + 2 * u][tk] = bf16_lo(xr[u]);
        s_x[b][seg * kXV + 2 * u + 1][tk] = bf16_hi(xr[u]);
      }
#pragma unroll
      for (int j = 0; j < kW4; ++j) {
        const int idx = (tid + 256 * j) * 4, ii = idx / (64 * EQ), e = idx % (64 * EQ);
        *reinterpret_cast<f32x4_t*>(&s_w[b][ii][e]) = wr4[j];
      }
    };
    load(0);
    store(0);
    __syncthreads();
    int b = 0;
    for (int i0 = 0; i0 < emb; i0 += kBK) {
      const bool more = i0 + kBK < emb;
      if (more) load(i0 + kBK);
#pragma unroll 2
      for (int ii = 0; ii < kBK; ++ii) {
        float xv[kTPW];
        const f32x4_t* px = reinterpret_cast<const f32x4_t*>(&s_x[b][ii][wave * kTPW]);
#pragma unroll
        for (int c = 0; c < kTPW / 4; ++c) {
          const f32x4_t v = px[c];
          xv[4 * c + 0] = v[0];
          xv[4 * c + 1] = v[1];
          xv[4 * c + 2] = v[2];
          xv[4 * c + 3] = v[3];
        }
        float wv[EQ];
#pragma unroll
        for (int q = 0; q < EQ; ++q) wv[q] = s_w[b][ii][lane + 64 * q];
#pragma unroll
        for (int tt = 0; tt < kTPW; ++tt)
#pragma unroll
          for (int q = 0; q < EQ; ++q) acc[tt][q] = __builtin_fmaf(xv[tt], wv[q], acc[tt][q]);
      }
      if (more) store(b ^ 1);  // the other buffer was last read before the previous barrier
      __syncthreads();
      b ^= 1;
    }
    if (bias) {
#pragma unroll
      for (int q = 0; q < EQ; ++q) {
        const int e = lane + 64 * q;
        const float b = e < E ? bias[e] : 0.0f;
#pragma unroll
        for (int tt = 0; tt < kTPW; ++tt) acc[tt][q] = acc[tt][q] + b;
      }
    }
  }

  // The logits go to LDS (into the w buffers: kTB x 64*EQ floats, free after
  // the last barrier), so the per-token loop below reads them by a runtime
  // token index. Each wave reads back only its own tokens.
  float* const s_l = &s_w[0][0][0];
#pragma unroll
  for (int tt = 0; tt < kTPW; ++tt)
#pragma unroll
    for (int q = 0; q < EQ; ++q) s_l[(wave * kTPW + tt) * 64 * EQ + lane + 64 * q] = acc[tt][q];

  // Top-k per token: k rounds of a wave-wide max over (key(logit), -expert).
  // Picked and padding experts hold candidate 0, which no real expert reaches.
#pragma unroll 1
  for (int tt = 0; tt < kTPW; ++tt) {
    const int64_t t = tw + tt;
    if (t >= T) break;  // wave-uniform
    uint64_t cand[EQ];
#pragma unroll
    for (int q = 0; q < EQ; ++q) {
      const int e = lane + 64 * q;
      const float l = s_l[(wave * kTPW + tt) * 64 * EQ + e];
      cand[q] = e < E ? (((uint64_t)order_key(l) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e)) : 0ull;
    }
    int my_e = 0;
    float my_l = 0.0f;
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0ull;
#pragma unroll
      for (int q = 0; q < EQ; ++q) best = cand[q] > best ? cand[q] : best;
      best = wave_max_u64(best);
      const int e = (int)(0xffffffffu - (uint32_t)best);
      const float l = key_value((uint32_t)(best >> 32));
#pragma unroll
      for (int q = 0; q < EQ; ++q)
        if (e == lane + 64 * q) cand[q] = 0ull;
      if (lane == j) {
        my_e = e;
        my_l = l;
      }
    }
    const float l0 = __shfl(my_l, 0);
    const float ex = lane < k ? expf(my_l - l0) : 0.0f;
    const float s = wave_sum(ex);
    if (lane < k) {
      topk_idx[t * k + lane] = my_e;
      topk_w[t * k + lane] = ex / s;
    }
  }
}

}  // namespace

hipError_t launch_route(int64_t T, int emb, int E, int k, const uint16_t* x, const float* wr, const float* bias,
                        const float* logits_in, int32_t* topk_idx, float* topk_w, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int eq = (E + 63) / 64;
  const int tb = (eq <= 2 ? 16 : 8) * kWaves;
  const dim3 grid((unsigned)((T + tb - 1) / tb)), block(256);
  switch (eq) {
    case 1: route_kernel<1, 16><<<grid, block, 0, stream>>>(T, emb, E, k, x, wr, bias, logits_in, topk_idx, topk_w); break;
    case 2: route_kernel<2, 16><<<grid, block, 0, stream>>>(T, emb, E, k, x, wr, bias, logits_in, topk_idx, topk_w); break;
    case 3: route_kernel<3, 8><<<grid, block, 0, stream>>>(T, emb, E, k, x, wr, bias, logits_in, topk_idx, topk_w); break;
    default: route_kernel<4, 8><<<grid, block, 0, stream>>>(T, emb, E, k, x, wr, bias, logits_in, topk_idx, topk_w); break;
  }
  return hipGetLastError();
}

}  // namespace moe
