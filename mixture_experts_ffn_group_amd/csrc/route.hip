// Router: logits, top-k and renormalised weights, one workgroup per 64 (or 32) tokens.
//
// Gate and top-k routing come first in the MoE block ("[DRAFT][JAX] Optimize
// MoE block", Flowchart), and the top-k weights are computed on the main
// compute units ("Gemma4 26B MoE on TPU v6e: MaxText layer/model
// optimizations", Commits table, commit 6).
//
// Logit contract (an integer decision hangs on it, so it is fixed exactly):
// logits[t, e] = fp32 fma chain over i = 0..emb-1 of x[t, i] * wr[i, e],
// starting from +0, then one fp32 add of bias[e].
// The chains run on the fp32 matrix cores: v_mfma_f32_32x32x1_2b_f32 has
// K = 1, so each instruction adds exactly one product to each of its 2 x 32 x
// 32 accumulators, and a sequence of them over i is a chain of fp32
// multiply-adds. Measured on the MI355X, every such chain is bitwise equal to
// the sequential fmaf chain (normal, signed-zero and subnormal operands and
// sums alike). Each emb step costs one MFMA per wave: 2048 multiply-adds at
// the fp32 matrix rate (157.3 TFLOP/s), twice the non-packed vector rate.
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

// Output layout of v_mfma_f32_32x32x1_2b_f32 (measured): lane l, register r ->
// block r/16, row ((r%16)/4)*8 + (l/32)*4 + r%4 of that block, column l%32;
// lane l feeds row l%32 (A) and column l%32 (B) of block l/32.
//
// MODE 0 (E <= 128): 64 tokens per workgroup. The two MFMA blocks are tokens
//   0-31 and 32-63; wave w owns experts 32w .. 32w+31.
// MODE 1 (E <= 256): 32 tokens per workgroup. The two blocks are experts
//   64w .. 64w+31 and 64w+32 .. 64w+63 of wave w, for the same 32 tokens.
template <int MODE>
__global__ __launch_bounds__(256) void route_kernel(int64_t T, int emb, int E, int k, const uint16_t* __restrict__ x,
                                                    const float* __restrict__ wr, const float* __restrict__ bias,
                                                    const float* __restrict__ logits_in, int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ topk_w) {
  constexpr int TB = MODE == 0 ? 64 : 32;  // tokens per workgroup
  constexpr int EP = MODE == 0 ? 128 : 256;  // expert columns (logit row stride)
  constexpr int EQ = EP / 64;              // experts per lane in the top-k
  constexpr int TPW = TB / kWaves;         // tokens per wave in the top-k
  static_assert(TB <= 2 * kBK, "the two w buffers must hold the logits of a workgroup's tokens");
  __shared__ __attribute__((aligned(16))) float s_x[2][kBK][TB];
  __shared__ __attribute__((aligned(16))) float s_w[2][kBK][EP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * TB;
  // Logits [TB][EP] go to LDS (into the w buffers, free after the last
  // barrier), so the per-token top-k loop reads them by a runtime index.
  float* const s_l = &s_w[0][0][0];

  if (logits_in) {
    for (int idx = tid; idx < TB * EP; idx += 256) {
      const int tok = idx / EP, e = idx % EP;
      const int64_t t = t0 + tok;
      s_l[idx] = (t < T && e < E) ? logits_in[t * E + e] : 0.0f;
    }
  } else {
    const int tok_a = MODE == 0 ? lane : (lane & 31);  // A operand: this lane's token
    const int exp_b = MODE == 0 ? 32 * wave + (lane & 31) : 64 * wave + lane;  // B operand: its expert
    const bool busy = (MODE == 0 ? 32 : 64) * wave < E;  // wave-uniform
    f32x32_t acc;
#pragma unroll
    for (int r = 0; r < 32; ++r) acc[r] = 0.0f;
    // Slices of kBK emb values are double-buffered: the next slice is loaded
    // into registers while the current one feeds the chains, then written to
    // the other LDS buffer; one barrier per slice.
    constexpr int kXV = TB * kBK / 256;  // x values per thread per slice: 8 or 4
    const int tk = tid / (kBK / kXV), seg = tid % (kBK / kXV);  // x: token tk of the block, kXV values at seg*kXV
    const int64_t tx = t0 + tk;
    const bool vec_w = (E & 3) == 0;
    constexpr int kW4 = kBK * EP / 4 / 256;  // float4 of the w slice per thread
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
        const int idx = (tid + 256 * j) * 4, ii = idx / EP, e = idx % EP;
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
        const int idx = (tid + 256 * j) * 4, ii = idx / EP, e = idx % EP;
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
      if (busy) {  // all operands of the slice first, so the chain runs while the reads land
        float xv[kBK], wv[kBK];
#pragma unroll
        for (int ii = 0; ii < kBK; ++ii) {
          xv[ii] = s_x[b][ii][tok_a];
          wv[ii] = s_w[b][ii][exp_b];
        }
#pragma unroll
        for (int ii = 0; ii < kBK; ++ii) acc = __builtin_amdgcn_mfma_f32_32x32x1f32(xv[ii], wv[ii], acc, 0, 0, 0);
      }
      if (more) store(b ^ 1);  // the other buffer was last read before the previous barrier
      __syncthreads();
      b ^= 1;
    }
    if (busy) {
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        const int blk = r >> 4, rr = r & 15;
        const int row = (rr >> 2) * 8 + (lane >> 5) * 4 + (rr & 3), col = lane & 31;
        const int tok = MODE == 0 ? 32 * blk + row : row;
        const int e = MODE == 0 ? 32 * wave + col : 64 * wave + 32 * blk + col;
        if (e < E) s_l[tok * EP + e] = bias ? acc[r] + bias[e] : acc[r];
      }
    }
  }
  __syncthreads();

  // Top-k per token: k rounds of a wave-wide max over (key(logit), -expert).
  // Picked and padding experts hold candidate 0, which no real expert reaches.
#pragma unroll 1
  for (int tt = 0; tt < TPW; ++tt) {
    const int tok = wave * TPW + tt;
    const int64_t t = t0 + tok;
    if (t >= T) break;  // wave-uniform
    uint64_t cand[EQ];
#pragma unroll
    for (int q = 0; q < EQ; ++q) {
      const int e = lane + 64 * q;
      const float l = s_l[tok * EP + e];
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
  const dim3 block(256);
  if (E <= 128) {
    route_kernel<0><<<dim3((unsigned)((T + 63) / 64)), block, 0, stream>>>(T, emb, E, k, x, wr, bias, logits_in,
                                                                          topk_idx, topk_w);
  } else {
    route_kernel<1><<<dim3((unsigned)((T + 31) / 32)), block, 0, stream>>>(T, emb, E, k, x, wr, bias, logits_in,
                                                                          topk_idx, topk_w);
  }
  return hipGetLastError();
}

}  // namespace moe
