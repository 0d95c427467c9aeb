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

// Direct global->LDS copy, 16 bytes per lane: lane L's 16 bytes at sbase + voff
// land at LDS byte address lds + 16 L (global_load_lds_dwordx4, M0 = lds).
// Issued from inline asm, so the kernel counts vmcnt itself before the barrier
// that publishes a stage.
__device__ __forceinline__ void g2lds16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(lds) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm_n() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
template <class T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const T*)(((uint64_t)hi << 32) | lo);
}

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

// Wave-wide reductions on DPP lane moves (GFX9 controls): the two quad
// permutations and row rotations by 4 and 8 reduce each 16-lane row, and the
// row broadcasts of lanes 15 and 31 carry the rows into lane 63, which is
// then read as a scalar. A few cycles per step, where a cross-lane shuffle
// through the LDS crossbar waits on its result every step.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROW_MASK, 0xf, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xb1, 0xf>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4e, 0xf>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x124, 0xf>(v));  // row_ror:4
  v = max(v, dpp_u32<0x128, 0xf>(v));  // row_ror:8
  v = max(v, dpp_u32<0x142, 0xa>(v));  // row_bcast:15 into rows 1, 3
  v = max(v, dpp_u32<0x143, 0xc>(v));  // row_bcast:31 into rows 2, 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ float wave_sum(float v) {
  auto add = [](float a, uint32_t b) { return a + __uint_as_float(b); };
  v = add(v, dpp_u32<0xb1, 0xf>(__float_as_uint(v)));
  v = add(v, dpp_u32<0x4e, 0xf>(__float_as_uint(v)));
  v = add(v, dpp_u32<0x124, 0xf>(__float_as_uint(v)));
  v = add(v, dpp_u32<0x128, 0xf>(__float_as_uint(v)));
  // rows 1 and 3 add the previous row's total; row 3 then adds rows 0 + 1 (carried by lane 31)
  const uint32_t b15 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), 0x142, 0xa, 0xf, false);
  v = v + __uint_as_float(b15);
  const uint32_t b31 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), 0x143, 0xc, 0xf, false);
  v = v + __uint_as_float(b31);
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 63));
}

// 16-lane (row) reductions with symmetric exchanges: quad swaps, then the
// half-row and row mirrors. Every lane combines its value with a partner's
// in the same association, so all 16 lanes end with the identical result.
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xb1, 0xf>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4e, 0xf>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x141, 0xf>(v));  // row_half_mirror
  v = max(v, dpp_u32<0x140, 0xf>(v));  // row_mirror
  return v;
}
__device__ __forceinline__ float row_sum(float v) {
  v = v + __uint_as_float(dpp_u32<0xb1, 0xf>(__float_as_uint(v)));
  v = v + __uint_as_float(dpp_u32<0x4e, 0xf>(__float_as_uint(v)));
  v = v + __uint_as_float(dpp_u32<0x141, 0xf>(__float_as_uint(v)));
  v = v + __uint_as_float(dpp_u32<0x140, 0xf>(__float_as_uint(v)));
  return v;
}

// Row maximum with each lane move feeding the max directly (every lane of a
// row has a source under these four patterns, so no lane keeps an old value).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t v) {
  return max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ uint32_t row_max_fused(uint32_t v) {
  v = dpp_max_step<0xb1>(v);   // quad_perm [1,0,3,2]
  v = dpp_max_step<0x4e>(v);   // quad_perm [2,3,0,1]
  v = dpp_max_step<0x141>(v);  // row_half_mirror
  v = dpp_max_step<0x140>(v);  // row_mirror
  return v;
}

// Batcher's odd-even merge sort network on N = 2^m elements (Knuth, TAOCP
// vol. 3, 5.3.4), as a compile-time list of compare-exchange pairs.
struct CxPair {
  int a, b;
};
template <int N>
struct OddEvenMergeNet {
  CxPair p[N * N] = {};
  int n = 0;
  constexpr OddEvenMergeNet() {
    for (int pp = 1; pp < N; pp <<= 1)
      for (int kk = pp; kk >= 1; kk >>= 1)
        for (int j = kk % pp; j + kk < N; j += 2 * kk)
          for (int i = 0; i < kk && i + j + kk < N; ++i)
            if ((i + j) / (2 * pp) == (i + j + kk) / (2 * pp)) p[n++] = CxPair{i + j, i + j + kk};
  }
};
template <int N>
__device__ __forceinline__ void sort_desc(uint64_t (&c)[N]) {
  constexpr OddEvenMergeNet<N> net{};
#pragma unroll
  for (int q = 0; q < net.n; ++q) {
    uint64_t& a = c[net.p[q].a];
    uint64_t& b = c[net.p[q].b];
    const bool sw = b > a;
    const uint64_t hi = sw ? b : a, lo = sw ? a : b;
    a = hi;
    b = lo;
  }
}

// Top-k for k <= 16, four tokens at a time per wave: token g of the group on
// lanes 16g..16g+15, lane r holding experts r + 16q as 64-bit candidates
// (key(logit), ~expert), sorted once in descending order. Each round takes
// the largest (key, -expert) of the row: one row maximum of the lanes' head
// keys; when some row has more than one lane holding its maximum key (equal
// logits, or only NaN and padding left at key 0), a second row maximum over
// those lanes' low words picks the lowest expert. The winning lane parks the
// expert in the token's logit row (already read into registers) and pops its
// head. Same picks as taking the largest (key, -expert) of the remaining
// candidates each round.
template <int TB, int EP>
__device__ __forceinline__ void route_topk16(float* s_l, int64_t T, int64_t t0, int E, int k,
                                             int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  constexpr int EQ = EP / 16;       // experts per lane
  constexpr int TPW = TB / kWaves;  // tokens per wave (a multiple of 8)
  constexpr int NG = 2;             // 4-token groups in flight per wave (independent chains)
  static_assert(TPW % (4 * NG) == 0, "whole group pairs per wave");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r = lane & 15;
#pragma unroll 1
  for (int t8 = 0; t8 < TPW; t8 += 4 * NG) {
    if (t0 + wave * TPW + t8 >= T) break;  // wave-uniform: no token of the groups exists
    float* row[NG];
    int64_t t[NG];
    uint64_t cand[NG][EQ];
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      const int tok = wave * TPW + t8 + 4 * u + g;
      t[u] = t0 + tok;
      row[u] = s_l + tok * EP;
#pragma unroll
      for (int q = 0; q < EQ; ++q) {
        const int e = r + 16 * q;
        const float l = row[u][e];
        cand[u][q] = e < E ? (((uint64_t)order_key(l) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e)) : 0ull;
      }
    }
#pragma unroll
    for (int u = 0; u < NG; ++u) sort_desc(cand[u]);
    float my_l[NG] = {}, l0[NG] = {};
    for (int j = 0; j < k; ++j) {
#pragma unroll
      for (int u = 0; u < NG; ++u) {
        const uint32_t hk = (uint32_t)(cand[u][0] >> 32), lo = (uint32_t)cand[u][0];
        const uint32_t key = row_max_fused(hk);
        bool win = hk == key;
        if (__builtin_popcountll(__ballot(win)) > 4) {  // wave-uniform: each of the 4 rows has a holder
          const uint32_t low = row_max_fused(win ? lo : 0u);
          win = win && lo == low;
        }
        const float l = key_value(key);
        if (j == 0) l0[u] = l;
        if (r == j) my_l[u] = l;
        if (win) row[u][j] = __int_as_float(min(max((int)(0xffffffffu - lo), 0), E - 1));
        // pop: the winner takes each neighbour through a bitwise select (v_bfi_b32) on an opaque
        // all-ones mask, so the shift is not rewritten as a candidate index chosen at run time
        uint32_t m = 0u - (uint32_t)win;
        asm volatile("" : "+v"(m));
#pragma unroll
        for (int q = 0; q < EQ; ++q) {
          const uint64_t nx = q + 1 < EQ ? cand[u][q + 1] : 0ull;
          const uint32_t h = ((uint32_t)(nx >> 32) & m) | ((uint32_t)(cand[u][q] >> 32) & ~m);
          const uint32_t l32 = ((uint32_t)nx & m) | ((uint32_t)cand[u][q] & ~m);
          cand[u][q] = ((uint64_t)h << 32) | l32;
        }
      }
    }
    // lane r reads back pick r, which another lane of the wave may have written (the wave's
    // LDS accesses run in order; the fence keeps the compiler from reusing lane r's earlier
    // read of that address, its logit)
    wave_lds_fence();
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      const float ex = r < k ? expf(my_l[u] - l0[u]) : 0.0f;
      const float sum = row_sum(ex);
      if (r < k && t[u] < T) {
        topk_idx[t[u] * k + r] = __float_as_int(row[u][r]);
        topk_w[t[u] * k + r] = ex / sum;
      }
    }
  }
}

// Top-k of the logits of a workgroup's TB tokens, held in LDS as [TB][EP]:
// one token per wave at a time (any k <= 64).
template <int TB, int EP>
__device__ __forceinline__ void route_topk(const float* s_l, int64_t T, int64_t t0, int E, int k,
                                           int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  constexpr int EQ = EP / 64;     // experts per lane
  constexpr int TPW = TB / kWaves;  // tokens per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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
      // the wave's largest (key, -expert): the largest key, then the lowest expert holding it
      const uint32_t key = wave_max_u32((uint32_t)(best >> 32));
      const uint32_t low = wave_max_u32((uint32_t)(best >> 32) == key ? (uint32_t)best : 0u);
      const int e = min(max((int)(0xffffffffu - low), 0), E - 1);
      const float l = key_value(key);
#pragma unroll
      for (int q = 0; q < EQ; ++q)
        if (e == lane + 64 * q) cand[q] = 0ull;
      if (lane == j) {
        my_e = e;
        my_l = l;
      }
    }
    const float l0 = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(my_l), 0));
    const float ex = lane < k ? expf(my_l - l0) : 0.0f;
    const float s = wave_sum(ex);
    if (lane < k) {
      topk_idx[t * k + lane] = my_e;
      topk_w[t * k + lane] = ex / s;
    }
  }
}

// Bias of the experts a lane's accumulators hold: MODE 0, expert 32*wave + lane%32 for both
// blocks; MODE 1, experts 64*wave + 32*blk + lane%32. Loaded together (one round trip); a load per
// accumulator at the logit store was waited one at a time.
template <int MODE>
__device__ __forceinline__ void lane_bias(const float* bias, int E, int wave, int lane, float (&bv)[2]) {
  bv[0] = bv[1] = 0.0f;
  if (!bias) return;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int e = MODE == 0 ? 32 * wave + (lane & 31) : 64 * wave + 32 * b + (lane & 31);
    if (e < E) bv[b] = bias[e];
  }
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
      float bv[2];
      lane_bias<MODE>(bias, E, wave, lane, bv);
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        const int blk = r >> 4, rr = r & 15;
        const int row = (rr >> 2) * 8 + (lane >> 5) * 4 + (rr & 3), col = lane & 31;
        const int tok = MODE == 0 ? 32 * blk + row : row;
        const int e = MODE == 0 ? 32 * wave + col : 64 * wave + 32 * blk + col;
        if (e < E) s_l[tok * EP + e] = bias ? acc[r] + bv[blk] : acc[r];
      }
    }
  }
  __syncthreads();

  if (k <= 16) route_topk16<TB, EP>(s_l, T, t0, E, k, topk_idx, topk_w);
  else route_topk<TB, EP>(s_l, T, t0, E, k, topk_idx, topk_w);
}


// The same logits with the operands copied global -> LDS by direct loads
// (global_load_lds_dwordx4) into a ring of NS stages, NS slices ahead of the
// one multiplied, so the latency of x (read once, from HBM) is covered
// by several slices of MFMAs rather than one. The x slice keeps its bf16 bits
// in LDS ([TB tokens][32] with 64-byte rows, 16-byte chunk c of token t at
// chunk c ^ ((t >> 2) & 3)) and is widened to fp32 (exact) as it is read;
// the Wr slice is [32][EP] fp32, as Wr is laid out. Each slice's operands
// are read into registers during the previous slice's MFMAs. Needs
// E % 4 == 0: a 16-byte copy of Wr holds four experts of one row.
template <int MODE>
__global__ __launch_bounds__(256) void route_ring_kernel(int64_t T, int emb, int E, int k,
                                                         const uint16_t* __restrict__ x, const float* __restrict__ wr,
                                                         const float* __restrict__ bias, int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w) {
  constexpr int TB = MODE == 0 ? 64 : 32;
  constexpr int EP = MODE == 0 ? 128 : 256;
  constexpr int NS = MODE == 0 ? 3 : 4;  // two workgroups per CU in MODE 0, one in MODE 1
  constexpr int kXS = TB * kBK * 2;      // x stage: 4 KB / 2 KB
  constexpr int kWS = kBK * EP * 4;      // Wr stage: 16 KB / 32 KB
  constexpr int kWI = kWS / 1024 / kWaves;  // 1 KB Wr copies per wave per slice: 4 / 8
  constexpr int nL = 1 + kWI;            // copies per wave per slice
  static_assert(NS * (kXS + kWS) >= TB * EP * 4, "the logits reuse the ring");
  __shared__ __attribute__((aligned(16))) uint8_t s_ring[NS * (kXS + kWS)];
  uint8_t* const s_xr = s_ring;              // NS x stages
  uint8_t* const s_wr = s_ring + NS * kXS;   // NS Wr stages
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int64_t t0 = (int64_t)blockIdx.x * TB;
  const int ns = emb / kBK;  // even: emb % 64 == 0

  // Per-lane copy offsets. x: MODE 0 wave w copies tokens 16w..16w+15 (1 KB),
  // MODE 1 tokens 8w..8w+7 (512 B, lanes 0-31); lane L -> token, physical
  // chunk L % 4 holding logical chunk (L % 4) ^ ((token >> 2) & 3). Tokens
  // past T read the last token (their logits are never used).
  const int xtok = (MODE == 0 ? 16 : 8) * wave + (lane >> 2);
  const int xlc = (lane & 3) ^ ((xtok >> 2) & 3);
  const uint16_t* const xbase = x + t0 * emb;
  const uint32_t xoff = (uint32_t)(((int64_t)min<int64_t>(xtok, T - 1 - t0) * emb + 8 * xlc) * 2);
  // Wr: copy j of wave w is 1 KB of the [32][EP] slice at byte (w * kWI + j) * 1024;
  // experts past E read expert 0 (never used).
  uint32_t woff[kWI];
#pragma unroll
  for (int j = 0; j < kWI; ++j) {
    const int byte = (wave * kWI + j) * 1024 + lane * 16;
    const int row = byte / (EP * 4), e = (byte % (EP * 4)) / 4;
    woff[j] = (uint32_t)((row * E + (e < E ? e : 0)) * 4);
  }
  const uint32_t lds_x = lds_addr(s_xr) + wave_u * (MODE == 0 ? 1024 : 512);
  const uint32_t lds_w = lds_addr(s_wr) + wave_u * kWI * 1024;
  auto issue = [&](int sl, int st) {  // slice sl's copies into stage st
    const uint16_t* xs = uniform_ptr(xbase + sl * kBK);
    if (MODE == 0 || lane < 32) g2lds16(xs, xoff, lds_x + st * kXS);
    const float* ws = uniform_ptr(wr + (int64_t)sl * kBK * E);
#pragma unroll
    for (int j = 0; j < kWI; ++j) g2lds16(ws, woff[j], lds_w + st * kWS + j * 1024);
  };

  const int tok_a = MODE == 0 ? lane : (lane & 31);  // A operand: this lane's token
  const int exp_b = MODE == 0 ? 32 * wave + (lane & 31) : 64 * wave + lane;  // B operand: its expert
  const bool busy = (MODE == 0 ? 32 : 64) * wave < E;  // wave-uniform
  // bias of this lane's experts, loaded before the copies: the latency hides under the MFMA loop,
  // and the loads being older than every copy, the copy waits below still count correctly
  float bv[2] = {0.0f, 0.0f};
  if (busy) lane_bias<MODE>(bias, E, wave, lane, bv);
  f32x32_t acc;
#pragma unroll
  for (int r = 0; r < 32; ++r) acc[r] = 0.0f;
  u32x4_t xq[2][4];
  float wv[2][kBK];
  auto read_ops = [&](int sl, int set) {
    const int st = sl % NS;
    const uint8_t* xt = s_xr + st * kXS;
    const float* wt = reinterpret_cast<const float*>(s_wr + st * kWS);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      xq[set][c] = *reinterpret_cast<const u32x4_t*>(xt + tok_a * 64 + ((c ^ ((tok_a >> 2) & 3)) << 4));
#pragma unroll
    for (int ii = 0; ii < kBK; ++ii) wv[set][ii] = wt[ii * EP + exp_b];
  };
  auto chain = [&](int set) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t v = xq[set][c][h];
        acc = __builtin_amdgcn_mfma_f32_32x32x1f32(__uint_as_float(v << 16), wv[set][8 * c + 2 * h], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x1f32(__uint_as_float(v & 0xffff0000u), wv[set][8 * c + 2 * h + 1],
                                                   acc, 0, 0, 0);
      }
  };
  // Slice j: wait for slice j + 1's copies, barrier (every wave has also
  // finished reading slice j into registers, so its stage takes slice j + NS),
  // read slice j + 1's operands under slice j's MFMAs, one read per MFMA.
  // Every step issues one slice's copies (past the end, a repeat of the last
  // slice into the free stage, whose data is never read), so every wait has
  // the same count.
  auto step = [&](int jj, int set) {
    wait_vm_n<(NS - 2) * nL>();
    __syncthreads();
    issue(min(jj + NS, ns - 1), jj % NS);
    if (busy) {
      read_ops(jj + 1, set ^ 1);
      chain(set);
#pragma unroll
      for (int i = 0; i < 2 * kBK / 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    }
  };
  for (int sl = 0; sl < NS; ++sl) issue(min(sl, ns - 1), sl);
  wait_vm_n<(NS - 1) * nL>();
  __syncthreads();
  if (busy) read_ops(0, 0);
  for (int j = 0; j + 2 < ns; j += 2) {
    step(j, 0);
    step(j + 1, 1);
  }
  step(ns - 2, 0);
  if (busy) chain(1);
  wait_vm_n<0>();   // the repeated copies past the end
  __syncthreads();  // the ring now takes the logits
  float* const s_l = reinterpret_cast<float*>(s_ring);
  if (busy) {
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      const int blk = r >> 4, rr = r & 15;
      const int row = (rr >> 2) * 8 + (lane >> 5) * 4 + (rr & 3), col = lane & 31;
      const int tok = MODE == 0 ? 32 * blk + row : row;
      const int e = MODE == 0 ? 32 * wave + col : 64 * wave + 32 * blk + col;
      if (e < E) s_l[tok * EP + e] = bias ? acc[r] + bv[blk] : acc[r];
    }
  }
  __syncthreads();
  if (k <= 16) route_topk16<TB, EP>(s_l, T, t0, E, k, topk_idx, topk_w);
  else route_topk<TB, EP>(s_l, T, t0, E, k, topk_idx, topk_w);
}

}  // namespace

hipError_t launch_route(int64_t T, int emb, int E, int k, const uint16_t* x, const float* wr, const float* bias,
                        const float* logits_in, int32_t* topk_idx, float* topk_w, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 block(256);
  if (!logits_in && (E & 3) == 0) {
    if (E <= 128)
      route_ring_kernel<0><<<dim3((unsigned)((T + 63) / 64)), block, 0, stream>>>(T, emb, E, k, x, wr, bias, topk_idx,
                                                                                 topk_w);
    else
      route_ring_kernel<1><<<dim3((unsigned)((T + 31) / 32)), block, 0, stream>>>(T, emb, E, k, x, wr, bias, topk_idx,
                                                                                 topk_w);
  } else if (E <= 128) {
    route_kernel<0><<<dim3((unsigned)((T + 63) / 64)), block, 0, stream>>>(T, emb, E, k, x, wr, bias, logits_in,
                                                                          topk_idx, topk_w);
  } else {
    route_kernel<1><<<dim3((unsigned)((T + 31) / 32)), block, 0, stream>>>(T, emb, E, k, x, wr, bias, logits_in,
                                                                          topk_idx, topk_w);
  }
  return hipGetLastError();
}

}  // namespace moe
