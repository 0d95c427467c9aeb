// Combine (unpermute + top-k weighted sum) and its backward.
//
// "MoE: fused TensorCore Pallas permute/combine kernels and split-expert wi
// layout for TPU v6e", Commits table: commit 1 fuses the unpermute with the
// top-k weighted sum, and its backward is a permutation for dx plus a
// reduction for the weight gradient; commit 2 notes that the permute backward
// is the combine forward with unit weights.
//
// One wave per token. The k source rows are gathered 16 bytes per lane and
// accumulated in fp32 with one fused multiply-add per pick, in pick order,
// then rounded once to bf16. Both kernels are HBM-bound streams. The rows
// they gather are read once and the rows they write are not read again by
// the kernel, so both go through non-temporal loads and stores (measured on
// the 32768-token workload with the Infinity Cache flushed: combine 5.2 ->
// 5.7 TB/s, its backward 4.2 -> 5.1 TB/s).
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kJB = 8;  // picks gathered per batch (loads in flight per lane)

__global__ __launch_bounds__(256) void combine_kernel(int64_t T, int emb, int k, const uint16_t* __restrict__ ys,
                                                      const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ w, uint16_t* __restrict__ y) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= T) return;
  const int64_t S = T * k;
  int32_t my_r = -1;
  float my_w = 0.0f;
  if (lane < k) {
    const int32_t r = slot_row[t * k + lane];
    if (r >= 0 && r < S) {
      my_r = r;
      my_w = w ? w[t * k + lane] : 1.0f;
    }
  }
  const int nch = emb >> 3;
  // Pick j lives in lane j, and the shuffles below read it from there. A shuffle does not return
  // the value of a lane outside the active set, so the chunk loop is wave-uniform and only the
  // loads and the store are masked: with a per-lane loop, a row of fewer than 64 chunks (or the
  // last, partial round of a longer one) left the lanes past its end, and with them every pick
  // held there when k exceeded the active lanes, out of the sum.
  for (int c0 = 0; c0 < nch; c0 += 64) {
    const int c = c0 + lane;
    const bool on = c < nch;
    float acc[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += kJB) {
      int32_t rr[kJB];
      float ww[kJB];
      u32x4_t v[kJB];
#pragma unroll
      for (int u = 0; u < kJB; ++u) {
        rr[u] = __shfl(my_r, (j0 + u) & 63);
        ww[u] = __shfl(my_w, (j0 + u) & 63);
        if (j0 + u >= k || !on) rr[u] = -1;
      }
#pragma unroll
      for (int u = 0; u < kJB; ++u)
        if (rr[u] >= 0) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(ys + (int64_t)rr[u] * emb + c * 8));
#pragma unroll
      for (int u = 0; u < kJB; ++u) {
        if (rr[u] < 0) continue;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          acc[2 * m] = __builtin_fmaf(ww[u], bf16_lo(v[u][m]), acc[2 * m]);
          acc[2 * m + 1] = __builtin_fmaf(ww[u], bf16_hi(v[u][m]), acc[2 * m + 1]);
        }
      }
    }
    if (!on) continue;
    u32x4_t o;
#pragma unroll
    for (int m = 0; m < 4; ++m) o[m] = pack_bf16x2(acc[2 * m], acc[2 * m + 1]);
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(y + t * emb + c * 8));
  }
}

// Backward, one wave per token. The dy row is read once: per group of up to
// kGB 16-byte chunks per lane it is held in registers while every pick j
// writes its scaled copy do = bf16(w_j * dy) to row slot_row[t*k + j] and,
// when the weight gradient is wanted, gathers that row of ys for the dot
// product <ys[row], dy> (all kGB loads of a pick in flight together). The
// wave's sum of pick j is kept in lane j. Measured at 2, 4, 6, 8 and 16
// chunks per group, and with two picks' loads in flight: 4 is the fastest.
constexpr int kGB = 4;

__global__ __launch_bounds__(256) void combine_bwd_kernel(int64_t T, int emb, int k, const uint16_t* __restrict__ dy,
                                                          const uint16_t* __restrict__ ys,
                                                          const int32_t* __restrict__ slot_row,
                                                          const float* __restrict__ w, uint16_t* __restrict__ dys,
                                                          float* __restrict__ dw) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= T) return;
  const int64_t S = T * k;
  int32_t my_r = -1;
  float my_w = 0.0f, my_dot = 0.0f;
  if (lane < k) {
    const int32_t r = slot_row[t * k + lane];
    my_w = w[t * k + lane];
    if (r >= 0 && r < S) my_r = r;
  }
  const bool want_dw = ys && dw;
  const int nch = emb >> 3;
  const uint16_t* dyr = dy + t * emb;
  for (int c0 = 0; c0 < nch; c0 += 64 * kGB) {
    u32x4_t d[kGB];
#pragma unroll
    for (int u = 0; u < kGB; ++u) {
      const int c = c0 + lane + 64 * u;
      if (c < nch) d[u] = ld16(dyr + c * 8);
    }
    for (int j = 0; j < k; ++j) {
      const int32_t r = __shfl(my_r, j);
      const float wj = __shfl(my_w, j);
      if (r < 0) continue;  // wave-uniform
      u32x4_t v[kGB];
      if (want_dw) {
#pragma unroll
        for (int u = 0; u < kGB; ++u) {
          const int c = c0 + lane + 64 * u;
          if (c < nch) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(ys + (int64_t)r * emb + c * 8));
        }
      }
#pragma unroll
      for (int u = 0; u < kGB; ++u) {
        const int c = c0 + lane + 64 * u;
        if (c >= nch) continue;
        u32x4_t o;
#pragma unroll
        for (int m = 0; m < 4; ++m) o[m] = pack_bf16x2(wj * bf16_lo(d[u][m]), wj * bf16_hi(d[u][m]));
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(dys + (int64_t)r * emb + c * 8));
      }
      if (want_dw) {
        float dot = 0.0f;
#pragma unroll
        for (int u = 0; u < kGB; ++u) {
          const int c = c0 + lane + 64 * u;
          if (c >= nch) continue;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            dot = __builtin_fmaf(bf16_lo(v[u][m]), bf16_lo(d[u][m]), dot);
            dot = __builtin_fmaf(bf16_hi(v[u][m]), bf16_hi(d[u][m]), dot);
          }
        }
#pragma unroll
        for (int s2 = 32; s2 >= 1; s2 >>= 1) dot += __shfl_xor(dot, s2);
        if (lane == j) my_dot += dot;
      }
    }
  }
  if (want_dw && lane < k) dw[t * k + lane] = my_r >= 0 ? my_dot : 0.0f;
}

}  // namespace

hipError_t launch_combine(int64_t T, int emb, int k, const uint16_t* ys, const int32_t* slot_row, const float* w,
                          uint16_t* y, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  combine_kernel<<<dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream>>>(T, emb, k, ys, slot_row, w, y);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(int64_t T, int emb, int k, const uint16_t* dy, const uint16_t* ys,
                              const int32_t* slot_row, const float* w, uint16_t* dys, float* dw, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  combine_bwd_kernel<<<dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream>>>(T, emb, k, dy, ys, slot_row, w, dys,
                                                                              dw);
  return hipGetLastError();
}

}  // namespace moe
