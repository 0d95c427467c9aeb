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
// then rounded once to bf16. Both kernels are HBM-bound streams.
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
  for (int c = lane; c < nch; c += 64) {
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
        if (j0 + u >= k) rr[u] = -1;
      }
#pragma unroll
      for (int u = 0; u < kJB; ++u)
        if (rr[u] >= 0) v[u] = ld16(ys + (int64_t)rr[u] * emb + c * 8);
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
    u32x4_t o;
#pragma unroll
    for (int m = 0; m < 4; ++m) o[m] = pack_bf16x2(acc[2 * m], acc[2 * m + 1]);
    st16(y + t * emb + c * 8, o);
  }
}

__global__ __launch_bounds__(256) void combine_bwd_kernel(int64_t T, int emb, int k, const uint16_t* __restrict__ dy,
                                                          const uint16_t* __restrict__ ys,
                                                          const int32_t* __restrict__ slot_row,
                                                          const float* __restrict__ w, uint16_t* __restrict__ dys,
                                                          float* __restrict__ dw) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= T) return;
  const int64_t S = T * k;
  const int nch = emb >> 3;
  const uint16_t* dyr = dy + t * emb;
  for (int j = 0; j < k; ++j) {
    const int32_t r = slot_row[t * k + j];
    const float wj = w[t * k + j];
    const bool ok = r >= 0 && r < S;
    float dot = 0.0f;
    if (ok) {
      for (int c = lane; c < nch; c += 64) {
        const u32x4_t d = ld16(dyr + c * 8);
        u32x4_t o;
#pragma unroll
        for (int m = 0; m < 4; ++m) o[m] = pack_bf16x2(wj * bf16_lo(d[m]), wj * bf16_hi(d[m]));
        st16(dys + (int64_t)r * emb + c * 8, o);
        if (ys && dw) {
          const u32x4_t v = ld16(ys + (int64_t)r * emb + c * 8);
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            dot = __builtin_fmaf(bf16_lo(v[m]), bf16_lo(d[m]), dot);
            dot = __builtin_fmaf(bf16_hi(v[m]), bf16_hi(d[m]), dot);
          }
        }
      }
    }
    if (ys && dw) {
#pragma unroll
      for (int s = 32; s >= 1; s >>= 1) dot += __shfl_xor(dot, s);
      if (lane == 0) dw[t * k + j] = dot;
    }
  }
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
