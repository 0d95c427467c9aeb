// Router backward with the picks held fixed: the top-k selection has no
// gradient, so the router's gradients flow only through the top-k weights,
// which are the softmax over each token's k picked logits. The weight
// gradient comes out of the combine backward's reduction ("MoE: fused
// TensorCore Pallas permute/combine kernels and split-expert wi layout for
// TPU v6e", Commits table, commit 1). With g = dtopk_w[t] and the forward's
// weights w:
//   dlogits[t, e_j] = w_j (g_j - sum_i w_i g_i)   (0 for experts not picked)
//   dWr[i, e] = sum_t x[t, i] dlogits[t, e],  dbias[e] = sum_t dlogits[t, e]
//   dx[t, :] += sum_j dlogits[t, e_j] Wr[:, e_j]
// dWr and dbias sum each expert's rows in expert-sorted (token) order, so the
// result does not depend on scheduling. All three are HBM-bound streams.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// One thread per token: the per-slot logit gradients.
__global__ __launch_bounds__(256) void rb_dl_kernel(int64_t T, int k, const float* __restrict__ w,
                                                    const float* __restrict__ g, float* __restrict__ dl) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  float s = 0.0f;
  for (int j = 0; j < k; ++j) s = __builtin_fmaf(w[t * k + j], g[t * k + j], s);
  for (int j = 0; j < k; ++j) dl[t * k + j] = w[t * k + j] * (g[t * k + j] - s);
}

// Wr [emb, E] -> WrT [E, emb] through a 32 x 32 LDS tile.
__global__ __launch_bounds__(256) void rb_transpose_kernel(int emb, int E, const float* __restrict__ wr,
                                                           float* __restrict__ wrt) {
  __shared__ float tile[32][33];
  const int i0 = blockIdx.x * 32, e0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int r = ty; r < 32; r += 8) {
    const int i = i0 + r, e = e0 + tx;
    tile[r][tx] = (i < emb && e < E) ? wr[(int64_t)i * E + e] : 0.0f;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int e = e0 + r, i = i0 + tx;
    if (e < E && i < emb) wrt[(int64_t)e * emb + i] = tile[tx][r];
  }
}

// One wave per (expert e, 512 columns): the expert's rows in sorted order,
// 8 columns per lane, fp32 fused multiply-adds in row order. dbias by the
// first column chunk.
__global__ __launch_bounds__(64) void rb_dwr_kernel(int emb, int E, int k, int64_t S, const uint16_t* __restrict__ x,
                                                    const int32_t* __restrict__ sorted_slot,
                                                    const int32_t* __restrict__ off, const float* __restrict__ dl,
                                                    float* __restrict__ dwr, float* __restrict__ dbias) {
  const int e = blockIdx.x, lane = threadIdx.x;
  const int c0 = blockIdx.y * 512 + lane * 8;  // this lane's first column
  int64_t lo = off[e], hi = off[e + 1];
  lo = lo < 0 ? 0 : (lo > S ? S : lo);
  hi = hi < lo ? lo : (hi > S ? S : hi);
  float acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = 0.0f;
  float db = 0.0f;
  const bool live = c0 < emb;
  int64_t r = lo;
  for (; r + 4 <= hi; r += 4) {  // four rows in flight
    int32_t sl[4];
    float d[4];
    u32x4_t v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      sl[q] = min(max(sorted_slot[r + q], 0), (int)(S - 1));
      d[q] = dl[sl[q]];
      if (live) v[q] = ld16(x + (int64_t)(sl[q] / k) * emb + c0);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      db += d[q];
      if (live)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          acc[2 * m] = __builtin_fmaf(bf16_lo(v[q][m]), d[q], acc[2 * m]);
          acc[2 * m + 1] = __builtin_fmaf(bf16_hi(v[q][m]), d[q], acc[2 * m + 1]);
        }
    }
  }
  for (; r < hi; ++r) {
    const int32_t sl = min(max(sorted_slot[r], 0), (int)(S - 1));
    const float d = dl[sl];
    db += d;
    if (live) {
      const u32x4_t v = ld16(x + (int64_t)(sl / k) * emb + c0);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        acc[2 * m] = __builtin_fmaf(bf16_lo(v[m]), d, acc[2 * m]);
        acc[2 * m + 1] = __builtin_fmaf(bf16_hi(v[m]), d, acc[2 * m + 1]);
      }
    }
  }
  if (live)
#pragma unroll
    for (int u = 0; u < 8; ++u) dwr[(int64_t)(c0 + u) * E + e] = acc[u];
  if (dbias && blockIdx.y == 0 && lane == 0) dbias[e] = db;
}

// One wave per token: dx[t] += sum_j dl[t, j] WrT[e_j], fp32 from the incoming
// bf16 value then the picks in order, one rounding.
__global__ __launch_bounds__(256) void rb_dx_kernel(int64_t T, int emb, int E, int k,
                                                    const int32_t* __restrict__ topk_idx,
                                                    const float* __restrict__ dl, const float* __restrict__ wrt,
                                                    uint16_t* __restrict__ dx) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= T) return;
  for (int c = lane * 8; c < emb; c += 512) {
    const u32x4_t v = ld16(dx + t * emb + c);
    float acc[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      acc[2 * m] = bf16_lo(v[m]);
      acc[2 * m + 1] = bf16_hi(v[m]);
    }
    for (int j = 0; j < k; ++j) {
      const int e = topk_idx[t * k + j];
      if ((unsigned)e >= (unsigned)E) continue;
      const float d = dl[t * k + j];
      const f32x4_t w0 = *reinterpret_cast<const f32x4_t*>(wrt + (int64_t)e * emb + c);
      const f32x4_t w1 = *reinterpret_cast<const f32x4_t*>(wrt + (int64_t)e * emb + c + 4);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc[u] = __builtin_fmaf(d, w0[u], acc[u]);
        acc[4 + u] = __builtin_fmaf(d, w1[u], acc[4 + u]);
      }
    }
    u32x4_t o;
#pragma unroll
    for (int m = 0; m < 4; ++m) o[m] = pack_bf16x2(acc[2 * m], acc[2 * m + 1]);
    st16(dx + t * emb + c, o);
  }
}

}  // namespace

hipError_t launch_route_bwd(int64_t T, int emb, int E, int k, const uint16_t* x, const float* wr,
                            const int32_t* topk_idx, const float* topk_w, const float* dtopk_w,
                            const int32_t* sorted_slot, const int32_t* group_offsets, float* dwr, float* dbias,
                            uint16_t* dx, float* dl, float* wrt, hipStream_t stream) {
  const int64_t S = T * k;
  if (T > 0) rb_dl_kernel<<<dim3((unsigned)((T + 255) / 256)), dim3(256), 0, stream>>>(T, k, topk_w, dtopk_w, dl);
  // also with no tokens: every group is then empty and dwr, dbias come out as exact zeros
  rb_dwr_kernel<<<dim3((unsigned)E, (unsigned)((emb + 511) / 512)), dim3(64), 0, stream>>>(
      emb, E, k, S, x, sorted_slot, group_offsets, dl, dwr, dbias);
  if (dx && T > 0) {
    rb_transpose_kernel<<<dim3((unsigned)((emb + 31) / 32), (unsigned)((E + 31) / 32)), dim3(256), 0, stream>>>(
        emb, E, wr, wrt);
    rb_dx_kernel<<<dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream>>>(T, emb, E, k, topk_idx, dl, wrt, dx);
  }
  return hipGetLastError();
}

}  // namespace moe
