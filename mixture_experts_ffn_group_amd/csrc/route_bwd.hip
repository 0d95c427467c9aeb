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
// result does not depend on scheduling. Everything here streams memory.
//
// Column split by XCD: workgroup L runs on XCD L % 8 (dispatch is round-robin
// over the XCDs), and every kernel that reads rows gives XCD q the columns
// [q * emb/8, (q+1) * emb/8). Each XCD then touches one eighth of Wr^T and of
// the x rows, which keeps Wr^T (E * emb * 4 bytes in all) resident in the
// XCD's own L2 while dx gathers it once per pick.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kXcd = 8;
constexpr int kRowsInFlight = 16;  // x rows loaded before their FMAs in the dWr reduction
constexpr int kPickBatch = 8;      // picks whose Wr^T rows are loaded before their FMAs in dx

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// One thread per expert-sorted row r: the logit gradient of its slot s, stored
// by slot (dl) and by row (dls), and the row's token (tok). The sum over the
// token's picks is the same fma chain for each of them, so all k rows of a
// token agree bit for bit.
__global__ __launch_bounds__(256) void rb_prep_kernel(int64_t S, int k, const float* __restrict__ w,
                                                      const float* __restrict__ g,
                                                      const int32_t* __restrict__ sorted_slot,
                                                      const int32_t* __restrict__ off, int E, float* __restrict__ dl,
                                                      float* __restrict__ dls, int32_t* __restrict__ tok) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int64_t n = off[E];
  n = n < 0 ? 0 : (n > S ? S : n);
  if (r >= n) return;
  const int64_t s = min(max((int64_t)sorted_slot[r], (int64_t)0), S - 1);
  const int64_t t = s / k;
  float sum = 0.0f;
  for (int j = 0; j < k; ++j) sum = __builtin_fmaf(w[t * k + j], g[t * k + j], sum);
  const float d = w[s] * (g[s] - sum);
  dl[s] = d;
  dls[r] = d;
  tok[r] = (int32_t)t;
}

// src [R, C] fp32 -> dst [C, R] through a 32 x 32 LDS tile.
__global__ __launch_bounds__(256) void rb_transpose_kernel(int R, int C, const float* __restrict__ src,
                                                           float* __restrict__ dst) {
  __shared__ float tile[32][33];
  const int r0 = blockIdx.x * 32, c0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int i = ty; i < 32; i += 8) {
    const int r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < R && c < C) ? src[(int64_t)r * C + c] : 0.0f;
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int c = c0 + i, r = r0 + tx;
    if (c < C && r < R) dst[(int64_t)c * R + r] = tile[tx][i];
  }
}

__device__ __forceinline__ void fma_row(float (&acc)[8], const u32x4_t& v, float d) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    acc[2 * m] = __builtin_fmaf(bf16_lo(v[m]), d, acc[2 * m]);
    acc[2 * m + 1] = __builtin_fmaf(bf16_hi(v[m]), d, acc[2 * m + 1]);
  }
}

// One wave per (XCD column slice, expert e, pass): lane task = pass * 64 + lane
// owns 8 columns of the slice and sums the expert's rows in sorted order with
// fp32 fmas. The rows' tokens and logit gradients come 64 at a time from one
// coalesced load and are broadcast with readlane; 16 rows of x are in flight.
// Output dWr^T [E, emb] (contiguous per lane); dbias from the first wave.
__global__ __launch_bounds__(64) void rb_dwr_kernel(int emb, int E, int64_t S, int ntask,
                                                    const uint16_t* __restrict__ x, const int32_t* __restrict__ tok,
                                                    const float* __restrict__ dls, const int32_t* __restrict__ off,
                                                    float* __restrict__ dwrt, float* __restrict__ dbias) {
  const int L = blockIdx.x, lane = threadIdx.x;
  const int xcd = L % kXcd;
  const int rest = L / kXcd;
  const int e = rest % E, pass = rest / E;
  const int task = pass * 64 + lane;
  const bool live = task < ntask;
  const int c0 = xcd * (emb / kXcd) + task * 8;
  // rows past group_offsets[E] have no token written by rb_prep_kernel: never read them
  int64_t n_all = off[E];
  n_all = n_all < 0 ? 0 : (n_all > S ? S : n_all);
  int64_t lo = off[e], hi = off[e + 1];
  lo = lo < 0 ? 0 : (lo > n_all ? n_all : lo);
  hi = hi < lo ? lo : (hi > n_all ? n_all : hi);
  float acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = 0.0f;
  float db = 0.0f;
  const uint16_t* xc = x + c0;
  for (int64_t r0 = lo; r0 < hi; r0 += 64) {
    const int n = (int)(hi - r0 < 64 ? hi - r0 : 64);
    int my_t = 0;
    float my_d = 0.0f;
    if (lane < n) {
      my_t = tok[r0 + lane];
      my_d = dls[r0 + lane];
    }
    int q = 0;
    for (; q + kRowsInFlight <= n; q += kRowsInFlight) {
      u32x4_t v[kRowsInFlight];
      float d[kRowsInFlight];
#pragma unroll
      for (int u = 0; u < kRowsInFlight; ++u) {
        const int t = __builtin_amdgcn_readlane(my_t, q + u);
        d[u] = readlane_f(my_d, q + u);
        if (live) v[u] = ld16(xc + (int64_t)t * emb);
      }
#pragma unroll
      for (int u = 0; u < kRowsInFlight; ++u) {
        db += d[u];
        if (live) fma_row(acc, v[u], d[u]);
      }
    }
    for (; q < n; ++q) {
      const int t = __builtin_amdgcn_readlane(my_t, q);
      const float d = readlane_f(my_d, q);
      db += d;
      if (live) fma_row(acc, ld16(xc + (int64_t)t * emb), d);
    }
  }
  if (live) {
    f32x4_t o0, o1;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      o0[u] = acc[u];
      o1[u] = acc[4 + u];
    }
    float* dst = dwrt + (int64_t)e * emb + c0;
    *reinterpret_cast<f32x4_t*>(dst) = o0;
    *reinterpret_cast<f32x4_t*>(dst + 4) = o1;
  }
  if (dbias && xcd == 0 && pass == 0 && lane == 0) dbias[e] = db;
}

// One thread per (token t, 8 columns of the XCD's slice): dx[t] += sum_j
// dl[t, j] WrT[e_j], fp32 from the incoming bf16 value then the picks in
// order, one rounding. A batch of picks' Wr^T rows is loaded before its FMAs.
__global__ __launch_bounds__(256) void rb_dx_kernel(int64_t T, int emb, int E, int k, int ntask,
                                                    const int32_t* __restrict__ topk_idx,
                                                    const float* __restrict__ dl, const float* __restrict__ wrt,
                                                    uint16_t* __restrict__ dx) {
  const int L = blockIdx.x;
  const int xcd = L % kXcd;
  const int64_t item = (int64_t)(L / kXcd) * 256 + threadIdx.x;
  if (item >= T * ntask) return;
  const int64_t t = item / ntask;
  const int task = (int)(item % ntask);
  const int c = xcd * (emb / kXcd) + task * 8;
  uint16_t* px = dx + t * emb + c;
  const u32x4_t v = ld16(px);
  float acc[8];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    acc[2 * m] = bf16_lo(v[m]);
    acc[2 * m + 1] = bf16_hi(v[m]);
  }
  for (int j0 = 0; j0 < k; j0 += kPickBatch) {
    int e[kPickBatch];
    float d[kPickBatch];
    f32x4_t w0[kPickBatch], w1[kPickBatch];
#pragma unroll
    for (int u = 0; u < kPickBatch; ++u) {
      const int j = j0 + u;
      e[u] = j < k ? topk_idx[t * k + j] : -1;
      d[u] = j < k ? dl[t * k + j] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kPickBatch; ++u) {
      if ((unsigned)e[u] < (unsigned)E) {
        const float* src = wrt + (int64_t)e[u] * emb + c;
        w0[u] = *reinterpret_cast<const f32x4_t*>(src);
        w1[u] = *reinterpret_cast<const f32x4_t*>(src + 4);
      }
    }
#pragma unroll
    for (int u = 0; u < kPickBatch; ++u) {
      if ((unsigned)e[u] < (unsigned)E) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[q] = __builtin_fmaf(d[u], w0[u][q], acc[q]);
          acc[4 + q] = __builtin_fmaf(d[u], w1[u][q], acc[4 + q]);
        }
      }
    }
  }
  u32x4_t o;
#pragma unroll
  for (int m = 0; m < 4; ++m) o[m] = pack_bf16x2(acc[2 * m], acc[2 * m + 1]);
  st16(px, o);
}

}  // namespace

hipError_t launch_route_bwd(int64_t T, int emb, int E, int k, const uint16_t* x, const float* wr,
                            const int32_t* topk_idx, const float* topk_w, const float* dtopk_w,
                            const int32_t* sorted_slot, const int32_t* group_offsets, float* dwr, float* dbias,
                            uint16_t* dx, float* dl, float* dls, int32_t* tok, float* wrt, float* dwrt,
                            hipStream_t stream) {
  const int64_t S = T * k;
  const int ntask = emb / (8 * kXcd);  // 8-column tasks per XCD slice (emb is a multiple of 64)
  if (S > 0)
    rb_prep_kernel<<<dim3((unsigned)((S + 255) / 256)), dim3(256), 0, stream>>>(S, k, topk_w, dtopk_w, sorted_slot,
                                                                               group_offsets, E, dl, dls, tok);
  // also with no tokens: every group is then empty and dwr, dbias come out as exact zeros
  const int npass = (ntask + 63) / 64;
  rb_dwr_kernel<<<dim3((unsigned)(kXcd * E * npass)), dim3(64), 0, stream>>>(emb, E, S, ntask, x, tok, dls,
                                                                            group_offsets, dwrt, dbias);
  rb_transpose_kernel<<<dim3((unsigned)((E + 31) / 32), (unsigned)((emb + 31) / 32)), dim3(256), 0, stream>>>(
      E, emb, dwrt, dwr);
  if (dx && T > 0) {
    rb_transpose_kernel<<<dim3((unsigned)((emb + 31) / 32), (unsigned)((E + 31) / 32)), dim3(256), 0, stream>>>(
        emb, E, wr, wrt);
    const int64_t nblk = (T * ntask + 255) / 256;
    rb_dx_kernel<<<dim3((unsigned)(kXcd * nblk)), dim3(256), 0, stream>>>(T, emb, E, k, ntask, topk_idx, dl, wrt,
                                                                         dx);
  }
  return hipGetLastError();
}

}  // namespace moe
