// Permute into expert-sorted order: histogram, scan, row scatter.
//
// The group_size histogram sits above the gather ("MoE: fused TensorCore
// Pallas permute/combine kernels and split-expert wi layout for TPU v6e",
// Commits table, commit 2), and the gather never builds the unsorted
// [tokens * top_k, emb] copy (same page, Context item 1): each token row is
// read once and written straight to its k sorted rows.
//
// Sorted order is by (expert, token). Tokens are cut into blocks of 64; for
// block b and expert e a 64-bit mask holds which of the block's tokens picked
// e (a token picks an expert at most once). Then
//   group_sizes[e] = sum_b popcount(mask[b][e]),
//   base[b][e]     = sum_{b' < b} popcount(mask[b'][e]),
//   row(t, j)      = group_offsets[e] + base[b][e] + popcount(mask[b][e] & lanes below t),
// which is the rank of token t among the tokens of expert e: the stable order.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// One wave per 64-token block: LDS 64-bit OR per (token, pick).
__global__ __launch_bounds__(256) void hist_kernel(int64_t T, int E, int k, int64_t nblk,
                                                   const int32_t* __restrict__ topk_idx, uint64_t* __restrict__ masks) {
  __shared__ unsigned long long s_m[4][kMaxExperts];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t blk = (int64_t)blockIdx.x * 4 + wave;
  for (int e = lane; e < E; e += 64) s_m[wave][e] = 0ull;
  __syncthreads();
  const int64_t t = blk * kPermuteBlock + lane;
  if (blk < nblk && t < T) {
    for (int j0 = 0; j0 < k; j0 += 8) {  // the picks' loads in flight together, 8 at a time
      int ev[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) ev[u] = j0 + u < k ? topk_idx[t * k + j0 + u] : -1;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if ((unsigned)ev[u] < (unsigned)E) atomicOr(&s_m[wave][ev[u]], 1ull << lane);
    }
  }
  __syncthreads();
  if (blk < nblk)
    for (int e = lane; e < E; e += 64) masks[blk * E + e] = s_m[wave][e];
}

// The scan: block_scan_kernel runs one workgroup per expert e. Thread i owns
// a contiguous chunk of the blocks; its chunk's mask counts, scanned across
// the workgroup, give base[b][e] = sum_{b' < b} popcount(mask[b'][e])
// (relative to the expert's first row) and group_sizes[e]. The rank kernels
// then scan group_sizes into group_offsets themselves. A single workgroup for
// all experts (the first form) took 22 us on the 32768-token workload: its
// 1.3 MB of mask reads and base writes all went through one CU. Permute,
// histogram to ranks, on that workload: 32.8 -> 16.0 us.
constexpr int kScanThreads = 256;
constexpr int kScanBatch = 16;  // mask loads in flight per thread

__global__ __launch_bounds__(kScanThreads) void block_scan_kernel(int64_t nblk, int E,
                                                                  const uint64_t* __restrict__ masks,
                                                                  int32_t* __restrict__ group_sizes,
                                                                  int32_t* __restrict__ base) {
  __shared__ int32_t s_wave[kScanThreads / 64];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t chunk = (nblk + kScanThreads - 1) / kScanThreads;
  const int64_t b0 = min((int64_t)tid * chunk, nblk), b1 = min(b0 + chunk, nblk);
  int32_t s = 0;
  {
    int64_t b = b0;
    for (; b + kScanBatch <= b1; b += kScanBatch) {
      uint64_t m[kScanBatch];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) m[u] = masks[(b + u) * E + e];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) s += __popcll(m[u]);
    }
    for (; b < b1; ++b) s += __popcll(masks[b * E + e]);
  }
  // exclusive scan of the threads' counts (chunks are in thread order)
  int32_t incl = s;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t n = __shfl_up(incl, d);
    if (lane >= d) incl += n;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int32_t run = incl - s, total = 0;
#pragma unroll
  for (int w = 0; w < kScanThreads / 64; ++w) {
    if (w < wave) run += s_wave[w];
    total += s_wave[w];
  }
  if (tid == 0) group_sizes[e] = total;
  int64_t b = b0;
  for (; b + kScanBatch <= b1; b += kScanBatch) {
    uint64_t m[kScanBatch];
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) m[u] = masks[(b + u) * E + e];
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      base[(b + u) * E + e] = run;
      run += __popcll(m[u]);
    }
  }
  for (; b < b1; ++b) {
    base[b * E + e] = run;
    run += __popcll(masks[b * E + e]);
  }
}

// group_offsets = exclusive scan of group_sizes (E <= 256), computed by every
// workgroup of the rank kernels into its LDS (256 threads, one per expert)
// instead of in a kernel of its own; workgroup 0 also writes group_offsets.
__device__ __forceinline__ void expert_offsets(int E, const int32_t* __restrict__ group_sizes,
                                               int32_t* __restrict__ group_offsets, int32_t* s_off,
                                               int32_t* s_wave) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t v = tid < E ? group_sizes[tid] : 0;
  int32_t incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t n = __shfl_up(incl, d);
    if (lane >= d) incl += n;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int32_t ex = incl - v;
  for (int w = 0; w < wave; ++w) ex += s_wave[w];
  if (tid < E) s_off[tid] = ex;
  if (blockIdx.x == 0) {
    if (tid < E) group_offsets[tid] = ex;
    if (tid == E - 1) group_offsets[E] = ex + v;
  }
  __syncthreads();
}

// T == 0: only group_offsets (all zero) is left to write.
__global__ __launch_bounds__(256) void expert_scan_kernel(int E, const int32_t* __restrict__ group_sizes,
                                                          int32_t* __restrict__ group_offsets) {
  __shared__ int32_t s_off[kMaxExperts], s_wave[4];
  expert_offsets(E, group_sizes, group_offsets, s_off, s_wave);
}

// One wave per token: read the row once (16 bytes per lane per chunk), write it to its k rows
// (non-temporal: the sorted copy is read back only by later kernels).
__global__ __launch_bounds__(256) void scatter_kernel(int64_t T, int emb, int E, int k, const uint16_t* __restrict__ x,
                                                      const int32_t* __restrict__ topk_idx,
                                                      const uint64_t* __restrict__ masks,
                                                      const int32_t* __restrict__ base,
                                                      const int32_t* __restrict__ group_sizes,
                                                      int32_t* __restrict__ group_offsets,
                                                      int32_t* __restrict__ sorted_slot,
                                                      int32_t* __restrict__ slot_row, uint16_t* __restrict__ xs) {
  __shared__ int32_t s_off[kMaxExperts], s_wave[4];
  expert_offsets(E, group_sizes, group_offsets, s_off, s_wave);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= T) return;
  const int64_t b = t / kPermuteBlock;
  const int tl = (int)(t % kPermuteBlock);
  const uint64_t below = (1ull << tl) - 1ull;
  int32_t my_r = -1;
  if (lane < k) {
    const int e = topk_idx[t * k + lane];
    if ((unsigned)e < (unsigned)E) {
      my_r = s_off[e] + base[b * E + e] + __popcll(masks[b * E + e] & below);
      sorted_slot[my_r] = (int32_t)(t * k + lane);
      slot_row[t * k + lane] = my_r;
    }
  }
  const int nch = emb >> 3;  // 16-byte chunks per row
  const uint16_t* src = x + t * emb;
  for (int c0 = 0; c0 < nch; c0 += 64 * 8) {
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = c0 + lane + 64 * u;
      if (c < nch) v[u] = ld16(src + c * 8);
    }
    for (int j = 0; j < k; ++j) {
      const int32_t r = __shfl(my_r, j);
      if (r < 0) continue;
      uint16_t* dst = xs + (int64_t)r * emb;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = c0 + lane + 64 * u;
        if (c < nch) __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4_t*>(dst + c * 8));
      }
    }
  }
}

// Index only (no row copy), one thread per slot s = t*k + j: the same stable
// rank as scatter_kernel, for callers that read the rows in place through
// sorted_slot (the grouped GEMM's row gather).
__global__ __launch_bounds__(256) void index_kernel(int64_t T, int E, int k, const int32_t* __restrict__ topk_idx,
                                                    const uint64_t* __restrict__ masks,
                                                    const int32_t* __restrict__ base,
                                                    const int32_t* __restrict__ group_sizes,
                                                    int32_t* __restrict__ group_offsets,
                                                    int32_t* __restrict__ sorted_slot,
                                                    int32_t* __restrict__ slot_row) {
  __shared__ int32_t s_off[kMaxExperts], s_wave[4];
  expert_offsets(E, group_sizes, group_offsets, s_off, s_wave);
  const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (s >= T * k) return;
  const int64_t t = s / k;
  const int64_t b = t / kPermuteBlock;
  const int tl = (int)(t % kPermuteBlock);
  const int e = topk_idx[s];
  if ((unsigned)e >= (unsigned)E) return;
  const int32_t r = s_off[e] + base[b * E + e] + __popcll(masks[b * E + e] & ((1ull << tl) - 1ull));
  sorted_slot[r] = (int32_t)s;
  slot_row[s] = r;
}

}  // namespace

// Fixed scratch of the allocation-free permute: the per-block expert masks
// and row bases, [nblk, E] uint64 then [nblk, E] int32, each region rounded up
// to 256 bytes. One copy per GPU, held until the process ends. Host code
// passes its device address (permute_scratch), never this name.
static __device__ __align__(256) uint8_t scratch[kPermuteScratchBytes];

// Device address of this GPU's copy of `scratch`, looked up once per device
// (with that device current) and kept.
hipError_t permute_scratch(uint8_t** out) {
  static std::mutex mu;
  static uint8_t* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<uint8_t*>(p);
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_permute_noalloc(int64_t T, int emb, int E, int k, const uint16_t* x, const int32_t* topk_idx,
                                  int32_t* group_sizes, int32_t* group_offsets, int32_t* sorted_slot,
                                  int32_t* slot_row, uint16_t* xs, hipStream_t stream) {
  const int64_t nblk = (T + kPermuteBlock - 1) / kPermuteBlock;
  const size_t masks = ((size_t)nblk * E * sizeof(uint64_t) + 255) / 256 * 256;
  const size_t base = ((size_t)nblk * E * sizeof(int32_t) + 255) / 256 * 256;
  if (masks + base > kPermuteScratchBytes) return hipErrorInvalidValue;  // checked by the caller first
  uint8_t* s = nullptr;
  if (hipError_t e = permute_scratch(&s)) return e;
  // every mask and base a call reads is written earlier in the same call, so the last call's contents
  // need no clearing
  return launch_permute(T, emb, E, k, x, topk_idx, group_sizes, group_offsets, sorted_slot, slot_row, xs,
                        reinterpret_cast<uint64_t*>(s), reinterpret_cast<int32_t*>(s + masks), stream);
}

hipError_t launch_permute(int64_t T, int emb, int E, int k, const uint16_t* x, const int32_t* topk_idx,
                          int32_t* group_sizes, int32_t* group_offsets, int32_t* sorted_slot, int32_t* slot_row,
                          uint16_t* xs, uint64_t* masks, int32_t* base, hipStream_t stream) {
  const int64_t nblk = (T + kPermuteBlock - 1) / kPermuteBlock;
  if (nblk > 0) {
    hist_kernel<<<dim3((unsigned)((nblk + 3) / 4)), dim3(256), 0, stream>>>(T, E, k, nblk, topk_idx, masks);
  }
  // The scans also run for T == 0 so that group_sizes / group_offsets are written (all zero).
  block_scan_kernel<<<dim3((unsigned)E), dim3(kScanThreads), 0, stream>>>(nblk, E, masks, group_sizes, base);
  // the rank kernels scan group_sizes themselves and write group_offsets
  if (T > 0) {
    if (xs)
      scatter_kernel<<<dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream>>>(
          T, emb, E, k, x, topk_idx, masks, base, group_sizes, group_offsets, sorted_slot, slot_row, xs);
    else
      index_kernel<<<dim3((unsigned)((T * k + 255) / 256)), dim3(256), 0, stream>>>(
          T, E, k, topk_idx, masks, base, group_sizes, group_offsets, sorted_slot, slot_row);
  } else {
    expert_scan_kernel<<<dim3(1), dim3(256), 0, stream>>>(E, group_sizes, group_offsets);
  }
  return hipGetLastError();
}

}  // namespace moe
