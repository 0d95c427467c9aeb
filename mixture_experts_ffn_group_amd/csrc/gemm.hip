// Ragged grouped GEMM on bf16 MFMA (gfx950) and its weight-gradient form.
//
// Forward: one grouped GEMM on the prefused weight wi [E, emb, 2*mlp], with
// only the GEMM output split into gate and up for SwiGLU ("Keep fused MoE
// weights intact through FSDP gather", Description). The SwiGLU runs in the
// epilogue on fp32 accumulators, so neither the weight nor the output is ever
// split or concatenated in memory: a 256-wide B tile holds 128 gate columns
// [n0, n0+128) and the matching 128 up columns [mlp+n0, mlp+n0+128) of the
// same wi[e], and the two accumulator sets sit in the same lanes.
// Backward: the transposed-RHS form C = A B[e]^T ("MoE: fused TensorCore
// Pallas permute/combine kernels ...", Related PRs, part 3), the SwiGLU
// backward as one concatenated [dgate | dup] ("Gemma4 26B MoE on TPU v6e",
// Commits table, commit 7), and the weight gradient dW[e] = X_e^T dH_e.
// Group-aware kernels do no masked dense work ("[DRAFT][JAX] Optimize MoE
// block", Changes): only the tiles a group needs are run, and the partial
// tile at a group edge is masked on store ("MoE: fused TensorCore Pallas
// permute/combine kernels ...", Tests: boundary-tile masking).
//
// Design (gfx950):
//  - Workgroup tile 256 x 256 x 64, 4 waves in 2 x 2, each wave 128 x 128 =
//    4 x 4 MFMA 32x32x16 bf16 blocks (256 fp32 accumulators per lane).
//  - A and B stages double-buffered in LDS (128 KB). Global loads of the next
//    k-slice are in flight while the current slice feeds the MFMAs.
//  - The weight side is the MFMA's first operand, so each lane ends with four
//    consecutive output columns per register group (8-byte stores).
//  - [k][n]-major B tiles (the NN weight, both wgrad operands) are read with
//    the gfx950 transposed LDS read ds_read_b64_tr_b16; [n][k]-major tiles with
//    ds_read_b128. Both layouts are XOR-swizzled on 16-byte chunks so the
//    reads are bank-conflict free.
//  - Persistent grid of one workgroup per CU. Each workgroup derives the
//    ragged tile list from the device-side group offsets itself (no host
//    sync). Tiles are numbered expert-major and dealt so that each XCD works
//    on a contiguous run of tiles that share A and B panels in its L2.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int BM = 256, BN = 256, BK = 64, NTHR = 256;
constexpr int kStageBytes = BM * BK * 2;  // one operand, one stage: 32 KB
constexpr int kLdsBytes = 4 * kStageBytes;

enum { OP_NN = 0, OP_NT = 1 };
enum { EPI_NONE = 0, EPI_SWIGLU = 1, EPI_SWIGLU_BWD = 2 };

struct GemmP {
  const uint16_t* A;
  const uint16_t* B;
  const float* aux_in;   // SWIGLU_BWD: saved h [M, 2N] fp32
  float* aux_out;        // SWIGLU: h [M, N] fp32 (optional)
  uint16_t* C;
  const int32_t* off;
  const int32_t* row_slot;  // optional: A row of output row r is row_slot[r] / slot_div
  const float* slot_scale;  // optional: output row r is scaled by slot_scale[row_slot[r]] (or [r])
  int E, M, K, N;
  int n_slots, slot_div;
};

struct WgradP {
  const uint16_t* A;
  const uint16_t* D;
  const int32_t* off;
  uint16_t* C;
  int E, M, P, Q;
};

// Tiles whose rows hold 8 16-byte chunks (64 bf16 along k): A [BM][BK], NT-B [BN][BK].
__device__ __forceinline__ int off_k8(int row, int c) { return row * 128 + ((c ^ (row & 7)) << 4); }
// Tiles whose rows hold 32 chunks (256 bf16 along n): NN-B [BK][BN], wgrad [BK][256].
__device__ __forceinline__ int off_n32(int krow, int c) { return krow * 512 + ((c ^ ((krow & 3) << 1)) << 4); }

__device__ __forceinline__ bf16x8_t lds_rd16(const uint8_t* base, int off) {
  return *reinterpret_cast<const bf16x8_t*>(base + off);
}

// MFMA operand from a [k][n] tile: lane l gets 8 k values (k0 + 8*(l/32) + 0..7)
// of column nbase + l%32. In each 16-lane group the transposed read returns,
// for output lane j, element m of source lane 4m + j/4; source lane i
// therefore points at row k0 + 4*rd + i/4, columns nbase + 16*(group&1) + 4*(i%4).
__device__ __forceinline__ bf16x8_t frag_tr(const uint8_t* tile, int lane, int k0, int nbase) {
  const int g = lane >> 4, i = lane & 15;
  const int kr = k0 + 8 * (g >> 1) + (i >> 2);
  const int nc = nbase + 16 * (g & 1) + 4 * (i & 3);
  const int within = (nc & 7) * 2;
  typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
  const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4*)(const_cast<uint8_t*>(tile) + off_n32(kr, nc >> 3) + within));
  const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4*)(const_cast<uint8_t*>(tile) + off_n32(kr + 4, nc >> 3) + within));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// MFMA operand from a [row][k] tile: lane l gets row rbase + l%32, k values k0 + 8*(l/32) + 0..7.
__device__ __forceinline__ bf16x8_t frag_k(const uint8_t* tile, int lane, int k0, int rbase) {
  return lds_rd16(tile, off_k8(rbase + (lane & 31), (k0 >> 3) + (lane >> 5)));
}

__device__ __forceinline__ f32x16_t mfma(bf16x8_t w, bf16x8_t x, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(w, x, c, 0, 0, 0);
}

__device__ __forceinline__ u32x2_t pack4(float a, float b, float c, float d) {
  u32x2_t v;
  v[0] = pack_bf16x2(a, b);
  v[1] = pack_bf16x2(c, d);
  return v;
}

// Block-wide inclusive scan of one int per thread (256 threads); s_wsum holds 4 ints.
__device__ __forceinline__ int block_incl_scan(int v, int* s_wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int n = __shfl_up(v, d);
    if (lane >= d) v += n;
  }
  if (lane == 63) s_wsum[wave] = v;
  __syncthreads();
  for (int w2 = 0; w2 < wave; ++w2) v += s_wsum[w2];
  return v;
}

// Column base (within the 256-wide B tile) of N-fragment f of wave column wn.
template <int EPI>
__device__ __forceinline__ int frag_col(int wn, int f) {
  if (EPI == EPI_SWIGLU) return f < 2 ? wn * 64 + f * 32 : 128 + wn * 64 + (f - 2) * 32;
  return wn * 128 + f * 32;
}

template <int OP, int EPI>
__global__ __launch_bounds__(NTHR, 1) void gemm_kernel(GemmP p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLdsBytes];
  __shared__ int s_lo[kMaxExperts], s_n[kMaxExperts], s_pref[kMaxExperts + 1], s_wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int mlp = EPI == EPI_SWIGLU ? p.N / 2 : p.N;
  const int tile_n = EPI == EPI_SWIGLU ? 128 : BN;
  const int ntn = (mlp + tile_n - 1) / tile_n;

  {  // ragged tile list: tiles of expert e = ceil(rows_e / BM) * ntn, prefix over experts
    int tiles = 0;
    if (tid < p.E) {
      int lo = p.off[tid], hi = p.off[tid + 1];
      lo = min(max(lo, 0), p.M);
      hi = min(max(hi, 0), p.M);
      const int n = hi > lo ? hi - lo : 0;
      s_lo[tid] = lo;
      s_n[tid] = n;
      tiles = ((n + BM - 1) / BM) * ntn;
    }
    const int incl = block_incl_scan(tiles, s_wsum);
    if (tid < p.E) s_pref[tid + 1] = incl;
    if (tid == 0) s_pref[0] = 0;
    __syncthreads();
  }
  const int total = s_pref[p.E];
  uint8_t* const As0 = smem;
  uint8_t* const Bs0 = smem + 2 * kStageBytes;

  // loader lanes
  const int ca = tid & 7, ra = tid >> 3;   // [row][k] tiles: chunk, first row (+32 per step)
  const int cb = tid & 31, kb = tid >> 5;  // [k][n] tiles: chunk, first k-row (+8 per step)

  for (int64_t it = 0;; ++it) {
    const int64_t tl = xcd_tile(it, blockIdx.x, gridDim.x);
    if (tl >= total) break;
    const int tile = (int)tl;
    int lo = 0, hi = p.E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid] <= tile) lo = mid;
      else hi = mid;
    }
    const int e = lo;
    const int local = tile - s_pref[e];
    const int mt = local / ntn, nt = local % ntn;
    const int m0 = s_lo[e] + mt * BM;
    const int m_end = s_lo[e] + s_n[e];
    const int n0 = nt * tile_n;
    const uint16_t* Bexp = p.B + (int64_t)e * p.K * p.N;

    // Per-tile operand bases with 32-bit offsets. Rows past the group end are
    // clamped to its last row and columns past N to a valid column: both only
    // feed outputs that are never stored. With a row gather, A rows are read in
    // place through the slot index (no permuted copy of A).
    const uint16_t* Ab;
    int a_off[8];
    if (p.row_slot) {
      Ab = p.A;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int s = min(max(p.row_slot[min(m0 + ra + 32 * i, m_end - 1)], 0), p.n_slots - 1);
        a_off[i] = (s / p.slot_div) * p.K + ca * 8;
      }
    } else {
      Ab = p.A + (int64_t)m0 * p.K;
#pragma unroll
      for (int i = 0; i < 8; ++i) a_off[i] = (min(m0 + ra + 32 * i, m_end - 1) - m0) * p.K + ca * 8;
    }
    int b_off[8];
    if (OP == OP_NT) {
#pragma unroll
      for (int i = 0; i < 8; ++i) b_off[i] = min(n0 + ra + 32 * i, p.N - 1) * p.K + ca * 8;
    } else {
      int col;
      if (EPI == EPI_SWIGLU) {
        const int c = cb < 16 ? n0 + cb * 8 : n0 + (cb - 16) * 8;
        col = c < mlp ? (cb < 16 ? c : mlp + c) : 0;
      } else {
        col = n0 + cb * 8;
        col = col < p.N ? col : 0;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) b_off[i] = (kb + 8 * i) * p.N + col;
    }

    u32x4_t ar[8], br[8];
    auto load = [&](int k0) {
      const uint16_t* Ak = Ab + k0;
#pragma unroll
      for (int i = 0; i < 8; ++i) ar[i] = ld16(Ak + a_off[i]);
      const uint16_t* Bk = OP == OP_NT ? Bexp + k0 : Bexp + (int64_t)k0 * p.N;
#pragma unroll
      for (int i = 0; i < 8; ++i) br[i] = ld16(Bk + b_off[i]);
    };
    auto store = [&](int stage) {
      uint8_t* As = As0 + stage * kStageBytes;
      uint8_t* Bs = Bs0 + stage * kStageBytes;
#pragma unroll
      for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4_t*>(As + off_k8(ra + 32 * i, ca)) = ar[i];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (OP == OP_NT) *reinterpret_cast<u32x4_t*>(Bs + off_k8(ra + 32 * i, ca)) = br[i];
        else *reinterpret_cast<u32x4_t*>(Bs + off_n32(kb + 8 * i, cb)) = br[i];
      }
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][f][r] = 0.0f;

    const int nk = p.K / BK;
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) load((kt + 1) * BK);
      const uint8_t* As = As0 + cur * kStageBytes;
      const uint8_t* Bs = Bs0 + cur * kStageBytes;
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        bf16x8_t af[4], bf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = frag_k(As, lane, ks * 16, wm * 128 + i * 32);
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          if (OP == OP_NT) bf[f] = frag_k(Bs, lane, ks * 16, frag_col<EPI>(wn, f));
          else bf[f] = frag_tr(Bs, lane, ks * 16, frag_col<EPI>(wn, f));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int f = 0; f < 4; ++f) acc[i][f] = mfma(bf[f], af[i], acc[i][f]);
      }
      if (kt + 1 < nk) store(cur ^ 1);
      __syncthreads();
    }

    // Epilogue. Lane holds rows m = tile row + lane%32 and, per register group q,
    // four consecutive columns 8q + 4*(lane/32) + 0..3 of each 32-wide fragment.
    const int hh = lane >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + wm * 128 + i * 32 + (lane & 31);
      if (m >= m_end) continue;
      if (p.slot_scale) {  // per-row scale in fp32 (e.g. the top-k weight of the row's slot)
        const int s = p.row_slot ? min(max(p.row_slot[m], 0), p.n_slots - 1) : m;
        const float sc = p.slot_scale[s];
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][f][r] *= sc;
      }
      if (EPI == EPI_NONE) {
        uint16_t* crow = p.C + (int64_t)m * p.N;
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = n0 + wn * 128 + f * 32 + 8 * q + 4 * hh;
            if (n < p.N)
              st8(crow + n, pack4(acc[i][f][4 * q], acc[i][f][4 * q + 1], acc[i][f][4 * q + 2], acc[i][f][4 * q + 3]));
          }
      } else if (EPI == EPI_SWIGLU) {
        uint16_t* arow = p.C + (int64_t)m * mlp;
        float* hrow = p.aux_out ? p.aux_out + (int64_t)m * 2 * mlp : nullptr;
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = n0 + wn * 64 + f * 32 + 8 * q + 4 * hh;
            if (col >= mlp) continue;
            float a[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) a[u] = silu_f(acc[i][f][4 * q + u]) * acc[i][f + 2][4 * q + u];
            st8(arow + col, pack4(a[0], a[1], a[2], a[3]));
            if (hrow) {  // h kept in fp32 for the backward: the gate/up values the SwiGLU used, unrounded
              f32x4_t gv, uv;
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                gv[u] = acc[i][f][4 * q + u];
                uv[u] = acc[i][f + 2][4 * q + u];
              }
              *reinterpret_cast<f32x4_t*>(hrow + col) = gv;
              *reinterpret_cast<f32x4_t*>(hrow + mlp + col) = uv;
            }
          }
      } else {  // EPI_SWIGLU_BWD: N = mlp, aux = saved h [M, 2N], C = dh [M, 2N]
        const float* hrow = p.aux_in + (int64_t)m * 2 * p.N;
        uint16_t* drow = p.C + (int64_t)m * 2 * p.N;
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = n0 + wn * 128 + f * 32 + 8 * q + 4 * hh;
            if (n >= p.N) continue;
            const f32x4_t g = *reinterpret_cast<const f32x4_t*>(hrow + n);
            const f32x4_t u = *reinterpret_cast<const f32x4_t*>(hrow + p.N + n);
            float dg[4], du[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float da = acc[i][f][4 * q + r];
              const float s = sigmoid_f(g[r]);
              dg[r] = da * u[r] * s * (1.0f + g[r] * (1.0f - s));
              du[r] = da * g[r] * s;
            }
            st8(drow + n, pack4(dg[0], dg[1], dg[2], dg[3]));
            st8(drow + p.N + n, pack4(du[0], du[1], du[2], du[3]));
          }
      }
    }
  }
}

// dW[e] [P, Q] = sum over rows r of group e of A[r]^T D[r]. The contraction runs
// over the group's rows, so both operands are [row][col] tiles read transposed.
// Rows past the group end load as zeros; an empty group writes exact zeros.
__global__ __launch_bounds__(NTHR, 1) void wgrad_kernel(WgradP p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int tp = (p.P + 255) / 256, tq = (p.Q + 255) / 256;
  const int64_t total = (int64_t)p.E * tp * tq;
  uint8_t* const As0 = smem;
  uint8_t* const Ds0 = smem + 2 * kStageBytes;
  const int cb = tid & 31, kb = tid >> 5;

  for (int64_t it = 0;; ++it) {
    const int64_t tl = xcd_tile(it, blockIdx.x, gridDim.x);
    if (tl >= total) break;
    const int e = (int)(tl / (tp * tq));
    const int loc = (int)(tl % (tp * tq));
    const int p0 = (loc / tq) * 256, q0 = (loc % tq) * 256;
    int lo = p.off[e], hi = p.off[e + 1];
    lo = min(max(lo, 0), p.M);
    hi = min(max(hi, 0), p.M);
    const int n = hi > lo ? hi - lo : 0;
    const int pc = p0 + cb * 8, qc = q0 + cb * 8;

    u32x4_t ar[8], dr[8];
    auto load = [&](int k0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = k0 + kb + 8 * i;
        ar[i] = u32x4_t{0u, 0u, 0u, 0u};
        dr[i] = u32x4_t{0u, 0u, 0u, 0u};
        if (row < n) {
          if (pc < p.P) ar[i] = ld16(p.A + (int64_t)(lo + row) * p.P + pc);
          if (qc < p.Q) dr[i] = ld16(p.D + (int64_t)(lo + row) * p.Q + qc);
        }
      }
    };
    auto store = [&](int stage) {
      uint8_t* As = As0 + stage * kStageBytes;
      uint8_t* Ds = Ds0 + stage * kStageBytes;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        *reinterpret_cast<u32x4_t*>(As + off_n32(kb + 8 * i, cb)) = ar[i];
        *reinterpret_cast<u32x4_t*>(Ds + off_n32(kb + 8 * i, cb)) = dr[i];
      }
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][f][r] = 0.0f;

    const int nk = (n + BK - 1) / BK;
    if (nk > 0) {
      load(0);
      store(0);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) load((kt + 1) * BK);
      const uint8_t* As = As0 + cur * kStageBytes;
      const uint8_t* Ds = Ds0 + cur * kStageBytes;
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        bf16x8_t af[4], df[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = frag_tr(As, lane, ks * 16, wm * 128 + i * 32);
#pragma unroll
        for (int f = 0; f < 4; ++f) df[f] = frag_tr(Ds, lane, ks * 16, wn * 128 + f * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int f = 0; f < 4; ++f) acc[i][f] = mfma(df[f], af[i], acc[i][f]);
      }
      if (kt + 1 < nk) store(cur ^ 1);
      __syncthreads();
    }

    const int hh = lane >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pr = p0 + wm * 128 + i * 32 + (lane & 31);
      if (pr >= p.P) continue;
      uint16_t* crow = p.C + ((int64_t)e * p.P + pr) * p.Q;
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int qq = q0 + wn * 128 + f * 32 + 8 * q + 4 * hh;
          if (qq < p.Q)
            st8(crow + qq, pack4(acc[i][f][4 * q], acc[i][f][4 * q + 1], acc[i][f][4 * q + 2], acc[i][f][4 * q + 3]));
        }
    }
  }
}

int persistent_grid() {
  int g = device_cu_count();
  g -= g % kNumXcd;
  return g < kNumXcd ? kNumXcd : g;
}

}  // namespace

hipError_t launch_grouped_gemm(int op, int epi, const uint16_t* A, const uint16_t* B, const float* aux_in,
                               float* aux_out, const int32_t* group_offsets, int E, int64_t M, int K, int N,
                               const int32_t* row_slot, int n_slots, int slot_div, const float* slot_scale,
                               uint16_t* C, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  GemmP p{A, B, aux_in, aux_out, C, group_offsets, row_slot, slot_scale, E, (int)M, K, N,
          row_slot ? n_slots : (int)M, slot_div > 0 ? slot_div : 1};
  const dim3 grid(persistent_grid()), block(NTHR);
  if (op == OP_NN && epi == EPI_NONE) gemm_kernel<OP_NN, EPI_NONE><<<grid, block, 0, stream>>>(p);
  else if (op == OP_NN && epi == EPI_SWIGLU) gemm_kernel<OP_NN, EPI_SWIGLU><<<grid, block, 0, stream>>>(p);
  else if (op == OP_NT && epi == EPI_NONE) gemm_kernel<OP_NT, EPI_NONE><<<grid, block, 0, stream>>>(p);
  else if (op == OP_NT && epi == EPI_SWIGLU_BWD) gemm_kernel<OP_NT, EPI_SWIGLU_BWD><<<grid, block, 0, stream>>>(p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_wgrad(const uint16_t* A, const uint16_t* D, const int32_t* group_offsets, int E, int64_t M, int P,
                        int Q, uint16_t* C, hipStream_t stream) {
  if (E == 0) return hipSuccess;
  WgradP p{A, D, group_offsets, C, E, (int)M, P, Q};
  wgrad_kernel<<<dim3(persistent_grid()), dim3(NTHR), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace moe
