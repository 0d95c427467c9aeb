// Grouped GEMM on MXFP8 operands ("[DRAFT][JAX] Optimize MoE block",
// Changes: MXFP8 quantization in the MoE block; Flowchart: grouped FC1
// quantize and GEMM), on gfx950's block-scaled matrix cores:
//   C[r, n] = sum_k A[r, k] * B[e][n, k]   for the rows r of group e,
// where A and B are E4M3 codes times the E8M0 scale of their 32-element K
// block (the layouts of mxfp8.hip: codes K-contiguous, scales one dword per
// row and 64-element slice). Epilogues: none (C [M, N] bf16) or SwiGLU on a
// prefused [gate | up] weight (C [M, N/2] bf16, gate = columns [0, N/2)).
// With a slot index the A rows (codes and scales) are read in place through
// it, so token rows quantized once serve all k of their expert rows. The
// SwiGLU epilogue can also write its output as MXFP8 (the operand of the next
// GEMM): each wave's 32 output columns are one block of each row.
//
// v_mfma_scale_f32_32x32x64_f8f6f4 multiplies 32 x 64 by 64 x 32 with one
// scale byte per lane and 32-element block. Its operand layout (pinned on the
// device): lane l holds row l % 32; bytes 0-15 are K elements 16h .. 16h+15
// and bytes 16-31 are 32+16h .. 32+16h+15, h = l / 32 (the same assignment
// for both operands), and its scale is that of row l % 32 and block h. The
// products of one instruction are summed to a precision fixed relative to the
// largest of them (probes: within 2^-11.8 of the largest product), then added
// to the fp32 accumulator.
//
// The kernel follows the bf16 grouped GEMM: 8 waves as 2 (M) x 4 (N), a
// 256 x 256 output tile per workgroup, each wave 128 x 64 (4 x 2 MFMA
// blocks); a persistent XCD-dealt grid over the ragged tile list built from
// the device group offsets; direct global->LDS copies into four stages. A
// k-slice is 64 elements (64 bytes per row, one MFMA deep); with it travel
// the two operands' scale dwords of the tile's 256 rows (waves 0-3 copy the A
// rows', waves 4-7 the B rows'), so every wave issues 5 copies per k-slice.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int MXT = 512;                        // threads: 8 waves
constexpr int MXN = 4;                          // LDS stages
constexpr int kMxOp = 256 * 64;                 // one operand tile per stage: 256 rows x 64 bytes
constexpr int kMxScl = 256 * 4;                 // one operand's scale dwords per stage
constexpr int kMxStage = 2 * kMxOp + 2 * kMxScl;  // 34 KB
enum { MXE_NONE = 0, MXE_SWIGLU = 1 };

struct MxGemmP {
  const uint8_t* A;   // codes [a_rows][K]
  const uint8_t* As;  // scales [K/64][a_rows][4]
  const int32_t* row_slot;  // optional: A row of output row r is row_slot[r] / slot_div
  const uint8_t* B;   // codes [E][N][K]
  const uint8_t* Bs;  // scales [E][K/64][N][4]
  const int32_t* off;
  uint16_t* C;    // bf16 output, or NULL
  uint8_t* Cq;    // SwiGLU only: MXFP8 codes of the output [M][N/2], or NULL
  uint8_t* Cqs;   // and its scales [N/128][M][4] (bytes 0 and 1 of each dword)
  int E, M, K, N;
  int a_rows, slot_div;
};

__device__ __forceinline__ void mx_g2lds16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(lds) : "memory");
}
__device__ __forceinline__ void mx_g2lds4(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" : : "v"(voff), "s"(sbase), "s"(lds) : "memory");
}
__device__ __forceinline__ void mx_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void mx_wait_5() { asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); }
__device__ __forceinline__ void mx_wait_10() { asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); }
__device__ __forceinline__ void mx_wait_20() { asm volatile("s_waitcnt vmcnt(20)" ::: "memory"); }
__device__ __forceinline__ void mx_wait_30() { asm volatile("s_waitcnt vmcnt(30)" ::: "memory"); }
__device__ __forceinline__ uint32_t mx_lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ int mx_opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}
template <class T>
__device__ __forceinline__ const T* mx_uniform(const T* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const T*)(((uint64_t)hi << 32) | lo);
}

// [row][k] tiles of 64-byte rows, 16-byte chunk c of a row at row*64 + ((c ^ ((row >> 2) & 3)) << 4)
__device__ __forceinline__ int mx_off(int row, int c) { return row * 64 + ((c ^ ((row >> 2) & 3)) << 4); }

// MFMA operand of tile row `row` for lane half h: chunks h and 2 + h.
__device__ __forceinline__ i32x8_t mx_frag(const uint8_t* tile, int row, int h) {
  const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(tile + mx_off(row, h));
  const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(tile + mx_off(row, 2 + h));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int EPI>
__device__ __forceinline__ int mx_col(int wn, int f) {
  if (EPI == MXE_SWIGLU) return f == 0 ? wn * 32 : 128 + wn * 32;
  return wn * 64 + f * 32;
}

__device__ __forceinline__ u32x2_t mx_pack4(float a, float b, float c, float d) {
  u32x2_t v;
  v[0] = pack_bf16x2(a, b);
  v[1] = pack_bf16x2(c, d);
  return v;
}

template <int NW>
__device__ __forceinline__ int mx_scan(int v, int* s_wsum) {
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

template <int EPI, bool GATHER>
__global__ __launch_bounds__(MXT, 1) void mx_gemm_kernel(MxGemmP p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[MXN * kMxStage];
  __shared__ __attribute__((aligned(16))) uint8_t s_stage[MXT / 64][2048];
  __shared__ int s_lo[kMaxExperts + 1], s_pref[kMaxExperts + 1], s_wsum[8];
  const int mlp = EPI == MXE_SWIGLU ? p.N / 2 : p.N;
  const int tile_n = EPI == MXE_SWIGLU ? 128 : 256;
  const int ntn = (mlp + tile_n - 1) / tile_n;
  {  // ragged tile list: tiles of expert e = ceil(rows_e / 256) * ntn, prefix over experts
    const int tid = threadIdx.x;
    int tiles = 0;
    if (tid <= p.E) s_lo[tid] = clamp_rows(p.off[tid], p.M);
    if (tid < p.E) tiles = group_tiles(clamp_rows(p.off[tid + 1], p.M) - clamp_rows(p.off[tid], p.M), ntn);
    const int incl = mx_scan<MXT / 64>(tiles, s_wsum);
    if (tid < p.E) s_pref[tid + 1] = incl;
    if (tid == 0) s_pref[0] = 0;
    __syncthreads();
  }
  const int total = s_pref[p.E];
  const int tid = mx_opaque((int)threadIdx.x), lane = tid & 63, wave = tid >> 6;
  // Wave w owns row half w / 4 and column quarter w % 4 (SIMD w % 4 holds one
  // wave of each row half), so a wave whose rows lie past the group end can
  // skip its MFMAs, as in the bf16 grouped GEMM.
  const int wm = wave >> 2, wn = wave & 3, h = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // Plain output (the wo GEMM): waves 0-3 issue every operand and scale copy
  // and no global store, waves 4-7 every store (non-temporal), as in the bf16
  // grouped GEMM; the copying waves' output crosses through the last ring
  // stage. Without its stores this GEMM runs in about half the time on the
  // 32768-token workload. The SwiGLU form keeps every wave copying and storing.
  constexpr bool SPLIT = EPI == MXE_NONE;
  constexpr int LPW = SPLIT ? 4 : 2;  // 1 KB copies per operand, k-slice and copying wave
  const bool loader = !SPLIT || wave_u < 4;
  const uint32_t lds0 = mx_lds_addr(smem);
  const int nk = p.K / 64;
  const int nslice_rows = p.a_rows;  // rows of A's scale slices
  // With the gather, output row r reads token row row_slot[r] / slot_div (clamped); this is that
  // row from an already loaded slot.
  auto slot_row = [&](int slot) -> int {
    const int t = slot / p.slot_div;
    return t < 0 ? 0 : (t >= p.a_rows ? p.a_rows - 1 : t);
  };
  int m0 = 0, m_end = 0, m_cls = 0, n0 = 0, e = 0;  // tile rows [m0, m_end); m_cls sets the multiply class
  const uint8_t* Bexp = p.B;
  const uint8_t* Bsexp = p.Bs;
  uint32_t a_off[LPW], b_off[LPW], s_off, s_off2 = 0;
  auto decode = [&](int64_t it) -> bool {
    const int64_t tl = xcd_tile(it, blockIdx.x, gridDim.x);
    if (tl >= total) return false;
    const RaggedTile rt = ragged_tile((int)tl, s_pref, p.E, ntn);
    e = __builtin_amdgcn_readfirstlane(rt.e);
    const int mt = rt.mt, nt = rt.nt;
    {  // a group of 257-512 rows runs as two equal halves (tile_rows)
      int r0, r1, rc;
      tile_rows(s_lo[e], max(s_lo[e + 1], s_lo[e]), mt, &r0, &r1, &rc);
      m0 = __builtin_amdgcn_readfirstlane(r0);
      m_end = __builtin_amdgcn_readfirstlane(r1);
      m_cls = __builtin_amdgcn_readfirstlane(rc);
    }
    n0 = __builtin_amdgcn_readfirstlane(nt * tile_n);
    Bexp = mx_uniform(p.B + (int64_t)e * p.N * p.K);
    Bsexp = mx_uniform(p.Bs + (int64_t)e * nk * p.N * 4);
    if (!loader) return true;
    // With the gather, every slot this lane needs is loaded first, into the offset registers
    // themselves (few others are free while the accumulators are live), and converted after:
    // loaded and used one at a time, each cost a round trip.
    const bool a_scale_row = SPLIT || wave_u < 4;  // s_off is an A scale row
    if (GATHER) {
#pragma unroll
      for (int j = 0; j < LPW; ++j)
        a_off[j] = (uint32_t)p.row_slot[min(m0 + (wave_u * LPW + j) * 16 + (lane >> 2), m_end - 1)];
      if (a_scale_row)
        s_off = (uint32_t)p.row_slot[min(m0 + (SPLIT ? wave_u : (wave_u & 3)) * 64 + lane, m_end - 1)];
    }
    // tile rows: block b = LPW*wave + j holds rows 16b .. 16b+15; lane L -> row 16b + L/4, physical chunk L%4
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int row = (wave_u * LPW + j) * 16 + (lane >> 2);
      const int c = (lane & 3) ^ ((row >> 2) & 3);
      const int r = GATHER ? slot_row((int)a_off[j]) : min(m0 + row, m_end - 1);
      a_off[j] = (uint32_t)r * (uint32_t)p.K + (uint32_t)c * 16u;
      int n;
      if (EPI == MXE_SWIGLU) {
        const int cc = n0 + (row & 127);
        n = cc < mlp ? (row < 128 ? cc : mlp + cc) : 0;
      } else {
        n = n0 + row < p.N ? n0 + row : p.N - 1;
      }
      b_off[j] = (uint32_t)n * (uint32_t)p.K + (uint32_t)c * 16u;
    }
    // scale rows: waves 0-3 copy A rows 64*wave + L, waves 4-7 B rows 64*(wave-4) + L (with the
    // roles split, waves 0-3 copy both: s_off for A, s_off2 for B)
    if (SPLIT) {
      const int row = wave_u * 64 + lane;
      s_off = (uint32_t)(GATHER ? slot_row((int)s_off) : min(m0 + row, m_end - 1)) * 4u;
      s_off2 = (uint32_t)(n0 + row < p.N ? n0 + row : p.N - 1) * 4u;
    } else {
      const int row = (wave_u & 3) * 64 + lane;
      if (wave_u < 4) {
        s_off = (uint32_t)(GATHER ? slot_row((int)s_off) : min(m0 + row, m_end - 1)) * 4u;
      } else {
        int n;
        if (EPI == MXE_SWIGLU) {
          const int cc = n0 + (row & 127);
          n = cc < mlp ? (row < 128 ? cc : mlp + cc) : 0;
        } else {
          n = n0 + row < p.N ? n0 + row : p.N - 1;
        }
        s_off = (uint32_t)n * 4u;
      }
    }
    return true;
  };
  auto issue_loads = [&](int kt) {
    if (!loader) return;
    const uint32_t st = lds0 + (uint32_t)(kt & (MXN - 1)) * kMxStage;
    const uint8_t* Ak = p.A + (int64_t)kt * 64;
    const uint8_t* Bk = Bexp + (int64_t)kt * 64;
#pragma unroll
    for (int j = 0; j < LPW; ++j) mx_g2lds16(Ak, a_off[j], st + wave_u * LPW * 1024 + j * 1024);
#pragma unroll
    for (int j = 0; j < LPW; ++j) mx_g2lds16(Bk, b_off[j], st + kMxOp + wave_u * LPW * 1024 + j * 1024);
    if (SPLIT) {
      mx_g2lds4(p.As + (int64_t)kt * nslice_rows * 4, s_off, st + 2 * kMxOp + wave_u * 256);
      mx_g2lds4(Bsexp + (int64_t)kt * p.N * 4, s_off2, st + 2 * kMxOp + kMxScl + wave_u * 256);
    } else if (wave_u < 4) {
      mx_g2lds4(p.As + (int64_t)kt * nslice_rows * 4, s_off, st + 2 * kMxOp + wave_u * 256);
    } else {
      mx_g2lds4(Bsexp + (int64_t)kt * p.N * 4, s_off, st + 2 * kMxOp + kMxScl + (wave_u - 4) * 256);
    }
  };
  // workgroup barrier after this wave's LDS reads; unlike __syncthreads it
  // does not wait for the wave's outstanding global stores
  auto kbarrier = []() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  // the copies of a k-slice have landed once at most those of the n k-slices issued after it are
  // outstanding (10 per k-slice and copying wave with the roles split)
  auto wait_after = [](int n) {
    if (n >= 3) mx_wait_30();
    else if (n == 2) mx_wait_20();
    else if (n == 1) mx_wait_10();
    else mx_wait_all();
  };

  if (!decode(0)) return;
  for (int s = 0; s < MXN; ++s)
    if (s < nk) issue_loads(s);
  for (int64_t it = 0;; ++it) {
    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][f][r] = 0.0f;

    if (SPLIT) {
      if (loader) wait_after(min(nk, MXN) - 1);  // the tile's first k-slice has landed
      kbarrier();
    } else {
      mx_wait_all();  // this wave's loads of the first k-slices (and the last tile's stores) are done
      __syncthreads();
    }
    // k-slice kt+1 has landed (younger are the copies of k-slices kt+2 and kt+3, where they exist);
    // every wave has read stage kt (its MFMAs consumed it) and k-slice kt+1 is visible
    auto kwait = [&](int kt) {
      if (SPLIT) {
        if (loader) wait_after(kt + 3 < nk ? 2 : (kt + 2 < nk ? 1 : 0));
        kbarrier();
      } else {
        if (kt + 3 < nk) mx_wait_10();
        else if (kt + 2 < nk) mx_wait_5();
        else mx_wait_all();
        __syncthreads();
      }
      if (kt + MXN < nk) issue_loads(kt + MXN);
    };
    // NI: the 32-row blocks of the wave that are multiplied, those holding a
    // row before the group end (1 to 4)
    auto kloop = [&](auto NIc) {
      constexpr int NI = decltype(NIc)::value;
      for (int kt = 0; kt < nk; ++kt) {
        const uint8_t* stg = smem + (kt & (MXN - 1)) * kMxStage;
        const uint8_t* As_t = stg;
        const uint8_t* Bs_t = stg + kMxOp;
        const uint8_t* Asc = stg + 2 * kMxOp;
        const uint8_t* Bsc = Asc + kMxScl;
        i32x8_t af[NI], bf[2];
        int sa[NI], sb[2];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int row = wm * 128 + i * 32 + (lane & 31);
          af[i] = mx_frag(As_t, row, h);
          sa[i] = Asc[row * 4 + h];
        }
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int row = mx_col<EPI>(wn, f) + (lane & 31);
          bf[f] = mx_frag(Bs_t, row, h);
          sb[f] = Bsc[row * 4 + h];
        }
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int f = 0; f < 2; ++f)
            acc[i][f] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[f], af[i], acc[i][f], 0, 0, 0, sb[f], 0,
                                                                          sa[i]);
        kwait(kt);
      }
    };
    // rows of this tile that hold outputs, from this wave's first row (wave-uniform)
    const int wrows = m_cls - (m0 + (wave_u >> 2) * 128);
    if (wrows > 96) {
      kloop(std::integral_constant<int, 4>{});
    } else if (wrows > 64) {
      kloop(std::integral_constant<int, 3>{});  // blocks from NI on keep zero accumulators; their rows are not stored
    } else if (wrows > 32) {
      kloop(std::integral_constant<int, 2>{});
    } else if (wrows > 0) {
      kloop(std::integral_constant<int, 1>{});
    } else {
      for (int kt = 0; kt < nk; ++kt) kwait(kt);  // no output rows: the waits, barriers and copies only
    }

    const int cm0 = m0, cm_end = m_end, cn0 = n0;
    const bool more = decode(it + 1);
    // with the roles split, the last stage carries the copying waves' output and is loaded after the epilogue
    if (more)
      for (int s = 0; s < (SPLIT ? MXN - 1 : MXN); ++s)
        if (s < nk) issue_loads(s);
    // Epilogue through this wave's 2 KB staging area (as the bf16 grouped GEMM): lane holds rows
    // m = tile row + lane%32 and, per register group q, columns 8q + 4*(lane/32) + 0..3 of a 32-wide block.
    const int hh = lane >> 5;
    uint8_t* const stg = s_stage[wave];
    auto stg64 = [&](int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); };
    auto stg128 = [&](int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); };
    const int r = lane & 31;
    if (EPI == MXE_NONE) {
      // Copying wave src's 128 x 64 block crosses in 8 KB of the last stage, 64 rows x 128 B per phase
      // (16-byte chunk c of row rr at rr*128 + ((c ^ ((rr >> 1) & 7)) << 4)); storing wave src + 4 stores it.
      const int src = wave_u & 3;
      uint8_t* const xr = smem + (MXN - 1) * kMxStage + (src < 2 ? 0 : kMxOp) + (src & 1) * 8192;
      const int wm_s = src >> 2, wn_s = src & 3;
      auto sto = [](uint16_t* ptr, u32x4_t v) { __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(ptr)); };
#pragma unroll
      for (int ph = 0; ph < 2; ++ph) {
        if (loader) {
#pragma unroll
          for (int ii = 0; ii < 2; ++ii) {
            const int i = 2 * ph + ii, rr = ii * 32 + r;
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
              for (int q = 0; q < 4; ++q)
                *reinterpret_cast<u32x2_t*>(xr + stg128(rr, f * 4 + q) + hh * 8) =
                    mx_pack4(acc[i][f][4 * q], acc[i][f][4 * q + 1], acc[i][f][4 * q + 2], acc[i][f][4 * q + 3]);
          }
        } else if (ph == 0) {
          // the storing wave's own block, 32 rows x 128 B at a time: rows 0-15 in its
          // staging area, rows 16-31 in that of its copying wave (unused here)
          uint8_t* const wb = r < 16 ? stg : s_stage[wave - 4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m0r = cm0 + wm * 128 + i * 32;
            const int n0w = cn0 + wn * 64;
            const int valid = min(8, (p.N - n0w) >> 3);
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
              for (int q = 0; q < 4; ++q)
                *reinterpret_cast<u32x2_t*>(wb + stg128(r & 15, f * 4 + q) + hh * 8) =
                    mx_pack4(acc[i][f][4 * q], acc[i][f][4 * q + 1], acc[i][f][4 * q + 2], acc[i][f][4 * q + 3]);
            wave_lds_fence();
            u32x4_t v[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
              v[kk] = *reinterpret_cast<const u32x4_t*>((kk < 2 ? stg : s_stage[wave - 4]) +
                                                        stg128(8 * (kk & 1) + (lane >> 3), lane & 7));
            wave_lds_fence();
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
              const int m = m0r + 8 * kk + (lane >> 3), c = lane & 7;
              if (m < cm_end && c < valid) sto(p.C + (int64_t)m * p.N + n0w + c * 8, v[kk]);
            }
          }
        }
        kbarrier();  // the copying waves' rows are in LDS
        if (!loader) {
          const int m0r = cm0 + wm_s * 128 + ph * 64;
          const int n0w = cn0 + wn_s * 64;
          const int valid = min(8, (p.N - n0w) >> 3);
          u32x4_t v[8];  // reads first, then the masked stores
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = *reinterpret_cast<const u32x4_t*>(xr + stg128(8 * j + (lane >> 3), lane & 7));
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int m = m0r + 8 * j + (lane >> 3), c = lane & 7;
            if (m < cm_end && c < valid) sto(p.C + (int64_t)m * p.N + n0w + c * 8, v[j]);
          }
        }
        kbarrier();  // read back: the region may be written again
      }
      if (more && MXN - 1 < nk) issue_loads(MXN - 1);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m0r = cm0 + wm * 128 + i * 32;
        const int c0 = cn0 + wn * 32;
        u32x2_t pk[4];  // this lane's 16 outputs, rounded to bf16: columns 8q + 4*hh + 0..3
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float a[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) a[u] = silu_f(acc[i][0][4 * q + u]) * acc[i][1][4 * q + u];
          pk[q] = mx_pack4(a[0], a[1], a[2], a[3]);
        }
        if (p.C) {
#pragma unroll
          for (int q = 0; q < 4; ++q) *reinterpret_cast<u32x2_t*>(stg + stg64(r, q) + hh * 8) = pk[q];
          const int valid = min(4, (mlp - c0) >> 3);
          wave_lds_fence();
          u32x4_t v[2];
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) v[k2] = *reinterpret_cast<const u32x4_t*>(stg + stg64(16 * k2 + (lane >> 2), lane & 3));
          wave_lds_fence();
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const int m = m0r + 16 * k2 + (lane >> 2), c = lane & 3;
            if (m < cm_end && c < valid) st16(p.C + (int64_t)m * mlp + c0 + c * 8, v[k2]);
          }
        }
        if (p.Cq && c0 < mlp) {
          // The wave's 32 columns are one MXFP8 block of each row (c0 is a multiple of 32 and mlp of 64):
          // quantize the bf16-rounded outputs, the same values moe_mx_quantize_rows would read back.
          float v[16];
          uint32_t am = 0;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v[4 * q] = bf16_lo(pk[q][0]);
            v[4 * q + 1] = bf16_hi(pk[q][0]);
            v[4 * q + 2] = bf16_lo(pk[q][1]);
            v[4 * q + 3] = bf16_hi(pk[q][1]);
#pragma unroll
            for (int u = 0; u < 4; ++u) am = max(am, __float_as_uint(v[4 * q + u]) & 0x7fffffffu);
          }
          am = max(am, (uint32_t)__shfl_xor((int)am, 32));  // the row's other 16 columns
          const int sc = mx_e8m0_code(am);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int ex = 127 - sc;
            const uint32_t word = mx_e4m3_x4(ldexpf(v[4 * q], ex), ldexpf(v[4 * q + 1], ex), ldexpf(v[4 * q + 2], ex),
                                             ldexpf(v[4 * q + 3], ex));
            *reinterpret_cast<uint32_t*>(stg + 1024 + r * 32 + 8 * q + 4 * hh) = word;  // [32 rows][32 codes]
          }
          wave_lds_fence();
          {
            const int rr = lane >> 1, c = lane & 1;
            const u32x4_t w = *reinterpret_cast<const u32x4_t*>(stg + 1024 + rr * 32 + c * 16);
            wave_lds_fence();
            const int m = m0r + rr;
            if (m < cm_end) st16(p.Cq + (int64_t)m * mlp + c0 + c * 16, w);
          }
          const int m = m0r + r;
          if (hh == 0 && m < cm_end) p.Cqs[((int64_t)(c0 >> 6) * p.M + m) * 4 + ((c0 >> 5) & 1)] = (uint8_t)sc;
        }
      }
    }
    if (!more) break;
  }
}

}  // namespace

hipError_t launch_grouped_gemm_mx(int epilogue, const uint8_t* A, const uint8_t* As, int64_t a_rows,
                                  const int32_t* row_slot, int slot_div, const uint8_t* B, const uint8_t* Bs,
                                  const int32_t* group_offsets, int E, int64_t M, int K, int N, uint16_t* C,
                                  uint8_t* Cq, uint8_t* Cqs, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  MxGemmP p{A, As, row_slot, B, Bs, group_offsets, C, Cq, Cqs, E, (int)M, K, N, (int)a_rows, slot_div};
  int g = device_cu_count();
  g -= g % kNumXcd;
  if (g < kNumXcd) g = kNumXcd;
  const dim3 grid(g), block(MXT);
  if (epilogue == MXE_SWIGLU) {
    if (row_slot) mx_gemm_kernel<MXE_SWIGLU, true><<<grid, block, 0, stream>>>(p);
    else mx_gemm_kernel<MXE_SWIGLU, false><<<grid, block, 0, stream>>>(p);
  } else {
    if (row_slot) mx_gemm_kernel<MXE_NONE, true><<<grid, block, 0, stream>>>(p);
    else mx_gemm_kernel<MXE_NONE, false><<<grid, block, 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace moe
