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
//  - Workgroup tile 256 x 256, k-slice 32, 8 waves in 2 (M) x 4 (N); each wave
//    owns 128 x 64 outputs = 4 x 2 MFMA 32x32x16 bf16 blocks (128 fp32
//    accumulators per lane), which leaves room for two waves per SIMD.
//  - Operands go global -> LDS with direct loads (global_load_lds_dwordx4,
//    1 KB per instruction) into a ring of four LDS stages, so three k-slices
//    are in flight ahead of the one being multiplied.
//  - [k][n]-major tiles (the NN weight, both wgrad operands) are read with the
//    gfx950 transposed LDS read ds_read_b64_tr_b16, [row][k]-major tiles with
//    ds_read_b128. Both layouts are XOR-swizzled on 16-byte chunks for the
//    64-bank LDS. The swizzle is applied to the global address each lane
//    copies, since a direct load writes 1 KB of LDS contiguously.
//  - LDS reads of the next 16-wide sub-slice are issued one per MFMA.
//  - The weight side is the MFMA's first operand, so each lane ends with four
//    consecutive output columns per register group. The epilogue stages each
//    32 x 32 block through LDS and stores whole 64-byte row segments.
//  - Persistent grid of one workgroup per CU. Each workgroup derives the
//    ragged tile list from the device-side group offsets itself (no host
//    sync). Tiles are numbered expert-major and dealt so that each XCD works
//    on a contiguous run of tiles that share A and B panels in its L2; the
//    first k-slices of a workgroup's next tile are loaded during the epilogue
//    of the current one.
//  - Waves 0-3 issue all operand copies and waves 4-7 all output stores
//    (non-temporal), so no wave's vmcnt waits cover stores; the copying
//    waves' output reaches the storing waves through the last ring stage.
//  - A wave whose 128 rows lie past the group end skips its MFMAs, and one
//    with at most 64 output rows multiplies only its first two 32-row blocks.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int BM = 256, BN = 256;

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

// LDS swizzle of [k][n] tiles, 512-byte rows of 32 16-byte chunks (NN weight
// [32][256], wgrad [64][256]): a transposed read covers 4 k-rows x 64 bytes
// per 16 lanes, and physical chunk = c ^ ((k & 3) << 2) moves each of those
// k-rows to its own quarter of the 256-byte bank window.
__device__ __forceinline__ int off_n32(int krow, int c) { return krow * 512 + ((c ^ ((krow & 3) << 2)) << 4); }

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

// Direct global->LDS copy, 16 bytes per lane: lane L's 16 bytes at sbase + voff
// land at LDS byte address lds + 16 L (global_load_lds_dwordx4, M0 = lds).
// Issued from inline asm, so the compiler's wait-count tracking does not order
// later LDS reads behind it; the kernel waits on vmcnt itself before the
// barrier that publishes a stage.
__device__ __forceinline__ void g2lds16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(lds) : "memory");
}
__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_vm_8() { asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); }
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// Opaque copy of a value: stops the compiler hoisting per-lane values computed
// from it out of the persistent tile loop (they would stay live, and spill,
// across every tile); they are recomputed per tile instead.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}
template <class T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const T*)(((uint64_t)hi << 32) | lo);
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

// Column base (within the 256-wide B tile) of N-fragment f (0, 1) of wave column wn (0..3).
// SwiGLU: fragment 0 holds 32 gate columns and fragment 1 the matching 32 up columns.
template <int EPI>
__device__ __forceinline__ int frag_col8(int wn, int f) {
  if (EPI == EPI_SWIGLU) return f == 0 ? wn * 32 : 128 + wn * 32;
  return wn * 64 + f * 32;
}

// Block-wide inclusive scan of one int per thread (NW waves); s_wsum holds NW ints.
template <int NW>
__device__ __forceinline__ int block_incl_scan_n(int v, int* s_wsum) {
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

constexpr int GTHR = 512;  // 8 waves: 2 along M x 4 along N, each wave 128 x 64
constexpr int GBK = 32;    // k-slice
constexpr int NST = 4;     // LDS stages (three k-slices in flight ahead of the one in use)
constexpr int kOpStage = 256 * GBK * 2;      // one operand, one stage: 16 KB
constexpr int kGemmLds = 2 * NST * kOpStage;  // 128 KB

// [row][k] tiles of 64-byte rows (A [BM][32], NT-B [BN][32]): four 16-byte chunks
// per row; a ds_read_b128 of 16 lanes covers 16 consecutive rows at one chunk,
// and c ^ ((row >> 2) & 3) spreads the four rows that share a 64-byte bank
// quarter over the four chunks.
__device__ __forceinline__ int off_k4(int row, int c) { return row * 64 + ((c ^ ((row >> 2) & 3)) << 4); }
// MFMA operand from a [row][k] tile: lane l gets row rbase + l%32, k values k0 + 8*(l/32) + 0..7.
__device__ __forceinline__ bf16x8_t frag_k4(const uint8_t* tile, int lane, int k0, int rbase) {
  return lds_rd16(tile, off_k4(rbase + (lane & 31), (k0 >> 3) + (lane >> 5)));
}
__device__ __forceinline__ void wait_vm_4() { asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); }

// GATHER: the A rows are read in place through p.row_slot. SCALE: every output row is scaled by
// p.slot_scale (indexed through p.row_slot with GATHER, else by the row). Separate instances, so that a
// scale without a gather never touches p.row_slot and a gather without a scale multiplies by nothing.
template <int OP, int EPI, bool GATHER, bool SCALE>
__global__ __launch_bounds__(GTHR, 1) void gemm_kernel(GemmP p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kGemmLds];
  // Output staging: 2 KB per wave, 32 rows x 64 bytes of the wave's output at a time.
  __shared__ __attribute__((aligned(16))) uint8_t s_stage[GTHR / 64][2048];
  __shared__ int s_lo[kMaxExperts + 1], s_pref[kMaxExperts + 1], s_wsum[8];
  const int mlp = EPI == EPI_SWIGLU ? p.N / 2 : p.N;
  const int tile_n = EPI == EPI_SWIGLU ? 128 : BN;
  const int ntn = (mlp + tile_n - 1) / tile_n;

  {  // ragged tile list: tiles of expert e = ceil(rows_e / BM) * ntn, prefix over experts
    const int tid = threadIdx.x;
    int tiles = 0;
    if (tid <= p.E) s_lo[tid] = clamp_rows(p.off[tid], p.M);
    if (tid < p.E) tiles = group_tiles(clamp_rows(p.off[tid + 1], p.M) - clamp_rows(p.off[tid], p.M), ntn);
    const int incl = block_incl_scan_n<GTHR / 64>(tiles, s_wsum);
    if (tid < p.E) s_pref[tid + 1] = incl;
    if (tid == 0) s_pref[0] = 0;
    __syncthreads();
  }
  const int total = s_pref[p.E];
  uint8_t* const As0 = smem;
  uint8_t* const Bs0 = smem + NST * kOpStage;

  // Loader: direct global->LDS copies, 1 KB per instruction (64 lanes x 16 B,
  // lane L at LDS base + 16 L); the swizzle is applied to the global address
  // each lane reads. Per wave 2 instructions per operand per k-slice; block
  // b = 2*wave + j of 1 KB:
  //  [row][k] tiles: rows 16b .. 16b+15; lane L -> row 16b + L/4, physical chunk
  //    L%4, logical chunk (L%4) ^ ((row >> 2) & 3).
  //  [k][n] tiles: k-rows 2b, 2b+1; lane L -> k-row 2b + L/32, physical chunk
  //    L%32, logical chunk (L%32) ^ ((k-row & 3) << 2).
  // Rows past the group end are clamped to its last row and columns past N to a
  // valid column: both only feed outputs that are never stored. With a row
  // gather, A rows are read in place through the slot index.
  const int tid = opaque((int)threadIdx.x), lane = tid & 63, wave = tid >> 6;
  // Wave w owns rows 128 * (w / 4) and columns 64 * (w % 4) of the tile
  // (wave-to-SIMD placement is w % 4), so every SIMD holds one wave of each
  // row half; a wave multiplies only its 32-row blocks that hold a row before
  // the group end, and one whose 128 rows all lie past it skips its MFMAs.
  const int wm = wave >> 2, wn = wave & 3;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // Roles (every epilogue but the SwiGLU backward, which copies h through the
  // ring): waves 0-3 issue all operand copies and no global store; waves 4-7
  // issue all global stores (their own output, and that of waves 0-3 after
  // it crosses one LDS stage) and no copy. vmcnt counts a wave's loads and
  // stores together, so in a wave that does both, the wait for a k-slice
  // issued after the previous tile's stores also waits for those stores: all
  // workgroups store at about the same moment, and that burst held up the
  // next tile (measured: the stores cost the wo GEMM half its time on the
  // 32768-token workload). With the roles split, the copying waves' waits
  // cover copies only and the stores drain while the next tile computes.
  constexpr bool SPLIT = EPI != EPI_SWIGLU_BWD;
  constexpr int LPW = SPLIT ? 4 : 2;  // 1 KB copies per operand, k-slice and copying wave
  const bool loader = !SPLIT || wave_u < 4;
  const uint32_t lds_a = lds_addr(As0) + wave_u * LPW * 1024, lds_b = lds_addr(Bs0) + wave_u * LPW * 1024;
  const int nk = p.K / GBK;
  int m0, m_end, m_cls, n0;  // tile rows [m0, m_end); m_cls sets the waves' multiply class
  const uint16_t *Ab, *Bexp;
  uint32_t a_off[LPW], b_off[LPW];
  // the copies of a k-slice have landed once at most those of the n k-slices
  // issued after it are outstanding (2 * LPW per k-slice); any stores in
  // between would only make the wait longer
  auto wait_loads_after = [](int n) {
    if (LPW == 4) {
      if (n >= 3) asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
      else if (n == 2) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      else if (n == 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
      if (n >= 2) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else if (n == 1) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
  };
  // workgroup barrier after this wave's LDS reads have completed; unlike
  // __syncthreads it does not wait for the wave's outstanding global stores
  auto kbarrier = []() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  // Tile `it` of this workgroup -> m0, m_end, n0, operand bases and per-lane offsets.
  auto decode = [&](int64_t it) -> bool {
    const int64_t tl = xcd_tile(it, blockIdx.x, gridDim.x);
    if (tl >= total) return false;
    // Tile order inside an expert (ragged_tile): with 4 or more row blocks the
    // row block varies fastest (measured: wo GEMM 1.01 -> 0.97 ms at 128
    // experts of ~2048 rows, K = 768); with 1 or 3 row blocks the column tile
    // varies fastest (the other order cost 12 % at 256 experts of ~256 rows,
    // K = 7168); with 2 row blocks the two equal halves of a column are adjacent.
    const RaggedTile rt = ragged_tile((int)tl, s_pref, p.E, ntn);
    const int e = rt.e, mt = rt.mt, nt = rt.nt;
    {  // a group of 257-512 rows runs as two equal halves (tile_rows)
      int r0, r1, rc;
      tile_rows(s_lo[e], max(s_lo[e + 1], s_lo[e]), mt, &r0, &r1, &rc);
      m0 = __builtin_amdgcn_readfirstlane(r0);
      m_end = __builtin_amdgcn_readfirstlane(r1);
      m_cls = __builtin_amdgcn_readfirstlane(rc);
    }
    n0 = __builtin_amdgcn_readfirstlane(nt * tile_n);
    Bexp = uniform_ptr(p.B + (int64_t)__builtin_amdgcn_readfirstlane(e) * p.K * p.N);
    Ab = GATHER ? p.A : uniform_ptr(p.A + (int64_t)m0 * p.K);
    if (!loader) return true;
    if (GATHER) {
      // all LPW slot loads first, into a_off itself (the current tile's offsets are dead by now and
      // few other registers are free with the accumulators live), then their conversion: loaded and
      // used one at a time they cost LPW round trips
#pragma unroll
      for (int j = 0; j < LPW; ++j) {
        const int row = (wave_u * LPW + j) * 16 + (lane >> 2);
        a_off[j] = (uint32_t)p.row_slot[min(m0 + row, m_end - 1)];
      }
#pragma unroll
      for (int j = 0; j < LPW; ++j) {
        const int row = (wave_u * LPW + j) * 16 + (lane >> 2);
        const int c = (lane & 3) ^ ((row >> 2) & 3);
        const int s = min(max((int)a_off[j], 0), p.n_slots - 1);
        a_off[j] = (uint32_t)((s / p.slot_div) * p.K + c * 8) * 2u;
      }
    } else {
#pragma unroll
      for (int j = 0; j < LPW; ++j) {
        const int row = (wave_u * LPW + j) * 16 + (lane >> 2);
        const int c = (lane & 3) ^ ((row >> 2) & 3);
        const int r = min(m0 + row, m_end - 1);
        a_off[j] = (uint32_t)((r - m0) * p.K + c * 8) * 2u;
      }
    }
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      if (OP == OP_NT) {
        const int row = (wave_u * LPW + j) * 16 + (lane >> 2);
        const int c = (lane & 3) ^ ((row >> 2) & 3);
        b_off[j] = (uint32_t)(min(n0 + row, p.N - 1) * p.K + c * 8) * 2u;
      } else {
        const int krow = (wave_u * LPW + j) * 2 + (lane >> 5);
        const int c = (lane & 31) ^ ((krow & 3) << 2);
        int col;
        if (EPI == EPI_SWIGLU) {
          const int cc = c < 16 ? n0 + c * 8 : n0 + (c - 16) * 8;
          col = cc < mlp ? (c < 16 ? cc : mlp + cc) : 0;
        } else {
          col = n0 + c * 8;
          col = col < p.N ? col : 0;
        }
        b_off[j] = (uint32_t)(krow * p.N + col) * 2u;
      }
    }
    return true;
  };
  auto issue_loads = [&](int kt) {
    if (!loader) return;
    const int k0 = kt * GBK;
    const uint16_t* Ak = Ab + k0;
    const uint16_t* Bk = OP == OP_NT ? Bexp + k0 : Bexp + (int64_t)k0 * p.N;
    const uint32_t st = (uint32_t)(kt & (NST - 1)) * kOpStage;
#pragma unroll
    for (int j = 0; j < LPW; ++j) g2lds16(Ak, a_off[j], lds_a + st + j * 1024);
#pragma unroll
    for (int j = 0; j < LPW; ++j) g2lds16(Bk, b_off[j], lds_b + st + j * 1024);
  };

  // The first NST k-slices of a tile are issued before the previous tile's
  // epilogue (every stage is free once its last barrier has passed), so their
  // latency overlaps the epilogue's math and stores.
  if (!decode(0)) return;
  for (int s = 0; s < NST; ++s)
    if (s < nk) issue_loads(s);
  for (int64_t it = 0;; ++it) {
    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][f][r] = 0.0f;

    bf16x8_t af[2][4], bf[2][2];
    // NI: the 32-row blocks of the wave that are multiplied, those holding a
    // row before the group end (1 to 4)
    auto read_frags = [&](auto NIc, int stage, int ks, int set) {
      constexpr int NI = decltype(NIc)::value;
      const uint8_t* As = As0 + stage * kOpStage;
      const uint8_t* Bs = Bs0 + stage * kOpStage;
#pragma unroll
      for (int i = 0; i < NI; ++i) af[set][i] = frag_k4(As, lane, ks * 16, wm * 128 + i * 32);
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        if (OP == OP_NT) bf[set][f] = frag_k4(Bs, lane, ks * 16, frag_col8<EPI>(wn, f));
        else bf[set][f] = frag_tr(Bs, lane, ks * 16, frag_col8<EPI>(wn, f));
      }
    };
    auto mfmas = [&](auto NIc, int set) {
      constexpr int NI = decltype(NIc)::value;
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int f = 0; f < 2; ++f) acc[i][f] = mfma(bf[set][f], af[set][i], acc[i][f]);
    };
    // Issue order inside a 16-wide sub-slice: one MFMA, then one LDS read of the
    // next sub-slice's fragments (two per MFMA with two row blocks, three with one).
    auto interleave = [&](auto NIc) {
      constexpr int NI = decltype(NIc)::value;
#pragma unroll
      for (int j = 0; j < 2 * NI; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, NI >= 3 ? 1 : (NI == 2 ? 2 : 3), 0);
      }
    };

    if (SPLIT) {
      if (loader) wait_loads_after(min(nk, NST) - 1);  // the tile's first k-slice has landed
      kbarrier();
    } else {
      wait_vm_all();  // this wave's loads of the first k-slices (and the last tile's stores) are done
      __syncthreads();
    }
    // rows of this tile that count for the multiply, from this wave's first row (wave-uniform)
    const int wrows = m_cls - (m0 + (wave_u >> 2) * 128);
    using NI4 = std::integral_constant<int, 4>;
    using NI3 = std::integral_constant<int, 3>;
    using NI2 = std::integral_constant<int, 2>;
    using NI1 = std::integral_constant<int, 1>;
    // k-slice kt on stage kt % NST. On entry its first 16-wide sub-slice is in
    // fragment set 0. The barrier sits before the second sub-slice: every wave
    // then holds all of stage kt % NST in registers, so the loads of k-slice
    // kt + NST can go into it during the second sub-slice, and k-slice kt+1
    // (issued NST-1 k-slices ago) must have landed. The next stage's first fragments are read under
    // the second sub-slice's MFMAs (also on the last k-slice, where they go
    // unused: it keeps the body one basic block).
    // wait for k-slice kt+1 (the loads issued after it: k-slices kt+2 and kt+3, where they exist), then barrier
    auto kwait = [&](int kt) {
      if (SPLIT) {
        if (loader) wait_loads_after(kt + 3 < nk ? 2 : (kt + 2 < nk ? 1 : 0));
        kbarrier();
      } else {
        if (kt + 3 < nk) wait_vm_8();
        else if (kt + 2 < nk) wait_vm_4();
        else wait_vm_all();
        __syncthreads();
      }
    };
    // Second sub-slice of k-slice kt: per row block i, its two MFMAs, then the read of
    // block i of the next stage's first fragments (and of one B fragment every other
    // block), then one A copy of k-slice kt + NST; the B copies follow the last MFMA.
    // Issued as one burst after the barrier (the first form), a copying wave's eight
    // copies held back its MFMAs until the last of them was accepted. Measured,
    // alternating on one box (32768-token workload, DeepSeek-V3 shape in brackets):
    // GEMM1 1.463 -> 1.437 ms (4.66 -> 4.57), GEMM2 0.964 -> 0.954 (2.465 -> 2.43).
    // Spreading the B copies over the MFMAs as well, one per MFMA or across both
    // sub-slices, was slower than the burst form.
    auto second_half = [&](auto NIc, int kt) {
      constexpr int NI = decltype(NIc)::value;
      const int nst = (kt + 1) & (NST - 1);
      const uint8_t* As = As0 + nst * kOpStage;
      const uint8_t* Bs = Bs0 + nst * kOpStage;
      const int kn = kt + NST;
      const bool cp = loader && kn < nk;
      const uint16_t* Ak = Ab + kn * GBK;
      const uint16_t* Bk = OP == OP_NT ? Bexp + kn * GBK : Bexp + (int64_t)(kn * GBK) * p.N;
      const uint32_t cst = (uint32_t)(kn & (NST - 1)) * kOpStage;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
#pragma unroll
        for (int f = 0; f < 2; ++f) acc[i][f] = mfma(bf[1][f], af[1][i], acc[i][f]);
        af[0][i] = frag_k4(As, lane, 0, wm * 128 + i * 32);
        if (i & 1) {
          const int f = i >> 1;
          if (OP == OP_NT) bf[0][f] = frag_k4(Bs, lane, 0, frag_col8<EPI>(wn, f));
          else bf[0][f] = frag_tr(Bs, lane, 0, frag_col8<EPI>(wn, f));
        }
        if (cp && i < LPW) g2lds16(Ak, a_off[i], lds_a + cst + i * 1024);
      }
#pragma unroll
      for (int f = NI / 2; f < 2; ++f) {  // the B fragments not read between the MFMAs
        if (OP == OP_NT) bf[0][f] = frag_k4(Bs, lane, 0, frag_col8<EPI>(wn, f));
        else bf[0][f] = frag_tr(Bs, lane, 0, frag_col8<EPI>(wn, f));
      }
      if (cp) {
#pragma unroll
        for (int j = NI; j < LPW; ++j) g2lds16(Ak, a_off[j], lds_a + cst + j * 1024);
#pragma unroll
        for (int j = 0; j < LPW; ++j) g2lds16(Bk, b_off[j], lds_b + cst + j * 1024);
      }
    };
    auto kloop = [&](auto NIc) {
      read_frags(NIc, 0, 0, 0);
      for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & (NST - 1);
        read_frags(NIc, st, 1, 1);
        mfmas(NIc, 0);
        interleave(NIc);
        kwait(kt);
        second_half(NIc, kt);
      }
    };
    if (wrows > 96) {
      kloop(NI4{});
    } else if (wrows > 64) {
      kloop(NI3{});  // blocks from NI on keep their zero accumulators; their rows are not stored
    } else if (wrows > 32) {
      kloop(NI2{});
    } else if (wrows > 0) {
      kloop(NI1{});
    } else {
      // no output rows: keep the copies and barriers of the k-loop only
      for (int kt = 0; kt < nk; ++kt) {
        kwait(kt);
        if (kt + NST < nk) issue_loads(kt + NST);
      }
    }

    // Next tile's first loads go out now; this tile's rows and columns are kept for the epilogue.
    const int cm0 = m0, cm_end = m_end, cn0 = n0;
    // optional per-row fp32 scale (the top-k weight of the row's slot), applied as values are read;
    // fetched before the prefetch so that its wait does not cover the next tile's loads
    float sc4[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    if (SCALE) {  // the four indices, then the four scales: two round trips
      int si[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) si[i] = min(cm0 + wm * 128 + i * 32 + (lane & 31), cm_end - 1);
      if (GATHER) {
#pragma unroll
        for (int i = 0; i < 4; ++i) si[i] = p.row_slot[si[i]];
#pragma unroll
        for (int i = 0; i < 4; ++i) si[i] = min(max(si[i], 0), p.n_slots - 1);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sc4[i] = p.slot_scale[si[i]];
    }
    // The scales are consumed here, before the copies go out. The copies are inline asm, which the
    // compiler does not count, so a first use in the epilogue would carry a vmcnt wait sized for the
    // compiler's own loads, covering the copies too; and since the loads are conditional, that wait
    // (and any reuse of their registers, even in the next k-loop) was kept on both paths.
    if (SCALE) {
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(sc4[i]));
    }
    const bool more = decode(it + 1);
    // The last stage carries the copying waves' output to the storing waves
    // and is loaded after the epilogue (the SwiGLU backward uses the whole
    // ring in its epilogue and issues all of these afterwards).
    if (SPLIT && more)
      for (int s = 0; s < NST - 1; ++s)
        if (s < nk) issue_loads(s);
    // Copying wave w's output crosses in an 8 KB region of stage NST-1 (w < 2:
    // the A half, else the B half); storing wave w + 4 moves it to memory.
    const int src = wave_u & 3;  // the copying wave whose output this wave handles
    uint8_t* const xr = (src < 2 ? As0 : Bs0) + (NST - 1) * kOpStage + (src & 1) * 8192;
    const int wm_s = src >> 2, wn_s = src & 3;
    // Epilogue. Lane holds rows m = tile row + lane%32 and, per register group q,
    // four consecutive columns 8q + 4*(lane/32) + 0..3 of each 32-wide fragment.
    // NONE and SWIGLU pass their output through this wave's 2 KB LDS staging
    // area and store whole row segments (128 B for NONE, 64 B for the SwiGLU
    // output): stores straight from the MFMA layout would write 8 bytes into
    // each of 32 rows per instruction.
    const int hh = lane >> 5;
    uint8_t* const stg = s_stage[wave];
    // [32 rows][64 B] block, 16-byte chunk c of row r at r*64 + ((c ^ ((r >> 2) & 3)) << 4)
    auto stg64 = [&](int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); };
    // [16 rows][128 B] block: r*128 + ((c ^ ((r >> 1) & 7)) << 4)
    auto stg128 = [&](int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); };
    const int r = lane & 31;
    // Output stores. With the roles split they are non-temporal: the output
    // is not read again by this kernel, and streaming it past L2 keeps the
    // operand panels there (measured: wo GEMM 1.020 -> 1.002 ms, GEMM 1
    // 1.539 -> 1.534 ms on the 32768-token workload).
    auto sto = [&](void* ptr, u32x4_t v) {
      if (SPLIT) __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(ptr));
      else st16(ptr, v);
    };
    // Read the staged block back, four lanes per row, and store rows m0r + 0..31,
    // 16 bytes at column byte offset 16 * (lane % 4) from row_ptr(m).
    auto drain = [&](int m0r, auto row_ptr, int valid_chunks) {
      wave_lds_fence();
      u32x4_t v[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) v[k] = *reinterpret_cast<const u32x4_t*>(stg + stg64(16 * k + (lane >> 2), lane & 3));
      wave_lds_fence();
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int m = m0r + 16 * k + (lane >> 2), c = lane & 3;
        if (m < cm_end && c < valid_chunks) sto(reinterpret_cast<uint16_t*>(row_ptr(m)) + c * 8, v[k]);
      }
    };
    // A copying wave's output crosses as [rows][bytes] in its region xr, 16-byte
    // chunk c of row rr at rr*128 + ((c ^ ((rr >> 1) & 7)) << 4) for the plain
    // output (64 rows of 128 B per phase) and rr*64 + ((c ^ ((rr >> 2) & 3)) << 4)
    // for the SwiGLU output (128 rows of 64 B); each storing wave reads it back
    // in whole row segments.
    auto xoff128 = [](int rr, int c) { return rr * 128 + ((c ^ ((rr >> 1) & 7)) << 4); };
    auto xoff64 = [](int rr, int c) { return rr * 64 + ((c ^ ((rr >> 2) & 3)) << 4); };
    if (EPI == EPI_NONE) {
#pragma unroll
      for (int ph = 0; ph < 2; ++ph) {
        if (loader) {
          // rows 64ph .. 64ph + 63 of this wave's 128 x 64 output block
#pragma unroll
          for (int ii = 0; ii < 2; ++ii) {
            const int i = 2 * ph + ii;
            const float sc = sc4[i];
            const int rr = ii * 32 + r;
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
              for (int q = 0; q < 4; ++q)
                *reinterpret_cast<u32x2_t*>(xr + xoff128(rr, f * 4 + q) + hh * 8) =
                    pack4(sc * acc[i][f][4 * q], sc * acc[i][f][4 * q + 1], sc * acc[i][f][4 * q + 2],
                          sc * acc[i][f][4 * q + 3]);
          }
        } else if (ph == 0) {
          // the storing wave's own output: both 32-column fragments form
          // 128-byte row segments, staged 32 rows at a time, 8 lanes per row
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float sc = sc4[i];
            const int m0r = cm0 + wm * 128 + i * 32;
            const int n0w = cn0 + wn * 64;
            const int valid = min(8, (p.N - n0w) >> 3);
            // the whole 32-row block at once: rows 0-15 in this wave's 2 KB, rows 16-31 in
            // that of its copying wave, which this epilogue leaves unused (four rounds per
            // tile instead of eight; 32768-token GEMM2 0.944 -> 0.933 ms, alternating)
            uint8_t* const wb = r < 16 ? stg : s_stage[wave - 4];
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
              for (int q = 0; q < 4; ++q)
                *reinterpret_cast<u32x2_t*>(wb + stg128(r & 15, f * 4 + q) + hh * 8) =
                    pack4(sc * acc[i][f][4 * q], sc * acc[i][f][4 * q + 1], sc * acc[i][f][4 * q + 2],
                          sc * acc[i][f][4 * q + 3]);
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
          // all eight reads go out before the first store: a read waited just
          // before its own masked store would serialize the LDS latencies
          u32x4_t v[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = *reinterpret_cast<const u32x4_t*>(xr + xoff128(8 * j + (lane >> 3), lane & 7));
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int m = m0r + 8 * j + (lane >> 3), c = lane & 7;
            if (m < cm_end && c < valid) sto(p.C + (int64_t)m * p.N + n0w + c * 8, v[j]);
          }
        }
        kbarrier();  // read back: the region may be written again
      }
    } else if (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sc = sc4[i];
        const int m0r = cm0 + wm * 128 + i * 32;
        const int c0 = cn0 + wn * 32;
        f32x4_t gv[4], uv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float a[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            gv[q][u] = sc * acc[i][0][4 * q + u];
            uv[q][u] = sc * acc[i][1][4 * q + u];
            a[u] = silu_f(gv[q][u]) * uv[q][u];
          }
          const u32x2_t pk = pack4(a[0], a[1], a[2], a[3]);
          if (loader) *reinterpret_cast<u32x2_t*>(xr + xoff64(i * 32 + r, q) + hh * 8) = pk;
          else *reinterpret_cast<u32x2_t*>(stg + stg64(r, q) + hh * 8) = pk;
        }
        if (!loader) drain(m0r, [&](int m) { return (void*)(p.C + (int64_t)m * mlp + c0); }, min(4, (mlp - c0) >> 3));
        if (p.aux_out) {  // h kept in fp32 for the backward: the gate/up values the SwiGLU used, unrounded
#pragma unroll
          for (int part = 0; part < 4; ++part) {  // gate cols 0-15, 16-31, then up cols 0-15, 16-31
            const int half = part >> 1, qq = part & 1;
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2)
              *reinterpret_cast<f32x4_t*>(stg + stg64(r, 2 * q2 + hh)) = half == 0 ? gv[2 * qq + q2] : uv[2 * qq + q2];
            const int cb = c0 + 16 * qq;
            // 16 fp32 columns = 64 bytes per row; valid 16-byte chunks of 4 columns
            drain(m0r, [&](int m) { return (void*)(p.aux_out + (int64_t)m * 2 * mlp + half * mlp + cb); },
                  min(4, (mlp - cb) >> 2));
          }
        }
      }
      kbarrier();  // the copying waves' rows are in LDS
      if (!loader) {
        const int m0r = cm0 + wm_s * 128;
        const int c0 = cn0 + wn_s * 32;
        const int valid = min(4, (mlp - c0) >> 3);
        u32x4_t v[8];  // reads first, then the masked stores
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = *reinterpret_cast<const u32x4_t*>(xr + xoff64(16 * j + (lane >> 2), lane & 3));
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int m = m0r + 16 * j + (lane >> 2), c = lane & 3;
          if (m < cm_end && c < valid) sto(p.C + (int64_t)m * mlp + c0 + c * 8, v[j]);
        }
      }
      kbarrier();  // read back: the stage may be loaded
    } else {
      // EPI_SWIGLU_BWD: N = mlp, aux = saved h [M, 2N] fp32, C = dh [M, 2N] bf16.
      // Work unit (i, f): the 32 x 32 accumulator block acc[i][f]. Its gate and
      // up values (32 fp32 columns of each, 128 bytes per row) are copied by
      // direct loads, eight lanes per 128-byte row segment, into one half of
      // this wave's 16 KB share of the operand ring, which is idle until the
      // next tile's loads go out; the copy of unit u + 1 is in flight while
      // unit u is computed. Reading h straight from the accumulator layout
      // would fetch 16 bytes from each of 32 rows per instruction. Region
      // layout: [gate | up] x [32 rows][128 B], 16-byte chunk c of row r at
      // r*128 + ((c ^ ((r >> 1) & 7)) << 4), so the accumulator-layout reads
      // (16 rows at one chunk per 16 lanes) hit distinct banks. dgate and dup
      // leave through the 2 KB staging area as 64-byte row segments.
      __syncthreads();  // every wave has read its last fragments from the ring
      const int wm_u = wave_u >> 2, wn_u = wave_u & 3;
      const int nunits = 2 * min(4, max(0, (cm_end - (cm0 + wm_u * 128) + 31) / 32));  // wave-uniform
      const uint32_t hreg = lds_addr(smem) + wave_u * 16384;
      auto issue_h = [&](int u) {
        const int m0r = cm0 + wm_u * 128 + (u >> 1) * 32;
        const int cf = cn0 + wn_u * 64 + (u & 1) * 32;
        const float* rowbase = uniform_ptr(p.aux_in + (int64_t)m0r * 2 * p.N);
        const uint32_t dst = hreg + (u & 1) * 8192;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = 8 * j + (lane >> 3);
          const int lc = (lane & 7) ^ ((row >> 1) & 7);
          const int rl = min(m0r + row, cm_end - 1) - m0r;
          int col = cf + 4 * lc;
          col = col < p.N ? col : 0;  // columns past N feed outputs that are never stored
          const uint32_t voff = (uint32_t)(rl * 2 * p.N + col) * 4u;
          g2lds16(rowbase, voff, dst + j * 1024);
          g2lds16(rowbase, voff + (uint32_t)p.N * 4u, dst + 4096 + j * 1024);
        }
      };
      if (nunits > 0) issue_h(0);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (u < nunits) {
          if (u + 1 < nunits) {
            issue_h(u + 1);
            wait_vm_8();  // unit u's copies (older than unit u + 1's eight) have landed
          } else {
            wait_vm_all();
          }
          const int i = u >> 1, f = u & 1;
          const float sc = sc4[i];
          const int m0r = cm0 + wm * 128 + i * 32;
          const int cf = cn0 + wn * 64 + f * 32;
          const uint8_t* hb = smem + wave_u * 16384 + (u & 1) * 8192;
          u32x2_t dgp[4], dup[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int off = r * 128 + (((2 * q + hh) ^ ((r >> 1) & 7)) << 4);
            const f32x4_t g = *reinterpret_cast<const f32x4_t*>(hb + off);
            const f32x4_t uu = *reinterpret_cast<const f32x4_t*>(hb + 4096 + off);
            float dg[4], du[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float da = sc * acc[i][f][4 * q + e];
              const float s = sigmoid_f(g[e]);
              dg[e] = da * uu[e] * s * (1.0f + g[e] * (1.0f - s));
              du[e] = da * g[e] * s;
            }
            dgp[q] = pack4(dg[0], dg[1], dg[2], dg[3]);
            dup[q] = pack4(du[0], du[1], du[2], du[3]);
          }
          const int valid = min(4, (p.N - cf) >> 3);
#pragma unroll
          for (int q = 0; q < 4; ++q) *reinterpret_cast<u32x2_t*>(stg + stg64(r, q) + hh * 8) = dgp[q];
          drain(m0r, [&](int m) { return (void*)(p.C + (int64_t)m * 2 * p.N + cf); }, valid);
#pragma unroll
          for (int q = 0; q < 4; ++q) *reinterpret_cast<u32x2_t*>(stg + stg64(r, q) + hh * 8) = dup[q];
          drain(m0r, [&](int m) { return (void*)(p.C + (int64_t)m * 2 * p.N + p.N + cf); }, valid);
        }
      }
      __syncthreads();  // every wave is done with its share of the ring
      if (more)
        for (int s = 0; s < NST; ++s)
          if (s < nk) issue_loads(s);
    }
    if (SPLIT && more && NST - 1 < nk) issue_loads(NST - 1);
    if (!more) break;
  }
}

// dW[e] [P, Q] = sum over the rows r of group e of A[r]^T D[r]. The contraction
// runs over the group's rows, so both operands are [row][col] tiles that the
// MFMA reads transposed (ds_read_b64_tr_b16), like the NN weight of the
// forward GEMM. Same workgroup shape, LDS ring and staged epilogue as
// gemm_kernel; tiles are (expert, 256-row block of P, 256-column block of Q),
// dealt to the XCDs by expert, and the k-loop runs over the expert's own rows.
// Rows past the group end must add nothing: each k-slice is copied with
// buffer loads whose range is exactly the slice's valid rows, and the
// hardware writes zeros for out-of-range lanes. An empty group writes exact
// zeros.
typedef int i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4_t buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);                           // range in bytes
  r[3] = 0x00020000;                                                            // 32-bit data format
  return r;
}
// Buffer -> LDS copy, 16 bytes per lane (lane L at lds + 16 L): lanes whose
// offset is at or past the resource's range read zeros.
__device__ __forceinline__ void b2lds16(i32x4_t rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(rsrc), "s"(lds) : "memory");
}

__global__ __launch_bounds__(GTHR, 1) void wgrad_kernel(WgradP p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kGemmLds];
  __shared__ __attribute__((aligned(16))) uint8_t s_stage[GTHR / 64][2048];
  // group offsets, clamped to [0, M], read once: a tile's rows are then known
  // without a global load between two tiles
  __shared__ int s_off[kMaxExperts + 1];
  for (int i = threadIdx.x; i <= p.E; i += GTHR) s_off[i] = clamp_rows(p.off[i], p.M);
  __syncthreads();
  const int tp = (p.P + 255) / 256, tq = (p.Q + 255) / 256;
  uint8_t* const As0 = smem;
  uint8_t* const Ds0 = smem + NST * kOpStage;
  const int tid = opaque((int)threadIdx.x), lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // Copying waves 0-3 and storing waves 4-7, as in gemm_kernel: the output
  // (dW, several times the operands) leaves through waves that never wait
  // on vmcnt, and the copying waves' waits cover copies only.
  const bool loader = wave_u < 4;
  const uint32_t lds_a = lds_addr(As0) + wave_u * 4 * 1024, lds_d = lds_addr(Ds0) + wave_u * 4 * 1024;
  auto wait_loads_after = [](int n) {  // 8 copies per k-slice and copying wave
    if (n >= 3) asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
    else if (n == 2) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if (n == 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  auto kbarrier = []() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  // Per tile: expert e, output block (p0, q0), the group's rows [lo, lo + n), nk k-slices.
  // Loader (both operands [k][n] tiles of 32 rows x 512 bytes): block b = 2*wave + j
  // holds k-rows 2b, 2b+1; lane L -> k-row 2b + L/32, physical chunk L%32,
  // logical chunk (L%32) ^ ((k-row & 3) << 2). Columns past P or Q read other
  // bytes of the slice (or zeros) and only feed outputs that are never stored.
  int e = 0, p0 = 0, q0 = 0, lo = 0, n = 0, nk = 0;
  // copy j of a k-slice covers k-rows 8*wave + 2j + {0, 1}; copies j and j + 2
  // share the chunk swizzle ((2j + lane/32) & 3 repeats with period 2) and lie
  // 4 k-rows apart, so only j = 0, 1 are kept
  uint32_t a_off[2], d_off[2];
  // Tiles are dealt by expert (wgrad_tile): XCD x takes experts x, x + 8, ...,
  // so an expert's operand rows are read into one XCD's L2 rather than into
  // all eight; inside an expert the dimension with fewer 256-blocks varies
  // fastest, so its panels stay in L2 while the other dimension's stream past
  // once each.
  auto decode = [&](int64_t it) -> bool {
    WgradTile wt;
    if (!wgrad_tile(it, blockIdx.x, gridDim.x, p.E, tp, tq, &wt)) return false;
    e = __builtin_amdgcn_readfirstlane(wt.e);
    p0 = __builtin_amdgcn_readfirstlane(wt.pt * 256);
    q0 = __builtin_amdgcn_readfirstlane(wt.qt * 256);
    const int l0 = s_off[e], h0 = s_off[e + 1];
    lo = __builtin_amdgcn_readfirstlane(l0);
    n = __builtin_amdgcn_readfirstlane(h0 > l0 ? h0 - l0 : 0);
    nk = (n + GBK - 1) / GBK;
    if (!loader) return true;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int krow = (wave_u * 4 + j) * 2 + (lane >> 5);
      const int c = (lane & 31) ^ ((krow & 3) << 2);
      a_off[j] = (uint32_t)(krow * p.P + p0 + c * 8) * 2u;
      d_off[j] = (uint32_t)(krow * p.Q + q0 + c * 8) * 2u;
    }
    return true;
  };
  auto issue_loads = [&](int kt) {
    if (!loader) return;
    const int r0 = lo + kt * GBK, rows = min(GBK, n - kt * GBK);
    const i32x4_t ra = buffer_rsrc(p.A + (int64_t)r0 * p.P, (uint32_t)(rows * p.P * 2));
    const i32x4_t rd = buffer_rsrc(p.D + (int64_t)r0 * p.Q, (uint32_t)(rows * p.Q * 2));
    const uint32_t st = (uint32_t)(kt & (NST - 1)) * kOpStage;
#pragma unroll
    for (int j = 0; j < 4; ++j) b2lds16(ra, a_off[j & 1] + (uint32_t)((j >> 1) * 8 * p.P), lds_a + st + j * 1024);
#pragma unroll
    for (int j = 0; j < 4; ++j) b2lds16(rd, d_off[j & 1] + (uint32_t)((j >> 1) * 8 * p.Q), lds_d + st + j * 1024);
  };

  if (!decode(0)) return;
  for (int s = 0; s < NST; ++s)
    if (s < nk) issue_loads(s);
  for (int64_t it = 0;; ++it) {
    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][f][r] = 0.0f;

    bf16x8_t af[2][4], df[2][2];
    auto read_frags = [&](int stage, int ks, int set) {
      const uint8_t* As = As0 + stage * kOpStage;
      const uint8_t* Ds = Ds0 + stage * kOpStage;
#pragma unroll
      for (int i = 0; i < 4; ++i) af[set][i] = frag_tr(As, lane, ks * 16, wm * 128 + i * 32);
#pragma unroll
      for (int f = 0; f < 2; ++f) df[set][f] = frag_tr(Ds, lane, ks * 16, wn * 64 + f * 32);
    };
    auto mfmas = [&](int set) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int f = 0; f < 2; ++f) acc[i][f] = mfma(df[set][f], af[set][i], acc[i][f]);
    };
    // 12 transposed reads per 8 MFMAs: two reads after each of the first four MFMAs, one after the rest
    auto interleave = [&]() {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    };

    if (loader) wait_loads_after(min(nk, NST) - 1);  // the tile's first k-slice has landed
    kbarrier();
    read_frags(0, 0, 0);
    // same k-slice schedule as gemm_kernel
    for (int kt = 0; kt < nk; ++kt) {
      const int st = kt & (NST - 1);
      read_frags(st, 1, 1);
      mfmas(0);
      interleave();
      if (loader) wait_loads_after(kt + 3 < nk ? 2 : (kt + 2 < nk ? 1 : 0));
      kbarrier();
      {
        // second sub-slice, as in gemm_kernel: per row block i its two MFMAs, the next
        // stage's fragment reads, then one A copy of k-slice kt + NST; the D copies last
        const int nst = (kt + 1) & (NST - 1);
        const uint8_t* As = As0 + nst * kOpStage;
        const uint8_t* Ds = Ds0 + nst * kOpStage;
        const int kn = kt + NST;
        const bool cp = loader && kn < nk;
        const int r0 = lo + kn * GBK, rows = min(GBK, n - kn * GBK);
        const uint32_t cst = (uint32_t)(kn & (NST - 1)) * kOpStage;
        const i32x4_t ra = buffer_rsrc(p.A + (int64_t)r0 * p.P, (uint32_t)(rows * p.P * 2));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int f = 0; f < 2; ++f) acc[i][f] = mfma(df[1][f], af[1][i], acc[i][f]);
          af[0][i] = frag_tr(As, lane, 0, wm * 128 + i * 32);
          if (i & 1) df[0][i >> 1] = frag_tr(Ds, lane, 0, wn * 64 + (i >> 1) * 32);
          if (cp) b2lds16(ra, a_off[i & 1] + (uint32_t)((i >> 1) * 8 * p.P), lds_a + cst + i * 1024);
        }
        if (cp) {
          const i32x4_t rd = buffer_rsrc(p.D + (int64_t)r0 * p.Q, (uint32_t)(rows * p.Q * 2));
#pragma unroll
          for (int j = 0; j < 4; ++j) b2lds16(rd, d_off[j & 1] + (uint32_t)((j >> 1) * 8 * p.Q), lds_d + cst + j * 1024);
        }
      }
    }

    const int ce = e, cp0 = p0, cq0 = q0;
    const bool more = decode(it + 1);
    // the last stage carries the copying waves' output; it is loaded after the epilogue
    if (more)
      for (int s = 0; s < NST - 1; ++s)
        if (s < nk) issue_loads(s);
    // Epilogue: 128-byte row segments (a wave's 64 columns), non-temporal: the
    // output is several times the operands and is not read back here, so it
    // streams past L2 instead of evicting the operand panels the next tiles read.
    const int hh = lane >> 5, r = lane & 31;
    uint8_t* const stg = s_stage[wave];
    auto stg128 = [&](int rr, int c) { return rr * 128 + ((c ^ ((rr >> 1) & 7)) << 4); };
    uint16_t* const Ce = p.C + (int64_t)ce * p.P * p.Q;
    // copying wave src's output crosses in 8 KB of stage NST-1, 64 rows x 128 B per phase
    const int src = wave_u & 3;
    uint8_t* const xr = (src < 2 ? As0 : Ds0) + (NST - 1) * kOpStage + (src & 1) * 8192;
    const int wm_s = src & 1, wn_s = src >> 1;
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
                  pack4(acc[i][f][4 * q], acc[i][f][4 * q + 1], acc[i][f][4 * q + 2], acc[i][f][4 * q + 3]);
        }
      } else if (ph == 0) {
        // the storing wave's own output, staged 32 rows x 128 B at a time: rows 0-15
        // in this wave's 2 KB, rows 16-31 in that of its copying wave (unused here)
        const int qw = cq0 + wn * 64;
        const int valid = min(8, (p.Q - qw) >> 3);
        uint8_t* const wb = r < 16 ? stg : s_stage[wave - 4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pr0 = cp0 + wm * 128 + i * 32;
#pragma unroll
          for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              *reinterpret_cast<u32x2_t*>(wb + stg128(r & 15, f * 4 + q) + hh * 8) =
                  pack4(acc[i][f][4 * q], acc[i][f][4 * q + 1], acc[i][f][4 * q + 2], acc[i][f][4 * q + 3]);
          wave_lds_fence();
          u32x4_t v[4];
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            v[kk] = *reinterpret_cast<const u32x4_t*>((kk < 2 ? stg : s_stage[wave - 4]) +
                                                      stg128(8 * (kk & 1) + (lane >> 3), lane & 7));
          wave_lds_fence();
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const int pr = pr0 + 8 * kk + (lane >> 3), c = lane & 7;
            if (pr < p.P && c < valid)
              __builtin_nontemporal_store(v[kk], reinterpret_cast<u32x4_t*>(Ce + (int64_t)pr * p.Q + qw + c * 8));
          }
        }
      }
      kbarrier();  // the copying waves' rows are in LDS
      if (!loader) {
        const int pr0 = cp0 + wm_s * 128 + ph * 64;
        const int qw = cq0 + wn_s * 64;
        const int valid = min(8, (p.Q - qw) >> 3);
        u32x4_t v[8];  // reads first, then the masked stores
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = *reinterpret_cast<const u32x4_t*>(xr + stg128(8 * j + (lane >> 3), lane & 7));
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int pr = pr0 + 8 * j + (lane >> 3), c = lane & 7;
          if (pr < p.P && c < valid)
            __builtin_nontemporal_store(v[j], reinterpret_cast<u32x4_t*>(Ce + (int64_t)pr * p.Q + qw + c * 8));
        }
      }
      kbarrier();  // read back: the region may be written again
    }
    if (more && NST - 1 < nk) issue_loads(NST - 1);
    if (!more) break;
  }
}

}  // namespace

int persistent_grid() {
  int g = device_cu_count();
  g -= g % kNumXcd;
  return g < kNumXcd ? kNumXcd : g;
}

hipError_t launch_grouped_gemm(int op, int epi, const uint16_t* A, const uint16_t* B, const float* aux_in,
                               float* aux_out, const int32_t* group_offsets, int E, int64_t M, int K, int N,
                               const int32_t* row_slot, int n_slots, int slot_div, const float* slot_scale,
                               uint16_t* C, hipStream_t stream, int grid_size) {
  if (M == 0) return hipSuccess;
  GemmP p{A, B, aux_in, aux_out, C, group_offsets, row_slot, slot_scale, E, (int)M, K, N,
          row_slot ? n_slots : (int)M, slot_div > 0 ? slot_div : 1};
  const dim3 grid(grid_size > 0 ? grid_size : persistent_grid()), block(GTHR);
  const bool g = row_slot != nullptr, sc = slot_scale != nullptr;
#define MOE_GEMM_LAUNCH(O, P)                                                           \
  if (g && sc) gemm_kernel<O, P, true, true><<<grid, block, 0, stream>>>(p);            \
  else if (g) gemm_kernel<O, P, true, false><<<grid, block, 0, stream>>>(p);            \
  else if (sc) gemm_kernel<O, P, false, true><<<grid, block, 0, stream>>>(p);           \
  else gemm_kernel<O, P, false, false><<<grid, block, 0, stream>>>(p);
  if (op == OP_NN && epi == EPI_NONE) { MOE_GEMM_LAUNCH(OP_NN, EPI_NONE) }
  else if (op == OP_NN && epi == EPI_SWIGLU) { MOE_GEMM_LAUNCH(OP_NN, EPI_SWIGLU) }
  else if (op == OP_NT && epi == EPI_NONE) { MOE_GEMM_LAUNCH(OP_NT, EPI_NONE) }
  else if (op == OP_NT && epi == EPI_SWIGLU_BWD) { MOE_GEMM_LAUNCH(OP_NT, EPI_SWIGLU_BWD) }
  else return hipErrorInvalidValue;
#undef MOE_GEMM_LAUNCH
  return hipGetLastError();
}

hipError_t launch_wgrad(const uint16_t* A, const uint16_t* D, const int32_t* group_offsets, int E, int64_t M, int P,
                        int Q, uint16_t* C, hipStream_t stream, int grid_size) {
  if (E == 0) return hipSuccess;
  WgradP p{A, D, group_offsets, C, E, (int)M, P, Q};
  wgrad_kernel<<<dim3(grid_size > 0 ? grid_size : persistent_grid()), dim3(GTHR), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace moe
