// Ragged tile lists of the persistent grouped GEMMs: which output tile a
// workgroup computes on its it-th turn. The GPU kernels and the host-side
// schedule query (moe_tile_schedule) both call these functions, so the CPU
// checks of the tile lists run this very code.
//
// Group-aware kernels run only the tiles a group needs ("[DRAFT][JAX] Optimize
// MoE block", Changes), and the partial tile at a group edge is masked on
// store ("MoE: fused TensorCore Pallas permute/combine kernels and
// split-expert wi layout for TPU v6e", Tests: boundary-tile masking).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kNumXcd = 8;       // MI355X: 8 XCDs, workgroups dealt round-robin across them
constexpr int kTileRows = 256;   // output rows per grouped-GEMM tile
constexpr int kWgradTile = 256;  // weight-gradient tiles are 256 x 256

// Persistent-grid tile index: workgroup w sits on XCD w % 8. Turn `it` of
// workgroup w takes tile it * G + (w % 8) * (G / 8) + w / 8, so at any moment
// each XCD works on a contiguous run of G / 8 tiles, and those tiles share
// operands in that XCD's L2. For each it, w -> tile is a bijection onto
// [it * G, (it + 1) * G). G must be a multiple of 8.
__host__ __device__ __forceinline__ int64_t xcd_tile(int64_t it, int w, int G) {
  return it * G + (int64_t)(w % kNumXcd) * (G / kNumXcd) + w / kNumXcd;
}

// Group offset clamped to [0, M].
__host__ __device__ __forceinline__ int clamp_rows(int v, int M) { return v < 0 ? 0 : (v > M ? M : v); }

// Tiles of a group of n rows: one per 256-row block and column tile (none for an empty group).
__host__ __device__ __forceinline__ int group_tiles(int n, int ntn) {
  return n > 0 ? ((n + kTileRows - 1) / kTileRows) * ntn : 0;
}

struct RaggedTile {
  int e;   // expert
  int mt;  // 256-row block inside the expert
  int nt;  // column tile
};

// Tile `tile` (< pref[E]) of the expert-major list, pref[e] being the number
// of tiles of experts before e. Inside an expert with 4 or more row blocks the
// row block varies fastest (the workgroups of an XCD share one weight panel
// while they sweep the expert's rows); with 1 or 3 row blocks the column tile
// varies fastest (all column tiles read the same row block at once). With
// exactly 2 row blocks the two halves of each column are adjacent (see
// tile_rows).
template <class Pref>
__host__ __device__ __forceinline__ RaggedTile ragged_tile(int tile, const Pref& pref, int E, int ntn) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pref[mid] <= tile) lo = mid;
    else hi = mid;
  }
  const int local = tile - pref[lo];
  const int nmt = (pref[lo + 1] - pref[lo]) / ntn;
  const bool rows_fast = nmt >= 4 || nmt == 2;
  RaggedTile t;
  t.e = lo;
  t.mt = rows_fast ? local % nmt : local / ntn;
  t.nt = rows_fast ? local / nmt : local % ntn;
  return t;
}

// Rows of row block mt of the group [lo, hi): the tile covers [*r0, *r1) and
// multiplies as if its rows ended at *rc (a wave's work depends on how many of
// its rows lie before *rc; rows from *r1 on are read clamped and never stored).
// A group of 257-512 rows is cut into two halves, the first ceil(n / 2) rows
// and the rest, both multiplied as ceil(n / 2) rows long. Two 256-row blocks
// would leave the second nearly empty when n is just above 256; that tile
// finishes early, drifts away from its partner and streams the whole weight
// panel again (measured: such groups fetch the weights 1.5 times). With equal
// halves, adjacent in the tile list (ragged_tile), the pair lands on
// neighbouring workgroups of one XCD. Every 2-tile unit of such a list then
// does equal work, so the two workgroups stay in step and share each weight
// k-slice in L2. Measured on 256 groups of 256 +- 16 rows (K = 7168 / 2048 /
// 4096 / 7168, N = 4096 / 7168 / 7168 / 2048), bitwise-equal outputs: GEMM1 +
// SwiGLU 4.78 -> 4.60 ms, GEMM2 2.58 -> 2.48 ms, the dlhs NT GEMM 5.54 -> 4.99
// ms, the SwiGLU-backward NT GEMM 3.17 -> 2.89 ms.
__host__ __device__ __forceinline__ void tile_rows(int lo, int hi, int mt, int* r0, int* r1, int* rc) {
  const int n = hi - lo;
  if (n > kTileRows && n <= 2 * kTileRows) {
    const int s = (n + 1) / 2;
    *r0 = lo + mt * s;
    *r1 = mt == 0 ? lo + s : hi;
    *rc = *r0 + s;
  } else {
    *r0 = lo + mt * kTileRows;
    *r1 = hi < *r0 + kTileRows ? hi : *r0 + kTileRows;
    *rc = hi;
  }
}

struct WgradTile {
  int e;   // expert
  int pt;  // 256-row block of dW (rows of P)
  int qt;  // 256-column block of dW (columns of Q)
};

// Weight-gradient deal: XCD x (workgroups w with w % 8 == x) takes experts
// x, x + 8, ..., each expert's tp * tq tiles in turn over its G / 8
// workgroups. Every expert has the same number of tiles whatever its row
// count, so the XCDs stay balanced when E is a multiple of 8, and an expert's
// operand rows are read into one XCD's L2. Inside an expert the dimension with
// fewer 256-blocks varies fastest. Returns false once the workgroup is done.
__host__ __device__ __forceinline__ bool wgrad_tile(int64_t it, int w, int G, int E, int tp, int tq, WgradTile* t) {
  const int per_xcd = G / kNumXcd;
  const int64_t j = it * per_xcd + w / kNumXcd;
  const int64_t per_e = (int64_t)tp * tq;
  const int64_t ee = w % kNumXcd + (int64_t)kNumXcd * (j / per_e);
  if (ee >= E) return false;
  const int loc = (int)(j % per_e);
  t->e = (int)ee;
  t->pt = tq <= tp ? loc / tq : loc % tp;
  t->qt = tq <= tp ? loc % tq : loc / tp;
  return true;
}

}  // namespace moe
