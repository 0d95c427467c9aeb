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
// while they sweep the expert's rows); with 1-3 row blocks the column tile
// varies fastest (all column tiles read the same row block at once).
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
  const bool rows_fast = nmt >= 4;
  RaggedTile t;
  t.e = lo;
  t.mt = rows_fast ? local % nmt : local / ntn;
  t.nt = rows_fast ? local / nmt : local % ntn;
  return t;
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
