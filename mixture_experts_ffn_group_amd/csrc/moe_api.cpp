// C ABI of the MoE FFN library: argument validation, workspace layout and the
// launch sequence of each entry point (declared in include/moe_ffn.h).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>
#include <algorithm>

#include "kernels.h"
#include "moe_ffn.h"
#include "tiles.h"

namespace moe {

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace moe

namespace {

thread_local char g_detail[512];

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  return status;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define NEED(p)                                                       \
  do {                                                                \
    if (!(p)) return fail(MOE_ERR_NULL, "argument %s is NULL", #p);   \
    if (!aligned16(p)) return fail(MOE_ERR_ALIGN, "argument %s is not 16-byte aligned", #p); \
  } while (0)
#define MAYBE(p)                                                      \
  do {                                                                \
    if ((p) && !aligned16(p)) return fail(MOE_ERR_ALIGN, "argument %s is not 16-byte aligned", #p); \
  } while (0)
// The workspace `ws` of `ws_bytes` must hold `n` bytes; it may be NULL when the call needs none
// (no tokens).
#define NEED_WS(n)                                                                                   \
  do {                                                                                               \
    const size_t need_ = (n);                                                                        \
    if (need_ > 0) NEED(ws);                                                                         \
    else MAYBE(ws);                                                                                  \
    if (ws_bytes < need_) return fail(MOE_ERR_WORKSPACE, "need %zu workspace bytes", need_);         \
  } while (0)

constexpr size_t kAlign = 256;
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int check_shape(const moe_shape_t* s) {
  if (!s) return fail(MOE_ERR_NULL, "shape is NULL");
  if (s->T < 0 || s->emb <= 0 || s->mlp <= 0 || s->E <= 0 || s->k <= 0)
    return fail(MOE_ERR_SHAPE, "need T >= 0 and emb, mlp, E, k > 0");
  if (s->k > s->E) return fail(MOE_ERR_SHAPE, "k (%d) > E (%d)", s->k, s->E);
  if (s->E > 256) return fail(MOE_ERR_UNSUPPORTED, "E (%d) > 256", s->E);
  if (s->k > 64) return fail(MOE_ERR_UNSUPPORTED, "k (%d) > 64", s->k);
  if (s->emb % 64) return fail(MOE_ERR_UNSUPPORTED, "emb (%d) is not a multiple of 64", s->emb);
  if (s->mlp % 64) return fail(MOE_ERR_UNSUPPORTED, "mlp (%d) is not a multiple of 64", s->mlp);
  if (s->T * (int64_t)s->k >= (int64_t(1) << 31)) return fail(MOE_ERR_UNSUPPORTED, "T*k >= 2^31");
  // token rows are read through 32-bit offsets when gathered (dy in the backward)
  if (s->T * (int64_t)s->emb >= (int64_t(1) << 31)) return fail(MOE_ERR_UNSUPPORTED, "T*emb >= 2^31");
  if ((int64_t)s->emb * 2 * s->mlp >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "emb*2*mlp >= 2^31 (per-expert weight too large)");
  if (s->T * (int64_t)s->k * 2 * s->mlp >= (int64_t(1) << 40))
    return fail(MOE_ERR_UNSUPPORTED, "activation too large");
  return MOE_OK;
}

// Region sizes of the permute workspace.
size_t masks_bytes(const moe_shape_t* s) {
  const int64_t nblk = (s->T + moe::kPermuteBlock - 1) / moe::kPermuteBlock;
  return round_up((size_t)nblk * s->E * sizeof(uint64_t));
}
size_t base_bytes(const moe_shape_t* s) {
  const int64_t nblk = (s->T + moe::kPermuteBlock - 1) / moe::kPermuteBlock;
  return round_up((size_t)nblk * s->E * sizeof(int32_t));
}
size_t permute_ws(const moe_shape_t* s) { return masks_bytes(s) + base_bytes(s); }

struct Carver {
  char* p;
  size_t used = 0;
  template <class T>
  T* take(size_t count) {
    T* r = reinterpret_cast<T*>(p + used);
    used += round_up(count * sizeof(T));
    return r;
  }
};

// Forward workspace: permute scratch, then routing and activations (used when no saved set is given).
size_t fwd_ws(const moe_shape_t* s) {
  const size_t S = (size_t)s->T * s->k;
  return permute_ws(s) + round_up(S * 4) * 2 /*topk idx, w*/ + round_up(s->E * 4) + round_up((s->E + 1) * 4) +
         round_up(S * 4) * 2 /*sorted_slot, slot_row*/ + round_up(S * s->emb * 2) /*xs*/ +
         round_up(S * s->mlp * 2) /*a*/ + round_up(S * s->emb * 2) /*o*/;
}
size_t bwd_ws(const moe_shape_t* s) {
  const size_t S = (size_t)s->T * s->k;
  return round_up(S * s->emb * 2) /*do*/ + round_up(S * 2 * s->mlp * 2) /*dh*/ + round_up(S * s->emb * 2) /*dxs*/;
}
// Backward that recomputes h (the saved set has none): h [S, 2*mlp] fp32, and the SwiGLU output the
// recomputing GEMM also writes, which shares the dxs buffer unless mlp > emb.
size_t bwd_remat_ws(const moe_shape_t* s) {
  const size_t S = (size_t)s->T * s->k;
  return bwd_ws(s) + round_up(S * 2 * s->mlp * 4) + (s->mlp > s->emb ? round_up(S * s->mlp * 2) : 0);
}

int check_gemm(int op, int epi, int64_t M, int K, int N, int E) {
  if (op != MOE_NN && op != MOE_NT) return fail(MOE_ERR_SHAPE, "op must be MOE_NN or MOE_NT");
  if (epi == MOE_EPI_SWIGLU && op != MOE_NN) return fail(MOE_ERR_UNSUPPORTED, "SWIGLU epilogue needs op NN");
  if (epi == MOE_EPI_SWIGLU_BWD && op != MOE_NT) return fail(MOE_ERR_UNSUPPORTED, "SWIGLU_BWD epilogue needs op NT");
  if (epi < MOE_EPI_NONE || epi > MOE_EPI_SWIGLU_BWD) return fail(MOE_ERR_SHAPE, "unknown epilogue %d", epi);
  if (M < 0 || K <= 0 || N <= 0 || E <= 0) return fail(MOE_ERR_SHAPE, "need M >= 0 and K, N, E > 0");
  if (E > 256) return fail(MOE_ERR_UNSUPPORTED, "E (%d) > 256", E);
  if (M >= (int64_t(1) << 31)) return fail(MOE_ERR_UNSUPPORTED, "M >= 2^31");
  if (K % 64) return fail(MOE_ERR_UNSUPPORTED, "K (%d) is not a multiple of 64", K);
  if (N % 8) return fail(MOE_ERR_UNSUPPORTED, "N (%d) is not a multiple of 8", N);
  if (epi == MOE_EPI_SWIGLU && (N % 16)) return fail(MOE_ERR_UNSUPPORTED, "SWIGLU needs (N/2) %% 8 == 0");
  if ((int64_t)K * N >= (int64_t(1) << 31)) return fail(MOE_ERR_UNSUPPORTED, "K*N >= 2^31");
  if ((int64_t)255 * K >= (int64_t(1) << 31)) return fail(MOE_ERR_UNSUPPORTED, "K too large");
  // upper bound of the ragged tile count must fit an int
  const int64_t ntn = epi == MOE_EPI_SWIGLU ? (N / 2 + 127) / 128 : (N + 255) / 256;
  if ((M / 256 + E) * ntn >= (int64_t(1) << 31)) return fail(MOE_ERR_UNSUPPORTED, "tile count too large");
  return MOE_OK;
}

int check_wgrad(int32_t E, int64_t M, int32_t P, int32_t Q) {
  if (M < 0 || P <= 0 || Q <= 0 || E <= 0) return fail(MOE_ERR_SHAPE, "need M >= 0 and P, Q, E > 0");
  if (E > 256) return fail(MOE_ERR_UNSUPPORTED, "E (%d) > 256", E);
  if (M >= (int64_t(1) << 31)) return fail(MOE_ERR_UNSUPPORTED, "M >= 2^31");
  if (P % 8 || Q % 8) return fail(MOE_ERR_UNSUPPORTED, "P and Q must be multiples of 8");
  if ((int64_t)E * ((P + 255) / 256) * ((Q + 255) / 256) >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "tile count too large");
  return MOE_OK;
}

// grid: 0 (one workgroup per compute unit) or a multiple of 8 up to 65536
int check_grid(int32_t grid) {
  if (grid < 0 || grid % moe::kNumXcd || grid > 65536)
    return fail(MOE_ERR_SHAPE, "grid (%d) must be 0 or a positive multiple of 8 up to 65536", grid);
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "null pointer";
    case MOE_ERR_SHAPE: return "invalid shape";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch error";
    case MOE_ERR_ALIGN: return "pointer not 16-byte aligned";
    default: return "unknown status";
  }
}

const char* moe_last_error_detail(void) { return g_detail; }

const char* moe_version(void) { return "moe_ffn 0.1 gfx950"; }

int moe_query_support(const moe_shape_t* shape) {
  g_detail[0] = 0;
  return check_shape(shape);
}

size_t moe_permute_workspace_bytes(const moe_shape_t* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  return permute_ws(shape);
}

size_t moe_workspace_bytes(const moe_shape_t* shape, int with_backward) {
  if (check_shape(shape) != MOE_OK) return 0;
  return with_backward == 2 ? bwd_remat_ws(shape) : with_backward ? bwd_ws(shape) : fwd_ws(shape);
}

// MXFP8 forward: permute scratch, routing and indices, token codes/scales, SwiGLU output codes/scales, o.
size_t fwd_mx_ws(const moe_shape_t* s) {
  const size_t S = (size_t)s->T * s->k, T = (size_t)s->T;
  return permute_ws(s) + round_up(S * 4) * 2 /*topk idx, w*/ + round_up(s->E * 4) + round_up((s->E + 1) * 4) +
         round_up(S * 4) * 2 /*sorted_slot, slot_row*/ + round_up(T * s->emb) + round_up(T * s->emb / 16) +
         round_up(S * s->mlp) + round_up(S * s->mlp / 16) + round_up(S * s->emb * 2) /*o*/;
}

size_t moe_workspace_bytes_mx(const moe_shape_t* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  if (shape->mlp % 64) return 0;
  return fwd_mx_ws(shape);
}

// per-slot logit gradients, then Wr transposed
size_t route_bwd_ws(const moe_shape_t* s) {
  return 3 * round_up(4 * (size_t)s->T * s->k) + 2 * round_up(4 * (size_t)s->E * s->emb);
}

size_t moe_route_bwd_workspace_bytes(const moe_shape_t* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  return route_bwd_ws(shape);
}

int moe_route(const moe_shape_t* s, const moe_bf16_t* x, const float* wr, const float* bias, const float* logits_in,
              int32_t* topk_idx, float* topk_w, moe_stream_t stream) {
  g_detail[0] = 0;
  if (int rc = check_shape(s)) return rc;
  if (s->T == 0) return MOE_OK;  // no tokens: nothing to route
  if (logits_in) {
    if (x || wr || bias) return fail(MOE_ERR_SHAPE, "with logits_in, x, wr and bias must be NULL");
    MAYBE(logits_in);
  } else {
    NEED(x);
    NEED(wr);
    MAYBE(bias);
  }
  NEED(topk_idx);
  NEED(topk_w);
  return hip_status(moe::launch_route(s->T, s->emb, s->E, s->k, x, wr, bias, logits_in, topk_idx, topk_w,
                                      (hipStream_t)stream),
                    "moe_route");
}

int moe_permute(const moe_shape_t* s, const moe_bf16_t* x, const int32_t* topk_idx, int32_t* group_sizes,
                int32_t* group_offsets, int32_t* sorted_slot, int32_t* slot_row, moe_bf16_t* xs, void* ws,
                size_t ws_bytes, moe_stream_t stream) {
  g_detail[0] = 0;
  if (int rc = check_shape(s)) return rc;
  NEED(group_sizes);
  NEED(group_offsets);
  if (s->T > 0) {
    NEED(topk_idx);
    NEED(sorted_slot);
    NEED(slot_row);
    MAYBE(xs);  // NULL: index only, the rows are not copied
    if (xs) NEED(x);
  }
  NEED_WS(permute_ws(s));
  char* w = static_cast<char*>(ws);
  uint64_t* masks = reinterpret_cast<uint64_t*>(w);
  int32_t* base = reinterpret_cast<int32_t*>(w + masks_bytes(s));
  return hip_status(moe::launch_permute(s->T, s->emb, s->E, s->k, x, topk_idx, group_sizes, group_offsets,
                                        sorted_slot, slot_row, xs, masks, base, (hipStream_t)stream),
                    "moe_permute");
}

int moe_permute_noalloc(const moe_shape_t* s, const moe_bf16_t* x, const int32_t* topk_idx, int32_t* group_sizes,
                        int32_t* group_offsets, int32_t* sorted_slot, int32_t* slot_row, moe_bf16_t* xs,
                        moe_stream_t stream) {
  g_detail[0] = 0;
  if (int rc = check_shape(s)) return rc;
  NEED(group_sizes);
  NEED(group_offsets);
  if (s->T > 0) {
    NEED(topk_idx);
    NEED(sorted_slot);
    NEED(slot_row);
    MAYBE(xs);
    if (xs) NEED(x);
  }
  if (permute_ws(s) > moe::kPermuteScratchBytes)
    return fail(MOE_ERR_WORKSPACE, "needs %zu bytes of scratch; the fixed scratch holds %zu (12 * ceil(T/64) * E)",
                permute_ws(s), moe::kPermuteScratchBytes);
  return hip_status(moe::launch_permute_noalloc(s->T, s->emb, s->E, s->k, x, topk_idx, group_sizes, group_offsets,
                                                sorted_slot, slot_row, xs, (hipStream_t)stream),
                    "moe_permute_noalloc");
}

int moe_grouped_gemm_grid(int op, int epilogue, const moe_bf16_t* A, const moe_bf16_t* B, const float* aux_in,
                          float* aux_out, const int32_t* group_offsets, int32_t E, int64_t M, int32_t K, int32_t N,
                          const moe_gemm_rows_t* rows, moe_bf16_t* C, int32_t grid, moe_stream_t stream) {
  g_detail[0] = 0;
  if (int rc = check_gemm(op, epilogue, M, K, N, E)) return rc;
  if (int rc = check_grid(grid)) return rc;
  NEED(B);
  NEED(group_offsets);
  if (M > 0) {
    NEED(A);
    NEED(C);
  }
  if (epilogue == MOE_EPI_SWIGLU_BWD) NEED(aux_in);
  if (epilogue == MOE_EPI_SWIGLU) MAYBE(aux_out);
  const int32_t* row_slot = nullptr;
  const float* slot_scale = nullptr;
  int n_slots = 0, slot_div = 1;
  if (rows) {
    row_slot = rows->row_slot;
    slot_scale = rows->slot_scale;
    n_slots = rows->n_slots;
    slot_div = rows->slot_div;
    MAYBE(slot_scale);
    if (row_slot) {
      if (n_slots <= 0 || slot_div <= 0) return fail(MOE_ERR_SHAPE, "row gather needs n_slots > 0 and slot_div > 0");
      if ((int64_t)(n_slots / slot_div) * K >= (int64_t(1) << 31))
        return fail(MOE_ERR_UNSUPPORTED, "gathered A too large (rows*K >= 2^31)");
    }
  }
  return hip_status(moe::launch_grouped_gemm(op, epilogue, A, B, aux_in, epilogue == MOE_EPI_SWIGLU ? aux_out : nullptr,
                                             group_offsets, E, M, K, N, row_slot, n_slots, slot_div, slot_scale, C,
                                             (hipStream_t)stream, grid),
                    "moe_grouped_gemm");
}

int moe_grouped_gemm(int op, int epilogue, const moe_bf16_t* A, const moe_bf16_t* B, const float* aux_in,
                     float* aux_out, const int32_t* group_offsets, int32_t E, int64_t M, int32_t K, int32_t N,
                     const moe_gemm_rows_t* rows, moe_bf16_t* C, moe_stream_t stream) {
  return moe_grouped_gemm_grid(op, epilogue, A, B, aux_in, aux_out, group_offsets, E, M, K, N, rows, C, 0, stream);
}

int moe_grouped_gemm_wgrad_grid(const moe_bf16_t* A, const moe_bf16_t* D, const int32_t* group_offsets, int32_t E,
                                int64_t M, int32_t P, int32_t Q, moe_bf16_t* C, int32_t grid, moe_stream_t stream) {
  g_detail[0] = 0;
  if (int rc = check_wgrad(E, M, P, Q)) return rc;
  if (int rc = check_grid(grid)) return rc;
  NEED(group_offsets);
  NEED(C);
  if (M > 0) {
    NEED(A);
    NEED(D);
  }
  return hip_status(moe::launch_wgrad(A, D, group_offsets, E, M, P, Q, C, (hipStream_t)stream, grid),
                    "moe_grouped_gemm_wgrad");
}

int moe_grouped_gemm_wgrad(const moe_bf16_t* A, const moe_bf16_t* D, const int32_t* group_offsets, int32_t E,
                           int64_t M, int32_t P, int32_t Q, moe_bf16_t* C, moe_stream_t stream) {
  return moe_grouped_gemm_wgrad_grid(A, D, group_offsets, E, M, P, Q, C, 0, stream);
}

int moe_tile_schedule(int32_t kind, const int32_t* group_offsets, int32_t E, int64_t M, int32_t N, int32_t Q,
                      int32_t grid, int32_t* tiles, int64_t capacity, int64_t* count) {
  g_detail[0] = 0;
  if (!group_offsets) return fail(MOE_ERR_NULL, "argument group_offsets is NULL");
  if (!count) return fail(MOE_ERR_NULL, "argument count is NULL");
  if (capacity < 0 || (capacity > 0 && !tiles)) return fail(MOE_ERR_NULL, "tiles is NULL with capacity > 0");
  if (grid <= 0) return fail(MOE_ERR_SHAPE, "grid must be given (> 0) for the host schedule");
  if (int rc = check_grid(grid)) return rc;
  int64_t n = 0;
  auto emit = [&](int w, int64_t it, int e, int r0, int r1, int c0, int c1) {
    if (n < capacity) {
      int32_t* t = tiles + 7 * n;
      t[0] = w, t[1] = (int32_t)it, t[2] = e, t[3] = r0, t[4] = r1, t[5] = c0, t[6] = c1;
    }
    ++n;
  };
  if (kind == MOE_SCHED_WGRAD) {
    if (int rc = check_wgrad(E, M, N, Q)) return rc;
    const int tp = (N + moe::kWgradTile - 1) / moe::kWgradTile, tq = (Q + moe::kWgradTile - 1) / moe::kWgradTile;
    for (int w = 0; w < grid; ++w) {
      moe::WgradTile t;
      for (int64_t it = 0; moe::wgrad_tile(it, w, grid, E, tp, tq, &t); ++it) {
        const int p0 = t.pt * moe::kWgradTile, q0 = t.qt * moe::kWgradTile;
        emit(w, it, t.e, p0, std::min(p0 + moe::kWgradTile, N), q0, std::min(q0 + moe::kWgradTile, Q));
      }
    }
  } else if (kind == MOE_SCHED_GEMM || kind == MOE_SCHED_GEMM_SWIGLU) {
    const bool swiglu = kind == MOE_SCHED_GEMM_SWIGLU;
    if (int rc = check_gemm(swiglu ? MOE_NN : MOE_NT, swiglu ? MOE_EPI_SWIGLU : MOE_EPI_NONE, M, 64, N, E)) return rc;
    const int width = swiglu ? N / 2 : N, tile_n = swiglu ? 128 : 256, ntn = (width + tile_n - 1) / tile_n;
    std::vector<int> lo(E + 1), pref(E + 1);
    for (int e = 0; e <= E; ++e) lo[e] = moe::clamp_rows(group_offsets[e], (int)M);
    pref[0] = 0;
    for (int e = 0; e < E; ++e) pref[e + 1] = pref[e] + moe::group_tiles(lo[e + 1] - lo[e], ntn);
    for (int w = 0; w < grid; ++w) {
      for (int64_t it = 0;; ++it) {
        const int64_t tl = moe::xcd_tile(it, w, grid);
        if (tl >= pref[E]) break;
        const moe::RaggedTile t = moe::ragged_tile((int)tl, pref, E, ntn);
        int r0, r1, rc;
        moe::tile_rows(lo[t.e], std::max(lo[t.e + 1], lo[t.e]), t.mt, &r0, &r1, &rc);
        const int n0 = t.nt * tile_n;
        emit(w, it, t.e, r0, r1, n0, std::min(n0 + tile_n, width));
      }
    }
  } else {
    return fail(MOE_ERR_SHAPE, "unknown schedule kind %d", kind);
  }
  *count = n;
  return MOE_OK;
}

int moe_combine(const moe_shape_t* s, const moe_bf16_t* ys, const int32_t* slot_row, const float* topk_w,
                moe_bf16_t* y, moe_stream_t stream) {
  g_detail[0] = 0;
  if (int rc = check_shape(s)) return rc;
  if (s->T > 0) {
    NEED(ys);
    NEED(slot_row);
    NEED(y);
    MAYBE(topk_w);
  }
  return hip_status(moe::launch_combine(s->T, s->emb, s->k, ys, slot_row, topk_w, y, (hipStream_t)stream),
                    "moe_combine");
}

int moe_combine_bwd(const moe_shape_t* s, const moe_bf16_t* dy, const moe_bf16_t* ys, const int32_t* slot_row,
                    const float* topk_w, moe_bf16_t* dys, float* dtopk_w, moe_stream_t stream) {
  g_detail[0] = 0;
  if (int rc = check_shape(s)) return rc;
  if (s->T > 0) {
    NEED(dy);
    NEED(slot_row);
    NEED(topk_w);
    NEED(dys);
    MAYBE(ys);
    MAYBE(dtopk_w);
  }
  return hip_status(moe::launch_combine_bwd(s->T, s->emb, s->k, dy, ys, slot_row, topk_w, dys, dtopk_w,
                                            (hipStream_t)stream),
                    "moe_combine_bwd");
}

int moe_route_bwd(const moe_shape_t* s, const moe_bf16_t* x, const float* wr, const int32_t* topk_idx,
                  const float* topk_w, const float* dtopk_w, const int32_t* sorted_slot,
                  const int32_t* group_offsets, float* dwr, float* dbias, moe_bf16_t* dx, void* ws, size_t ws_bytes,
                  moe_stream_t stream) {
  g_detail[0] = 0;
  if (int rc = check_shape(s)) return rc;
  NEED(wr);
  NEED(group_offsets);
  NEED(dwr);
  MAYBE(dbias);
  if (s->T > 0) {  // with no tokens, per-token buffers may be empty (NULL)
    NEED(x);
    NEED(topk_idx);
    NEED(topk_w);
    NEED(dtopk_w);
    NEED(sorted_slot);
    MAYBE(dx);
  }
  NEED_WS(route_bwd_ws(s));
  Carver c{static_cast<char*>(ws)};
  float* dl = c.take<float>(s->T * s->k);
  float* dls = c.take<float>(s->T * s->k);
  int32_t* tok = c.take<int32_t>(s->T * s->k);
  float* wrt = c.take<float>((int64_t)s->E * s->emb);
  float* dwrt = c.take<float>((int64_t)s->E * s->emb);
  return hip_status(moe::launch_route_bwd(s->T, s->emb, s->E, s->k, x, wr, topk_idx, topk_w, dtopk_w, sorted_slot,
                                          group_offsets, dwr, dbias, s->T > 0 ? dx : nullptr, dl, dls, tok, wrt,
                                          dwrt, (hipStream_t)stream),
                    "moe_route_bwd");
}

int moe_mx_quantize_rows(const moe_bf16_t* src, int64_t src_rows, int32_t K, const int32_t* row_index,
                         int32_t row_div, int64_t M, uint8_t* codes, uint8_t* scales, moe_stream_t stream) {
  g_detail[0] = 0;
  if (M < 0 || src_rows < 0 || K <= 0) return fail(MOE_ERR_SHAPE, "need M, src_rows >= 0 and K > 0");
  if (K % 64) return fail(MOE_ERR_UNSUPPORTED, "K (%d) is not a multiple of 64", K);
  if (M * (K / 8) >= (int64_t(1) << 31) * 256) return fail(MOE_ERR_UNSUPPORTED, "M*K too large");
  if (M == 0) return MOE_OK;
  if (src_rows == 0) return fail(MOE_ERR_SHAPE, "no source rows for %lld output rows", (long long)M);
  if (row_index && row_div <= 0) return fail(MOE_ERR_SHAPE, "row_div must be > 0");
  NEED(src);
  MAYBE(row_index);
  NEED(codes);
  NEED(scales);
  return hip_status(moe::launch_mx_quantize_rows(src, src_rows, K, row_index, row_index ? row_div : 1, M, codes,
                                                  scales, (hipStream_t)stream),
                    "moe_mx_quantize_rows");
}

int moe_mx_quantize_weight(const moe_bf16_t* w, int32_t E, int32_t K, int32_t N, uint8_t* codes, uint8_t* scales,
                           moe_stream_t stream) {
  g_detail[0] = 0;
  if (E <= 0 || K <= 0 || N <= 0) return fail(MOE_ERR_SHAPE, "need E, K, N > 0");
  if (K % 64) return fail(MOE_ERR_UNSUPPORTED, "K (%d) is not a multiple of 64", K);
  if ((int64_t)E * (K / 64) * N >= (int64_t(1) << 31) * 256) return fail(MOE_ERR_UNSUPPORTED, "E*K*N too large");
  NEED(w);
  NEED(codes);
  NEED(scales);
  return hip_status(moe::launch_mx_quantize_weight(w, E, K, N, codes, scales, (hipStream_t)stream),
                    "moe_mx_quantize_weight");
}

int moe_grouped_gemm_mx(int32_t epilogue, const uint8_t* A, const uint8_t* A_scales, int64_t a_rows,
                        const int32_t* row_slot, int32_t slot_div, const uint8_t* B, const uint8_t* B_scales,
                        const int32_t* group_offsets, int32_t E, int64_t M, int32_t K, int32_t N, moe_bf16_t* C,
                        uint8_t* C_codes, uint8_t* C_scales, moe_stream_t stream) {
  g_detail[0] = 0;
  if ((C_codes != nullptr) != (C_scales != nullptr)) return fail(MOE_ERR_NULL, "C_codes and C_scales go together");
  if (C_codes && epilogue != MOE_EPI_SWIGLU) return fail(MOE_ERR_UNSUPPORTED, "an MXFP8 output needs SWIGLU");
  if (C_codes && (N / 2) % 64) return fail(MOE_ERR_UNSUPPORTED, "an MXFP8 output needs (N/2) %% 64 == 0");
  if (epilogue != MOE_EPI_NONE && epilogue != MOE_EPI_SWIGLU)
    return fail(MOE_ERR_UNSUPPORTED, "the MXFP8 GEMM has the NONE and SWIGLU epilogues");
  if (M < 0 || K <= 0 || N <= 0 || E <= 0) return fail(MOE_ERR_SHAPE, "need M >= 0 and K, N, E > 0");
  if (E > 256) return fail(MOE_ERR_UNSUPPORTED, "E (%d) > 256", E);
  if (K % 64) return fail(MOE_ERR_UNSUPPORTED, "K (%d) is not a multiple of 64", K);
  if (N % 8) return fail(MOE_ERR_UNSUPPORTED, "N (%d) is not a multiple of 8", N);
  if (epilogue == MOE_EPI_SWIGLU && N % 16) return fail(MOE_ERR_UNSUPPORTED, "SWIGLU needs (N/2) %% 8 == 0");
  if (!row_slot && a_rows != M) return fail(MOE_ERR_SHAPE, "without row_slot, a_rows must equal M");
  if (row_slot && (a_rows <= 0 || slot_div <= 0)) return fail(MOE_ERR_SHAPE, "row gather needs a_rows, slot_div > 0");
  if (a_rows * K >= (int64_t(1) << 32) || (int64_t)N * K >= (int64_t(1) << 32))
    return fail(MOE_ERR_UNSUPPORTED, "a_rows*K and N*K must be below 2^32 bytes");
  if (M >= (int64_t(1) << 31)) return fail(MOE_ERR_UNSUPPORTED, "M >= 2^31");
  const int64_t ntn = epilogue == MOE_EPI_SWIGLU ? (N / 2 + 127) / 128 : (N + 255) / 256;
  if ((M / 256 + E) * ntn >= (int64_t(1) << 31)) return fail(MOE_ERR_UNSUPPORTED, "tile count too large");
  NEED(group_offsets);
  NEED(B);
  NEED(B_scales);
  if (M > 0) {
    NEED(A);
    NEED(A_scales);
    MAYBE(row_slot);
    if (C_codes) {
      MAYBE(C);
      NEED(C_codes);
      NEED(C_scales);
    } else {
      NEED(C);
    }
  }
  return hip_status(moe::launch_grouped_gemm_mx(epilogue, A, A_scales, a_rows, row_slot, row_slot ? slot_div : 1, B,
                                                 B_scales, group_offsets, E, M, K, N, C, C_codes, C_scales,
                                                 (hipStream_t)stream),
                    "moe_grouped_gemm_mx");
}

int moe_ffn_fwd_mx(const moe_shape_t* s, const moe_bf16_t* x, const float* wr, const float* bias,
                   const float* logits_in, const uint8_t* wi_codes, const uint8_t* wi_scales, const uint8_t* wo_codes,
                   const uint8_t* wo_scales, moe_bf16_t* y, void* ws, size_t ws_bytes, moe_stream_t stream) {
  g_detail[0] = 0;
  if (int rc = check_shape(s)) return rc;
  if (s->mlp % 64) return fail(MOE_ERR_UNSUPPORTED, "the MXFP8 forward needs mlp %% 64 == 0");
  if ((int64_t)s->T * s->emb >= (int64_t(1) << 32) || (int64_t)s->T * s->k * s->mlp >= (int64_t(1) << 32))
    return fail(MOE_ERR_UNSUPPORTED, "T*emb and T*k*mlp must be below 2^32");
  const bool any = s->T > 0;
  if (any) {
    NEED(x);
    NEED(y);
  }
  NEED(wi_codes);
  NEED(wi_scales);
  NEED(wo_codes);
  NEED(wo_scales);
  if (logits_in) {
    if (wr || bias) return fail(MOE_ERR_SHAPE, "with logits_in, wr and bias must be NULL");
    MAYBE(logits_in);
  } else {
    NEED(wr);
    MAYBE(bias);
  }
  NEED_WS(fwd_mx_ws(s));
  if (!any) return MOE_OK;
  const int64_t T = s->T, S = T * s->k;
  const int emb = s->emb, mlp = s->mlp, E = s->E, k = s->k;
  const hipStream_t st = (hipStream_t)stream;
  Carver c{static_cast<char*>(ws)};
  uint64_t* masks = c.take<uint64_t>(((T + moe::kPermuteBlock - 1) / moe::kPermuteBlock) * E);
  int32_t* base = c.take<int32_t>(((T + moe::kPermuteBlock - 1) / moe::kPermuteBlock) * E);
  int32_t* topk_idx = c.take<int32_t>(S);
  float* topk_w = c.take<float>(S);
  int32_t* group_sizes = c.take<int32_t>(E);
  int32_t* group_offsets = c.take<int32_t>(E + 1);
  int32_t* sorted_slot = c.take<int32_t>(S);
  int32_t* slot_row = c.take<int32_t>(S);
  uint8_t* xq = c.take<uint8_t>(T * emb);
  uint8_t* xqs = c.take<uint8_t>(T * emb / 16);
  uint8_t* aq = c.take<uint8_t>(S * mlp);
  uint8_t* aqs = c.take<uint8_t>(S * mlp / 16);
  moe_bf16_t* o = c.take<moe_bf16_t>(S * emb);
  if (int rc = hip_status(moe::launch_route(T, emb, E, k, logits_in ? nullptr : x, wr, bias, logits_in, topk_idx,
                                            topk_w, st),
                          "route"))
    return rc;
  if (int rc = hip_status(moe::launch_permute(T, emb, E, k, x, topk_idx, group_sizes, group_offsets, sorted_slot,
                                              slot_row, nullptr, masks, base, st),
                          "permute"))
    return rc;
  // each token row quantized once; GEMM 1 reads its codes and scales through sorted_slot
  if (int rc = hip_status(moe::launch_mx_quantize_rows(x, T, emb, nullptr, 1, T, xq, xqs, st), "quantize x"))
    return rc;
  if (int rc = hip_status(moe::launch_grouped_gemm_mx(MOE_EPI_SWIGLU, xq, xqs, T, sorted_slot, k, wi_codes,
                                                      wi_scales, group_offsets, E, S, emb, 2 * mlp, nullptr, aq, aqs,
                                                      st),
                          "gemm1"))
    return rc;
  if (int rc = hip_status(moe::launch_grouped_gemm_mx(MOE_EPI_NONE, aq, aqs, S, nullptr, 1, wo_codes, wo_scales,
                                                      group_offsets, E, S, mlp, emb, o, nullptr, nullptr, st),
                          "gemm2"))
    return rc;
  return hip_status(moe::launch_combine(T, emb, k, o, slot_row, topk_w, y, st), "combine");
}

int moe_ffn_fwd(const moe_shape_t* s, const moe_bf16_t* x, const float* wr, const float* bias, const float* logits_in,
                const moe_bf16_t* wi, const moe_bf16_t* wo, moe_bf16_t* y, const moe_saved_t* saved, void* ws,
                size_t ws_bytes, moe_stream_t stream) {
  g_detail[0] = 0;
  if (int rc = check_shape(s)) return rc;
  const bool any = s->T > 0;  // with no tokens, per-token buffers may be empty (NULL)
  if (any) {
    NEED(x);
    NEED(y);
  }
  NEED(wi);
  NEED(wo);
  if (logits_in) {
    if (wr || bias) return fail(MOE_ERR_SHAPE, "with logits_in, wr and bias must be NULL");
    MAYBE(logits_in);
  } else {
    NEED(wr);
    MAYBE(bias);
  }
  NEED_WS(fwd_ws(s));
  if (saved) {
    NEED(saved->group_sizes);
    NEED(saved->group_offsets);
    if (any) {
      NEED(saved->topk_idx);
      NEED(saved->topk_w);
      NEED(saved->sorted_slot);
      NEED(saved->slot_row);
      NEED(saved->xs);
      MAYBE(saved->h);  // NULL: h is not kept, and moe_ffn_bwd recomputes it
      NEED(saved->a);
      NEED(saved->o);
    }
  }
  const int64_t T = s->T, S = T * s->k;
  Carver c{static_cast<char*>(ws)};
  uint64_t* masks = c.take<uint64_t>(((T + moe::kPermuteBlock - 1) / moe::kPermuteBlock) * s->E);
  int32_t* base = c.take<int32_t>(((T + moe::kPermuteBlock - 1) / moe::kPermuteBlock) * s->E);
  moe_saved_t v;
  v.topk_idx = c.take<int32_t>(S);
  v.topk_w = c.take<float>(S);
  v.group_sizes = c.take<int32_t>(s->E);
  v.group_offsets = c.take<int32_t>(s->E + 1);
  v.sorted_slot = c.take<int32_t>(S);
  v.slot_row = c.take<int32_t>(S);
  v.xs = c.take<moe_bf16_t>(S * s->emb);
  v.a = c.take<moe_bf16_t>(S * s->mlp);
  v.o = c.take<moe_bf16_t>(S * s->emb);
  v.h = nullptr;
  if (saved) v = *saved;
  const hipStream_t st = (hipStream_t)stream;
  const int emb = s->emb, mlp = s->mlp, E = s->E, k = s->k;
  if (int rc = hip_status(moe::launch_route(T, emb, E, k, logits_in ? nullptr : x, wr, bias, logits_in, v.topk_idx,
                                            v.topk_w, st),
                          "route"))
    return rc;
  // Inference (nothing saved): the permute builds only the index, and GEMM1 reads each
  // token row of x in place through sorted_slot, so the expert-sorted copy xs is never
  // written. Training keeps xs, which the weight gradient reads.
  const bool gather = saved == nullptr;
  if (int rc = hip_status(moe::launch_permute(T, emb, E, k, x, v.topk_idx, v.group_sizes, v.group_offsets,
                                              v.sorted_slot, v.slot_row, gather ? nullptr : v.xs, masks, base, st),
                          "permute"))
    return rc;
  if (int rc = hip_status(moe::launch_grouped_gemm(MOE_NN, MOE_EPI_SWIGLU, gather ? x : v.xs, wi, nullptr, v.h,
                                                   v.group_offsets, E, S, emb, 2 * mlp, gather ? v.sorted_slot : nullptr,
                                                   gather ? (int)S : 0, gather ? k : 1, nullptr, v.a, st),
                          "gemm1"))
    return rc;
  if (int rc = hip_status(moe::launch_grouped_gemm(MOE_NN, MOE_EPI_NONE, v.a, wo, nullptr, nullptr, v.group_offsets,
                                                   E, S, mlp, emb, nullptr, 0, 1, nullptr, v.o, st),
                          "gemm2"))
    return rc;
  return hip_status(moe::launch_combine(T, emb, k, v.o, v.slot_row, v.topk_w, y, st), "combine");
}

int moe_ffn_bwd(const moe_shape_t* s, const moe_bf16_t* dy, const moe_saved_t* saved, const moe_bf16_t* wi,
                const moe_bf16_t* wo, moe_bf16_t* dx, moe_bf16_t* dwi, moe_bf16_t* dwo, float* dtopk_w, void* ws,
                size_t ws_bytes, moe_stream_t stream) {
  g_detail[0] = 0;
  if (int rc = check_shape(s)) return rc;
  if (!saved) return fail(MOE_ERR_NULL, "saved is NULL");
  NEED(saved->group_offsets);
  if (s->T > 0) {  // with no tokens, per-token buffers may be empty (NULL)
    NEED(dy);
    NEED(saved->topk_w);
    NEED(saved->sorted_slot);
    NEED(saved->slot_row);
    NEED(saved->xs);
    MAYBE(saved->h);  // NULL: recomputed here from xs and wi
    NEED(saved->a);
    NEED(saved->o);
  }
  NEED(wi);
  NEED(wo);
  MAYBE(dx);
  MAYBE(dwi);
  MAYBE(dwo);
  MAYBE(dtopk_w);
  const bool remat = saved->h == nullptr;
  NEED_WS(remat ? bwd_remat_ws(s) : bwd_ws(s));
  const int64_t T = s->T, S = T * s->k;
  const int emb = s->emb, mlp = s->mlp, E = s->E, k = s->k;
  const hipStream_t st = (hipStream_t)stream;
  Carver c{static_cast<char*>(ws)};
  moe_bf16_t* d_o = c.take<moe_bf16_t>(S * emb);
  moe_bf16_t* dh = c.take<moe_bf16_t>(S * 2 * mlp);
  moe_bf16_t* dxs = c.take<moe_bf16_t>(S * emb);
  const float* h = saved->h;
  // combine backward: do (the permutation part) and dtopk_w (the reduction part)
  if (int rc = hip_status(moe::launch_combine_bwd(T, emb, k, dy, dtopk_w ? saved->o : nullptr, saved->slot_row,
                                                  saved->topk_w, d_o, dtopk_w, st),
                          "combine_bwd"))
    return rc;
  if (dwo) {
    if (int rc = hip_status(moe::launch_wgrad(saved->a, d_o, saved->group_offsets, E, S, mlp, emb, dwo, st), "dwo"))
      return rc;
  }
  if (!dx && !dwi) return MOE_OK;
  if (remat && S > 0) {
    // Recompute h = xs . wi[e] with the forward's own GEMM (same kernel, same inputs: the same bits as a
    // saved h). Its SwiGLU output is not needed and goes to the dxs buffer, which is written only later.
    float* hr = c.take<float>(S * 2 * mlp);
    moe_bf16_t* a_tmp = mlp > emb ? c.take<moe_bf16_t>(S * mlp) : dxs;
    if (int rc = hip_status(moe::launch_grouped_gemm(MOE_NN, MOE_EPI_SWIGLU, saved->xs, wi, nullptr, hr,
                                                     saved->group_offsets, E, S, emb, 2 * mlp, nullptr, 0, 1,
                                                     nullptr, a_tmp, st),
                            "recompute h"))
      return rc;
    h = hr;
  }
  // da = w * (dy . wo[e]^T): dy rows read in place through sorted_slot, the top-k weight applied in fp32
  if (int rc = hip_status(moe::launch_grouped_gemm(MOE_NT, MOE_EPI_SWIGLU_BWD, dy, wo, h, nullptr,
                                                   saved->group_offsets, E, S, emb, mlp, saved->sorted_slot, (int)S, k,
                                                   saved->topk_w, dh, st),
                          "dh"))
    return rc;
  if (dwi) {
    if (int rc = hip_status(moe::launch_wgrad(saved->xs, dh, saved->group_offsets, E, S, emb, 2 * mlp, dwi, st),
                            "dwi"))
      return rc;
  }
  if (dx) {
    if (int rc = hip_status(moe::launch_grouped_gemm(MOE_NT, MOE_EPI_NONE, dh, wi, nullptr, nullptr,
                                                     saved->group_offsets, E, S, 2 * mlp, emb, nullptr, 0, 1, nullptr,
                                                     dxs, st),
                            "dxs"))
      return rc;
    if (int rc = hip_status(moe::launch_combine(T, emb, k, dxs, saved->slot_row, nullptr, dx, st), "dx")) return rc;
  }
  return MOE_OK;
}

}  // extern "C"
