// Launch entry points of the gfx950 kernels (host side). Shapes and buffers
// are validated by the C-ABI layer before any of these is called; each
// returns the HIP status of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kPermuteBlock = 64;  // tokens per histogram block

// Number of compute units of the current device (cached per device).
int device_cu_count();

hipError_t launch_route(int64_t T, int emb, int E, int k, const uint16_t* x, const float* wr, const float* bias,
                        const float* logits_in, int32_t* topk_idx, float* topk_w, hipStream_t stream);

// masks: [nblk, E] uint64, base: [nblk, E] int32, nblk = ceil(T / 64).
hipError_t launch_permute(int64_t T, int emb, int E, int k, const uint16_t* x, const int32_t* topk_idx,
                          int32_t* group_sizes, int32_t* group_offsets, int32_t* sorted_slot, int32_t* slot_row,
                          uint16_t* xs, uint64_t* masks, int32_t* base, hipStream_t stream);

// The same permute on the library's fixed per-GPU scratch (kPermuteScratchBytes): no workspace argument,
// no allocation. The masks and bases ([nblk, E] uint64, [nblk, E] int32, each rounded up to 256 bytes) must
// fit; concurrent calls on one GPU share the scratch and race.
constexpr size_t kPermuteScratchBytes = size_t(4) << 20;
hipError_t launch_permute_noalloc(int64_t T, int emb, int E, int k, const uint16_t* x, const int32_t* topk_idx,
                                  int32_t* group_sizes, int32_t* group_offsets, int32_t* sorted_slot,
                                  int32_t* slot_row, uint16_t* xs, hipStream_t stream);

// grid: workgroups of the persistent grid (a multiple of 8); 0 = persistent_grid().
// row_slot (nullable): output row r reads A row row_slot[r] / slot_div, row_slot values in [0, n_slots).
// slot_scale (nullable): output row r is scaled by slot_scale[row_slot[r]] (or slot_scale[r]).
hipError_t launch_grouped_gemm(int op, int epi, const uint16_t* A, const uint16_t* B, const float* aux_in,
                               float* aux_out, const int32_t* group_offsets, int E, int64_t M, int K, int N,
                               const int32_t* row_slot, int n_slots, int slot_div, const float* slot_scale,
                               uint16_t* C, hipStream_t stream, int grid = 0);

hipError_t launch_wgrad(const uint16_t* A, const uint16_t* D, const int32_t* group_offsets, int E, int64_t M, int P,
                        int Q, uint16_t* C, hipStream_t stream, int grid = 0);

// Workgroups of the persistent GEMM grid: one per compute unit, rounded down to a multiple of 8 (at least 8).
int persistent_grid();

hipError_t launch_combine(int64_t T, int emb, int k, const uint16_t* ys, const int32_t* slot_row, const float* w,
                          uint16_t* y, hipStream_t stream);

hipError_t launch_combine_bwd(int64_t T, int emb, int k, const uint16_t* dy, const uint16_t* ys,
                              const int32_t* slot_row, const float* w, uint16_t* dys, float* dw, hipStream_t stream);

// Router backward, picks held fixed. dl: [T*k] fp32 scratch; wrt: [E, emb] fp32 scratch (used when dx != NULL).
hipError_t launch_mx_quantize_rows(const uint16_t* src, int64_t src_rows, int K, const int32_t* row_index, int row_div,
                                   int64_t M, uint8_t* codes, uint8_t* scales, hipStream_t stream);
hipError_t launch_mx_quantize_weight(const uint16_t* w, int E, int K, int N, uint8_t* codes, uint8_t* scales,
                                     hipStream_t stream);
hipError_t launch_grouped_gemm_mx(int epilogue, const uint8_t* A, const uint8_t* As, int64_t a_rows,
                                  const int32_t* row_slot, int slot_div, const uint8_t* B, const uint8_t* Bs,
                                  const int32_t* group_offsets, int E, int64_t M, int K, int N, uint16_t* C,
                                  uint8_t* Cq, uint8_t* Cqs, hipStream_t stream);
hipError_t launch_route_bwd(int64_t T, int emb, int E, int k, const uint16_t* x, const float* wr,
                            const int32_t* topk_idx, const float* topk_w, const float* dtopk_w,
                            const int32_t* sorted_slot, const int32_t* group_offsets, float* dwr, float* dbias,
                            uint16_t* dx, float* dl, float* dls, int32_t* tok, float* wrt, float* dwrt,
                            hipStream_t stream);

}  // namespace moe
