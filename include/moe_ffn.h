/*
 * moe_ffn.h -- C ABI of the MI355X (gfx950) sparse-MoE expert-FFN library.
 *
 * The forward pipeline follows the flow in "Keep fused MoE weights intact
 * through FSDP gather" (Description): the prefused expert weight feeds ONE
 * grouped GEMM and only the GEMM output is split into gate and up for SwiGLU.
 * Around it sit the router and the permute/combine pair of "MoE: fused
 * TensorCore Pallas permute/combine kernels and split-expert wi layout for
 * TPU v6e" (Context item 1; Commits table, commits 1 and 2), and the second
 * grouped GEMM of "[DRAFT][JAX] Optimize MoE block" (Flowchart).
 *
 * Conventions for every call:
 *  - Tensor arguments are DEVICE pointers to dense row-major buffers unless
 *    stated. bf16 tensors are passed as raw 16-bit patterns (moe_bf16_t).
 *    Every pointer must be 16-byte aligned.
 *  - The caller owns all memory, the workspace included. The library never
 *    allocates, frees, synchronises or copies between host and device. A
 *    workspace whose required size is 0 (no tokens) may be NULL.
 *  - Calls only enqueue work on `stream` (a hipStream_t; NULL = the null
 *    stream) and return. Results are ready when the stream reaches them.
 *  - Arguments are validated before anything is enqueued. A call that
 *    returns an error has enqueued nothing, except MOE_ERR_HIP, which reports
 *    a launch failure (the HIP error text is in moe_last_error_detail()).
 *  - Index data produced on the device (expert ids, offsets, rows) is not
 *    re-validated on the host. Out-of-range values give unspecified results
 *    but never an access outside the buffers described here.
 *  - The library holds no mutable global state apart from the thread-local
 *    error text. Calls on different streams with separate buffers may run
 *    concurrently.
 *
 * Shapes: T tokens, emb model width, mlp per-expert hidden width, E experts,
 * k experts per token, S = T * k routed rows.
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t moe_bf16_t; /* raw bf16 bit pattern */
typedef void* moe_stream_t;  /* hipStream_t */

typedef struct {
  int64_t T;
  int32_t emb, mlp, E, k;
} moe_shape_t;

enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,       /* sizes inconsistent or out of range */
  MOE_ERR_UNSUPPORTED = 3, /* valid but outside what the kernels support (moe_query_support) */
  MOE_ERR_WORKSPACE = 4,   /* workspace missing or too small */
  MOE_ERR_HIP = 5,         /* a kernel launch failed */
  MOE_ERR_ALIGN = 6        /* a pointer is not 16-byte aligned */
};

enum { MOE_NN = 0, MOE_NT = 1 };
enum { MOE_EPI_NONE = 0, MOE_EPI_SWIGLU = 1, MOE_EPI_SWIGLU_BWD = 2 };

/* Text of a status code (static storage). */
const char* moe_status_str(int status);
/* Detail of the last error on the calling thread ("" if none). */
const char* moe_last_error_detail(void);
/* Library version string. */
const char* moe_version(void);

/*
 * moe_query_support: MOE_OK if the layer kernels accept this shape, else the
 * reason (MOE_ERR_SHAPE / MOE_ERR_UNSUPPORTED, detail text set). Supported:
 * 0 <= T, T*k < 2^31, T*emb < 2^31; emb % 64 == 0; mlp % 64 == 0; 1 <= k <= 64; k <= E <= 256.
 * The pages' own Pallas kernels guard a similar envelope (a capability check
 * on dtype, width multiple of 128 lanes, row count = tokens * k and k <= 128;
 * "MoE: fused TensorCore Pallas permute/combine kernels ...", Code Review).
 * Here an unsupported shape is an error, never a fallback.
 */
int moe_query_support(const moe_shape_t* shape);

/*
 * Workspace sizes in bytes (host computation, no device access).
 *  moe_permute_workspace_bytes: scratch of moe_permute (per-block expert
 *    masks and row bases).
 *  moe_workspace_bytes: scratch of moe_ffn_fwd (with_backward = 0: routing,
 *    indices and the xs/a/o activations when no saved set is given) or of
 *    moe_ffn_bwd (with_backward = 1: the do/dh/dxs activations; 2: also h,
 *    for a saved set whose h is NULL).
 */
size_t moe_permute_workspace_bytes(const moe_shape_t* shape);
size_t moe_workspace_bytes(const moe_shape_t* shape, int with_backward);
/* moe_route_bwd_workspace_bytes: scratch of moe_route_bwd (per-slot logit
 * gradients, the sorted rows' tokens and gradients, and [E, emb] copies of
 * the router weight and its gradient). */
size_t moe_route_bwd_workspace_bytes(const moe_shape_t* shape);

/*
 * moe_route -- gate and top-k routing ("[DRAFT][JAX] Optimize MoE block",
 * Flowchart; top-k weights on the main compute units in "Gemma4 26B MoE on
 * TPU v6e: MaxText layer/model optimizations", Commits table, commit 6).
 *  x [T, emb] bf16; wr [emb, E] fp32; bias [E] fp32 or NULL (added to the
 *  logits, may hold -inf to disable an expert).
 *  logits_in [T, E] fp32 or NULL: when given, these are the logits (x, wr
 *  and bias must then be NULL).
 *  Outputs topk_idx [T, k] int32 and topk_w [T, k] fp32.
 * Logits are the fp32 fused-multiply-add chain over emb in ascending order
 * starting from 0, then + bias (one fp32 add). Picks are in descending logit
 * order; equal logits go to the lower expert id (+0 equals -0). The weights
 * are the softmax over the k picked logits (which equals the full softmax
 * renormalised over the picks). NaN logits give unspecified picks.
 */
int moe_route(const moe_shape_t* shape, const moe_bf16_t* x, const float* wr, const float* bias,
              const float* logits_in, int32_t* topk_idx, float* topk_w, moe_stream_t stream);

/*
 * moe_permute -- group_size histogram, then the gather of tokens into
 * expert-sorted order ("MoE: fused TensorCore Pallas permute/combine
 * kernels ...", Commits table, commit 2: the histogram moves above the
 * gather). The unsorted [T*k, emb] copy is never built (same page, Context
 * item 1): each token row is read once and written to its k sorted rows.
 *  x [T, emb] bf16, topk_idx [T, k] int32 in [0, E), distinct per token.
 *  Outputs: group_sizes [E], group_offsets [E + 1] (exclusive prefix,
 *  group_offsets[E] = S), sorted_slot [S] (row r holds slot t*k + j),
 *  slot_row [S] (its inverse), xs [S, emb] bf16 (row r = x[sorted_slot[r]/k]).
 *  Row order: by expert, then by token (stable), so it is unique.
 *  xs may be NULL: then only the index is built (group_sizes, group_offsets,
 *  sorted_slot, slot_row) and x may be NULL too. A grouped GEMM then reads
 *  the token rows in place through sorted_slot (moe_gemm_rows_t with
 *  slot_div = k) instead of from a sorted copy.
 *  ws: at least moe_permute_workspace_bytes(shape) bytes of device memory.
 */
int moe_permute(const moe_shape_t* shape, const moe_bf16_t* x, const int32_t* topk_idx, int32_t* group_sizes,
                int32_t* group_offsets, int32_t* sorted_slot, int32_t* slot_row, moe_bf16_t* xs, void* ws,
                size_t ws_bytes, moe_stream_t stream);

/*
 * moe_permute_noalloc -- moe_permute without a workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation). Same arguments, outputs and
 * errors as moe_permute, minus ws / ws_bytes. Its masks and row bases live in
 * a fixed scratch array of the library, 4 MiB per GPU (allocated when the
 * library's device code is loaded on that GPU and held until the process
 * ends); it needs 12 * ceil(T / 64) * E bytes (each of its two regions
 * rounded up to 256), so T <= 174,720 at E = 128 and T <= 87,360 at E = 256;
 * a larger shape returns MOE_ERR_WORKSPACE and enqueues nothing. The call
 * allocates nothing. All calls on one GPU share that GPU's scratch, which
 * keeps the last call's contents: calls that may overlap on one GPU (several
 * streams, several threads) race and must be serialised by the caller.
 */
int moe_permute_noalloc(const moe_shape_t* shape, const moe_bf16_t* x, const int32_t* topk_idx,
                        int32_t* group_sizes, int32_t* group_offsets, int32_t* sorted_slot, int32_t* slot_row,
                        moe_bf16_t* xs, moe_stream_t stream);

/* Optional row mapping of a grouped GEMM (see moe_grouped_gemm). */
typedef struct {
  const int32_t* row_slot;  /* [M] device, or NULL: output row r reads A row row_slot[r] / slot_div */
  int32_t n_slots;          /* row_slot values lie in [0, n_slots); A then has n_slots / slot_div rows */
  int32_t slot_div;         /* >= 1 (k when row_slot holds slots t*k + j and A is [T, K]) */
  const float* slot_scale;  /* device or NULL: output row r is scaled, in fp32 before the epilogue, by
                               slot_scale[row_slot[r]] ([n_slots]), or by slot_scale[r] ([M]) without row_slot */
} moe_gemm_rows_t;

/*
 * moe_grouped_gemm -- ragged grouped GEMM over expert groups, bf16 in, fp32
 * accumulate, bf16 out. Row r of the output belongs to the expert e with
 * group_offsets[e] <= r < group_offsets[e + 1] (device array [E + 1]); rows
 * at or past group_offsets[E] are not written. Groups may be empty.
 *  op MOE_NN: B is [E, K, N] (B[e] is K x N).  op MOE_NT: B is [E, N, K]
 *  (C = A B[e]^T, the transposed-RHS backward form of "MoE: fused TensorCore
 *  Pallas permute/combine kernels ...", Related PRs, part 3).
 *  A [M, K] bf16, or with rows->row_slot the rows are gathered in place from
 *  A [n_slots / slot_div, K] (no permuted copy is made).
 *  Epilogues:
 *   MOE_EPI_NONE: C [M, N].
 *   MOE_EPI_SWIGLU (op NN, N = 2*mlp, the prefused [gate | up] weight of
 *    "Keep fused MoE weights intact through FSDP gather", Description):
 *    C [M, mlp] = silu(h[:, :mlp]) * h[:, mlp:] with h = A B[e] kept in fp32;
 *    aux_out [M, 2*mlp] fp32 receives h when non-NULL (saved for backward).
 *   MOE_EPI_SWIGLU_BWD (op NT, N = mlp): da = A B[e]^T; aux_in = saved h
 *    [M, 2*mlp] fp32; C [M, 2*mlp] = [da*u*s*(1 + g*(1 - s)) | da*silu(g)]
 *    with g = h[:, :mlp], u = h[:, mlp:], s = sigmoid(g) -- one concatenated
 *    gradient, as in the gate/up split VJP of "Gemma4 26B MoE on TPU v6e",
 *    Commits table, commit 7.
 *  rows: NULL, or a row gather and/or per-row fp32 scale (moe_gemm_rows_t).
 *  Needs K % 64 == 0, N % 8 == 0 (SWIGLU: mlp % 8 == 0), M < 2^31.
 */
int moe_grouped_gemm(int op, int epilogue, const moe_bf16_t* A, const moe_bf16_t* B, const float* aux_in,
                     float* aux_out, const int32_t* group_offsets, int32_t E, int64_t M, int32_t K, int32_t N,
                     const moe_gemm_rows_t* rows, moe_bf16_t* C, moe_stream_t stream);

/*
 * moe_grouped_gemm_wgrad -- weight gradient of a grouped GEMM: for every
 * expert e, C[e] [P, Q] = sum over rows r of group e of A[r]^T D[r] (the
 * gradients of the grouped GEMM, "MoE: fused TensorCore Pallas
 * permute/combine kernels ...", Tests). A [M, P], D [M, Q] bf16;
 * C [E, P, Q] bf16; an empty group gives exact zeros. fp32 accumulate.
 * Needs P % 8 == 0, Q % 8 == 0.
 */
int moe_grouped_gemm_wgrad(const moe_bf16_t* A, const moe_bf16_t* D, const int32_t* group_offsets, int32_t E,
                           int64_t M, int32_t P, int32_t Q, moe_bf16_t* C, moe_stream_t stream);

/*
 * moe_grouped_gemm_grid / moe_grouped_gemm_wgrad_grid -- the same calls with
 * the size of the persistent grid given: `grid` workgroups (0, or a positive
 * multiple of 8 up to 65536; 0 = one per compute unit, which is what
 * moe_grouped_gemm and moe_grouped_gemm_wgrad launch). The result does not
 * depend on the grid: every output tile is computed whole by one workgroup,
 * in the same order of k. A small grid makes each workgroup run many tiles
 * in turn; tests use it to cover the persistent loop's tile-to-tile hand-over
 * (loads of the next tile issued during the current tile's epilogue) on
 * shapes small enough for an element-by-element comparison.
 */
int moe_grouped_gemm_grid(int op, int epilogue, const moe_bf16_t* A, const moe_bf16_t* B, const float* aux_in,
                          float* aux_out, const int32_t* group_offsets, int32_t E, int64_t M, int32_t K, int32_t N,
                          const moe_gemm_rows_t* rows, moe_bf16_t* C, int32_t grid, moe_stream_t stream);
int moe_grouped_gemm_wgrad_grid(const moe_bf16_t* A, const moe_bf16_t* D, const int32_t* group_offsets, int32_t E,
                                int64_t M, int32_t P, int32_t Q, moe_bf16_t* C, int32_t grid, moe_stream_t stream);

/*
 * moe_tile_schedule -- HOST call, no device access: the tile list that the
 * persistent grouped GEMMs run on a grid of `grid` workgroups (a positive
 * multiple of 8), computed by the same functions the kernels call. The pages'
 * grouped GEMM runs only the tiles a group needs, masking the partial tile at
 * a group edge ("MoE: fused TensorCore Pallas permute/combine kernels ...",
 * Tests: boundary-tile masking; "[DRAFT][JAX] Optimize MoE block", Changes:
 * group-aware kernels).
 *  kind MOE_SCHED_GEMM: moe_grouped_gemm with the plain output, N output
 *   columns. MOE_SCHED_GEMM_SWIGLU: the SwiGLU epilogue, N = 2*mlp (mlp
 *   output columns). MOE_SCHED_WGRAD: moe_grouped_gemm_wgrad with C[e]
 *   [N, Q] (N is P there); Q is ignored by the other kinds.
 *  group_offsets: HOST array [E + 1], read as the kernels read theirs.
 *  tiles: HOST array [capacity][7] int32 or NULL when capacity is 0; tile i
 *   is {workgroup, turn, expert, row0, row1, col0, col1}: rows [row0, row1)
 *   of the output (of dW[e] for WGRAD) and columns [col0, col1) that the
 *   workgroup computes on that turn, past group ends and widths excluded.
 *   GEMM row blocks are 256 rows, except that a group of 257-512 rows runs
 *   as two halves (its first ceil(n/2) rows, then the rest) whose tiles of
 *   each column are adjacent in the list.
 *  *count receives the number of tiles (tiles beyond capacity are counted,
 *   not written).
 */
enum { MOE_SCHED_GEMM = 0, MOE_SCHED_GEMM_SWIGLU = 1, MOE_SCHED_WGRAD = 2 };
int moe_tile_schedule(int32_t kind, const int32_t* group_offsets, int32_t E, int64_t M, int32_t N, int32_t Q,
                      int32_t grid, int32_t* tiles, int64_t capacity, int64_t* count);

/*
 * moe_combine -- unpermute plus top-k weighted sum ("MoE: fused TensorCore
 * Pallas permute/combine kernels ...", Commits table, commit 1):
 *  y[t] = sum_{j<k} topk_w[t, j] * ys[slot_row[t*k + j]], accumulated in fp32
 *  by fused multiply-add in j order, rounded once to bf16.
 *  ys [S, emb] bf16; slot_row [S]; topk_w [T, k] fp32 or NULL for unit
 *  weights (the permute backward, same table, commit 2); y [T, emb] bf16.
 */
int moe_combine(const moe_shape_t* shape, const moe_bf16_t* ys, const int32_t* slot_row, const float* topk_w,
                moe_bf16_t* y, moe_stream_t stream);

/*
 * moe_combine_bwd -- backward of moe_combine (same table, commit 1: a
 * permutation for dx and a reduction for the weight gradient):
 *  dys[slot_row[t*k + j]] = bf16(topk_w[t, j] * dy[t]);
 *  dtopk_w[t, j] = sum_n ys[slot_row[t*k + j], n] * dy[t, n] (fp32; skipped
 *  when ys or dtopk_w is NULL).
 */
int moe_combine_bwd(const moe_shape_t* shape, const moe_bf16_t* dy, const moe_bf16_t* ys, const int32_t* slot_row,
                    const float* topk_w, moe_bf16_t* dys, float* dtopk_w, moe_stream_t stream);

/* Caller-owned activations of one forward pass, kept for the backward. All
   device pointers: topk_idx [T,k], topk_w [T,k], group_sizes [E],
   group_offsets [E+1], sorted_slot [S], slot_row [S], xs [S,emb] bf16,
   h [S,2*mlp] fp32 (the gate/up pre-activations, unrounded) or NULL, a
   [S,mlp] bf16, o [S,emb] bf16. With h NULL the forward does not keep the
   gate/up values and the backward recomputes them (the Gemma4 workload of
   "MoE: fused TensorCore Pallas permute/combine kernels ...", Context, runs
   with full rematerialisation): 8*S*mlp fewer bytes held between the passes
   for one more GEMM1 in the backward. */
typedef struct {
  int32_t* topk_idx;
  float* topk_w;
  int32_t* group_sizes;
  int32_t* group_offsets;
  int32_t* sorted_slot;
  int32_t* slot_row;
  moe_bf16_t* xs;
  float* h;
  moe_bf16_t* a;
  moe_bf16_t* o;
} moe_saved_t;

/*
 * moe_route_bwd -- gradients of the router, the picks held fixed: the top-k
 * selection has no gradient, so they flow through the top-k weights only,
 * which are the softmax over each token's k picked logits. The incoming
 * gradient dtopk_w is the combine backward's reduction ("MoE: fused
 * TensorCore Pallas permute/combine kernels ...", Commits table, commit 1).
 * With g = dtopk_w[t] and the forward's weights w:
 *   dlogits[t, e_j] = w_j (g_j - sum_i w_i g_i)   (0 for experts not picked)
 *   dwr[i, e]  = sum_t x[t, i] dlogits[t, e]      (fp32, [emb, E], overwritten)
 *   dbias[e]   = sum_t dlogits[t, e]              (fp32 [E], or NULL)
 *   dx[t, :]  += sum_j dlogits[t, e_j] wr[:, e_j] (bf16 [T, emb] in/out, or NULL)
 *  x [T, emb] bf16 and wr [emb, E] fp32 are the forward's router inputs;
 *  topk_idx, topk_w [T, k] its routing; sorted_slot [S] and group_offsets
 *  [E+1] its permute index (moe_permute); dtopk_w [T, k] fp32 (moe_combine_bwd
 *  or moe_ffn_bwd).
 *  Order: dwr and dbias sum each expert's rows in expert-sorted (token)
 *  order with fp32 fused multiply-adds; the sum of s in dlogits runs over the
 *  picks in order; dx adds the k terms to the incoming value in fp32, in
 *  pick order, then rounds once. Results do not depend on scheduling.
 *  ws: at least moe_route_bwd_workspace_bytes(shape) bytes.
 */
int moe_route_bwd(const moe_shape_t* shape, const moe_bf16_t* x, const float* wr, const int32_t* topk_idx,
                  const float* topk_w, const float* dtopk_w, const int32_t* sorted_slot,
                  const int32_t* group_offsets, float* dwr, float* dbias, moe_bf16_t* dx, void* ws, size_t ws_bytes,
                  moe_stream_t stream);

/*
 * MXFP8 ("[DRAFT][JAX] Optimize MoE block", Changes: MXFP8 quantization in
 * the MoE block), in the OCP microscaling format: 32 consecutive elements
 * along the contraction dimension K share a power-of-two scale held as E8M0
 * (code c is 2^(c-127)), and the elements are FP8 E4M3 (bias 7, largest
 * finite 448). A block's scale is 2^(floor(log2(amax)) - 8), code clamped to
 * [0, 254], code 0 for an all-zero block; each element is v / scale rounded
 * to the nearest E4M3 value, ties to an even mantissa, magnitudes past 448
 * saturating, the sign kept. Inputs must be finite (otherwise the codes are
 * unspecified). Layouts, both K-contiguous:
 *   codes  [rows][K] bytes;
 *   scales [K/64][rows][4] bytes: bytes 0 and 1 hold the scales of blocks
 *          2j and 2j+1 of slice j of the row, bytes 2 and 3 are zero.
 * K must be a multiple of 64.
 *
 * moe_mx_quantize_rows -- rows of src [src_rows, K] bf16: output row r is
 *  source row row_index[r] / row_div (clamped into [0, src_rows)) when
 *  row_index is given (a gather through sorted_slot with row_div = k builds
 *  the expert-sorted rows directly), else row r. codes [M, K], scales
 *  [K/64][M][4].
 */
int moe_mx_quantize_rows(const moe_bf16_t* src, int64_t src_rows, int32_t K, const int32_t* row_index,
                         int32_t row_div, int64_t M, uint8_t* codes, uint8_t* scales, moe_stream_t stream);

/*
 * moe_mx_quantize_weight -- expert weights w [E, K, N] bf16 (the layout of wi
 *  and wo) in blocks of 32 along K, transposed to K-contiguous rows:
 *  codes [E, N, K], scales [E][K/64][N][4].
 */
int moe_mx_quantize_weight(const moe_bf16_t* w, int32_t E, int32_t K, int32_t N, uint8_t* codes, uint8_t* scales,
                           moe_stream_t stream);

/*
 * moe_grouped_gemm_mx -- grouped GEMM on MXFP8 operands ("[DRAFT][JAX]
 *  Optimize MoE block", Flowchart: grouped FC1 quantize and GEMM), on the
 *  block-scaled fp8 matrix cores: C[r, :] = A[r, :] . B[e]^T for the rows r
 *  of group e, A and B being E4M3 codes times their 32-element blocks' E8M0
 *  scales. A: codes [a_rows, K] and scales [K/64][a_rows][4]
 *  (moe_mx_quantize_rows); row r of the product reads A row
 *  row_slot[r] / slot_div (clamped into [0, a_rows)) when row_slot is given
 *  (token rows quantized once, read in place through sorted_slot with
 *  slot_div = k), else A row r, and then a_rows must equal M.
 *  B: codes [E, N, K] and scales [E][K/64][N][4] (moe_mx_quantize_weight).
 *  epilogue MOE_EPI_NONE: C [M, N] bf16; MOE_EPI_SWIGLU: B is a prefused
 *  [gate | up] weight and C [M, N/2] bf16 is silu(gate) * up, computed in
 *  fp32 and rounded once. With SWIGLU the output can also (or instead: C may
 *  then be NULL) be written as MXFP8, C_codes [M, N/2] and C_scales
 *  [N/128][M][4], the operand of the next MXFP8 GEMM: the bf16-rounded values
 *  quantized as moe_mx_quantize_rows would (bytes 2 and 3 of the scale dwords
 *  are left unwritten; (N/2) % 64 == 0). C_codes and C_scales are both given
 *  or both NULL. Accumulation is fp32 across 64-element K steps;
 *  within a step the hardware sums the scaled products to a precision fixed
 *  relative to the largest of them. Rows of C outside [group_offsets[0],
 *  group_offsets[E]) are not written. K % 64 == 0, N % 8 == 0 (N % 16 for
 *  SWIGLU), E <= 256, a_rows*K and N*K below 2^32.
 */
int moe_grouped_gemm_mx(int32_t epilogue, const uint8_t* A, const uint8_t* A_scales, int64_t a_rows,
                        const int32_t* row_slot, int32_t slot_div, const uint8_t* B, const uint8_t* B_scales,
                        const int32_t* group_offsets, int32_t E, int64_t M, int32_t K, int32_t N, moe_bf16_t* C,
                        uint8_t* C_codes, uint8_t* C_scales, moe_stream_t stream);

/*
 * moe_ffn_fwd_mx -- the MoE FFN forward with MXFP8 grouped GEMMs (inference):
 *  route and index-only permute as in moe_ffn_fwd; each token row of x
 *  quantized once (moe_mx_quantize_rows); GEMM 1 on the prefused weight reads
 *  the token codes through sorted_slot and writes its SwiGLU output as MXFP8;
 *  GEMM 2; combine into y [T, emb] bf16. The expert weights come quantized:
 *  wi_codes [E, 2*mlp, emb] and wi_scales [E][emb/64][2*mlp][4] from
 *  moe_mx_quantize_weight(wi), wo_codes [E, emb, mlp] and wo_scales
 *  [E][mlp/64][emb][4] from moe_mx_quantize_weight(wo). mlp % 64 == 0;
 *  T*emb and T*k*mlp below 2^32. Router inputs as in moe_route.
 *  ws: at least moe_workspace_bytes_mx(shape) bytes (0: unsupported shape).
 */
size_t moe_workspace_bytes_mx(const moe_shape_t* shape);
int moe_ffn_fwd_mx(const moe_shape_t* shape, const moe_bf16_t* x, const float* wr, const float* bias,
                   const float* logits_in, const uint8_t* wi_codes, const uint8_t* wi_scales, const uint8_t* wo_codes,
                   const uint8_t* wo_scales, moe_bf16_t* y, void* ws, size_t ws_bytes, moe_stream_t stream);

/*
 * moe_ffn_fwd -- the whole MoE FFN forward: route, permute, grouped GEMM on
 * the prefused wi [E, emb, 2*mlp] with the SwiGLU epilogue, grouped GEMM on
 * wo [E, mlp, emb], combine. y [T, emb] bf16.
 *  Router inputs as in moe_route. saved: NULL for inference (intermediates
 *  live in the workspace and h is not produced), else every pointer in it
 *  but h must be set and receives the intermediates (h NULL: not kept).
 *  For inference the expert-sorted copy xs is not written: the permute builds
 *  only the index and GEMM1 gathers x rows through sorted_slot, the
 *  single-device half of the fused MoE kernel of "Fused MoE Kernel
 *  integration and optimization - #3388" (Summary). With saved, xs is built
 *  (the weight gradient reads it).
 *  ws: at least moe_workspace_bytes(shape, 0) bytes.
 */
int moe_ffn_fwd(const moe_shape_t* shape, const moe_bf16_t* x, const float* wr, const float* bias,
                const float* logits_in, const moe_bf16_t* wi, const moe_bf16_t* wo, moe_bf16_t* y,
                const moe_saved_t* saved, void* ws, size_t ws_bytes, moe_stream_t stream);

/*
 * moe_ffn_bwd -- backward of moe_ffn_fwd with the routing held fixed, for
 * the loss sum(dy * y): combine backward, NT grouped GEMM on wo with the
 * SwiGLU-backward epilogue, NT grouped GEMM on wi, permute backward
 * (combine with unit weights), and the two weight-gradient grouped GEMMs.
 * The wo GEMM reads dy rows in place through sorted_slot and applies each
 * row's top-k weight in fp32, so its input is never rounded after scaling.
 *  dy [T, emb] bf16; saved from a moe_ffn_fwd call with the same shape and
 *  weights. Outputs (each may be NULL to skip it): dx [T, emb] bf16,
 *  dwi [E, emb, 2*mlp] bf16, dwo [E, mlp, emb] bf16, dtopk_w [T, k] fp32.
 *  If saved->h is NULL, h is first recomputed from xs and wi by the
 *  forward's own GEMM, which gives the same bits as a kept h, so the
 *  gradients are identical either way.
 *  ws: at least moe_workspace_bytes(shape, 1) bytes, or
 *  moe_workspace_bytes(shape, 2) if saved->h is NULL.
 */
int moe_ffn_bwd(const moe_shape_t* shape, const moe_bf16_t* dy, const moe_saved_t* saved, const moe_bf16_t* wi,
                const moe_bf16_t* wo, moe_bf16_t* dx, moe_bf16_t* dwi, moe_bf16_t* dwo, float* dtopk_w, void* ws,
                size_t ws_bytes, moe_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_FFN_H */
