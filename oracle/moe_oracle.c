/*
 * moe_oracle.c -- plain, slow CPU reference of the sparse-MoE expert FFN.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The GPU library never
 * links, includes or calls it, and this file includes nothing of the GPU
 * library. No blocking, fusion or reordering: every function is the plain
 * definition written out, one token (or one row) at a time.
 *
 * Precision. REAL is the accumulation type of the FFN arithmetic; the build
 * compiles this file twice, with REAL = float (fp32 accumulation, the
 * reference the GPU outputs are held to) and REAL = double (used for the
 * finite-difference gradient checks). Inputs are passed as typed buffers
 * (bf16 bit patterns, fp32 or fp64), converted exactly on load. Router
 * logits are always fp32, computed by one fixed fused-multiply-add chain,
 * because an integer decision (the top-k pick) hangs on them and both sides
 * must take it in the same precision.
 *
 * What is computed, and where the pages state it:
 *  - route: gate + top-k ("[DRAFT][JAX] Optimize MoE block", Flowchart: gate
 *    and top-k routing ahead of the grouped GEMMs); top-k weights and the
 *    per-expert group_size histogram ("Gemma4 26B MoE on TPU v6e: MaxText
 *    layer/model optimizations", Commits table, commit 6).
 *  - dispatch/permute: tokens gathered into expert-sorted order with unit
 *    weights ("MoE: fused TensorCore Pallas permute/combine kernels and
 *    split-expert wi layout for TPU v6e", Commits table, commit 2), without
 *    an unsorted [tokens*top_k, emb] copy (same page, Context item 1).
 *  - one grouped GEMM on the prefused [E, emb, 2*mlp] weight, the output
 *    split into gate and up for SwiGLU ("Keep fused MoE weights intact
 *    through FSDP gather", Description: the updated flow); gate is the first
 *    half (the gate/up split custom VJP in "Gemma4 26B MoE on TPU v6e",
 *    Code Review, concatenates [grad_gate, grad_up] in that order).
 *  - grouped FC2 GEMM on wo [E, mlp, emb] ("[DRAFT][JAX] Optimize MoE block",
 *    Flowchart: activation and grouped FC2 GEMM).
 *  - combine = unpermute + top-k weighted sum ("MoE: fused TensorCore Pallas
 *    permute/combine kernels ...", Commits table, commit 1); its backward is a
 *    permutation for dx and a reduction for the weight gradient (same entry),
 *    and the permute backward is the combine forward with unit weights
 *    (commit 2).
 *  - router backward through the renormalised top-k softmax, picks held
 *    fixed (R7).
 *
 * Readings taken where the pages are silent (each is a choice, not a quote):
 *  R1 logits[t,e] = (fma chain over i = 0..emb-1 of x[t,i]*Wr[i,e], from 0.0f)
 *     + bias[e], all fp32.
 *  R2 top-k selects on logits; larger logit first, equal logits -> lower
 *     expert id; IEEE equality (so -0 == +0); -inf may be picked; NaN is
 *     rejected.
 *  R3 pick order j = 0..k-1 is that descending order.
 *  R4 weights w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k picks
 *     (softmax over all E, then renormalised over the picks, is the same
 *     number), evaluated in double, stored as float.
 *  R5 expert-sorted order = key (expert asc, token asc); a token picks an
 *     expert at most once, so the key is unique.
 *  R6 silu(g) = g / (1 + exp(-g)); SwiGLU a = silu(gate) * up.
 *  R7 the router backward holds the picks fixed (the selection has no
 *     gradient) and uses the forward's saved weights.
 *  R8 MXFP8 ("[DRAFT][JAX] Optimize MoE block", Changes: MXFP8 quantization
 *     of the MoE block) follows the OCP microscaling format: blocks of 32
 *     consecutive elements along the contraction dimension share one
 *     power-of-two scale stored as E8M0 (code c means 2^(c-127)), and the
 *     elements are FP8 E4M3 (OCP "FN": bias 7, largest finite 448, no
 *     infinities). The scale is 2^(floor(log2(amax)) - 8), 8 being the
 *     exponent of E4M3's largest normal, its code clamped to [0, 254]; an
 *     all-zero block takes code 0. Each element is v / scale (exact: a
 *     power-of-two rescaling) rounded to the nearest E4M3 value, ties to an
 *     even mantissa, magnitudes above 448 saturating to 448, the sign kept
 *     (also on zero).
 *  R9 the pages fix only fp32 accumulation. Between stages the layer stores
 *     its activations (a, o, do = w * dy, dh, dxs) in bf16, rounded to
 *     nearest with ties to even. The reference keeps every intermediate in
 *     REAL. The backward functions can instead round them to bf16 where the
 *     layer stores them (stored_bf16): each term of dW is a product of two
 *     stored factors, and dtopk_w is a dot product over emb of the stored o,
 *     so the storage alone moves those results by more than a bf16 output
 *     rounding does.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_REAL
#define ORACLE_REAL float
#endif
typedef ORACLE_REAL real;

/* buffer element types */
enum { ORC_BF16 = 0, ORC_F32 = 1, ORC_F64 = 2 };
/* status codes */
enum { ORC_OK = 0, ORC_EINVAL = 1, ORC_ENAN = 2, ORC_ERANGE = 3, ORC_EDUP = 4, ORC_ENOMEM = 5 };

int orc_real_bytes(void) { return (int)sizeof(real); }

static double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* One element of a typed buffer, exactly converted. */
static double elem(const void* p, int dt, int64_t i) {
  if (dt == ORC_BF16) return bf16_value(((const uint16_t*)p)[i]);
  if (dt == ORC_F32) return (double)((const float*)p)[i];
  return ((const double*)p)[i];
}

/* n consecutive elements of a typed buffer starting at element off, into dst. */
static void load_row(const void* p, int dt, int64_t off, int64_t n, real* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = (real)elem(p, dt, off + i);
}

static int valid_dt(int dt) { return dt == ORC_BF16 || dt == ORC_F32 || dt == ORC_F64; }

/* v rounded to the nearest bf16 value, ties to even (reading R9): the value a bf16 store keeps. A double
   is first rounded to float. */
static real round_bf16(real v) {
  float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) != 0x7f800000u) u += 0x7fffu + ((u >> 16) & 1u); /* finite: carry into the kept bits */
  u &= 0xffff0000u;
  memcpy(&f, &u, 4);
  return (real)f;
}

static real silu(real g) { return (real)((double)g / (1.0 + exp(-(double)g))); }
static real sigmoid(real g) { return (real)(1.0 / (1.0 + exp(-(double)g))); }

/* ---------------------------------------------------------------- router */

/* logits [T, E] fp32 from x [T, emb] (bf16 or fp32) and Wr [emb, E] fp32 (R1). */
int orc_router_logits(int64_t T, int32_t emb, int32_t E, const void* x, int x_dt, const float* wr,
                      const float* bias, float* logits) {
  if (T < 0 || emb <= 0 || E <= 0 || !x || !wr || !logits) return ORC_EINVAL;
  if (x_dt != ORC_BF16 && x_dt != ORC_F32) return ORC_EINVAL;
  float* acc = (float*)malloc(sizeof(float) * (size_t)E);
  if (!acc) return ORC_ENOMEM;
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t e = 0; e < E; ++e) acc[e] = 0.0f;
    /* every (t, e) is its own chain over i ascending; the loop over e only
       runs the E independent chains side by side */
    for (int32_t i = 0; i < emb; ++i) {
      float xv = (float)elem(x, x_dt, t * (int64_t)emb + i);
      const float* w = wr + (int64_t)i * E;
      for (int32_t e = 0; e < E; ++e) acc[e] = fmaf(xv, w[e], acc[e]);
    }
    for (int32_t e = 0; e < E; ++e) logits[t * (int64_t)E + e] = bias ? acc[e] + bias[e] : acc[e];
  }
  free(acc);
  return ORC_OK;
}

/* top-k on logits (R2, R3) and renormalised weights (R4). */
int orc_topk(int64_t T, int32_t E, int32_t k, const float* logits, int32_t* topk_idx, float* topk_w) {
  if (T < 0 || E <= 0 || k <= 0 || k > E || !logits || !topk_idx || !topk_w) return ORC_EINVAL;
  unsigned char* taken = (unsigned char*)malloc((size_t)E);
  if (!taken) return ORC_ENOMEM;
  int rc = ORC_OK;
  for (int64_t t = 0; t < T && rc == ORC_OK; ++t) {
    const float* l = logits + t * (int64_t)E;
    for (int32_t e = 0; e < E; ++e) {
      if (isnan(l[e])) rc = ORC_ENAN;
      taken[e] = 0;
    }
    if (rc != ORC_OK) break;
    for (int32_t j = 0; j < k; ++j) {
      int32_t best = -1;
      for (int32_t e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e; /* strict: equal keeps the lower id */
      }
      taken[best] = 1;
      topk_idx[t * k + j] = best;
    }
    double l0 = (double)l[topk_idx[t * k]];
    double s = 0.0;
    for (int32_t j = 0; j < k; ++j) s += exp((double)l[topk_idx[t * k + j]] - l0);
    for (int32_t j = 0; j < k; ++j) topk_w[t * k + j] = (float)(exp((double)l[topk_idx[t * k + j]] - l0) / s);
  }
  free(taken);
  return rc;
}

/* ---------------------------------------------------------------- dispatch */

/* group_sizes [E], group_offsets [E+1], sorted_slot [S], slot_row [S] from
   topk_idx [T, k]; slot s = t*k + j; row order by key (expert, token) (R5). */
int orc_dispatch(int64_t T, int32_t E, int32_t k, const int32_t* topk_idx, int32_t* group_sizes,
                 int32_t* group_offsets, int32_t* sorted_slot, int32_t* slot_row) {
  if (T < 0 || E <= 0 || k <= 0 || !topk_idx || !group_sizes || !group_offsets || !sorted_slot || !slot_row)
    return ORC_EINVAL;
  for (int64_t t = 0; t < T; ++t)
    for (int32_t j = 0; j < k; ++j) {
      int32_t e = topk_idx[t * k + j];
      if (e < 0 || e >= E) return ORC_ERANGE;
      for (int32_t j2 = 0; j2 < j; ++j2)
        if (topk_idx[t * k + j2] == e) return ORC_EDUP;
    }
  for (int32_t e = 0; e < E; ++e) group_sizes[e] = 0;
  for (int64_t s = 0; s < T * k; ++s) group_sizes[topk_idx[s]] += 1;
  group_offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) group_offsets[e + 1] = group_offsets[e] + group_sizes[e];
  int64_t r = 0;
  for (int32_t e = 0; e < E; ++e)
    for (int64_t t = 0; t < T; ++t)
      for (int32_t j = 0; j < k; ++j)
        if (topk_idx[t * k + j] == e) {
          sorted_slot[r] = (int32_t)(t * k + j);
          slot_row[t * k + j] = (int32_t)r;
          ++r;
        }
  return ORC_OK;
}

/* xs [S, emb] bf16: row r is token sorted_slot[r] / k of x, bit for bit. */
int orc_permute(int64_t T, int32_t emb, int32_t k, const uint16_t* x, const int32_t* sorted_slot, uint16_t* xs) {
  if (T < 0 || emb <= 0 || k <= 0 || !x || !sorted_slot || !xs) return ORC_EINVAL;
  for (int64_t r = 0; r < T * k; ++r) {
    int64_t s = sorted_slot[r];
    if (s < 0 || s >= T * k) return ORC_ERANGE;
    memcpy(xs + r * emb, x + (s / k) * emb, sizeof(uint16_t) * (size_t)emb);
  }
  return ORC_OK;
}

/* ---------------------------------------------------------------- one expert on one token */

typedef struct {
  int32_t emb, mlp;
  real *xrow, *h, *a, *o, *wrow, *dyrow, *dov, *da, *dh, *dxs;
} scratch_t;

static int scratch_init(scratch_t* s, int32_t emb, int32_t mlp) {
  int64_t w = emb > 2 * mlp ? emb : 2 * mlp;
  s->emb = emb;
  s->mlp = mlp;
  real* base = (real*)calloc((size_t)(emb * 5 + 2 * mlp * 2 + mlp * 2 + w), sizeof(real));
  if (!base) return ORC_ENOMEM;
  s->xrow = base;
  s->dyrow = s->xrow + emb;
  s->o = s->dyrow + emb;
  s->dov = s->o + emb;
  s->dxs = s->dov + emb;
  s->h = s->dxs + emb;
  s->dh = s->h + 2 * mlp;
  s->a = s->dh + 2 * mlp;
  s->da = s->a + mlp;
  s->wrow = s->da + mlp;
  return ORC_OK;
}
static void scratch_free(scratch_t* s) { free(s->xrow); }

/* h = x . wi[e] (2*mlp columns), a = silu(h[:mlp]) * h[mlp:], o = a . wo[e]; with round_a, a is rounded
   to bf16 (kept so in s->a) before o. */
static void expert_forward_r(scratch_t* s, int32_t e, const void* wi, int wi_dt, const void* wo, int wo_dt,
                             int round_a) {
  const int32_t emb = s->emb, mlp = s->mlp, n2 = 2 * mlp;
  for (int32_t c = 0; c < n2; ++c) s->h[c] = 0;
  for (int32_t i = 0; i < emb; ++i) {
    load_row(wi, wi_dt, ((int64_t)e * emb + i) * n2, n2, s->wrow);
    for (int32_t c = 0; c < n2; ++c) s->h[c] += s->xrow[i] * s->wrow[c];
  }
  for (int32_t c = 0; c < mlp; ++c) s->a[c] = silu(s->h[c]) * s->h[mlp + c];
  if (round_a)
    for (int32_t c = 0; c < mlp; ++c) s->a[c] = round_bf16(s->a[c]);
  for (int32_t n = 0; n < emb; ++n) s->o[n] = 0;
  for (int32_t c = 0; c < mlp; ++c) {
    load_row(wo, wo_dt, ((int64_t)e * mlp + c) * emb, emb, s->wrow);
    for (int32_t n = 0; n < emb; ++n) s->o[n] += s->a[c] * s->wrow[n];
  }
}

/* given dov = d(loss)/d(o): da = dov . wo[e]^T, dh = [dgate | dup], dxs = dh . wi[e]^T;
   with round_dh, dh is rounded to bf16 (kept so in s->dh) before dxs */
static void expert_backward_r(scratch_t* s, int32_t e, const void* wi, int wi_dt, const void* wo, int wo_dt,
                              int round_dh) {
  const int32_t emb = s->emb, mlp = s->mlp, n2 = 2 * mlp;
  for (int32_t c = 0; c < mlp; ++c) {
    load_row(wo, wo_dt, ((int64_t)e * mlp + c) * emb, emb, s->wrow);
    real acc = 0;
    for (int32_t n = 0; n < emb; ++n) acc += s->dov[n] * s->wrow[n];
    s->da[c] = acc;
  }
  for (int32_t c = 0; c < mlp; ++c) {
    real g = s->h[c], u = s->h[mlp + c], sg = sigmoid(g);
    s->dh[c] = s->da[c] * u * sg * ((real)1 + g * ((real)1 - sg)); /* d silu(g)/dg = sg (1 + g (1 - sg)) */
    s->dh[mlp + c] = s->da[c] * silu(g);
  }
  if (round_dh)
    for (int32_t c = 0; c < n2; ++c) s->dh[c] = round_bf16(s->dh[c]);
  for (int32_t i = 0; i < emb; ++i) {
    load_row(wi, wi_dt, ((int64_t)e * emb + i) * n2, n2, s->wrow);
    real acc = 0;
    for (int32_t c = 0; c < n2; ++c) acc += s->dh[c] * s->wrow[c];
    s->dxs[i] = acc;
  }
}

static void expert_forward(scratch_t* s, int32_t e, const void* wi, int wi_dt, const void* wo, int wo_dt) {
  expert_forward_r(s, e, wi, wi_dt, wo, wo_dt, 0);
}
static void expert_backward(scratch_t* s, int32_t e, const void* wi, int wi_dt, const void* wo, int wo_dt) {
  expert_backward_r(s, e, wi, wi_dt, wo, wo_dt, 0);
}

static int check_common(int32_t emb, int32_t mlp, int32_t E, int32_t k, int x_dt, int wi_dt, int wo_dt) {
  if (emb <= 0 || mlp <= 0 || E <= 0 || k <= 0 || k > E) return ORC_EINVAL;
  if (!valid_dt(x_dt) || !valid_dt(wi_dt) || !valid_dt(wo_dt)) return ORC_EINVAL;
  return ORC_OK;
}

/* ---------------------------------------------------------------- full layer, per token */

/* Forward for the listed tokens: y[i] = sum_j topk_w[t,j] * FFN_{topk_idx[t,j]}(x[t]), t = tokens[i].
   Optional per-(token, pick) intermediates: h [n, k, 2mlp], a [n, k, mlp], o [n, k, emb]. */
int orc_ffn_fwd_tokens(int32_t emb, int32_t mlp, int32_t E, int32_t k, const void* x, int x_dt,
                       const int32_t* topk_idx, const float* topk_w, const void* wi, int wi_dt, const void* wo,
                       int wo_dt, int64_t ntok, const int64_t* tokens, real* y, real* h_out, real* a_out,
                       real* o_out) {
  int rc = check_common(emb, mlp, E, k, x_dt, wi_dt, wo_dt);
  if (rc) return rc;
  if (!x || !topk_idx || !topk_w || !wi || !wo || (ntok > 0 && (!tokens || !y))) return ORC_EINVAL;
  scratch_t s;
  if (scratch_init(&s, emb, mlp)) return ORC_ENOMEM;
  for (int64_t q = 0; q < ntok; ++q) {
    int64_t t = tokens[q];
    load_row(x, x_dt, t * emb, emb, s.xrow);
    real* yr = y + q * emb;
    for (int32_t n = 0; n < emb; ++n) yr[n] = 0;
    for (int32_t j = 0; j < k; ++j) {
      int32_t e = topk_idx[t * k + j];
      if (e < 0 || e >= E) {
        rc = ORC_ERANGE;
        goto done;
      }
      expert_forward(&s, e, wi, wi_dt, wo, wo_dt);
      real w = (real)topk_w[t * k + j];
      for (int32_t n = 0; n < emb; ++n) yr[n] += w * s.o[n];
      if (h_out) memcpy(h_out + (q * k + j) * 2 * mlp, s.h, sizeof(real) * 2 * (size_t)mlp);
      if (a_out) memcpy(a_out + (q * k + j) * mlp, s.a, sizeof(real) * (size_t)mlp);
      if (o_out) memcpy(o_out + (q * k + j) * emb, s.o, sizeof(real) * (size_t)emb);
    }
  }
done:
  scratch_free(&s);
  return rc;
}

/* Backward for the listed tokens, routing held fixed, loss L = sum(dy * y):
   dx[i] = sum_j (FFN_e)'(x[t])^T (w_j dy[t]),  dtopk_w[i, j] = <FFN_e(x[t]), dy[t]>.
   stored_bf16 != 0 takes reading R9 into the backward: a is rounded to bf16 before o = a . wo[e], o
   before the dtopk_w dot product, dh before dxs = dh . wi[e]^T, and dxs before the sum over picks. */
int orc_ffn_bwd_tokens(int32_t emb, int32_t mlp, int32_t E, int32_t k, const void* x, int x_dt,
                       const int32_t* topk_idx, const float* topk_w, const void* wi, int wi_dt, const void* wo,
                       int wo_dt, const void* dy, int dy_dt, int64_t ntok, const int64_t* tokens, real* dx,
                       real* dtopk_w, int32_t stored_bf16) {
  int rc = check_common(emb, mlp, E, k, x_dt, wi_dt, wo_dt);
  if (rc) return rc;
  if (!valid_dt(dy_dt) || !x || !topk_idx || !topk_w || !wi || !wo || !dy) return ORC_EINVAL;
  if (ntok > 0 && (!tokens || !dx)) return ORC_EINVAL;
  scratch_t s;
  if (scratch_init(&s, emb, mlp)) return ORC_ENOMEM;
  for (int64_t q = 0; q < ntok; ++q) {
    int64_t t = tokens[q];
    load_row(x, x_dt, t * emb, emb, s.xrow);
    load_row(dy, dy_dt, t * emb, emb, s.dyrow);
    real* dxr = dx + q * emb;
    for (int32_t i = 0; i < emb; ++i) dxr[i] = 0;
    for (int32_t j = 0; j < k; ++j) {
      int32_t e = topk_idx[t * k + j];
      if (e < 0 || e >= E) {
        rc = ORC_ERANGE;
        goto done;
      }
      expert_forward_r(&s, e, wi, wi_dt, wo, wo_dt, stored_bf16);
      real w = (real)topk_w[t * k + j];
      real dw = 0;
      if (stored_bf16)
        for (int32_t n = 0; n < emb; ++n) s.o[n] = round_bf16(s.o[n]);
      for (int32_t n = 0; n < emb; ++n) dw += s.o[n] * s.dyrow[n];
      if (dtopk_w) dtopk_w[q * k + j] = dw;
      for (int32_t n = 0; n < emb; ++n) s.dov[n] = w * s.dyrow[n];
      expert_backward_r(&s, e, wi, wi_dt, wo, wo_dt, stored_bf16);
      if (stored_bf16)
        for (int32_t i = 0; i < emb; ++i) s.dxs[i] = round_bf16(s.dxs[i]);
      for (int32_t i = 0; i < emb; ++i) dxr[i] += s.dxs[i];
    }
  }
done:
  scratch_free(&s);
  return rc;
}

/* Weight gradients of one expert e over its routed slots (slot = t*k + j, listed in
   expert-sorted order): dwi_e [emb, 2mlp] = sum x[t]^T dh, dwo_e [mlp, emb] = sum a^T do.
   An expert with no slots gets exact zeros.
   stored_bf16 != 0 takes the layer's storage reading R9 into the two products: the factors a,
   do = w * dy and dh, which the layer hands from one stage to the next in bf16, are each rounded to
   bf16 before they enter the sums (da itself is formed from the unrounded w * dy). The sums stay in
   REAL. */
int orc_ffn_wgrad_expert(int32_t emb, int32_t mlp, int32_t E, int32_t k, const void* x, int x_dt,
                         const int32_t* topk_idx, const float* topk_w, const void* wi, int wi_dt, const void* wo,
                         int wo_dt, const void* dy, int dy_dt, int32_t e, int64_t nslots, const int64_t* slots,
                         real* dwi_e, real* dwo_e, int32_t stored_bf16) {
  int rc = check_common(emb, mlp, E, k, x_dt, wi_dt, wo_dt);
  if (rc) return rc;
  if (!valid_dt(dy_dt) || e < 0 || e >= E || !dwi_e || !dwo_e) return ORC_EINVAL;
  if (nslots > 0 && (!slots || !x || !dy || !topk_idx || !topk_w || !wi || !wo)) return ORC_EINVAL;
  const int32_t n2 = 2 * mlp;
  for (int64_t i = 0; i < (int64_t)emb * n2; ++i) dwi_e[i] = 0;
  for (int64_t i = 0; i < (int64_t)mlp * emb; ++i) dwo_e[i] = 0;
  scratch_t s;
  if (scratch_init(&s, emb, mlp)) return ORC_ENOMEM;
  for (int64_t q = 0; q < nslots; ++q) {
    int64_t slot = slots[q], t = slot / k;
    if (topk_idx[slot] != e) {
      rc = ORC_ERANGE;
      break;
    }
    load_row(x, x_dt, t * emb, emb, s.xrow);
    load_row(dy, dy_dt, t * emb, emb, s.dyrow);
    expert_forward_r(&s, e, wi, wi_dt, wo, wo_dt, stored_bf16);
    real w = (real)topk_w[slot];
    for (int32_t n = 0; n < emb; ++n) s.dov[n] = w * s.dyrow[n];
    expert_backward(&s, e, wi, wi_dt, wo, wo_dt);
    if (stored_bf16) { /* a was rounded by the forward */
      for (int32_t n = 0; n < emb; ++n) s.dov[n] = round_bf16(s.dov[n]);
      for (int32_t c = 0; c < n2; ++c) s.dh[c] = round_bf16(s.dh[c]);
    }
    for (int32_t c = 0; c < mlp; ++c)
      for (int32_t n = 0; n < emb; ++n) dwo_e[(int64_t)c * emb + n] += s.a[c] * s.dov[n];
    for (int32_t i = 0; i < emb; ++i)
      for (int32_t c = 0; c < n2; ++c) dwi_e[(int64_t)i * n2 + c] += s.xrow[i] * s.dh[c];
  }
  scratch_free(&s);
  return rc;
}

/* ---------------------------------------------------------------- single stages on given inputs */

/* Expert owning row r under exclusive offsets off[0..E] (off[E] = rows covered); -1 if none. */
static int32_t expert_of_row(const int32_t* off, int32_t E, int64_t r) {
  for (int32_t e = 0; e < E; ++e)
    if (r >= off[e] && r < off[e + 1]) return e;
  return -1;
}

/* Grouped GEMM over rows [r0, r1) of A [M, K]; row r belongs to the expert e with
   off[e] <= r < off[e+1].
   op 0 (NN): B[e] is [K, N] row-major;  op 1 (NT): B[e] is [N, K] row-major (C = A B[e]^T).
   epi 0: C[r] = A[r] B[e]                                  (width N)
   epi 1: h = A[r] B[e]; C[r][c] = silu(h[c]) h[N/2 + c]     (width N/2)
   epi 2: da = A[r] B[e] (width N); aux = saved h [M, 2N];
          C[r] = [da u sg (1 + g (1 - sg)) | da silu(g)]     (width 2N), g = aux[r][c], u = aux[r][N + c]
   Rows outside every group are left untouched. C is [(r1 - r0), width]. */
int orc_grouped_gemm(int32_t op, int32_t epi, const void* A, int a_dt, const void* B, int b_dt, const void* aux,
                     int aux_dt, const int32_t* off, int32_t E, int64_t M, int32_t K, int32_t N, int64_t r0,
                     int64_t r1, real* C) {
  if ((op != 0 && op != 1) || epi < 0 || epi > 2 || !A || !B || !off || !C || E <= 0 || K <= 0 || N <= 0)
    return ORC_EINVAL;
  if (!valid_dt(a_dt) || !valid_dt(b_dt) || r0 < 0 || r1 > M || r0 > r1) return ORC_EINVAL;
  if (epi == 1 && (N % 2)) return ORC_EINVAL;
  if (epi == 2 && (!aux || !valid_dt(aux_dt))) return ORC_EINVAL;
  const int32_t width = epi == 0 ? N : (epi == 1 ? N / 2 : 2 * N);
  real* arow = (real*)malloc(sizeof(real) * (size_t)K);
  real* acc = (real*)malloc(sizeof(real) * (size_t)N);
  if (!arow || !acc) {
    free(arow);
    free(acc);
    return ORC_ENOMEM;
  }
  for (int64_t r = r0; r < r1; ++r) {
    int32_t e = expert_of_row(off, E, r);
    if (e < 0) continue;
    load_row(A, a_dt, r * K, K, arow);
    for (int32_t n = 0; n < N; ++n) {
      real s = 0;
      for (int32_t kk = 0; kk < K; ++kk) {
        int64_t bi = op == 0 ? ((int64_t)e * K + kk) * N + n : ((int64_t)e * N + n) * K + kk;
        s += arow[kk] * (real)elem(B, b_dt, bi);
      }
      acc[n] = s;
    }
    real* cr = C + (r - r0) * width;
    if (epi == 0) {
      for (int32_t n = 0; n < N; ++n) cr[n] = acc[n];
    } else if (epi == 1) {
      for (int32_t c = 0; c < N / 2; ++c) cr[c] = silu(acc[c]) * acc[N / 2 + c];
    } else {
      for (int32_t c = 0; c < N; ++c) {
        real g = (real)elem(aux, aux_dt, r * 2 * (int64_t)N + c);
        real u = (real)elem(aux, aux_dt, r * 2 * (int64_t)N + N + c);
        real sg = sigmoid(g);
        cr[c] = acc[c] * u * sg * ((real)1 + g * ((real)1 - sg));
        cr[N + c] = acc[c] * silu(g);
      }
    }
  }
  free(arow);
  free(acc);
  return ORC_OK;
}

/* Weight-gradient grouped GEMM for one expert: C [P, Q] = sum over rows r of group e of A[r]^T D[r],
   A [M, P], D [M, Q]. An empty group gives exact zeros. */
int orc_grouped_wgrad(const void* A, int a_dt, const void* D, int d_dt, const int32_t* off, int32_t E, int64_t M,
                      int32_t P, int32_t Q, int32_t e, real* C) {
  if (!A || !D || !off || !C || E <= 0 || P <= 0 || Q <= 0 || e < 0 || e >= E) return ORC_EINVAL;
  if (!valid_dt(a_dt) || !valid_dt(d_dt) || off[e] < 0 || off[e + 1] > M || off[e] > off[e + 1]) return ORC_EINVAL;
  real* arow = (real*)malloc(sizeof(real) * (size_t)P);
  real* drow = (real*)malloc(sizeof(real) * (size_t)Q);
  if (!arow || !drow) {
    free(arow);
    free(drow);
    return ORC_ENOMEM;
  }
  for (int64_t i = 0; i < (int64_t)P * Q; ++i) C[i] = 0;
  for (int64_t r = off[e]; r < off[e + 1]; ++r) {
    load_row(A, a_dt, r * P, P, arow);
    load_row(D, d_dt, r * Q, Q, drow);
    for (int32_t p = 0; p < P; ++p)
      for (int32_t q = 0; q < Q; ++q) C[(int64_t)p * Q + q] += arow[p] * drow[q];
  }
  free(arow);
  free(drow);
  return ORC_OK;
}

/* Combine: y[t] = sum_j w[t,j] * ys[slot_row[t*k + j]] in j order; w NULL means unit weights. */
int orc_combine(int64_t T, int32_t emb, int32_t k, const void* ys, int ys_dt, const int32_t* slot_row,
                const float* w, real* y) {
  if (T < 0 || emb <= 0 || k <= 0 || !ys || !slot_row || !y || !valid_dt(ys_dt)) return ORC_EINVAL;
  for (int64_t t = 0; t < T; ++t) {
    real* yr = y + t * emb;
    for (int32_t n = 0; n < emb; ++n) yr[n] = 0;
    for (int32_t j = 0; j < k; ++j) {
      int64_t r = slot_row[t * k + j];
      if (r < 0 || r >= T * k) return ORC_ERANGE;
      real wj = w ? (real)w[t * k + j] : (real)1;
      for (int32_t n = 0; n < emb; ++n) yr[n] += wj * (real)elem(ys, ys_dt, r * emb + n);
    }
  }
  return ORC_OK;
}

/* Combine backward: dys[slot_row[t*k+j]] = w[t,j] * dy[t] (the permutation part) and
   dw[t,j] = <ys[slot_row[t*k+j]], dy[t]> (the reduction part; skipped when ys or dw is NULL). */
/* Router backward with the picks held fixed: the top-k selection is
   piecewise constant in the logits, so gradients flow only through the
   weights. For token t the weights are the softmax over its k picked logits
   (R4), w_j = exp(l_j) / sum_i exp(l_i), whose Jacobian is
   dw_j/dl_m = w_j (delta_jm - w_m). With g = dtopk_w[t]:
     dl[t, e_j] = w_j (g_j - sum_i w_i g_i), every other logit of t gets 0;
   and through l = x Wr + bias:
     dWr[i, e] = sum_t x[t, i] dl[t, e],  dbias[e] = sum_t dl[t, e],
     dx[t, i]  = sum_e dl[t, e] Wr[i, e].
   w and g are the forward's saved weights and the incoming gradient. The
   routing gradients complete training ("MoE: fused TensorCore Pallas
   permute/combine kernels ...", Commits table, commit 1: the combine
   backward's weight-gradient reduction is what feeds them). */
int orc_router_bwd(int64_t T, int32_t emb, int32_t E, int32_t k, const void* x, int x_dt, const float* wr,
                   const int32_t* topk_idx, const float* topk_w, const void* g, int g_dt, real* dlogits, real* dwr,
                   real* dbias, real* dx) {
  if (T < 0 || emb <= 0 || E <= 0 || k <= 0 || k > E || !x || !wr || !topk_idx || !topk_w || !g || !dlogits ||
      !dwr || !valid_dt(x_dt) || !valid_dt(g_dt))
    return ORC_EINVAL;
  for (int64_t t = 0; t < T; ++t)
    for (int32_t j = 0; j < k; ++j) {
      int32_t e = topk_idx[t * k + j];
      if (e < 0 || e >= E) return ORC_ERANGE;
    }
  for (int64_t i = 0; i < T * (int64_t)E; ++i) dlogits[i] = 0;
  for (int64_t t = 0; t < T; ++t) {
    real s = 0;
    for (int32_t j = 0; j < k; ++j) s += (real)topk_w[t * k + j] * (real)elem(g, g_dt, t * k + j);
    for (int32_t j = 0; j < k; ++j) {
      real wj = (real)topk_w[t * k + j];
      dlogits[t * E + topk_idx[t * k + j]] = wj * ((real)elem(g, g_dt, t * k + j) - s);
    }
  }
  for (int64_t i = 0; i < (int64_t)emb * E; ++i) dwr[i] = 0;
  if (dbias)
    for (int32_t e = 0; e < E; ++e) dbias[e] = 0;
  for (int64_t t = 0; t < T; ++t)
    for (int32_t e = 0; e < E; ++e) {
      real d = dlogits[t * E + e];
      if (d == 0) continue;
      if (dbias) dbias[e] += d;
      for (int32_t i = 0; i < emb; ++i) dwr[(int64_t)i * E + e] += (real)elem(x, x_dt, t * emb + i) * d;
    }
  if (dx)
    for (int64_t t = 0; t < T; ++t)
      for (int32_t i = 0; i < emb; ++i) {
        real acc = 0;
        for (int32_t e = 0; e < E; ++e) acc += dlogits[t * E + e] * (real)wr[(int64_t)i * E + e];
        dx[t * emb + i] = acc;
      }
  return ORC_OK;
}

int orc_combine_bwd(int64_t T, int32_t emb, int32_t k, const void* dy, int dy_dt, const void* ys, int ys_dt,
                    const int32_t* slot_row, const float* w, real* dys, real* dw) {
  if (T < 0 || emb <= 0 || k <= 0 || !dy || !slot_row || !w || !dys || !valid_dt(dy_dt)) return ORC_EINVAL;
  if (ys && !valid_dt(ys_dt)) return ORC_EINVAL;
  for (int64_t t = 0; t < T; ++t)
    for (int32_t j = 0; j < k; ++j) {
      int64_t r = slot_row[t * k + j];
      if (r < 0 || r >= T * k) return ORC_ERANGE;
      real wj = (real)w[t * k + j];
      real acc = 0;
      for (int32_t n = 0; n < emb; ++n) {
        real d = (real)elem(dy, dy_dt, t * emb + n);
        dys[r * emb + n] = wj * d;
        if (ys && dw) acc += (real)elem(ys, ys_dt, r * emb + n) * d;
      }
      if (ys && dw) dw[t * k + j] = acc;
    }
  return ORC_OK;
}

/* ------------------------------------------------------------------ MXFP8 */

/* Value of an E4M3 ("FN") code: sign, 4-bit exponent (bias 7), 3-bit
 * mantissa; exponent 0 is subnormal (m/8 * 2^-6). Codes 0x7f / 0xff are NaN
 * and never produced by the quantizer. */
double orc_e4m3_value(uint8_t c) {
  const double sgn = (c & 0x80) ? -1.0 : 1.0;
  const int e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  return e == 0 ? sgn * ldexp((double)m, -9) : sgn * ldexp(8.0 + m, e - 10);
}

/* Nearest E4M3 code to v (ties to even mantissa, |v| > 448 saturates). v is
 * finite. Works on the exact value: the grid spacing below 2^-6 is 2^-9,
 * and in [2^e, 2^(e+1)) it is 2^(e-3). */
static uint8_t e4m3_encode(double v) {
  const uint8_t sgn = signbit(v) ? 0x80 : 0x00;
  double a = fabs(v);
  if (a >= 448.0) return (uint8_t)(sgn | 0x7e);
  int e;
  frexp(a, &e); /* a = f * 2^e, f in [0.5, 1): a in [2^(e-1), 2^e) */
  int ex = e - 1;
  if (ex < -6) ex = -6; /* subnormal range shares the spacing of [2^-6, 2^-5) */
  const double q = ldexp(1.0, ex - 3);
  const double n = a / q; /* exact: q is a power of two */
  double r = floor(n);
  const double frac = n - r;
  if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
  const double val = r * q;
  if (val > 448.0) return (uint8_t)(sgn | 0x7e);
  if (val == 0.0) return sgn;
  if (val < ldexp(1.0, -6)) return (uint8_t)(sgn | (int)(val / ldexp(1.0, -9))); /* subnormal: m */
  int ev;
  frexp(val, &ev);
  const int E = ev - 1; /* val in [2^E, 2^(E+1)) */
  const int m = (int)(val / ldexp(1.0, E - 3)) - 8;
  return (uint8_t)(sgn | ((E + 7) << 3) | m);
}

/* MXFP8 quantization of x [M, K] (bf16 bit patterns, row-major) in blocks of
 * 32 along K: codes [M, K] E4M3 and scales [M, K/32] E8M0 (reading R8).
 * K must be a multiple of 32; non-finite inputs are rejected. */
int orc_mx_quantize(int64_t M, int32_t K, const uint16_t* x, uint8_t* codes, uint8_t* scales) {
  if (M < 0 || K <= 0 || K % 32) return ORC_EINVAL;
  for (int64_t r = 0; r < M; ++r)
    for (int32_t b = 0; b < K / 32; ++b) {
      const uint16_t* blk = x + r * K + (int64_t)b * 32;
      double amax = 0.0;
      for (int i = 0; i < 32; ++i) {
        const double v = bf16_value(blk[i]);
        if (!isfinite(v)) return ORC_ENAN;
        if (fabs(v) > amax) amax = fabs(v);
      }
      int code = 0;
      if (amax > 0.0) {
        int e;
        frexp(amax, &e);
        code = (e - 1) - 8 + 127; /* floor(log2(amax)) - 8, biased */
        if (code < 0) code = 0;
        if (code > 254) code = 254;
      }
      scales[r * (K / 32) + b] = (uint8_t)code;
      const double inv = ldexp(1.0, 127 - code);
      for (int i = 0; i < 32; ++i) codes[r * K + (int64_t)b * 32 + i] = e4m3_encode(bf16_value(blk[i]) * inv);
    }
  return ORC_OK;
}
