// Device helpers shared by the gfx950 kernels of the MoE FFN library.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

#include "tiles.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x32_t __attribute__((ext_vector_type(32)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kMaxExperts = 256;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Two floats -> two bf16 (round to nearest even), lo in bits 0..15: one v_cvt_pk_bf16_f32 with
// both sources. Converting the two values separately gives one convert each plus a shift and an
// OR to merge them: four instructions per pair in every GEMM epilogue.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// silu(g) = g * sigmoid(g), sigmoid(g) = 1 / (1 + e^-g), with the hardware reciprocal (about 1 ulp of
// fp32) instead of an IEEE division: every caller rounds the result to bf16 (2^-9 relative) right after,
// and the division sequence cost the SwiGLU epilogue ~3 us per tile (measured at 8 k-slices per tile).
// Large |g| still gives silu -> 0 (e^-g = inf, reciprocal 0) or g.
__device__ __forceinline__ float silu_f(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }
__device__ __forceinline__ float sigmoid_f(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// The lanes of one wave hand values to each other through LDS with no barrier between the
// write and the read. The hardware runs a wave's LDS instructions in order, so the read sees the
// other lanes' writes; the compiler, reasoning lane by lane, does not know that. Where a lane
// wrote nothing to an address since it last read it (a staging block written by half the lanes,
// then read back by all), it may reuse the value it read before: it did so once the reads of such
// a block were issued together, and half the stored rows were stale. This empty asm with a memory
// clobber stands between each write phase and the read phase that follows, and between that read
// phase and the next write phase; it emits no instruction.
__device__ __forceinline__ void wave_lds_fence() { asm volatile("" ::: "memory"); }

// 16-byte global load / store.
__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }
__device__ __forceinline__ void st8(void* p, u32x2_t v) { *reinterpret_cast<u32x2_t*>(p) = v; }

__device__ __forceinline__ int popc64(uint64_t v) { return __popcll(v); }

// MXFP8 element and scale encodings (OCP microscaling, E4M3 elements with an
// E8M0 scale per 32-element block; see mxfp8.hip).
// E8M0 code of a block whose largest magnitude has fp32 bits amax_bits:
// 2^(floor(log2(amax)) - 8) biased by 127, clamped to [0, 254], 0 for zero.
__device__ __forceinline__ int mx_e8m0_code(uint32_t amax_bits) {
  if (amax_bits == 0) return 0;
  const int e = (int)(amax_bits >> 23) - 127;  // floor(log2(amax)); fp32 subnormals give -127 (clamped below)
  const int c = e - 8 + 127;
  return c < 0 ? 0 : (c > 254 ? 254 : c);
}
// Four E4M3 codes, byte i from value i, of values already divided by their block's scale (so below 512
// in magnitude): nearest value, ties to an even mantissa, magnitudes past 448 saturating, the sign kept.
// gfx950's packed conversion (v_cvt_pk_fp8_f32, to the OCP E4M3 format) rounds to nearest even and keeps
// subnormals; the clamp to +-448 first turns its overflow case into the saturation. Checked on the MI355X
// against an integer-arithmetic encoder of the same rule on every finite bf16 value (the quantizers only
// ever convert bf16 values times a power of two), a million random fp32 values and every rounding tie:
// identical codes.
__device__ __forceinline__ uint32_t mx_e4m3_x4(float a, float b, float c, float d) {
  const auto cl = [](float v) { return fminf(fmaxf(v, -448.0f), 448.0f); };
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), lo, true);
}

}  // namespace moe
