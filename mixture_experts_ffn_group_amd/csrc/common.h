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
// E4M3 code of v (finite, below 512 in magnitude): nearest value, ties to an
// even mantissa, magnitudes past 448 saturating, the sign kept.
__device__ __forceinline__ uint32_t mx_e4m3_code(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sgn = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a >= 0x43e00000u) return sgn | 0x7eu;  // |v| >= 448
  if (a < 0x3c800000u) {                     // |v| < 2^-6: multiples of 2^-9, nearest-even
    const uint32_t m = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);  // 0..8; 8 is code 0x08
    return sgn | m;
  }
  // keep 3 mantissa bits, round half to even on bit 20; a carry moves into the exponent
  const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;  // (biased fp32 exponent << 3) | mantissa
  const uint32_t c = r - ((127u - 7u) << 3);
  return sgn | (c > 0x7eu ? 0x7eu : c);
}

}  // namespace moe
