// Device helpers shared by the gfx950 kernels of the MoE FFN library.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

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
constexpr int kNumXcd = 8;   // MI355X: 8 XCDs, workgroups dealt round-robin across them
constexpr int kMaxExperts = 256;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Two floats -> two bf16 (round to nearest even, hardware convert), lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __hip_bfloat162 v = __float22bfloat162_rn(make_float2(lo, hi));
  return *reinterpret_cast<uint32_t*>(&v);
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }
__device__ __forceinline__ float sigmoid_f(float g) { return 1.0f / (1.0f + __expf(-g)); }

// 16-byte global load / store.
__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }
__device__ __forceinline__ void st8(void* p, u32x2_t v) { *reinterpret_cast<u32x2_t*>(p) = v; }

__device__ __forceinline__ int popc64(uint64_t v) { return __popcll(v); }

// Persistent-grid tile index: workgroup w sits on XCD w % 8. Tile sequence
// number `it` of workgroup w is it * G + (w % 8) * (G / 8) + w / 8, so at any
// moment each XCD works on a contiguous run of G / 8 tiles and those tiles
// share operands in that XCD's L2. G must be a multiple of 8.
__device__ __forceinline__ int64_t xcd_tile(int64_t it, int w, int G) {
  return it * G + (int64_t)(w % kNumXcd) * (G / kNumXcd) + w / kNumXcd;
}

}  // namespace moe
