// MXFP8 quantization for the MoE block's grouped GEMMs ("[DRAFT][JAX]
// Optimize MoE block", Changes: MXFP8 quantization in the MoE block),
// in the OCP microscaling format: 32 consecutive elements along the
// contraction dimension K share a power-of-two scale held as E8M0 (code c is
// 2^(c-127)); the elements are FP8 E4M3 (bias 7, largest finite 448, no
// infinities, 0x7f/0xff NaN). The scale of a block is 2^(floor(log2(amax)) -
// 8), 8 being the exponent of the largest normal E4M3, with the code clamped
// to [0, 254] and code 0 for an all-zero block; each element is v / scale
// (exact) rounded to the nearest E4M3 value with ties to an even mantissa,
// magnitudes past 448 saturating, the sign kept.
//
// Layouts (both sides of the MXFP8 GEMM are K-contiguous):
//   codes  [rows][K] bytes;
//   scales [K/64][rows][4] bytes: for the 64-element slice j of a row, bytes
//          0 and 1 are the scales of blocks 2j and 2j+1, bytes 2 and 3 are 0.
//          One dword per row and slice, so that a tile's scales for one
//          k-slice are one contiguous run.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// Rows: thread (row r, 8 consecutive elements); 8 threads cover one 64-element slice of a row.
// Source row of output row r: row_index ? row_index[r] / row_div : r (clamped into the source).
__global__ __launch_bounds__(256) void mxq_rows_kernel(const uint16_t* __restrict__ src, int64_t src_rows, int K,
                                                       const int32_t* __restrict__ row_index, int row_div, int64_t M,
                                                       uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int per_row = K / 8;
  const int64_t r = t / per_row;
  if (r >= M) return;  // whole 8-lane groups leave together: per_row is a multiple of 8
  const int c8 = (int)(t % per_row);
  int64_t sr = r;
  if (row_index) {
    sr = row_index[r] / row_div;
    sr = sr < 0 ? 0 : (sr >= src_rows ? src_rows - 1 : sr);
  }
  const u32x4_t v = ld16(src + sr * K + (int64_t)c8 * 8);
  float x[8];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    x[2 * m] = bf16_lo(v[m]);
    x[2 * m + 1] = bf16_hi(v[m]);
  }
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) am = max(am, __float_as_uint(x[i]) & 0x7fffffffu);
  // block of 32 = 4 consecutive threads (aligned in the wave: per_row and c8 are multiples of 8 per slice)
  am = max(am, (uint32_t)__shfl_xor((int)am, 1));
  am = max(am, (uint32_t)__shfl_xor((int)am, 2));
  const int sc = mx_e8m0_code(am);
  const int ex = 127 - sc;
  u32x2_t out;
  out[0] = mx_e4m3_x4(ldexpf(x[0], ex), ldexpf(x[1], ex), ldexpf(x[2], ex), ldexpf(x[3], ex));
  out[1] = mx_e4m3_x4(ldexpf(x[4], ex), ldexpf(x[5], ex), ldexpf(x[6], ex), ldexpf(x[7], ex));
  *reinterpret_cast<u32x2_t*>(codes + r * K + (int64_t)c8 * 8) = out;
  const int sc_odd = __shfl_xor(sc, 4);  // the other block of this 64-element slice
  if ((c8 & 7) == 0) {
    const int64_t j = c8 / 8;
    *reinterpret_cast<uint32_t*>(scales + (j * M + r) * 4) = (uint32_t)sc | ((uint32_t)sc_odd << 8);
  }
}

// Weights [E][K][N] -> codes [E][N][K], scales [E][K/64][N][4]: thread (expert e, column n, slice j) reads the
// column's 64 elements of the slice (adjacent threads read adjacent columns) and writes them contiguously.
__global__ __launch_bounds__(256) void mxq_weight_kernel(const uint16_t* __restrict__ w, int E, int K, int N,
                                                         uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int nj = K / 64;
  const int64_t total = (int64_t)E * nj * N;
  if (t >= total) return;
  const int n = (int)(t % N);
  const int64_t q = t / N;
  const int j = (int)(q % nj);
  const int e = (int)(q / nj);
  const uint16_t* col = w + (int64_t)e * K * N + (int64_t)j * 64 * N + n;
  int sc2[2];
  uint8_t* dst = codes + ((int64_t)e * N + n) * K + (int64_t)j * 64;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    float x[32];
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      x[i] = __uint_as_float((uint32_t)col[(int64_t)(32 * b + i) * N] << 16);
      am = max(am, __float_as_uint(x[i]) & 0x7fffffffu);
    }
    const int sc = mx_e8m0_code(am);
    sc2[b] = sc;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      u32x4_t o;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float* xv = x + 16 * g + 4 * d;
        const int ex = 127 - sc;
        o[d] = mx_e4m3_x4(ldexpf(xv[0], ex), ldexpf(xv[1], ex), ldexpf(xv[2], ex), ldexpf(xv[3], ex));
      }
      st16(dst + 32 * b + 16 * g, o);
    }
  }
  *reinterpret_cast<uint32_t*>(scales + (((int64_t)e * nj + j) * N + n) * 4) =
      (uint32_t)sc2[0] | ((uint32_t)sc2[1] << 8);
}

}  // namespace

hipError_t launch_mx_quantize_rows(const uint16_t* src, int64_t src_rows, int K, const int32_t* row_index, int row_div,
                                   int64_t M, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t threads = M * (K / 8);
  if (threads > 0)
    mxq_rows_kernel<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream>>>(src, src_rows, K, row_index,
                                                                                     row_div, M, codes, scales);
  return hipGetLastError();
}

hipError_t launch_mx_quantize_weight(const uint16_t* w, int E, int K, int N, uint8_t* codes, uint8_t* scales,
                                     hipStream_t stream) {
  const int64_t threads = (int64_t)E * (K / 64) * N;
  if (threads > 0)
    mxq_weight_kernel<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream>>>(w, E, K, N, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
