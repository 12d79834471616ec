// Device helpers shared by the gfx950 kernels of the routed-MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;  // CDNA wavefront width

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;  // one MFMA A/B fragment
typedef __attribute__((ext_vector_type(4))) float f32x4;    // 16x16 MFMA accumulator
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4; // 16-byte load unit

// bf16 bit pattern -> float (exact: a bf16 is the upper half of a binary32).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest, ties to even (quiet NaN kept).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

// Where moe_forward's down GEMMs put the row of flat index i = t * top_k + j: the first pick
// of each token (j = 0, the largest routing weight, since picks are in key order) in fp32
// at row t of y0 [M, H]; every other pick rounded to bf16 (nearest even) at row i of
// y [M * top_k, H].  A token whose weight sits on one pick would otherwise carry that
// pick's bf16 rounding into its output unaveraged.
struct YRow {
  size_t off;   // element offset of the row in y0 (first pick) or y
  bool first;
};
__device__ __forceinline__ YRow y_row(int i, int top_k, int ncols) {
  const int t = i / top_k;
  const bool first = i == t * top_k;
  return YRow{(size_t)(first ? t : i) * ncols, first};
}
// values n .. n + 3 of the row
__device__ __forceinline__ void store_y4(uint16_t* __restrict__ y, float* __restrict__ y0,
                                         YRow r, int n, float a, float b, float c, float d) {
  if (r.first) {
    *reinterpret_cast<float4*>(y0 + r.off + n) = make_float4(a, b, c, d);
  } else {
    uint2 v;
    v.x = pack_bf16x2(a, b);
    v.y = pack_bf16x2(c, d);
    *reinterpret_cast<uint2*>(y + r.off + n) = v;
  }
}

// 16-byte global load / store through the vector memory path.
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).  Lane l supplies A row (l % 16) and
// B column (l % 16), eight consecutive K values each for the K group l / 16; it receives
// D rows 4 * (l / 16) + q, q = 0..3, of column l % 16.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// MXFP8 weights: 16 E4M3 codes (K values k..k+15 of one row, all in one 32-value scale
// block) and the block's E8M0 scale byte -> the two bf16 MFMA fragments of K values
// k..k+7 (lo) and k+8..k+15 (hi).  The products code * 2^(byte - 127) are exact in bf16.
__device__ __forceinline__ void mx_dequant16(u32x4 codes, uint32_t scale_byte, u32x4& lo,
                                             u32x4& hi) {
  const float scale = __uint_as_float(scale_byte ? scale_byte << 23 : 0x00400000u);
#define MOE_CVT(word, high) \
  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, scale, high))
  lo = u32x4{MOE_CVT(codes[0], false), MOE_CVT(codes[0], true), MOE_CVT(codes[1], false),
             MOE_CVT(codes[1], true)};
  hi = u32x4{MOE_CVT(codes[2], false), MOE_CVT(codes[2], true), MOE_CVT(codes[3], false),
             MOE_CVT(codes[3], true)};
#undef MOE_CVT
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

}  // namespace moe
