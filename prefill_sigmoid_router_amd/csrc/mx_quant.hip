// MXFP8 expert weights: quantize bf16 weights and dequantize them back.
//
// AlphaMoE page (FlashInfer PR #6511 analysis), section 1: the routed-MoE kernels read
// block-scaled narrow weights so that a decode step streams fewer bytes.  The format here
// is the OCP Microscaling (MX) v1.0 one with FP8 E4M3 elements: one E8M0 scale byte per 32
// consecutive values of a row (along K), shared exponent s = floor(log2(max |v|)) - 8 (8 is
// the exponent of E4M3's largest normal, 448), elements E4M3(v / 2^s) rounded to nearest
// even and clamped to +-448; a block of zeros gets scale byte 0.
//
// One thread per 32-value block.  Every step is exact integer or power-of-two arithmetic,
// so the codes match any correct implementation of the conversion bit for bit.
#include "device_common.h"
#include "launchers.h"

namespace moe {

namespace {

constexpr int kMxBlock = 32;

// |v| < 512 and finite (v = bf16 value / 2^s): E4M3 code, round to nearest even, 448 max.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (!(a < 448.0f)) {
    code = 0x7Eu;
  } else if (a < 0x1p-6f) {
    code = (uint32_t)rintf(a * 512.0f);  // subnormal grid 2^-9; 8 becomes 0x08 = 2^-6
  } else {
    const uint32_t ab = __float_as_uint(a);
    const int ex = (int)(ab >> 23) - 127;  // -6 .. 8
    const uint32_t m = ab & 0x7FFFFFu;
    uint32_t q = m >> 20;
    const uint32_t rem = m & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;  // a carry moves to the exponent
    code = ((uint32_t)(ex + 7) << 3) + q;
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return code ? (code | sign) : 0u;
}

__global__ __launch_bounds__(256) void mx_quantize_kernel(const uint16_t* __restrict__ w,
                                                          int64_t nblocks,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = ld16(w + b * kMxBlock + 8 * i);
  uint32_t amax = 0;  // largest |value| as bf16 bits (ordered like the magnitudes)
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      amax = max(amax, v[i][j] & 0x7FFFu);
      amax = max(amax, (v[i][j] >> 16) & 0x7FFFu);
    }
  int s = -127;
  if (amax != 0) {
    const int field = (int)(amax >> 7);
    const int fl = field ? field - 127 : (31 - __clz((int)(amax & 0x7Fu))) - 133;  // floor(log2)
    s = min(127, max(-127, fl - 8));
  }
  scales[b] = (uint8_t)(s + 127);
  const float inv = __uint_as_float((uint32_t)(127 - s) << 23);  // 2^-s, s <= 119 here
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t c0 = e4m3_code(bf16lo(v[i][j]) * inv);
      const uint32_t c1 = e4m3_code(bf16hi(v[i][j]) * inv);
      const int e = 8 * i + 2 * j;  // element index of c0
      if ((e & 3) == 0) out[e >> 2] = c0 | (c1 << 8);
      else out[e >> 2] |= (c0 << 16) | (c1 << 24);
    }
  st16(codes + b * kMxBlock, u32x4{out[0], out[1], out[2], out[3]});
  st16(codes + b * kMxBlock + 16, u32x4{out[4], out[5], out[6], out[7]});
}

// One thread per 16 codes (half a block): the same conversion the MXFP8 GEMMs use.
__global__ __launch_bounds__(256) void mx_dequantize_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            int64_t nhalves,
                                                            uint16_t* __restrict__ w) {
  const int64_t h = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (h >= nhalves) return;
  u32x4 lo, hi;
  mx_dequant16(ld16(codes + h * 16), scales[h >> 1], lo, hi);
  st16(w + h * 16, lo);
  st16(w + h * 16 + 8, hi);
}

}  // namespace

hipError_t launch_mx_quantize(const uint16_t* w, int64_t rows, int K, uint8_t* codes,
                              uint8_t* scales, hipStream_t s) {
  const int64_t nblocks = rows * (K / kMxBlock);
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(mx_quantize_kernel, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, s,
                     w, nblocks, codes, scales);
  return hipGetLastError();
}

hipError_t launch_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int K,
                                uint16_t* w, hipStream_t s) {
  const int64_t nhalves = rows * (K / 16);
  if (nhalves == 0) return hipSuccess;
  hipLaunchKernelGGL(mx_dequantize_kernel, dim3((unsigned)((nhalves + 255) / 256)), dim3(256), 0,
                     s, codes, scales, nhalves, w);
  return hipGetLastError();
}

}  // namespace moe
