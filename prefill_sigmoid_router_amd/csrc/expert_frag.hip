// Grouped expert GEMMs on prepared weights (the offline weight re-layout of the AlphaMoE
// page, FlashInfer PR #6511 analysis, section 2: the down kernel streams W2 from panels
// prepared once, prepare_*_k256).  Here the panels are laid out in MFMA-fragment order so
// that every weight load of a wave is 1 KiB of contiguous memory -- eight whole 128-byte
// lines -- that lands directly in the A operand of v_mfma_f32_16x16x32_bf16: no LDS staging,
// no barrier between the waves for weights.  Only the token rows, which all 8 waves share,
// go through an LDS ring (whole-line global_load_lds copies, XOR-swizzled, as in the tiled
// kernels).
//
// Prepared layout (bf16, 16-byte groups of 8 values; "frag" = 64 lanes x 16 bytes):
//   W13p [E][I/256][8 waves][H/32 K steps][4 tiles][64 lanes][8 values]
//        wave w, N tile n, tile j: rows n*256 + 32w + 16j + lane%16 of the gate half (j < 2)
//        or I + n*256 + 32w + 16(j-2) + lane%16 of the up half (j >= 2);
//        K values 32 s + 8 (lane / 16) + v of step s.
//   W2p  [E][ceil(H/512)][8][I/32][4][64][8]
//        rows n*512 + 64w + 16j + lane%16 (zero past H), K values as above.
// A wave's whole weight stream for one (expert, N tile) is contiguous: (K/32) x 4 KiB.
//
// MXFP4 weights (OCP MX: E2M1 elements, one E8M0 scale byte per 32 values along K) use the
// same panel order: for wave w, N tile n, K step s (one 32-value block), lane l holds the 8
// values of tile j as 4 code bytes (value 2b in the low nibble of byte b, 2b + 1 in the
// high one), the 4 tiles' bytes together (16 bytes per lane, 1 KiB per step and wave), and
// the step's scale bytes follow as [16 rows][4 tiles] (64 bytes per step and wave):
//   W13q [E][I/256][8][H/32][64 lanes][4 tiles][4 bytes], W13s [E][I/256][8][H/32][16][4]
//   W2q  [E][ceil(H/512)][8][I/32][64][4][4],             W2s  [E][ceil(H/512)][8][I/32][16][4]
// with the rows of the bf16 panels (rows past H: codes and scale bytes 0).  Each step's 4
// weight fragments are dequantized in registers with v_cvt_scalef32_pk_bf16_fp4 (exact).
//
// MXFP8 weights (OCP MX: E4M3 elements, one E8M0 scale byte per 32 values along K, the
// natural format of moe_mx_quantize) re-laid-out into the same order: per (wave, N tile,
// K step) two 1 KiB halves, half h holding tiles 2h and 2h + 1 -- lane l's 16 bytes are the
// 8 codes of tile 2h then the 8 of tile 2h + 1 (value v in byte v) -- and the scale bytes as
// for MXFP4:
//   W13c8 [E][I/256][8][H/32][2 halves][64 lanes][2 tiles][8 bytes], W13s8 as W13s
//   W2c8  [E][ceil(H/512)][8][I/32][2][64][2][8],                   W2s8 as W2s
// dequantized in registers with v_cvt_scalef32_pk_bf16_fp8 (exact).
//
// Item = one token tile (BM = 64 or 128 plan rows of one expert) x one N tile (up: 256 act
// columns = 512 weight rows; down: 512 output columns), 8 wave streams of 64 weight rows;
// a 128-row tile's item runs on an 8-wave workgroup, a 64-row tile's on two 4-wave
// workgroups taking 4 streams each.  Each wave owns 4 weight row tiles (64 rows) x all
// BM/16 token tiles.  Per MFMA K step of 32 values a wave loads its 4 weight fragments
// (4 KiB for bf16) into a register ring of RS steps (the weights of RS - 1 steps in flight
// while one step is computed), and per K chunk of 64 values 2 KiB per 16 token rows, split
// over the workgroup's waves, into an LDS ring of TS stages.
#include <algorithm>

#include "device_common.h"
#include "launchers.h"
#include "tiled_common.h"

namespace moe {

constexpr int kFragWaves = 8;
constexpr int kFragKC = 64;            // K values per chunk (2 MFMA K steps)
constexpr int kFragRS = 4;             // weight register ring, in K steps of 32 values (bf16)
constexpr int kFragRS4 = 6;            // the same for MXFP4 codes (128-row tiles)
constexpr int kFragRS4Small = 16;      // ... and 64-row tiles, whose accumulators leave room
                                       // (decode: 510 -> 472 us per layer against 6 steps)
constexpr int kFragRS8 = 4;            // the same for MXFP8 codes (128-row tiles)
constexpr int kFragRS8Small = 8;       // ... and 64-row tiles
constexpr int kFragTS = 4;             // token LDS ring stages
constexpr int kFragNT = 2;             // cache policy bits of a nontemporal load (gfx950)

// weight formats of the fragment GEMMs
constexpr int kWBf16 = 0;   // bf16 panels (moe_prepare_weights)
constexpr int kWMx8 = 1;    // MXFP8 panels (moe_mx_prepare_weights)
constexpr int kWMx4 = 2;    // MXFP4 panels (moe_mx4_quantize)

int frag_up_columns() { return 256; }

// ---------------------------------------------------------------------------------------
// Preparation: natural row-major [rows, K] stacks -> fragment panels.  One thread per
// 16-byte group of the output; it reads the 16 bytes (8 consecutive K values of one row)
// from the natural layout.  Rows past the weight (W2 with H not a multiple of 512) are 0.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prepare_w13_kernel(const uint16_t* __restrict__ w13,
                                                          int E, int H, int I,
                                                          uint16_t* __restrict__ out) {
  const size_t groups = (size_t)E * 2 * I * H / 8;
  const int steps = H / 32;
  for (size_t g = (size_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups;
       g += (size_t)gridDim.x * blockDim.x) {
    size_t r = g;
    const int lane = (int)(r % 64); r /= 64;
    const int j = (int)(r % 4); r /= 4;
    const int s = (int)(r % steps); r /= steps;
    const int w = (int)(r % kFragWaves); r /= kFragWaves;
    const int n = (int)(r % (I / 256)); r /= (I / 256);
    const int e = (int)r;
    const int col = n * 256 + 32 * w + 16 * (j & 1) + (lane & 15);
    const int row = j < 2 ? col : I + col;
    const int k = 32 * s + 8 * (lane >> 4);
    st16(out + g * 8, ld16(w13 + ((size_t)e * 2 * I + row) * H + k));
  }
}

__global__ __launch_bounds__(256) void prepare_w2_kernel(const uint16_t* __restrict__ w2, int E,
                                                         int H, int I,
                                                         uint16_t* __restrict__ out) {
  const int nt = (H + 511) / 512;
  const size_t groups = (size_t)E * nt * 512 * I / 8;
  const int steps = I / 32;
  for (size_t g = (size_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups;
       g += (size_t)gridDim.x * blockDim.x) {
    size_t r = g;
    const int lane = (int)(r % 64); r /= 64;
    const int j = (int)(r % 4); r /= 4;
    const int s = (int)(r % steps); r /= steps;
    const int w = (int)(r % kFragWaves); r /= kFragWaves;
    const int n = (int)(r % nt); r /= nt;
    const int e = (int)r;
    const int row = n * 512 + 64 * w + 16 * j + (lane & 15);
    const int k = 32 * s + 8 * (lane >> 4);
    const u32x4 v = row < H ? ld16(w2 + ((size_t)e * H + row) * I + k) : u32x4{0, 0, 0, 0};
    st16(out + g * 8, v);
  }
}

size_t frag_w13_elems(int E, int H, int I) { return (size_t)E * 2 * I * H; }
size_t frag_w2_elems(int E, int H, int I) { return (size_t)E * ((H + 511) / 512) * 512 * I; }

hipError_t launch_prepare_weights(const uint16_t* w13, const uint16_t* w2, int E, int H, int I,
                                  uint16_t* w13p, uint16_t* w2p, hipStream_t s) {
  if (H % 64 != 0 || I % 256 != 0) return hipErrorInvalidValue;
  const long g13 = (long)(frag_w13_elems(E, H, I) / 8);
  const long g2 = (long)(frag_w2_elems(E, H, I) / 8);
  const long grid13 = std::min<long>((g13 + 255) / 256, 1L << 20);
  const long grid2 = std::min<long>((g2 + 255) / 256, 1L << 20);
  if (w13 != nullptr) {
    hipLaunchKernelGGL(prepare_w13_kernel, dim3((unsigned)grid13), dim3(256), 0, s, w13, E, H, I,
                       w13p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (w2 != nullptr) {
    hipLaunchKernelGGL(prepare_w2_kernel, dim3((unsigned)grid2), dim3(256), 0, s, w2, E, H, I,
                       w2p);
    return hipGetLastError();
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------------------
// MXFP8 panels from the natural MXFP8 stacks (codes [rows, K], scale bytes [rows, K/32]):
// a byte permutation.  One thread per (expert, N tile, wave, step, lane), as the MXFP4
// quantizer below: the lane's 8 codes of each of the 4 tiles; lanes 0..15 also move the
// scale bytes of row `lane`.
// ---------------------------------------------------------------------------------------
template <bool UP>
__global__ __launch_bounds__(256) void mx8_prepare_panels_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int E, int H, int I,
    uint8_t* __restrict__ pcodes, uint8_t* __restrict__ pscales) {
  const int K = UP ? H : I;
  const int steps = K / 32;
  const int nnt = UP ? I / 256 : (H + 511) / 512;
  const size_t threads = (size_t)E * nnt * kFragWaves * steps * 64;
  for (size_t g = (size_t)blockIdx.x * blockDim.x + threadIdx.x; g < threads;
       g += (size_t)gridDim.x * blockDim.x) {
    size_t r = g;
    const int lane = (int)(r % 64); r /= 64;
    const int st = (int)(r % steps); r /= steps;
    const int wv = (int)(r % kFragWaves); r /= kFragWaves;
    const int n = (int)(r % nnt); r /= nnt;
    const int e = (int)r;
    uint2 word[4];
    uint32_t sbyte[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int row;
      bool on = true;
      if (UP) {
        const int col = n * 256 + 32 * wv + 16 * (j & 1) + (lane & 15);
        row = j < 2 ? col : I + col;
      } else {
        row = n * 512 + 64 * wv + 16 * j + (lane & 15);
        on = row < H;
      }
      word[j] = make_uint2(0u, 0u);
      sbyte[j] = 0u;
      if (!on) continue;
      const size_t grow = (size_t)e * (UP ? 2 * I : H) + row;
      word[j] = *reinterpret_cast<const uint2*>(codes + grow * K + 32 * st + 8 * (lane >> 4));
      sbyte[j] = scales[grow * steps + st];
    }
    const size_t stepi = (((size_t)e * nnt + n) * kFragWaves + wv) * steps + st;
    st16(pcodes + stepi * 2048 + lane * 16, u32x4{word[0].x, word[0].y, word[1].x, word[1].y});
    st16(pcodes + stepi * 2048 + 1024 + lane * 16, u32x4{word[2].x, word[2].y, word[3].x, word[3].y});
    if (lane < 16)
      *reinterpret_cast<uint32_t*>(pscales + stepi * 64 + lane * 4) =
          sbyte[0] | (sbyte[1] << 8) | (sbyte[2] << 16) | (sbyte[3] << 24);
  }
}

size_t mx8_codes_bytes(int E, int H, int I, bool w13) {
  return w13 ? (size_t)E * 2 * I * H : (size_t)E * ((H + 511) / 512) * 512 * I;
}

hipError_t launch_mx8_prepare(const uint8_t* codes, const uint8_t* scales, bool w13, int E, int H,
                              int I, uint8_t* pcodes, uint8_t* pscales, hipStream_t s) {
  if (H % 64 != 0 || I % 256 != 0) return hipErrorInvalidValue;
  const size_t threads = mx8_codes_bytes(E, H, I, w13) / 32;
  const long grid = std::min<long>((long)((threads + 255) / 256), 1L << 20);
  if (w13)
    hipLaunchKernelGGL(mx8_prepare_panels_kernel<true>, dim3((unsigned)grid), dim3(256), 0, s,
                       codes, scales, E, H, I, pcodes, pscales);
  else
    hipLaunchKernelGGL(mx8_prepare_panels_kernel<false>, dim3((unsigned)grid), dim3(256), 0, s,
                       codes, scales, E, H, I, pcodes, pscales);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// MXFP4 panels: quantization (natural bf16 stacks -> panels) and dequantization back
// ---------------------------------------------------------------------------------------
// E2M1 code of x (the weight times 2^-s, |x| < 8 by the choice of s): the nearest of
// 0, 0.5, 1, 1.5, 2, 3, 4, 6, a tie going to the neighbour with mantissa bit 0 -- the
// comparisons below put every midpoint on that side; above 6 the largest.  Zero of either
// sign, and anything that rounds to it, is +0.
__device__ __forceinline__ uint32_t e2m1_code(float x) {
  const float a = fabsf(x);
  const uint32_t c = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                   : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
  return (x < 0.0f && c != 0u) ? (c | 8u) : c;
}

// E8M0 byte of a 32-value block from its largest bf16 magnitude pattern: s = floor(log2
// amax) - 2 = exponent field - 129 for a normal maximum, clamped to [-127, 127] (zero and
// subnormal maxima give -127, byte 0).
__device__ __forceinline__ int mx4_scale_exp(uint32_t amax_bits) {
  const int e = (int)((amax_bits >> 7) & 0xFF);
  const int s = e > 0 ? e - 129 : -127;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// 4 code bytes (8 E2M1 values) and their block's scale byte -> one bf16 MFMA fragment (8
// values, exact: a 4-bit significand times a power of two).
__device__ __forceinline__ u32x4 mx4_dequant8(uint32_t codes, uint32_t scale_byte) {
  const float scale = __uint_as_float(scale_byte ? scale_byte << 23 : 0x00400000u);
#define MOE_CVT4(b) \
  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, b))
  return u32x4{MOE_CVT4(0), MOE_CVT4(1), MOE_CVT4(2), MOE_CVT4(3)};
#undef MOE_CVT4
}

// 8 E4M3 codes (two words, value v in byte v) and their block's scale byte -> one bf16 MFMA
// fragment (exact: a 4-bit significand times a power of two)
__device__ __forceinline__ u32x4 mx8_dequant8(uint32_t c0, uint32_t c1, uint32_t scale_byte) {
  const float scale = __uint_as_float(scale_byte ? scale_byte << 23 : 0x00400000u);
#define MOE_CVT8(w, hi) \
  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, hi))
  return u32x4{MOE_CVT8(c0, false), MOE_CVT8(c0, true), MOE_CVT8(c1, false), MOE_CVT8(c1, true)};
#undef MOE_CVT8
}

// One thread per (expert, N tile, wave, step, lane): for each of the 4 tiles, the row's
// 32-value block of this step (read whole, for its maximum), its scale, and the lane's 8
// values encoded into 4 bytes; lanes 0..15 also write the scale bytes of row `lane`.
// W13 rows (gate / up interleaved per N tile) when UP, else W2 rows (zero past H).
template <bool UP>
__global__ __launch_bounds__(256) void mx4_quantize_panels_kernel(
    const uint16_t* __restrict__ w, int E, int H, int I, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales) {
  const int K = UP ? H : I;
  const int steps = K / 32;
  const int nnt = UP ? I / 256 : (H + 511) / 512;
  const size_t threads = (size_t)E * nnt * kFragWaves * steps * 64;
  for (size_t g = (size_t)blockIdx.x * blockDim.x + threadIdx.x; g < threads;
       g += (size_t)gridDim.x * blockDim.x) {
    size_t r = g;
    const int lane = (int)(r % 64); r /= 64;
    const int st = (int)(r % steps); r /= steps;
    const int wv = (int)(r % kFragWaves); r /= kFragWaves;
    const int n = (int)(r % nnt); r /= nnt;
    const int e = (int)r;
    uint32_t word[4], sbyte[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int row;
      bool on = true;
      if (UP) {
        const int col = n * 256 + 32 * wv + 16 * (j & 1) + (lane & 15);
        row = j < 2 ? col : I + col;
      } else {
        row = n * 512 + 64 * wv + 16 * j + (lane & 15);
        on = row < H;
      }
      word[j] = 0u;
      sbyte[j] = 0u;
      if (!on) continue;
      const uint16_t* blk = w + ((size_t)e * (UP ? 2 * I : H) + row) * K + 32 * st;
      u32x4 v[4];
      uint32_t amax = 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[q] = ld16(blk + 8 * q);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const uint32_t lo = v[q][h] & 0x7FFFu, hi = (v[q][h] >> 16) & 0x7FFFu;
          amax = max(amax, max(lo, hi));
        }
      }
      const int sexp = mx4_scale_exp(amax);
      sbyte[j] = (uint32_t)(sexp + 127);
      const float inv = __uint_as_float((uint32_t)(127 - sexp) << 23);   // 2^-s, exact
      const u32x4 mine = v[lane >> 4];                                     // this lane's 8 values
      uint32_t packed = 0u;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t c0 = e2m1_code(bf16lo(mine[h]) * inv);
        const uint32_t c1 = e2m1_code(bf16hi(mine[h]) * inv);
        packed |= (c0 | (c1 << 4)) << (8 * h);
      }
      word[j] = packed;
    }
    const size_t stepi = (((size_t)e * nnt + n) * kFragWaves + wv) * steps + st;
    st16(codes + stepi * 1024 + lane * 16, u32x4{word[0], word[1], word[2], word[3]});
    if (lane < 16)
      *reinterpret_cast<uint32_t*>(scales + stepi * 64 + lane * 4) =
          sbyte[0] | (sbyte[1] << 8) | (sbyte[2] << 16) | (sbyte[3] << 24);
  }
}

// The inverse: panels -> natural bf16 rows (with the GEMMs' dequantization), same threads.
template <bool UP>
__global__ __launch_bounds__(256) void mx4_dequantize_panels_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int E, int H, int I,
    uint16_t* __restrict__ w) {
  const int K = UP ? H : I;
  const int steps = K / 32;
  const int nnt = UP ? I / 256 : (H + 511) / 512;
  const size_t threads = (size_t)E * nnt * kFragWaves * steps * 64;
  for (size_t g = (size_t)blockIdx.x * blockDim.x + threadIdx.x; g < threads;
       g += (size_t)gridDim.x * blockDim.x) {
    size_t r = g;
    const int lane = (int)(r % 64); r /= 64;
    const int st = (int)(r % steps); r /= steps;
    const int wv = (int)(r % kFragWaves); r /= kFragWaves;
    const int n = (int)(r % nnt); r /= nnt;
    const int e = (int)r;
    const size_t stepi = (((size_t)e * nnt + n) * kFragWaves + wv) * steps + st;
    const u32x4 c = ld16(codes + stepi * 1024 + lane * 16);
    const uint32_t sc = *reinterpret_cast<const uint32_t*>(scales + stepi * 64 + (lane & 15) * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int row;
      if (UP) {
        const int col = n * 256 + 32 * wv + 16 * (j & 1) + (lane & 15);
        row = j < 2 ? col : I + col;
      } else {
        row = n * 512 + 64 * wv + 16 * j + (lane & 15);
        if (row >= H) continue;
      }
      st16(w + ((size_t)e * (UP ? 2 * I : H) + row) * K + 32 * st + 8 * (lane >> 4),
           mx4_dequant8(c[j], (sc >> (8 * j)) & 0xFFu));
    }
  }
}

size_t mx4_codes_bytes(int E, int H, int I, bool w13) {
  return w13 ? (size_t)E * 2 * I * H / 2 : (size_t)E * ((H + 511) / 512) * 512 * I / 2;
}
size_t mx4_scales_bytes(int E, int H, int I, bool w13) {
  return w13 ? (size_t)E * 2 * I * H / 32 : (size_t)E * ((H + 511) / 512) * 512 * I / 32;
}

hipError_t launch_mx4_quantize(const uint16_t* w, bool w13, int E, int H, int I, uint8_t* codes,
                               uint8_t* scales, hipStream_t s) {
  if (H % 64 != 0 || I % 256 != 0) return hipErrorInvalidValue;
  const size_t threads = mx4_codes_bytes(E, H, I, w13) / 16;
  const long grid = std::min<long>((long)((threads + 255) / 256), 1L << 20);
  if (w13)
    hipLaunchKernelGGL(mx4_quantize_panels_kernel<true>, dim3((unsigned)grid), dim3(256), 0, s, w,
                       E, H, I, codes, scales);
  else
    hipLaunchKernelGGL(mx4_quantize_panels_kernel<false>, dim3((unsigned)grid), dim3(256), 0, s, w,
                       E, H, I, codes, scales);
  return hipGetLastError();
}

hipError_t launch_mx4_dequantize(const uint8_t* codes, const uint8_t* scales, bool w13, int E,
                                 int H, int I, uint16_t* w, hipStream_t s) {
  if (H % 64 != 0 || I % 256 != 0) return hipErrorInvalidValue;
  const size_t threads = mx4_codes_bytes(E, H, I, w13) / 16;
  const long grid = std::min<long>((long)((threads + 255) / 256), 1L << 20);
  if (w13)
    hipLaunchKernelGGL(mx4_dequantize_panels_kernel<true>, dim3((unsigned)grid), dim3(256), 0, s,
                       codes, scales, E, H, I, w);
  else
    hipLaunchKernelGGL(mx4_dequantize_panels_kernel<false>, dim3((unsigned)grid), dim3(256), 0, s,
                       codes, scales, E, H, I, w);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// The GEMM
// ---------------------------------------------------------------------------------------
template <int BM>
struct FragCfg {
  static constexpr int MT = BM / 16;                  // token row tiles
  static constexpr int TSTAGE = MT * 2048;            // bytes of one token chunk
  static constexpr int TCOPIES = MT * 2;              // 1 KiB copies per token chunk
};

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left open) through the builtin, which the
// compiler's own wait insertion takes into account -- it then adds no wait of its own for
// the loads this one already covers.  gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt[5:4] << 14.
template <int N>
__device__ __forceinline__ void frag_wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Buffer resource over one wave's weight stream (`bytes` long, 4-byte aligned base): raw,
// untyped 32-bit data.  Every load the GEMMs issue through it stays inside `bytes` (steps
// past the last one are clamped to it).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// One work item: plan rows start..start+nlive-1 of expert e (their flat indices row_ids[r])
// against N tile `ntile` of the prepared weights, computing the first NA token tiles (at
// least the tiles holding real rows: the inner loop then has no branch, which keeps the
// compiler's own load waits exact).  The ring is a __restrict__ parameter so that the
// compiler can tell the token copies in flight apart from the LDS reads (without it, it
// drains every load before each fragment read).
template <int BM, bool UP, int WPOL, int NA, int WF, int NWG>
__device__ __forceinline__ void frag_item(
    unsigned char* __restrict__ tlds, const uint16_t* __restrict__ tok_src,
    const void* __restrict__ wp, const uint8_t* __restrict__ wsc,
    const int32_t* __restrict__ row_ids, int start, int nlive, int e, int ntile, int part,
    int n_ntiles, int K, int ncols, int I, int top_k, uint16_t* __restrict__ act,
    uint16_t* __restrict__ y, float* __restrict__ y0) {
  using C = FragCfg<BM>;
  constexpr int MT = C::MT;
  constexpr int TS = kFragTS;
  // weight ring depth in K steps and loads per step: bf16 4 fragments (16 VGPRs a step);
  // MXFP8 two 16-byte loads of codes and one 4-byte load of scale bytes (9 VGPRs a step);
  // MXFP4 one 16-byte load of codes and one of scale bytes (5 VGPRs a step)
  constexpr int RS = WF == kWMx4   ? (BM == 64 ? kFragRS4Small : kFragRS4)
                     : WF == kWMx8 ? (BM == 64 ? kFragRS8Small : kFragRS8)
                                   : kFragRS;
  constexpr int WPS = WF == kWMx4 ? 2 : WF == kWMx8 ? 3 : 4;
  constexpr int WREGS = WF == kWMx4 ? 1 : WF == kWMx8 ? 2 : 4;   // 16-byte loads of codes
  constexpr int SB = 1024 * WREGS;                                 // bytes per step and wave
  // token copies: copy f (0 .. TCOPIES-1) of a chunk covers rows 8h..8h+7 (h = f % 2) of
  // token tile f / 2; wave w of the NWG issues copies w, w + NWG, ...
  constexpr int TCPW = C::TCOPIES / NWG;
  static_assert(TCPW * NWG == C::TCOPIES, "token copies must split evenly over the waves");
  // Every chunk issues the token copies of chunk c + TS - 1, then the weights of steps
  // 2c + RS and 2c + 1 + RS (WPS loads each) -- always, with the chunk and step clamped to
  // the last one, so the count of this wave's loads issued after the token copies of chunk c
  // is fixed: 2 WPS + (TS - 2) (TCPW + 2 WPS) in the steady state, at least
  // (TS - 2) TCPW + WPS RS after the prologue (token copies of chunks 0..TS-2, then the
  // weights of steps 0..RS-1).
  constexpr int kAfterT = 2 * WPS + (TS - 2) * (TCPW + 2 * WPS);
  constexpr int kAfterT0 = (TS - 2) * TCPW + RS * WPS;
  constexpr int kWaitT = kAfterT < kAfterT0 ? kAfterT : kAfterT0;
  static_assert(kWaitT <= 63, "vmcnt range");
  // The weights of step st were issued at the end of step st - RS (or in the prologue);
  // after them this wave issued at least the weights of RS - 1 more steps and the token
  // copies of one chunk start, so they have landed once at most that many loads are
  // outstanding.
  constexpr int kWaitW = WPS * (RS - 1) + TCPW;

  // the wave index as a scalar: the weight stream's base is the same for the whole wave;
  // a workgroup of NWG < 8 waves takes part `part` of the panel's 8 wave streams
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pw = part * NWG + wave;
  const int lane = threadIdx.x & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int nch = K / kFragKC;
  const int nsteps = K / 32;

  // this wave's weight stream (nsteps x 4 KiB, contiguous): fragment (step s, tile j) at byte
  // s * 4096 + j * 1024, lane l's 16 bytes at + 16 l; loaded through a buffer resource (the
  // step offset in a scalar register, one vector register for all lanes' offsets)
  // (MXFP8 / MXFP4: codes nsteps x 2 / 1 KiB, scale bytes nsteps x 64 B, lane l's scale
  // word -- row l % 16 of the 4 tiles -- at 4 (l % 16))
  const size_t stream = ((size_t)e * n_ntiles + ntile) * kFragWaves + pw;
  const __amdgpu_buffer_rsrc_t wrsrc =
      stream_rsrc(static_cast<const uint8_t*>(wp) + stream * nsteps * SB, nsteps * SB);
  const __amdgpu_buffer_rsrc_t srsrc = stream_rsrc(
      WF != kWBf16 ? wsc + stream * nsteps * 64 : static_cast<const uint8_t*>(wp), nsteps * 64);
  const int lane_off = lane * 16;
  const int scale_off = (lane & 15) * 4;
  // token copies of this wave; rows past the tile's real rows read its first row
  const uint16_t* tsrc[TCPW];
#pragma unroll
  for (int i = 0; i < TCPW; ++i) {
    const int f = wave + NWG * i;
    const int rt = f >> 1, h = f & 1;
    const int r = 16 * rt + 8 * h + (lane >> 3);
    const int koff = 8 * ((lane & 7) ^ (lane >> 3) ^ h);
    const bool on = r < nlive;
    if (UP) {
      const int sid = row_ids[on ? r : 0];
      tsrc[i] = tok_src + (size_t)(sid < 0 ? 0 : sid / top_k) * K + koff;
    } else {
      tsrc[i] = tok_src + (size_t)(start + (on ? r : 0)) * K + koff;
    }
  }
  auto issue_t = [&](int c) {  // into stage c % TS; c is clamped to the last chunk
    const int cc = c < nch ? c : nch - 1;
    unsigned char* base = tlds + (size_t)(c % TS) * C::TSTAGE;
#pragma unroll
    for (int i = 0; i < TCPW; ++i)
      __builtin_amdgcn_global_load_lds((global_void*)(tsrc[i] + cc * kFragKC),
                                       (lds_void*)(base + (wave + NWG * i) * 1024), 16, 0, 0);
  };
  const int frag_off = (li >> 3) * 1024 + (li & 7) * 128;
  auto tfrag = [&](int c, int t, int ks) -> u32x4 {
    const int q = (lg + 4 * ks) ^ (li & 7) ^ (li >> 3);
    return *reinterpret_cast<const u32x4*>(tlds + (size_t)(c % TS) * C::TSTAGE + t * 2048 +
                                           frag_off + q * 16);
  };
  // bf16: wr[slot][j] is fragment j; MXFP8: wr[slot][h] holds the code words of tiles 2h
  // and 2h + 1; MXFP4: wr[slot][0] holds the 4 tiles' code words; wsr[slot] the scale bytes
  u32x4 wr[RS][WREGS];
  uint32_t wsr[WF != kWBf16 ? RS : 1];
  auto issue_w = [&](int st, int slot) {  // st is clamped to the last step
    const int ss = st < nsteps ? st : nsteps - 1;
#pragma unroll
    for (int j = 0; j < WREGS; ++j)
      wr[slot][j] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrsrc, lane_off, ss * SB + j * 1024, WPOL));
    if constexpr (WF != kWBf16)
      wsr[slot] = __builtin_amdgcn_raw_buffer_load_b32(srsrc, scale_off, ss * 64, WPOL);
  };

  static_assert(NA >= 1 && NA <= MT, "computed token tiles");
  f32x4 acc[4][NA];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int s = 0; s < NA; ++s) acc[j][s] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int p = 0; p < TS - 1; ++p) issue_t(p);
#pragma unroll
  for (int u = 0; u < RS; ++u) issue_w(u, u);

  // step st (ring slot u % RS, u compile-time after unrolling): on a chunk's first step wait
  // for its token copies, publish them and start the copies TS - 1 chunks ahead; NA token
  // tiles x 4 weight tiles of MFMAs; the weights RS steps ahead into the freed slot
  auto step = [&](int st, int u) {
    const int c = st >> 1, ks = u & 1;
    if (ks == 0) {
      // this wave's token copies of chunk c have landed ...
      frag_wait_vmcnt<kWaitT>();
      // ... for every wave, and chunk c - 1 is consumed: stage (c + TS - 1) % TS is free
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      issue_t(c + TS - 1);
    }
    frag_wait_vmcnt<kWaitW>();   // this step's weights are in registers
    // keep the dequantization of this step's codes below the wait: the empty asm takes the
    // registers as inputs and outputs, so nothing computed from them moves above it (the
    // compiler would otherwise hoist the scale arithmetic of later steps and drain every
    // load to feed it)
    if constexpr (WF == kWMx4) asm volatile("" : "+v"(wr[u % RS][0]), "+v"(wsr[u % RS]));
    if constexpr (WF == kWMx8)
      asm volatile("" : "+v"(wr[u % RS][0]), "+v"(wr[u % RS][1]), "+v"(wsr[u % RS]));
    u32x4 wa[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (WF == kWMx4) {
        wa[j] = mx4_dequant8(wr[u % RS][0][j], (wsr[u % RS] >> (8 * j)) & 0xFFu);
      } else if constexpr (WF == kWMx8) {
        const u32x4 h = wr[u % RS][j >> 1];
        wa[j] = mx8_dequant8(h[2 * (j & 1)], h[2 * (j & 1) + 1], (wsr[u % RS] >> (8 * j)) & 0xFFu);
      } else {
        wa[j] = wr[u % RS][j];
      }
    }
    issue_w(st + RS, u % RS);
#pragma unroll
    for (int s = 0; s < NA; ++s) {
      const u32x4 xb = tfrag(c, s, ks);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j][s] = mfma16x16x32(wa[j], xb, acc[j][s]);
    }
  };
  // whole groups of 2 RS steps (whole chunks) without a branch, then the rest
  int s0 = 0;
  for (; s0 + 2 * RS <= nsteps; s0 += 2 * RS) {
#pragma unroll
    for (int u = 0; u < 2 * RS; ++u) step(s0 + u, u);
  }
#pragma unroll
  for (int u = 0; u < 2 * RS; ++u)
    if (s0 + u < nsteps) step(s0 + u, u);
  // the clamped loads past the last step are discarded: let them land before the registers
  // and the ring are reused
  frag_wait_vmcnt<0>();

  // epilogue (as in the tiled kernels): act rows in bf16 for the up GEMM, y rows for the
  // down GEMM (bf16, a token's first pick fp32: store_y4), real rows only
#pragma unroll
  for (int s = 0; s < NA; ++s) {
    const int r = 16 * s + li;
    if (r >= nlive) continue;
    if (UP) {
      const int col0 = ntile * 256 + 32 * pw;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int n = col0 + 16 * h + 4 * lg;
        float a[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) a[q] = silu_f32(acc[h][s][q]) * acc[2 + h][s][q];
        uint2 v;
        v.x = pack_bf16x2(a[0], a[1]);
        v.y = pack_bf16x2(a[2], a[3]);
        *reinterpret_cast<uint2*>(act + (size_t)(start + r) * I + n) = v;
      }
    } else {
      const YRow yr = y_row(row_ids[r], top_k, ncols);
      const int col0 = ntile * 512 + 64 * pw;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = col0 + 16 * j + 4 * lg;
        if (n < ncols)
          store_y4(y, y0, yr, n, acc[j][s][0], acc[j][s][1], acc[j][s][2], acc[j][s][3]);
      }
    }
  }
}

// Work items (tile, N tile) in expert-major order: the tiles of one expert for its first N
// tile, then for the next, and so on, expert after expert; each XCD takes an equal
// contiguous share, so the ~32 items it runs at a time are a few N tiles of one expert
// (its tiles share each weight line through the XCD's L2) or all N tiles of the one tile of
// a cold expert (which share its token rows).  Items of expert e occupy the logical range
// [first tile x n_ntiles, (first tile + tiles) x n_ntiles), so item L belongs to the expert
// of tile L / n_ntiles.
struct ExpertMajorWalk {
  TiledWalk w;
  const int2* groups;
  int n_ntiles;
  int expert_tiles = 0;   // token tiles of the expert of the last item
  __device__ ExpertMajorWalk(int ntl, int nnt, const int2* g) : w(ntl, nnt), groups(g), n_ntiles(nnt) {}
  __device__ bool next(int& ntile, int& ti) {
    int a, b;
    if (!w.next(a, b)) return false;
    const int logical = a * w.ntiles_live + b;
    const int2 g = groups[logical / n_ntiles];
    const int local = logical - g.x * n_ntiles;
    ntile = local / g.y;
    ti = g.x + local % g.y;
    expert_tiles = g.y;
    return true;
  }
};

template <int BM, bool UP, int WPOL, int WF, int NWG>
__global__ __launch_bounds__(64 * NWG) void expert_frag_kernel(
    const uint16_t* __restrict__ tok_src, const void* __restrict__ wp,
    const uint8_t* __restrict__ wsc,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ block_expert,
    const int2* __restrict__ tiles, const int2* __restrict__ tile_groups,
    const int32_t* __restrict__ num_tiles, int n_ntiles, int K, int ncols, int I, int top_k,
    int block, uint16_t* __restrict__ act, uint16_t* __restrict__ y, float* __restrict__ y0) {
  __shared__ __align__(16) unsigned char tlds[kFragTS * FragCfg<BM>::TSTAGE];
  // items: (tile, N tile of the panels, part); a workgroup of NWG waves does 8 / NWG parts
  // of an N tile, the parts counted as N tiles of their own in the walk
  constexpr int PARTS = kFragWaves / NWG;
  ExpertMajorWalk walk(*num_tiles, n_ntiles * PARTS, tile_groups);
  int nt_part, ti;
  while (walk.next(nt_part, ti)) {
    const int ntile = nt_part / PARTS, part = nt_part % PARTS;
    const int2 tile = tiles[ti];
    // token tiles computed: all of them, or the first quarter (64-row tiles) / half
    // (128-row tiles) when that holds every real row (padding rows hold copies of the first
    // row); each choice is its own branch-free loop, which keeps the compiler's own load
    // waits exact
    constexpr int MT = FragCfg<BM>::MT;
    constexpr int NS = BM == 64 ? 1 : MT / 2;
    // In the up GEMM of a launch that keeps weights cached (several tiles share the hot
    // experts' weights), the weights of an expert with a single token tile are copied
    // nontemporally: they are read by that one item per N tile, and cached they would evict
    // the lines the hot experts' tiles share (M=2048, bf16 panels: up 3,021 -> 2,832 us,
    // layer 5,156 -> 5,017 us; nontemporal for every tile costs 3 %).  Only the up GEMM (the
    // down GEMM's added instantiations spill) and 128-row tiles (with 64-row MXFP4 tiles the
    // added copies leave one wave per SIMD).
    if (UP && WPOL == 0 && BM == 128 && walk.expert_tiles == 1) {
      if (tile.y <= 16 * NS)
        frag_item<BM, UP, kFragNT, NS, WF, NWG>(tlds, tok_src, wp, wsc, sorted_ids + tile.x,
                                                tile.x, tile.y, block_expert[tile.x / block],
                                                ntile, part, n_ntiles, K, ncols, I, top_k, act,
                                                y, y0);
      else
        frag_item<BM, UP, kFragNT, MT, WF, NWG>(tlds, tok_src, wp, wsc, sorted_ids + tile.x,
                                                tile.x, tile.y, block_expert[tile.x / block],
                                                ntile, part, n_ntiles, K, ncols, I, top_k, act,
                                                y, y0);
    } else if (tile.y <= 16 * NS) {
      frag_item<BM, UP, WPOL, NS, WF, NWG>(tlds, tok_src, wp, wsc, sorted_ids + tile.x, tile.x,
                                            tile.y, block_expert[tile.x / block], ntile, part,
                                            n_ntiles, K, ncols, I, top_k, act, y, y0);
    } else {
      frag_item<BM, UP, WPOL, MT, WF, NWG>(tlds, tok_src, wp, wsc, sorted_ids + tile.x, tile.x,
                                            tile.y, block_expert[tile.x / block], ntile, part,
                                            n_ntiles, K, ncols, I, top_k, act, y, y0);
    }
    __syncthreads();  // the next item's first token copies reuse the ring
  }
}

template <int BM, bool UP, int WPOL, int WF = kWBf16>
static hipError_t launch_frag(const uint16_t* src, const void* wp, const uint8_t* wsc,
                              const int32_t* sorted_ids,
                              const int32_t* block_expert, const int2* tiles,
                              const int2* tile_groups, const int32_t* num_tiles, int max_tiles,
                              int K, int ncols, int I, int top_k, int block, uint16_t* act,
                              uint16_t* y, float* y0, hipStream_t s) {
  const int per_ntile = UP ? 256 : 512;
  if (K % kFragKC != 0 || (UP && I % per_ntile != 0)) return hipErrorInvalidValue;
  const int n_ntiles = (ncols + per_ntile - 1) / per_ntile;
  // 64-row tiles (few tokens per expert): workgroups of 4 waves, each item half a panel N
  // tile, two workgroups per CU walking their XCD's share (twice the items of 8-wave
  // workgroups: a CU's last item is a smaller share of its work); 128-row tiles: 8 waves,
  // one item per workgroup
  constexpr int NWG = BM == 64 ? 4 : 8;
  const long items = (long)max_tiles * n_ntiles * (kFragWaves / NWG);
  const long grid = BM == 64 ? walk_grid(items, 80 * 1024) : (items + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL((expert_frag_kernel<BM, UP, WPOL, WF, NWG>), dim3((unsigned)grid),
                     dim3(64 * NWG), 0, s, src, wp, wsc, sorted_ids, block_expert, tiles,
                     tile_groups, num_tiles, n_ntiles, K, ncols, I, top_k, block, act, y, y0);
  return hipGetLastError();
}


hipError_t launch_expert_up_frag(const uint16_t* x, const uint16_t* w13p, const int32_t* sorted_ids,
                                 const int32_t* block_expert, const int2* tiles,
                                 const int2* tile_groups, const int32_t* num_tiles, int max_tiles,
                                 int tile_rows, bool stream_weights, int H, int I, int top_k,
                                 int block, uint16_t* act, hipStream_t s) {
#define MOE_FRAG_UP(BM, POL)                                                                    \
  return launch_frag<BM, true, POL>(x, w13p, nullptr, sorted_ids, block_expert, tiles,        \
                                    tile_groups,                                              \
                                    num_tiles, max_tiles, H, I, I, top_k, block, act, nullptr, \
                                    nullptr, s)
  if (tile_rows == 64) {
    if (stream_weights) MOE_FRAG_UP(64, kFragNT);
    MOE_FRAG_UP(64, 0);
  }
  if (tile_rows == 128) {
    if (stream_weights) MOE_FRAG_UP(128, kFragNT);
    MOE_FRAG_UP(128, 0);
  }
#undef MOE_FRAG_UP
  return hipErrorInvalidValue;
}

hipError_t launch_expert_down_frag(const uint16_t* act, const uint16_t* w2p,
                                   const int32_t* sorted_ids, const int32_t* block_expert,
                                   const int2* tiles, const int2* tile_groups,
                                   const int32_t* num_tiles, int max_tiles, int tile_rows,
                                   bool stream_weights, int H, int I, int top_k, int block,
                                   uint16_t* y, float* y0, hipStream_t s) {
#define MOE_FRAG_DOWN(BM, POL)                                                                  \
  return launch_frag<BM, false, POL>(act, w2p, nullptr, sorted_ids, block_expert, tiles,       \
                                     tile_groups, num_tiles, max_tiles, I, H, I, top_k, block, \
                                     nullptr, y, y0, s)
  if (tile_rows == 64) {
    if (stream_weights) MOE_FRAG_DOWN(64, kFragNT);
    MOE_FRAG_DOWN(64, 0);
  }
  if (tile_rows == 128) {
    if (stream_weights) MOE_FRAG_DOWN(128, kFragNT);
    MOE_FRAG_DOWN(128, 0);
  }
#undef MOE_FRAG_DOWN
  return hipErrorInvalidValue;
}

hipError_t launch_expert_up_frag_mx(const uint16_t* x, const uint8_t* w13c, const uint8_t* w13s,
                                   bool fp4, const int32_t* sorted_ids,
                                   const int32_t* block_expert, const int2* tiles,
                                   const int2* tile_groups, const int32_t* num_tiles,
                                   int max_tiles, int tile_rows, bool stream_weights, int H, int I,
                                   int top_k, int block, uint16_t* act, hipStream_t s) {
#define MOE_FRAGMX_UP(BM, POL, WF)                                                              \
  return launch_frag<BM, true, POL, WF>(x, w13c, w13s, sorted_ids, block_expert, tiles,         \
                                        tile_groups, num_tiles, max_tiles, H, I, I, top_k,      \
                                        block, act, nullptr, nullptr, s)
#define MOE_FRAGMX_UP_FMT(WF)                   \
  if (tile_rows == 64) {                        \
    if (stream_weights) MOE_FRAGMX_UP(64, kFragNT, WF); \
    MOE_FRAGMX_UP(64, 0, WF);                   \
  }                                             \
  if (tile_rows == 128) {                       \
    if (stream_weights) MOE_FRAGMX_UP(128, kFragNT, WF); \
    MOE_FRAGMX_UP(128, 0, WF);                  \
  }
  if (fp4) {
    MOE_FRAGMX_UP_FMT(kWMx4)
  } else {
    MOE_FRAGMX_UP_FMT(kWMx8)
  }
#undef MOE_FRAGMX_UP_FMT
#undef MOE_FRAGMX_UP
  return hipErrorInvalidValue;
}

hipError_t launch_expert_down_frag_mx(const uint16_t* act, const uint8_t* w2c, const uint8_t* w2s,
                                     bool fp4, const int32_t* sorted_ids,
                                     const int32_t* block_expert, const int2* tiles,
                                     const int2* tile_groups, const int32_t* num_tiles,
                                     int max_tiles, int tile_rows, bool stream_weights, int H,
                                     int I, int top_k, int block, uint16_t* y, float* y0,
                                     hipStream_t s) {
#define MOE_FRAGMX_DOWN(BM, POL, WF)                                                            \
  return launch_frag<BM, false, POL, WF>(act, w2c, w2s, sorted_ids, block_expert, tiles,        \
                                         tile_groups, num_tiles, max_tiles, I, H, I, top_k,     \
                                         block, nullptr, y, y0, s)
#define MOE_FRAGMX_DOWN_FMT(WF)                 \
  if (tile_rows == 64) {                        \
    if (stream_weights) MOE_FRAGMX_DOWN(64, kFragNT, WF); \
    MOE_FRAGMX_DOWN(64, 0, WF);                 \
  }                                             \
  if (tile_rows == 128) {                       \
    if (stream_weights) MOE_FRAGMX_DOWN(128, kFragNT, WF); \
    MOE_FRAGMX_DOWN(128, 0, WF);                \
  }
  if (fp4) {
    MOE_FRAGMX_DOWN_FMT(kWMx4)
  } else {
    MOE_FRAGMX_DOWN_FMT(kWMx8)
  }
#undef MOE_FRAGMX_DOWN_FMT
#undef MOE_FRAGMX_DOWN
  return hipErrorInvalidValue;
}

}  // namespace moe
