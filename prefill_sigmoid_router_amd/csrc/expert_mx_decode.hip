// Grouped expert GEMMs on MXFP8 weights (E4M3 codes, one E8M0 scale byte per 32 values
// along K) with the codes copied into LDS whole lines at a time and dequantized from there
// straight into the MFMA operands.  moe_forward_mx runs them for every MXFP8 GEMM but the up
// GEMM from 64 tokens per expert.
//
// AlphaMoE page (FlashInfer PR #6511 analysis), sections 1-4: the up kernel gathers the
// token tile of an expert and streams that expert's weights, the down kernel streams W2;
// its weights are block-scaled low-precision codes.  Trainium2 megakernel page, first
// paragraph, rules 1-2: keep the working set on chip, split each weight stream over many
// programs so that small-batch decode runs at memory bandwidth.
//
// Workgroup: 8 waves, 256 weight rows (up: the gate and up rows of 128 act columns; down:
// 256 output columns; each wave 2 row tiles of 16) x a BM-row token tile of one expert (32,
// 64 or 128 rows).  K runs in chunks of 128 values: one 128-byte line of codes per weight
// row (32 KiB) and 256 bytes of bf16 token row per token row (BM/4 KiB), both copied
// global -> LDS with global_load_lds_dwordx4 into a 3-stage ring (two chunks in flight; 2
// stages for 128-row tiles), the codes nontemporally when each expert's weights are read by
// about one token tile.  The scale bytes of 8 chunks (32 per row, 8 KiB per workgroup)
// arrive with 4-byte copies into a 2-stage ring, issued six chunks before their first use:
// scale requests are an eighth of the code requests.  A wave reads 8 codes per lane
// (ds_read_b64) for each MFMA fragment and converts them with the block's scale
// (v_cvt_scalef32_pk_bf16_fp8, exact in bf16) straight into the A operand of
// v_mfma_f32_16x16x32_bf16; token fragments are ds_read_b128.  The 16-byte slots of a row
// are XOR-swizzled by the row's index so both fragment reads are free of bank conflicts.
// One workgroup per CU walks its XCD's share of the (tile, N tile) items.
#include "device_common.h"
#include "launchers.h"
#include "tiled_common.h"

namespace moe {

namespace {

constexpr int kNT = 2;                                // cache policy bits of a nontemporal load
constexpr int kKC = 128;                              // K values (code bytes) per chunk
constexpr int kRows = 256;                            // weight rows per workgroup
constexpr int kWaves = 8;                             // 2 per SIMD (4: decode up 506 -> 486 us)
constexpr int kTW = 16 / kWaves;                      // row tiles per wave
constexpr int kGroup = 8;                             // chunks per scale stage
constexpr int kCodeStage = kRows * kKC;               // 32 KiB
constexpr int kScaleStage = kRows * kGroup * 4;       // 32 scale bytes per row
constexpr int kCodeCopies = kCodeStage / 1024 / kWaves;    // 1 KiB copies per wave per chunk
constexpr int kScaleCopies = kScaleStage / 256 / kWaves;   // 256-byte copies per wave per group
static_assert(kCodeCopies * kWaves * 1024 == kCodeStage && kScaleCopies * kWaves * 256 == kScaleStage,
              "copies must split evenly over the waves");

// Ring of a BM-row token tile: 3 stages (two chunks in flight) when they fit the LDS next to
// the scale ring, else 2.
template <int BM>
struct MxdCfg {
  static constexpr int MT = BM / 16;                  // token row tiles
  static constexpr int TOK_STAGE = BM * kKC * 2;      // bf16 token rows of a chunk
  static constexpr int STAGE = kCodeStage + TOK_STAGE;
  static constexpr int S = 3 * STAGE + 2 * kScaleStage <= 160 * 1024 ? 3 : 2;
  static constexpr int LDS = S * STAGE + 2 * kScaleStage;
  static constexpr int TOK_COPIES = TOK_STAGE / 1024 / kWaves;
  static constexpr int PER_CHUNK = kCodeCopies + TOK_COPIES;
  static_assert(TOK_COPIES * kWaves * 1024 == TOK_STAGE, "token copies must split evenly");
  static_assert((S - 1) * PER_CHUNK + kScaleCopies <= 63, "the copies in flight must fit vmcnt");
  static_assert(LDS <= 160 * 1024, "the rings must fit the LDS");
};

// 8 codes (K values k..k+7 of one row, all in one 32-value scale block) and the block's
// scale byte -> one bf16 MFMA fragment; code * 2^(byte - 127) is exact in bf16.
__device__ __forceinline__ u32x4 dequant8(uint2 codes, uint32_t scale_byte) {
  const float scale = __uint_as_float(scale_byte ? scale_byte << 23 : 0x00400000u);
  return u32x4{
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.x, scale, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.x, scale, true)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.y, scale, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.y, scale, true))};
}

// One work item (token tile ti x N tile ntile) through the rings `ring` (kStages stages of
// codes + token rows) and `sring` (2 stages of scale bytes).  The rings come in as
// __restrict__ pointers, as in the bf16 tiled GEMMs: the compiler then leaves the ordering
// of the global -> LDS copies and the LDS reads to the explicit waits and barriers below
// (otherwise it drains every copy in flight before each chunk's first LDS read).
// This wave's kTW of the 16 row tiles: up -> gate tiles w kTW/2 .. and the up tiles 8 later
// (act columns 16 w kTW/2 .. of the N tile); down -> tiles w kTW ...
template <int BM, int WPOL, bool UP>
__device__ __forceinline__ void mx_decode_item(
    unsigned char* __restrict__ ring, unsigned char* __restrict__ sring, int ntile, int ti,
    const uint16_t* __restrict__ tok_src, const uint8_t* __restrict__ wc,
    const uint8_t* __restrict__ ws, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int2* __restrict__ tiles, int K, int ncols,
    int I, int top_k, int block, uint16_t* __restrict__ act, uint16_t* __restrict__ y,
    float* __restrict__ y0) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int nch = K / kKC;
  const int ngroups = (nch + kGroup - 1) / kGroup;
  const int srow = K / 32;
  const int rows_e = UP ? 2 * I : ncols;
  int wtile[kTW];
#pragma unroll
  for (int j = 0; j < kTW; ++j)
    wtile[j] = UP ? ((j < kTW / 2) ? kTW / 2 * wave + j : 8 + kTW / 2 * wave + (j - kTW / 2))
                  : kTW * wave + j;
  // weight row, within the expert, of workgroup row R of N tile nt
  auto wrow = [&](int nt, int R) -> int {
    const int t = R >> 4, rr = R & 15;
    if (UP) return t < 8 ? nt * 128 + 16 * t + rr : I + nt * 128 + 16 * (t - 8) + rr;
    const int row = nt * kRows + R;
    return row < ncols ? row : 0;                       // rows past H: read, never stored
  };

  const int2 tile = tiles[ti];
  using C = MxdCfg<BM>;
  const int start = tile.x, nlive = tile.y;           // nlive <= BM
  const size_t ebase = (size_t)block_expert[start / block] * rows_e;

  // code copy f = kCodeCopies * wave + i: rows 8f .. 8f+7, lane l row 8f + l/8; its 16
  // bytes land in slot l % 8 of the row's line and hold code bytes 16 q of the chunk,
  // q = (l % 8) ^ (row % 8) ^ (row % 16) / 8
  const uint8_t* csrc[kCodeCopies];
#pragma unroll
  for (int i = 0; i < kCodeCopies; ++i) {
    const int R = 8 * (kCodeCopies * wave + i) + (lane >> 3);
    const int q = (lane & 7) ^ (R & 7) ^ ((R >> 3) & 1);
    csrc[i] = wc + (ebase + wrow(ntile, R)) * K + 16 * q;
  }
  // token copy f = TOK_COPIES * wave + i: token rows 4f .. 4f+3, lane l row r = 4f + l/16,
  // slot l % 16 holding K values 8 (l % 16 ^ r % 16) of the chunk; rows past the tile's
  // real rows read its first row (never stored)
  const uint16_t* tsrc[C::TOK_COPIES];
#pragma unroll
  for (int i = 0; i < C::TOK_COPIES; ++i) {
    const int r = 4 * (C::TOK_COPIES * wave + i) + (lane >> 4);
    const int koff = 8 * ((lane & 15) ^ (r & 15));
    const bool on = r < nlive;
    size_t trow;
    if (UP) {
      const int sid = sorted_ids[start + (on ? r : 0)];
      trow = (size_t)(sid < 0 ? 0 : sid / top_k);
    } else {
      trow = (size_t)start + (on ? r : 0);
    }
    tsrc[i] = tok_src + trow * K + koff;
  }
  // scale copy f = kScaleCopies * wave + i: rows 8f .. 8f+7, lane l row 8f + l/8, bytes
  // 4 (l % 8) of the group's 32; pieces past the row's last scale byte read its first
  const uint8_t* ssrc[kScaleCopies];
#pragma unroll
  for (int i = 0; i < kScaleCopies; ++i) {
    const int R = 8 * (kScaleCopies * wave + i) + (lane >> 3);
    ssrc[i] = ws + (ebase + wrow(ntile, R)) * srow;
  }
  const int spiece = 4 * (lane & 7);

  auto issue_chunk = [&](int c) {
    unsigned char* base = ring + (c % C::S) * C::STAGE;
#pragma unroll
    for (int i = 0; i < kCodeCopies; ++i)
      __builtin_amdgcn_global_load_lds((global_void*)(csrc[i] + c * kKC),
                                       (lds_void*)(base + (kCodeCopies * wave + i) * 1024), 16, 0,
                                       WPOL);
#pragma unroll
    for (int i = 0; i < C::TOK_COPIES; ++i)
      __builtin_amdgcn_global_load_lds(
          (global_void*)(tsrc[i] + c * kKC),
          (lds_void*)(base + kCodeStage + (C::TOK_COPIES * wave + i) * 1024), 16, 0, 0);
  };
  auto issue_scales = [&](int g) {
    unsigned char* base = sring + (g & 1) * kScaleStage;
    const int b = g * 32 + spiece;
    const int off = b + 4 <= srow ? b : 0;
#pragma unroll
    for (int i = 0; i < kScaleCopies; ++i)
      __builtin_amdgcn_global_load_lds((global_void*)(ssrc[i] + off),
                                       (lds_void*)(base + (kScaleCopies * wave + i) * 256), 4, 0,
                                       0);
  };

  f32x4 acc[kTW][C::MT];
#pragma unroll
  for (int j = 0; j < kTW; ++j)
#pragma unroll
    for (int s = 0; s < C::MT; ++s) acc[j][s] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int mt_active = (nlive + 15) >> 4;

  auto compute = [&](int c) {
    const unsigned char* base = ring + (c % C::S) * C::STAGE;
    const unsigned char* sb = sring + ((c / kGroup) & 1) * kScaleStage + (c % kGroup) * 4;
    uint32_t sc[kTW];                                  // scale bytes of the 4 K steps
#pragma unroll
    for (int j = 0; j < kTW; ++j)
      sc[j] = *reinterpret_cast<const uint32_t*>(sb + (16 * wtile[j] + li) * 32);
#pragma unroll
    for (int ks = 0; ks < kKC / 32; ++ks) {
      // codes K 32 ks + 8 lg .. + 8 of row li: 16-byte slot 2 ks + lg / 2, half lg % 2
      const int cq = ((2 * ks + (lg >> 1)) ^ (li & 7) ^ (li >> 3)) * 16 + (lg & 1) * 8;
      u32x4 wa[kTW];
#pragma unroll
      for (int j = 0; j < kTW; ++j) {
        const uint2 cw = *reinterpret_cast<const uint2*>(base + wtile[j] * 2048 + li * 128 + cq);
        wa[j] = dequant8(cw, (sc[j] >> (8 * ks)) & 0xFFu);
      }
#pragma unroll
      for (int s = 0; s < C::MT; ++s) {
        if (s < mt_active) {
          const u32x4 xb = *reinterpret_cast<const u32x4*>(
              base + kCodeStage + (16 * s + li) * 256 + (((4 * ks + lg) ^ li) * 16));
#pragma unroll
          for (int j = 0; j < kTW; ++j) acc[j][s] = mfma16x16x32(wa[j], xb, acc[j][s]);
        }
      }
    }
  };

  // The scales of group g + 1 go out right before chunk 8 g + 2; each wait counts the
  // copies issued after the chunk it needs (loads return in order): with 3 stages the
  // next chunk's (and the scales sent just before it), with 2 stages none.
  issue_scales(0);
#pragma unroll
  for (int p = 0; p < C::S - 1; ++p)
    if (p < nch) issue_chunk(p);
  for (int c = 0; c < nch; ++c) {
    const int n1 = c + 1;
    if (C::S == 2 || n1 >= nch) wait_vmcnt<0>();
    else if (n1 % kGroup == 2 && n1 / kGroup + 1 < ngroups) wait_vmcnt<C::PER_CHUNK + kScaleCopies>();
    else wait_vmcnt<C::PER_CHUNK>();
    // chunk c landed for every wave and chunk c - 1 is consumed; a bare barrier keeps the
    // copies in flight
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int q = c + C::S - 1;
    if (q < nch) {
      if (q % kGroup == 2 && q / kGroup + 1 < ngroups) issue_scales(q / kGroup + 1);
      issue_chunk(q);
    }
    compute(c);
  }

#pragma unroll
  for (int s = 0; s < C::MT; ++s) {
    if (s >= mt_active) continue;
    const int r = 16 * s + li;
    if (r >= nlive) continue;                          // padding rows are never read
    if (UP) {
#pragma unroll
      for (int h = 0; h < kTW / 2; ++h) {
        const int n = ntile * 128 + 16 * (kTW / 2 * wave + h) + 4 * lg;
        float a[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) a[q] = silu_f32(acc[h][s][q]) * acc[kTW / 2 + h][s][q];
        uint2 v;
        v.x = pack_bf16x2(a[0], a[1]);
        v.y = pack_bf16x2(a[2], a[3]);
        *reinterpret_cast<uint2*>(act + (size_t)(start + r) * I + n) = v;
      }
    } else {
      const YRow yr = y_row(sorted_ids[start + r], top_k, ncols);
#pragma unroll
      for (int j = 0; j < kTW; ++j) {
        const int n = ntile * kRows + 16 * (kTW * wave + j) + 4 * lg;
        if (n < ncols)
          store_y4(y, y0, yr, n, acc[j][s][0], acc[j][s][1], acc[j][s][2], acc[j][s][3]);
      }
    }
  }
}

template <int BM, int WPOL, bool UP>
__global__ __launch_bounds__(64 * kWaves) void expert_mx_decode_kernel(
    const uint16_t* __restrict__ tok_src, const uint8_t* __restrict__ wc,
    const uint8_t* __restrict__ ws, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int2* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, int n_ntiles, int K, int ncols, int I, int top_k,
    int block, uint16_t* __restrict__ act, uint16_t* __restrict__ y, float* __restrict__ y0) {
  using C = MxdCfg<BM>;
  __shared__ __align__(16) unsigned char lds[C::LDS];
  TiledWalk walk(*num_tiles, n_ntiles);
  int ntile, ti;
  while (walk.next(ntile, ti)) {
    mx_decode_item<BM, WPOL, UP>(lds, lds + C::S * C::STAGE, ntile, ti, tok_src, wc, ws, sorted_ids,
                       block_expert, tiles, K, ncols, I, top_k, block, act, y, y0);
    __syncthreads();  // the next item's first copies reuse the rings
  }
}

template <int BM, int WPOL, bool UP>
hipError_t launch_mx_lds(const uint16_t* src, const uint8_t* wc, const uint8_t* ws,
                         const int32_t* sorted_ids, const int32_t* block_expert, const int2* tiles,
                         const int32_t* num_tiles, int max_tiles, int K, int ncols, int I,
                         int top_k, int block, uint16_t* act, uint16_t* y, float* y0,
                         hipStream_t s) {
  if (K % kKC != 0 || (UP && I % 128 != 0) || (uintptr_t)ws % 4 != 0) return hipErrorInvalidValue;
  const int per_ntile = UP ? 128 : kRows;
  const int n_ntiles = (ncols + per_ntile - 1) / per_ntile;
  const long items = (long)max_tiles * n_ntiles;
  const long grid = walk_grid(items, MxdCfg<BM>::LDS);
  hipLaunchKernelGGL((expert_mx_decode_kernel<BM, WPOL, UP>), dim3((unsigned)grid),
                     dim3(64 * kWaves), 0, s, src, wc, ws, sorted_ids, block_expert, tiles,
                     num_tiles, n_ntiles, K, ncols, I, top_k, block, act, y, y0);
  return hipGetLastError();
}

template <bool UP>
hipError_t launch_mx_lds_rows(const uint16_t* src, const uint8_t* wc, const uint8_t* ws,
                              const int32_t* sorted_ids, const int32_t* block_expert,
                              const int2* tiles, const int32_t* num_tiles, int max_tiles,
                              int tile_rows, bool stream_weights, int K, int ncols, int I,
                              int top_k, int block, uint16_t* act, uint16_t* y, float* y0,
                              hipStream_t s) {
#define MOE_MXL(BM, POL)                                                                      \
  return launch_mx_lds<BM, POL, UP>(src, wc, ws, sorted_ids, block_expert, tiles, num_tiles, \
                                    max_tiles, K, ncols, I, top_k, block, act, y, y0, s)
  if (tile_rows == 32) {
    if (stream_weights) MOE_MXL(32, kNT);
    MOE_MXL(32, 0);
  }
  if (tile_rows == 64) {
    if (stream_weights) MOE_MXL(64, kNT);
    MOE_MXL(64, 0);
  }
  if (tile_rows == 128) {
    if (stream_weights) MOE_MXL(128, kNT);
    MOE_MXL(128, 0);
  }
#undef MOE_MXL
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_expert_up_mx_lds(const uint16_t* x, const uint8_t* w13c, const uint8_t* w13s,
                                   const int32_t* sorted_ids, const int32_t* block_expert,
                                   const int2* tiles, const int32_t* num_tiles, int max_tiles,
                                   int tile_rows, bool stream_weights, int H, int I, int top_k,
                                   int block, uint16_t* act, hipStream_t s) {
  return launch_mx_lds_rows<true>(x, w13c, w13s, sorted_ids, block_expert, tiles, num_tiles,
                                  max_tiles, tile_rows, stream_weights, H, I, I, top_k, block,
                                  act, nullptr, nullptr, s);
}

hipError_t launch_expert_down_mx_lds(const uint16_t* act, const uint8_t* w2c, const uint8_t* w2s,
                                     const int32_t* sorted_ids, const int32_t* block_expert,
                                     const int2* tiles, const int32_t* num_tiles, int max_tiles,
                                     int tile_rows, bool stream_weights, int H, int I, int top_k,
                                     int block, uint16_t* y, float* y0, hipStream_t s) {
  return launch_mx_lds_rows<false>(act, w2c, w2s, sorted_ids, block_expert, tiles, num_tiles,
                                   max_tiles, tile_rows, stream_weights, I, H, I, top_k, block,
                                   nullptr, y, y0, s);
}

}  // namespace moe
