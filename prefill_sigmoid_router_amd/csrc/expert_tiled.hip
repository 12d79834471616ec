// Grouped expert GEMMs for plans whose experts carry many tokens (batched decode and
// prefill): LDS-tiled MFMA kernels.
//
// AlphaMoE page (FlashInfer PR #6511 analysis), section 4: the up kernel of the large
// batch and prefill routes gathers a tile of tokens per expert; section 2: the down
// kernel streams W2 in deep K panels.  Trainium2 megakernel page, first paragraph,
// rule 1: keep the working set on chip -- the weight chunk in LDS is shared by all token
// rows of the tile, and the M tiles of one expert run on one XCD at the same time so
// they share the weight stream through that XCD's L2.
//
// Workgroup tile: BM plan rows of one expert (a tile of the align kernel's list) x 128
// weight rows (up: 64 gate + 64 up rows = 64 act columns; down: 128 output columns), K in
// chunks of 64.  Both operands go global -> registers -> LDS in MFMA fragment order: a
// fragment is 16 rows x 32 K values, 1 KiB, lane l holding row l%16, K values
// 8*(l/16)..+8, so every global load instruction reads 16 rows x 64 contiguous bytes and
// every LDS read of a fragment is one conflict-free 1 KiB ds_read_b128.  PF chunks are
// in flight in registers while the current chunk is multiplied out of LDS (one barrier
// per chunk).  Wave w owns weight row tiles {w, w+4} (up: the gate and up rows of the
// same act columns) against every token row tile that holds real entries.
//
// Work order: the hardware hands workgroup p to XCD p % 8.  Each XCD gets an equal,
// contiguous share of the live (tile, N tile) items (the tile count is read on the
// device), ordered N tile by N tile.
#include <type_traits>

#include "device_common.h"
#include "launchers.h"

namespace moe {

constexpr int kTileKC = 64;                     // K values per chunk
constexpr int kTileKS = kTileKC / 32;           // MFMA K steps per chunk
constexpr int kTileWT = 8;                      // 16-row weight tiles per workgroup
constexpr int kXcds = 8;                        // MI355X: 8 XCDs, round-robin dispatch
#ifndef MOE_TILE_PF
#define MOE_TILE_PF 2
#endif
constexpr int kTilePF = MOE_TILE_PF;            // chunks in flight in registers

template <int BM>
struct TiledCfg {
  static constexpr int MT = BM / 16;                        // token row tiles
  static constexpr int FRAGS = (kTileWT + MT) * kTileKS;    // fragments per chunk
  static constexpr int FPW = FRAGS / 4;                     // fragments staged per wave
};

// Fragment f of a chunk: f < kTileWT*kTileKS are weight fragments (row tile f / kTileKS,
// K step f % kTileKS), the rest token fragments.
template <int BM, bool UP>
__global__ __launch_bounds__(256) void expert_tiled_kernel(
    const uint16_t* __restrict__ tok_src, const uint16_t* __restrict__ w,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ block_expert,
    const int2* __restrict__ tiles, const int32_t* __restrict__ num_tiles, int n_ntiles, int K,
    int ncols, int I, int top_k, int block, uint16_t* __restrict__ act, float* __restrict__ y) {
  using C = TiledCfg<BM>;
  __shared__ __align__(16) unsigned char lds[2 * C::FRAGS * 1024];

  const int ntiles_live = *num_tiles;
  const int live_items = ntiles_live * n_ntiles;
  const int per_xcd = (live_items + kXcds - 1) / kXcds;
  const int slot = blockIdx.x / kXcds;
  if (slot >= per_xcd) return;
  const int logical = (blockIdx.x % kXcds) * per_xcd + slot;
  if (logical >= live_items) return;
  const int ntile = logical / ntiles_live;
  const int ti = logical % ntiles_live;
  const int2 tile = tiles[ti];
  const int start = tile.x, nlive = tile.y;
  const int mt_active = (nlive + 15) >> 4;
  const int e = block_expert[start / block];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lg = lane >> 4;

  // source row pointer (at K offset 8 * lg) of every fragment this wave stages
  const uint16_t* src[C::FPW];
  bool src_on[C::FPW];
  int src_ks[C::FPW];
  const size_t wexp = UP ? (size_t)e * 2 * I * K : (size_t)e * ncols * K;
#pragma unroll
  for (int i = 0; i < C::FPW; ++i) {
    const int f = wave * C::FPW + i;
    if (f < kTileWT * kTileKS) {
      const int rt = f / kTileKS;
      src_ks[i] = f % kTileKS;
      int row;
      if (UP) row = (rt < 4) ? ntile * 64 + rt * 16 + li : I + ntile * 64 + (rt - 4) * 16 + li;
      else row = ntile * 128 + rt * 16 + li;
      src_on[i] = UP || row < ncols;
      src[i] = w + wexp + (size_t)(src_on[i] ? row : 0) * K + 8 * lg;
    } else {
      const int g = f - kTileWT * kTileKS;
      const int mt = g / kTileKS;
      src_ks[i] = g % kTileKS;
      const int r = 16 * mt + li;
      src_on[i] = r < nlive;
      const int prow = start + (src_on[i] ? r : 0);
      src[i] = UP ? tok_src + (size_t)(src_on[i] ? sorted_ids[prow] / top_k : 0) * K + 8 * lg
                  : tok_src + (size_t)prow * K + 8 * lg;
    }
  }

  const int nch = (K + kTileKC - 1) / kTileKC;
  const u32x4 z4 = u32x4{0, 0, 0, 0};
  u32x4 R[kTilePF][C::FPW];
  auto issue = [&](int c, u32x4 (&dst)[C::FPW]) {
#pragma unroll
    for (int i = 0; i < C::FPW; ++i) {
      const int k = c * kTileKC + src_ks[i] * 32;
      dst[i] = (src_on[i] && k + 8 * lg + 8 <= K) ? ld16(src[i] + k) : z4;
    }
  };
  auto stash = [&](int buf, const u32x4 (&v)[C::FPW]) {
#pragma unroll
    for (int i = 0; i < C::FPW; ++i) {
      const int f = wave * C::FPW + i;
      *reinterpret_cast<u32x4*>(lds + ((size_t)(buf * C::FRAGS + f) * 64 + lane) * 16) = v[i];
    }
  };
  auto frag = [&](int buf, int f) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(lds + ((size_t)(buf * C::FRAGS + f) * 64 + lane) * 16);
  };

  f32x4 acc[2][C::MT];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int s = 0; s < C::MT; ++s) acc[j][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  // chunk c lives in register stage c % PF until it is stashed into LDS buffer c % 2;
  // the stage index is a compile-time constant so the stages stay in registers
  auto body = [&](int c, auto stage_c) {
    constexpr int st = decltype(stage_c)::value;   // = c % kTilePF
    const int buf = c & 1;
    if (c + kTilePF < nch) issue(c + kTilePF, R[st]);  // R[st] (chunk c) is already in LDS
#pragma unroll
    for (int ks = 0; ks < kTileKS; ++ks) {
      const u32x4 wa0 = frag(buf, wave * kTileKS + ks);
      const u32x4 wa1 = frag(buf, (wave + 4) * kTileKS + ks);
#pragma unroll
      for (int s = 0; s < C::MT; ++s) {
        if (s < mt_active) {
          const u32x4 xb = frag(buf, (kTileWT + s) * kTileKS + ks);
          acc[0][s] = mfma16x16x32(wa0, xb, acc[0][s]);
          acc[1][s] = mfma16x16x32(wa1, xb, acc[1][s]);
        }
      }
    }
    if (c + 1 < nch) stash(buf ^ 1, R[(st + 1) % kTilePF]);
    __syncthreads();
  };

#pragma unroll
  for (int p = 0; p < kTilePF; ++p)
    if (p < nch) issue(p, R[p]);
  stash(0, R[0]);
  __syncthreads();
  for (int c = 0; c < nch; c += kTilePF) {
    body(c, std::integral_constant<int, 0>{});
    if (c + 1 < nch) body(c + 1, std::integral_constant<int, 1 % kTilePF>{});
    if (kTilePF > 2 && c + 2 < nch) body(c + 2, std::integral_constant<int, 2 % kTilePF>{});
    if (kTilePF > 3 && c + 3 < nch) body(c + 3, std::integral_constant<int, 3 % kTilePF>{});
  }

  // epilogue: D rows 4*lg+q of weight tile, column li of token tile s
#pragma unroll
  for (int s = 0; s < C::MT; ++s) {
    if (s >= mt_active) continue;
    const int r = 16 * s + li;
    if (UP) {
      const int n = ntile * 64 + wave * 16 + 4 * lg;
      float a[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) a[q] = silu_f32(acc[0][s][q]) * acc[1][s][q];
      uint2 v;
      v.x = pack_bf16x2(a[0], a[1]);
      v.y = pack_bf16x2(a[2], a[3]);
      *reinterpret_cast<uint2*>(act + (size_t)(start + r) * I + n) = v;
    } else if (r < nlive) {
      const int dst = sorted_ids[start + r];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = ntile * 128 + (wave + 4 * j) * 16 + 4 * lg;
        if (n < ncols)
          *reinterpret_cast<float4*>(y + (size_t)dst * ncols + n) =
              make_float4(acc[j][s][0], acc[j][s][1], acc[j][s][2], acc[j][s][3]);
      }
    }
  }
}

template <int BM, bool UP>
static hipError_t launch_tiled(const uint16_t* src, const uint16_t* w, const int32_t* sorted_ids,
                               const int32_t* block_expert, const int2* tiles,
                               const int32_t* num_tiles, int max_tiles, int n_ntiles, int K,
                               int ncols, int I, int top_k, int block, uint16_t* act, float* y,
                               hipStream_t s) {
  const long total = (long)max_tiles * n_ntiles;
  const long grid = (total + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL((expert_tiled_kernel<BM, UP>), dim3((unsigned)grid), dim3(256), 0, s, src, w,
                     sorted_ids, block_expert, tiles, num_tiles, n_ntiles, K, ncols, I, top_k, block,
                     act, y);
  return hipGetLastError();
}

hipError_t launch_expert_up_tiled(const uint16_t* x, const uint16_t* w13, const int32_t* sorted_ids,
                                  const int32_t* block_expert, const int2* tiles,
                                  const int32_t* num_tiles, int max_tiles, int tile_rows, int M,
                                  int H, int I, int top_k, int block, uint16_t* act,
                                  hipStream_t s) {
  (void)M;
  const int nt = I / 64;
  if (tile_rows == 64)
    return launch_tiled<64, true>(x, w13, sorted_ids, block_expert, tiles, num_tiles, max_tiles, nt,
                                  H, I, I, top_k, block, act, nullptr, s);
  if (tile_rows == 128)
    return launch_tiled<128, true>(x, w13, sorted_ids, block_expert, tiles, num_tiles, max_tiles, nt,
                                   H, I, I, top_k, block, act, nullptr, s);
  return hipErrorInvalidValue;
}

hipError_t launch_expert_down_tiled(const uint16_t* act, const uint16_t* w2,
                                    const int32_t* sorted_ids, const int32_t* block_expert,
                                    const int2* tiles, const int32_t* num_tiles, int max_tiles,
                                    int tile_rows, int M, int H, int I, int top_k, int block,
                                    float* y, hipStream_t s) {
  (void)M;
  const int nt = (H + 127) / 128;
  if (tile_rows == 64)
    return launch_tiled<64, false>(act, w2, sorted_ids, block_expert, tiles, num_tiles, max_tiles,
                                   nt, I, H, I, top_k, block, nullptr, y, s);
  if (tile_rows == 128)
    return launch_tiled<128, false>(act, w2, sorted_ids, block_expert, tiles, num_tiles, max_tiles,
                                    nt, I, H, I, top_k, block, nullptr, y, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
