// Grouped expert GEMMs of the routed-MoE layer over the align plan: weight-streaming
// kernels for 16-row token tiles.  moe_forward uses them for bf16 weights only when I is
// not a multiple of 256 (the LDS-tiled kernels serve every size otherwise), for MXFP8
// weights below 16 tokens per expert, and moe_expert_up / moe_expert_down always.
//
// AlphaMoE page (FlashInfer PR #6511 analysis), sections 1-4: the up kernel gathers the
// token tile of an expert and streams that expert's weights, the down kernel streams
// W2; the route chain is up -> down -> finalize.  Trainium2 megakernel page, first
// paragraph, rule 2: split each weight stream over many programs so that small-batch
// decode runs at memory bandwidth.
//
// MI355X layout.  One workgroup = one 16-row tile of plan rows (one expert) x 16 output
// columns (up: 16 gate + 16 up weight rows; down: 32 columns, two 16-row halves).  Its
// 4 waves split the weight rows and the two halves of K; the partial sums meet through
// LDS at the end, so every wave holds a single 16-row weight stream.  Every wave streams
// its 16 weight rows straight from HBM into the A operand of v_mfma_f32_16x16x32_bf16 in
// the instruction's natural layout -- lane l reads 16 bytes of row l%16 at K offset
// 8*(l/16), so one load instruction covers 16 rows x 64 contiguous bytes -- with U
// K steps of 32 per batch and the next batch in flight while the MFMAs of this one run.
// Token rows (x for up, act for down) are the B operand, gathered by plan row; rows past
// the tile's real entries read as zero.  A K tail that is not a whole step is read with
// per-lane predicates.
//
// D fragment of lane l: weight rows 4*(l/16)+q (q = 0..3) for token column l%16, so a
// lane writes 4 consecutive outputs of one token row (8 bytes of act, 16 bytes of y).
#include "device_common.h"
#include "launchers.h"

namespace moe {

// K steps of 32 per streamed batch.  Measured on MI355X (M=8, H=7168, I=2048): the up
// kernel's 16-row x 3584-long weight streams gain 2% from 8 steps (128 VGPRs, 3 workgroups
// per CU) over 4 or 6; the down kernel's 1024-long ones are at the read rate with 4.
constexpr int kUpStreamU = 8;
constexpr int kDownStreamU = 4;

// acc[j] += W_j(16 rows) . B(16 rows)^T over len K values.  wr[j] / br point at this
// lane's first element (row start + K offset + 8 * (lane / 16)).  MASKED: lanes with
// br_live false read B as zero (their loads are skipped).  Otherwise every lane loads its B
// row -- the caller points a lane without a real entry at lane 0's row, so it adds no cache
// lines and its unused output column stays finite -- and the compiler, which drains the
// next batch's loads before the MFMAs when loads sit under a lane mask, keeps them in
// flight (measured at M=8: up 1,057 -> 1,000 us unmasked; down 494 masked, 512 unmasked).
template <int NW, int U, bool MASKED>
__device__ __forceinline__ void stream_k(const uint16_t* const (&wr)[NW], const uint16_t* br,
                                         bool br_live, int len, int lg, f32x4 (&acc)[NW]) {
  const u32x4 z4 = u32x4{0, 0, 0, 0};
  const int full = len / (32 * U);
  u32x4 wa[2][NW][U], xa[2][U];
  if (full > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int j = 0; j < NW; ++j) wa[0][j][u] = ld16(wr[j] + 32 * u);
      xa[0][u] = (!MASKED || br_live) ? ld16(br + 32 * u) : z4;
    }
  }
  for (int m = 0; m < full; m += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int mm = m + h;
      if (mm < full) {
        if (mm + 1 < full) {
          const int kn = (mm + 1) * 32 * U;
#pragma unroll
          for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int j = 0; j < NW; ++j) wa[h ^ 1][j][u] = ld16(wr[j] + kn + 32 * u);
            xa[h ^ 1][u] = (!MASKED || br_live) ? ld16(br + kn + 32 * u) : z4;
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int j = 0; j < NW; ++j) acc[j] = mfma16x16x32(wa[h][j][u], xa[h][u], acc[j]);
      }
    }
  }
  for (int k = full * 32 * U; k < len; k += 32) {  // tail, 32 at a time
    const bool in = k + 8 * lg + 8 <= len;
    const u32x4 xb = (in && (!MASKED || br_live)) ? ld16(br + k) : z4;
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const u32x4 wv = in ? ld16(wr[j] + k) : z4;
      acc[j] = mfma16x16x32(wv, xb, acc[j]);
    }
  }
}

// MXFP8 weights: acc += W(16 rows) . B(16 rows)^T over ng groups of 256 K values (4
// chunks of 64, 8 scale bytes).  wr points at this lane's 16 E4M3 codes of the first chunk
// (row start + K offset + 16 * (lane / 16)), sr at the row's scale bytes of the first group
// (8-byte aligned), br at the lane's B row + the same K offset as wr.  A chunk's 16 codes
// dequantize (exactly, to bf16) into two MFMA fragments: K values 16*lg..+8 and
// 16*lg+8..+16 of the chunk, paired with the same K values of B -- the MFMA sums over its
// K group whatever the order, so this only permutes K.  Scales: a byte load per chunk costs
// as many cache-line requests as the codes, so one 8-byte load per row brings two groups'
// scales -- lanes 0-31 load the even group, lanes 32-63 the odd one, and a lane-half swap
// (v_permlane32_swap) gives every lane both; chunk u of a group uses byte 2u + lg / 2.
template <int NW>
__device__ __forceinline__ void stream_mx(const uint8_t* const (&wr)[NW],
                                          const uint8_t* const (&sr)[NW], const uint16_t* br,
                                          int ng, f32x4 (&acc)[NW]) {
  constexpr int U = 4;
  const int upper = (threadIdx.x & 63) >> 5;   // also lg / 2
  const int sshift = 8 * upper;
  u32x4 wc[2][NW][U], xa[2][U], xb[2][U];
  uint2 sp[NW];                                // pair load in flight: group 2p + upper
  auto fetch = [&](int g, u32x4 (&cw)[NW][U], u32x4 (&a)[U], u32x4 (&b)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = g * U + u;
#pragma unroll
      for (int j = 0; j < NW; ++j) cw[j][u] = ld16(wr[j] + 64 * c);
      a[u] = ld16(br + 64 * c);
      b[u] = ld16(br + 64 * c + 8);
    }
  };
  auto fetch_scales = [&](int g) {             // g even: groups g and g + 1 (if any)
    const int gg = min(g + upper, ng - 1);
#pragma unroll
    for (int j = 0; j < NW; ++j) sp[j] = *reinterpret_cast<const uint2*>(sr[j] + 8 * gg);
  };
  auto mma = [&](const u32x4 (&cw)[NW][U], const uint2 (&sv)[NW], const u32x4 (&a)[U],
                 const u32x4 (&b)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        const uint32_t word = u < 2 ? sv[j].x : sv[j].y;
        const uint32_t sbyte = (word >> (16 * (u & 1) + sshift)) & 0xFFu;
        u32x4 lo, hi;
        mx_dequant16(cw[j][u], sbyte, lo, hi);
        acc[j] = mfma16x16x32(lo, a[u], acc[j]);
        acc[j] = mfma16x16x32(hi, b[u], acc[j]);
      }
  };
  if (ng <= 0) return;
  fetch_scales(0);
  fetch(0, wc[0], xa[0], xb[0]);
  for (int m = 0; m < ng; m += 2) {
    if (m + 1 < ng) fetch(m + 1, wc[1], xa[1], xb[1]);
    uint2 s_even[NW], s_odd[NW];
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const auto rx = __builtin_amdgcn_permlane32_swap(sp[j].x, sp[j].x, false, false);
      const auto ry = __builtin_amdgcn_permlane32_swap(sp[j].y, sp[j].y, false, false);
      s_even[j] = uint2{rx[0], ry[0]};
      s_odd[j] = uint2{rx[1], ry[1]};
    }
    mma(wc[0], s_even, xa[0], xb[0]);
    if (m + 2 < ng) {
      fetch_scales(m + 2);
      fetch(m + 2, wc[0], xa[0], xb[0]);
    }
    if (m + 1 < ng) mma(wc[1], s_odd, xa[1], xb[1]);
  }
}

// Work item of a workgroup: a 16-row plan tile.  From the tile list when given, else the
// blockIdx.y-th 16 rows of the plan (skipped when past the plan or without real rows).
__device__ __forceinline__ bool tile_of(const int2* tiles, const int32_t* num_tiles,
                                        const int32_t* sorted_ids, const int32_t* num_padded,
                                        int sentinel, int& start, int& nlive) {
  const int y = blockIdx.y;
  if (tiles != nullptr) {
    if (y >= *num_tiles) return false;
    const int2 t = tiles[y];
    start = t.x;
    nlive = t.y;
    return true;
  }
  start = y * 16;
  if (start >= *num_padded) return false;
  // real entries precede the sentinel padding inside an expert's run
  const int lane = threadIdx.x & 63;
  const bool live = lane < 16 && sorted_ids[start + lane] < sentinel;
  nlive = __popcll(__ballot(live));
  return nlive > 0;
}

// Up + SwiGLU: the four waves are {gate rows, up rows} x {low K half, high K half} of 16
// act columns; the three partial sums meet wave 0 through LDS, which applies
// silu(gate) * up and writes the bf16 act row fragment.
template <int U>
__global__ __launch_bounds__(256) void expert_up_stream_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w13,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ num_padded, const int2* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, int H, int I, int top_k, int block, int sentinel,
    uint16_t* __restrict__ act) {
  __shared__ f32x4 red[3][kWave];
  int start, nlive;
  if (!tile_of(tiles, num_tiles, sorted_ids, num_padded, sentinel, start, nlive)) return;
  const int e = block_expert[start / block];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int gu = wave & 1, wk = wave >> 1;
  const bool live = li < nlive;
  const int tok = sorted_ids[start + (live ? li : 0)] / top_k;  // dead lanes: lane 0's row
  const int n0 = blockIdx.x * 16;
  const int khalf = H >> 1;
  const int kb = wk * khalf + 8 * lg;
  const uint16_t* wr[1] = {w13 + (size_t)e * 2 * I * H + (size_t)(gu * I + n0 + li) * H + kb};
  f32x4 acc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
  stream_k<1, U, false>(wr, x + (size_t)tok * H + kb, live, khalf, lg, acc);
  if (wave != 0) red[wave - 1][lane] = acc[0];   // wave 1: up low-K, 2: gate high-K, 3: up high-K
  __syncthreads();
  if (wave != 0) return;
  const f32x4 g = acc[0] + red[1][lane];
  const f32x4 u = red[0][lane] + red[2][lane];
  float a[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) a[q] = live ? silu_f32(g[q]) * u[q] : 0.0f;  // sentinel rows: 0
  uint2 v;
  v.x = pack_bf16x2(a[0], a[1]);
  v.y = pack_bf16x2(a[2], a[3]);
  *reinterpret_cast<uint2*>(act + (size_t)(start + li) * I + n0 + 4 * lg) = v;
}

template <int U>
__global__ __launch_bounds__(256) void expert_down_stream_kernel(
    const uint16_t* __restrict__ act, const uint16_t* __restrict__ w2,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ num_padded, const int2* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, int H, int I, int block, int sentinel,
    float* __restrict__ y) {
  __shared__ f32x4 red[2][kWave];
  int start, nlive;
  if (!tile_of(tiles, num_tiles, sorted_ids, num_padded, sentinel, start, nlive)) return;
  const int e = block_expert[start / block];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int wn = wave & 1, wk = wave >> 1;

  const bool live = li < nlive;
  const int n0 = blockIdx.x * 32 + wn * 16;
  const bool n_in = n0 < H;  // H is a multiple of 16: a wave's 16 columns are all in or all out
  const int khalf = I >> 1;
  const int kb = wk * khalf + 8 * lg;
  const uint16_t* wr[1] = {w2 + (size_t)e * H * I + (size_t)(n_in ? n0 + li : 0) * I + kb};
  f32x4 acc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
  if (n_in) stream_k<1, U, true>(wr, act + (size_t)(start + li) * I + kb, live, khalf, lg, acc);

  if (wk == 1) red[wn][lane] = acc[0];
  __syncthreads();
  if (wk == 1 || !n_in || !live) return;
  acc[0] += red[wn][lane];
  const int dst = sorted_ids[start + li];
  *reinterpret_cast<float4*>(y + (size_t)dst * H + n0 + 4 * lg) =
      make_float4(acc[0][0], acc[0][1], acc[0][2], acc[0][3]);
}

// Up + SwiGLU on MXFP8 W13 (codes [E, 2I, H], scale bytes [E, 2I, H/32]): 16 CG act
// columns per workgroup.  Each of the four waves streams the gate and the up rows of all
// CG column groups over a quarter of K (whole 256-value groups), so one fragment of x
// feeds 2 CG MFMAs; the quarters meet wave 0 through LDS in a fixed order.  H is a
// multiple of 256, the scale rows 8-byte aligned.
template <int CG>
__global__ __launch_bounds__(256) void expert_up_mx_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ w13c,
    const uint8_t* __restrict__ w13s, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    const int2* __restrict__ tiles, const int32_t* __restrict__ num_tiles, int H, int I,
    int top_k, int block, int sentinel, uint16_t* __restrict__ act) {
  constexpr int NS = 2 * CG;  // weight streams per wave: gate and up of each group
  __shared__ f32x4 red[3][NS][kWave];
  int start, nlive;
  if (!tile_of(tiles, num_tiles, sorted_ids, num_padded, sentinel, start, nlive)) return;
  const int e = block_expert[start / block];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lg = lane >> 4;
  const bool live = li < nlive;
  const int tok = sorted_ids[start + (live ? li : 0)] / top_k;  // dead lanes: lane 0's row
  const int n0 = blockIdx.x * 16 * CG;
  const int ng = H / 256;                                  // groups of 256 K values
  const int g0 = wave * ng / 4, g1 = (wave + 1) * ng / 4;  // this wave's share of K
  const int kb = 256 * g0;
  const uint8_t* wr[NS];
  const uint8_t* sr[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {   // stream j: group j / 2, gate (j even) or up (j odd)
    const size_t row = (size_t)e * 2 * I + (j & 1) * I + n0 + 16 * (j >> 1) + li;
    wr[j] = w13c + row * H + kb + 16 * lg;
    sr[j] = w13s + row * (H / 32) + kb / 32;
  }
  f32x4 acc[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  stream_mx<NS>(wr, sr, x + (size_t)tok * H + kb + 16 * lg, g1 - g0, acc);
  if (wave != 0)
#pragma unroll
    for (int j = 0; j < NS; ++j) red[wave - 1][j][lane] = acc[j];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    const f32x4 g = ((acc[2 * c] + red[0][2 * c][lane]) + red[1][2 * c][lane]) + red[2][2 * c][lane];
    const f32x4 u =
        ((acc[2 * c + 1] + red[0][2 * c + 1][lane]) + red[1][2 * c + 1][lane]) + red[2][2 * c + 1][lane];
    float a[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) a[q] = live ? silu_f32(g[q]) * u[q] : 0.0f;  // sentinel rows: 0
    uint2 v;
    v.x = pack_bf16x2(a[0], a[1]);
    v.y = pack_bf16x2(a[2], a[3]);
    *reinterpret_cast<uint2*>(act + (size_t)(start + li) * I + n0 + 16 * c + 4 * lg) = v;
  }
}

// Down on MXFP8 W2 (codes [E, H, I], scale bytes [E, H, I/32]): 32 NC output columns per
// workgroup; waves = 2 column groups x 2 halves of K (whole 256-value groups), each
// streaming NC 16-row tiles of W2 against one act fragment; I is a multiple of 256.
template <int NC>
__global__ __launch_bounds__(256) void expert_down_mx_kernel(
    const uint16_t* __restrict__ act, const uint8_t* __restrict__ w2c,
    const uint8_t* __restrict__ w2s, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    const int2* __restrict__ tiles, const int32_t* __restrict__ num_tiles, int H, int I,
    int block, int sentinel, float* __restrict__ y) {
  __shared__ f32x4 red[2][NC][kWave];
  int start, nlive;
  if (!tile_of(tiles, num_tiles, sorted_ids, num_padded, sentinel, start, nlive)) return;
  const int e = block_expert[start / block];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int wn = wave & 1, wk = wave >> 1;
  const bool live = li < nlive;
  const int n0 = blockIdx.x * 32 * NC + wn * 16 * NC;
  const int ng = I / 256;                                  // groups of 256 K values
  const int g0 = wk * ng / 2, g1 = (wk + 1) * ng / 2;      // this wave's half of K
  const int kb = 256 * g0;
  const uint8_t* wr[NC];
  const uint8_t* sr[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int n = n0 + 16 * j;
    const size_t row = (size_t)e * H + (n < H ? n + li : 0);   // H % 16 == 0
    wr[j] = w2c + row * I + kb + 16 * lg;
    sr[j] = w2s + row * (I / 32) + kb / 32;
  }
  f32x4 acc[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int arow = start + (live ? li : 0);  // dead lanes read lane 0's row
  if (n0 < H) stream_mx<NC>(wr, sr, act + (size_t)arow * I + kb + 16 * lg, g1 - g0, acc);
  if (wk == 1)
#pragma unroll
    for (int j = 0; j < NC; ++j) red[wn][j][lane] = acc[j];
  __syncthreads();
  if (wk == 1 || !live) return;
  const int dst = sorted_ids[start + li];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int n = n0 + 16 * j;
    if (n < H) {
      const f32x4 d = acc[j] + red[wn][j][lane];
      *reinterpret_cast<float4*>(y + (size_t)dst * H + n + 4 * lg) = make_float4(d[0], d[1], d[2], d[3]);
    }
  }
}

hipError_t launch_expert_up(const uint16_t* x, const uint16_t* w13, const int32_t* sorted_ids,
                            const int32_t* block_expert, const int32_t* num_padded,
                            const int2* tiles, const int32_t* num_tiles, int max_tiles, int M,
                            int H, int I, int top_k, int block, uint16_t* act, hipStream_t s) {
  dim3 grid(I / 16, max_tiles);
  hipLaunchKernelGGL((expert_up_stream_kernel<kUpStreamU>), grid, dim3(256), 0, s, x, w13, sorted_ids,
                     block_expert, num_padded, tiles, num_tiles, H, I, top_k, block, M * top_k,
                     act);
  return hipGetLastError();
}

hipError_t launch_expert_down(const uint16_t* act, const uint16_t* w2, const int32_t* sorted_ids,
                              const int32_t* block_expert, const int32_t* num_padded,
                              const int2* tiles, const int32_t* num_tiles, int max_tiles, int M,
                              int H, int I, int top_k, int block, float* y, hipStream_t s) {
  dim3 grid((H + 31) / 32, max_tiles);
  hipLaunchKernelGGL((expert_down_stream_kernel<kDownStreamU>), grid, dim3(256), 0, s, act, w2,
                     sorted_ids, block_expert, num_padded, tiles, num_tiles, H, I, block,
                     M * top_k, y);
  return hipGetLastError();
}

// Act column groups per up workgroup and W2 tiles per down wave.  Measured at M=8
// (interleaved runs): one column group is fastest for up (two: +11 %, the 298 registers
// leave one wave per SIMD); two W2 tiles per wave take down from 425 to 393 us (four spill).
constexpr int kMxUpCG = 1;
constexpr int kMxDownNC = 2;

hipError_t launch_expert_up_mx(const uint16_t* x, const uint8_t* w13c, const uint8_t* w13s,
                               const int32_t* sorted_ids, const int32_t* block_expert,
                               const int32_t* num_padded, const int2* tiles,
                               const int32_t* num_tiles, int max_tiles, int M, int H, int I,
                               int top_k, int block, uint16_t* act, hipStream_t s) {
  if (H % 256 != 0 || I % (16 * kMxUpCG) != 0 || (uintptr_t)w13s % 8 != 0)
    return hipErrorInvalidValue;
  dim3 grid(I / (16 * kMxUpCG), max_tiles);
  hipLaunchKernelGGL((expert_up_mx_kernel<kMxUpCG>), grid, dim3(256), 0, s, x, w13c, w13s,
                     sorted_ids, block_expert, num_padded, tiles, num_tiles, H, I, top_k, block,
                     M * top_k, act);
  return hipGetLastError();
}

hipError_t launch_expert_down_mx(const uint16_t* act, const uint8_t* w2c, const uint8_t* w2s,
                                 const int32_t* sorted_ids, const int32_t* block_expert,
                                 const int32_t* num_padded, const int2* tiles,
                                 const int32_t* num_tiles, int max_tiles, int M, int H, int I,
                                 int top_k, int block, float* y, hipStream_t s) {
  if (I % 256 != 0 || (uintptr_t)w2s % 8 != 0) return hipErrorInvalidValue;
  dim3 grid((H + 32 * kMxDownNC - 1) / (32 * kMxDownNC), max_tiles);
  hipLaunchKernelGGL((expert_down_mx_kernel<kMxDownNC>), grid, dim3(256), 0, s, act, w2c, w2s,
                     sorted_ids, block_expert, num_padded, tiles, num_tiles, H, I, block,
                     M * top_k, y);
  return hipGetLastError();
}

}  // namespace moe
