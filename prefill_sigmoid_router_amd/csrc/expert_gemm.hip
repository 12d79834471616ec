// Grouped expert GEMMs of the routed-MoE layer over the align plan: weight-streaming
// kernels for 16-row token tiles.  moe_forward uses them only when I is not a multiple of
// 256 (the LDS-tiled kernels serve every size otherwise); moe_expert_up / moe_expert_down
// always.
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
#include <type_traits>

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
  // K halves split on a multiple of 8 values, so both start on a 16-byte boundary (H is a
  // multiple of 8, not necessarily of 16)
  const int klo = ((H >> 1) + 7) & ~7;
  const int kb = (wk ? klo : 0) + 8 * lg;
  const int klen = wk ? H - klo : klo;
  const uint16_t* wr[1] = {w13 + (size_t)e * 2 * I * H + (size_t)(gu * I + n0 + li) * H + kb};
  f32x4 acc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
  stream_k<1, U, false>(wr, x + (size_t)tok * H + kb, live, klen, lg, acc);
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

template <int U, typename Y>
__global__ __launch_bounds__(256) void expert_down_stream_kernel(
    const uint16_t* __restrict__ act, const uint16_t* __restrict__ w2,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ num_padded, const int2* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, int H, int I, int top_k, int block, int sentinel,
    Y* __restrict__ y, float* __restrict__ y0) {
  __shared__ f32x4 red[2][kWave];
  int start, nlive;
  if (!tile_of(tiles, num_tiles, sorted_ids, num_padded, sentinel, start, nlive)) return;
  const int e = block_expert[start / block];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int wn = wave & 1, wk = wave >> 1;

  const bool live = li < nlive;
  const int n0 = blockIdx.x * 32 + wn * 16;
  // a wave's 16 output columns: all in, all out, or (H a multiple of 8 only) the first 8 in;
  // weight rows past H read row 0 and their outputs are never stored
  const bool n_in = n0 < H;
  const int khalf = I >> 1;  // I is a multiple of 16: both halves start on 16 bytes
  const int kb = wk * khalf + 8 * lg;
  const uint16_t* wr[1] = {w2 + (size_t)e * H * I + (size_t)(n0 + li < H ? n0 + li : 0) * I + kb};
  f32x4 acc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
  if (n_in) stream_k<1, U, true>(wr, act + (size_t)(start + li) * I + kb, live, khalf, lg, acc);

  if (wk == 1) red[wn][lane] = acc[0];
  __syncthreads();
  if (wk == 1 || !n_in || !live || n0 + 4 * lg >= H) return;  // columns n0 + 4 lg .. + 3
  acc[0] += red[wn][lane];
  const int dst = sorted_ids[start + li];
  if constexpr (std::is_same<Y, float>::value) {
    *reinterpret_cast<float4*>(y + (size_t)dst * H + n0 + 4 * lg) =
        make_float4(acc[0][0], acc[0][1], acc[0][2], acc[0][3]);
  } else {                                           // first picks fp32, the others bf16
    store_y4(y, y0, y_row(dst, top_k, H), n0 + 4 * lg, acc[0][0], acc[0][1], acc[0][2],
             acc[0][3]);
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

template <typename Y>
static hipError_t launch_down_rows(const uint16_t* act, const uint16_t* w2, const int32_t* sorted_ids,
                              const int32_t* block_expert, const int32_t* num_padded,
                              const int2* tiles, const int32_t* num_tiles, int max_tiles, int M,
                              int H, int I, int top_k, int block, Y* y, float* y0,
                              hipStream_t s) {
  dim3 grid((H + 31) / 32, max_tiles);
  hipLaunchKernelGGL((expert_down_stream_kernel<kDownStreamU, Y>), grid, dim3(256), 0, s, act, w2,
                     sorted_ids, block_expert, num_padded, tiles, num_tiles, H, I, top_k, block,
                     M * top_k, y, y0);
  return hipGetLastError();
}

hipError_t launch_expert_down(const uint16_t* act, const uint16_t* w2, const int32_t* sorted_ids,
                              const int32_t* block_expert, const int32_t* num_padded,
                              const int2* tiles, const int32_t* num_tiles, int max_tiles, int M,
                              int H, int I, int top_k, int block, float* y, hipStream_t s) {
  return launch_down_rows(act, w2, sorted_ids, block_expert, num_padded, tiles, num_tiles,
                          max_tiles, M, H, I, top_k, block, y, nullptr, s);
}
hipError_t launch_expert_down(const uint16_t* act, const uint16_t* w2, const int32_t* sorted_ids,
                              const int32_t* block_expert, const int32_t* num_padded,
                              const int2* tiles, const int32_t* num_tiles, int max_tiles, int M,
                              int H, int I, int top_k, int block, uint16_t* y, float* y0,
                              hipStream_t s) {
  return launch_down_rows(act, w2, sorted_ids, block_expert, num_padded, tiles, num_tiles,
                          max_tiles, M, H, I, top_k, block, y, y0, s);
}

}  // namespace moe
