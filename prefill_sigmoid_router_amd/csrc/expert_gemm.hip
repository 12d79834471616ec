// Grouped expert GEMMs of the routed-MoE layer over the align plan.
//
// AlphaMoE page (FlashInfer PR #6511 analysis), sections 1-4: the up kernel gathers the
// token tile of an expert and streams that expert's weights, the down kernel streams
// W2 in deep K panels; the route chain is up -> down -> finalize.  Trainium2 megakernel
// page, first paragraph, rule 2: split each weight stream over many programs so that
// small-batch decode runs at memory bandwidth.
//
// MI355X layout: one workgroup = one plan block (block rows of one expert) x one N tile;
// every wave owns 16-row weight tiles and streams them straight from HBM into MFMA
// A-fragments (v_mfma_f32_16x16x32_bf16).  The token rows are the B operand, gathered by
// plan row.  Each lane reads 16*P contiguous bytes of its weight row per K step: inside
// one K step of 32*P values, lane group g = lane/16 covers [g*8P, (g+1)*8P) and MFMA p
// takes values g*8P + 8p .. +8 -- a permutation of K applied identically to A and B,
// so the sum is unchanged while every weight row is read in 64-byte runs.  Only the
// 16-row groups of a block that hold at least one real entry are computed; the weight
// fragments of a K step are loaded once and reused by every such group.
//
// D fragment of lane l: weight rows 4*(l/16)+q (q = 0..3) for token column l%16, so a
// lane writes 4 consecutive outputs of one token row (8 bytes of act, 16 bytes of y).
#include "device_common.h"
#include "launchers.h"

namespace moe {

template <int NS, int NT, int P>
__global__ __launch_bounds__(256) void expert_up_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w13,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ num_padded, int H, int I, int top_k, int block, int sentinel,
    uint16_t* __restrict__ act) {
  const int b = blockIdx.y;
  if (b * block >= *num_padded) return;  // workgroup-uniform
  const int e = block_expert[b];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lg = lane >> 4;

  int tok[NS];
  bool live[NS], active[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int v = sorted_ids[b * block + 16 * s + li];
    live[s] = v < sentinel;
    tok[s] = live[s] ? v / top_k : 0;
    active[s] = __ballot(live[s]) != 0ull;
  }

  const int nbase = blockIdx.x * (64 * NT) + wave * (16 * NT);
  const uint16_t* wexp = w13 + (size_t)e * 2 * I * H;
  const uint16_t* wg_row[NT];
  const uint16_t* wu_row[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = nbase + 16 * nt + li;
    wg_row[nt] = wexp + (size_t)n * H;
    wu_row[nt] = wexp + (size_t)(I + n) * H;
  }

  f32x4 accg[NT][NS], accu[NT][NS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      accg[nt][s] = f32x4{0.f, 0.f, 0.f, 0.f};
      accu[nt][s] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  for (int k0 = 0; k0 < H; k0 += 32 * P) {
    const int kl = k0 + lg * 8 * P;
    u32x4 wg[NT][P], wu[NT][P], xf[NS][P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int kk = kl + 8 * p;
      const bool in = kk < H;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        wg[nt][p] = in ? ld16(wg_row[nt] + kk) : u32x4{0, 0, 0, 0};
        wu[nt][p] = in ? ld16(wu_row[nt] + kk) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int s = 0; s < NS; ++s)
        xf[s][p] = (active[s] && live[s] && in) ? ld16(x + (size_t)tok[s] * H + kk)
                                                : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (!active[s]) continue;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          accg[nt][s] = mfma16x16x32(wg[nt][p], xf[s][p], accg[nt][s]);
          accu[nt][s] = mfma16x16x32(wu[nt][p], xf[s][p], accu[nt][s]);
        }
      }
  }

#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (!active[s]) continue;
    const size_t r = (size_t)b * block + 16 * s + li;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = nbase + 16 * nt + 4 * lg;
      float a[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) a[q] = silu_f32(accg[nt][s][q]) * accu[nt][s][q];
      uint2 v;
      v.x = pack_bf16x2(a[0], a[1]);
      v.y = pack_bf16x2(a[2], a[3]);
      *reinterpret_cast<uint2*>(act + r * I + n) = v;
    }
  }
}

template <int NS, int NT, int P>
__global__ __launch_bounds__(256) void expert_down_kernel(
    const uint16_t* __restrict__ act, const uint16_t* __restrict__ w2,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ num_padded, int H, int I, int block, int sentinel,
    float* __restrict__ y) {
  const int b = blockIdx.y;
  if (b * block >= *num_padded) return;  // workgroup-uniform
  const int e = block_expert[b];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lg = lane >> 4;

  int dst[NS];
  bool live[NS], active[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int v = sorted_ids[b * block + 16 * s + li];
    live[s] = v < sentinel;
    dst[s] = v;
    active[s] = __ballot(live[s]) != 0ull;
  }

  const int nbase = blockIdx.x * (64 * NT) + wave * (16 * NT);
  if (nbase >= H) return;  // wave-uniform (H is a multiple of 16); no barriers below
  const uint16_t* wexp = w2 + (size_t)e * H * I;
  const uint16_t* w_row[NT];
  bool nt_in[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    nt_in[nt] = nbase + 16 * nt < H;
    w_row[nt] = wexp + (size_t)(nt_in[nt] ? nbase + 16 * nt + li : 0) * I;
  }
  const uint16_t* a_row[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) a_row[s] = act + ((size_t)b * block + 16 * s + li) * I;

  f32x4 acc[NT][NS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int s = 0; s < NS; ++s) acc[nt][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < I; k0 += 32 * P) {
    const int kl = k0 + lg * 8 * P;
    u32x4 wf[NT][P], af[NS][P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int kk = kl + 8 * p;
      const bool in = kk < I;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        wf[nt][p] = (in && nt_in[nt]) ? ld16(w_row[nt] + kk) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < NS; ++s)
        af[s][p] = (active[s] && in) ? ld16(a_row[s] + kk) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (!active[s]) continue;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt][s] = mfma16x16x32(wf[nt][p], af[s][p], acc[nt][s]);
      }
  }

#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (!live[s]) continue;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (!nt_in[nt]) continue;
      const int n = nbase + 16 * nt + 4 * lg;
      float4 v;
      v.x = acc[nt][s][0];
      v.y = acc[nt][s][1];
      v.z = acc[nt][s][2];
      v.w = acc[nt][s][3];
      *reinterpret_cast<float4*>(y + (size_t)dst[s] * H + n) = v;
    }
  }
}

template <int NS>
static hipError_t up_for_block(const uint16_t* x, const uint16_t* w13, const int32_t* sorted_ids,
                               const int32_t* block_expert, const int32_t* num_padded, int M,
                               int H, int I, int top_k, int block, int capacity, uint16_t* act,
                               hipStream_t s) {
  constexpr int NT = 1, P = NS <= 2 ? 4 : (NS == 4 ? 2 : 1);
  dim3 grid(I / (64 * NT), capacity / block);
  hipLaunchKernelGGL((expert_up_kernel<NS, NT, P>), grid, dim3(256), 0, s, x, w13, sorted_ids,
                     block_expert, num_padded, H, I, top_k, block, M * top_k, act);
  return hipGetLastError();
}

template <int NS>
static hipError_t down_for_block(const uint16_t* act, const uint16_t* w2,
                                 const int32_t* sorted_ids, const int32_t* block_expert,
                                 const int32_t* num_padded, int M, int H, int I, int top_k,
                                 int block, int capacity, float* y, hipStream_t s) {
  constexpr int NT = 2, P = NS <= 2 ? 4 : (NS == 4 ? 2 : 1);
  dim3 grid((H + 64 * NT - 1) / (64 * NT), capacity / block);
  hipLaunchKernelGGL((expert_down_kernel<NS, NT, P>), grid, dim3(256), 0, s, act, w2, sorted_ids,
                     block_expert, num_padded, H, I, block, M * top_k, y);
  return hipGetLastError();
}

hipError_t launch_expert_up(const uint16_t* x, const uint16_t* w13, const int32_t* sorted_ids,
                            const int32_t* block_expert, const int32_t* num_padded, int M, int H,
                            int E, int I, int top_k, int block, int capacity, uint16_t* act,
                            hipStream_t s) {
  (void)E;
  switch (block) {
    case 16: return up_for_block<1>(x, w13, sorted_ids, block_expert, num_padded, M, H, I, top_k, block, capacity, act, s);
    case 32: return up_for_block<2>(x, w13, sorted_ids, block_expert, num_padded, M, H, I, top_k, block, capacity, act, s);
    case 64: return up_for_block<4>(x, w13, sorted_ids, block_expert, num_padded, M, H, I, top_k, block, capacity, act, s);
    case 128: return up_for_block<8>(x, w13, sorted_ids, block_expert, num_padded, M, H, I, top_k, block, capacity, act, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_expert_down(const uint16_t* act, const uint16_t* w2, const int32_t* sorted_ids,
                              const int32_t* block_expert, const int32_t* num_padded, int M,
                              int H, int E, int I, int top_k, int block, int capacity, float* y,
                              hipStream_t s) {
  (void)E;
  switch (block) {
    case 16: return down_for_block<1>(act, w2, sorted_ids, block_expert, num_padded, M, H, I, top_k, block, capacity, y, s);
    case 32: return down_for_block<2>(act, w2, sorted_ids, block_expert, num_padded, M, H, I, top_k, block, capacity, y, s);
    case 64: return down_for_block<4>(act, w2, sorted_ids, block_expert, num_padded, M, H, I, top_k, block, capacity, y, s);
    case 128: return down_for_block<8>(act, w2, sorted_ids, block_expert, num_padded, M, H, I, top_k, block, capacity, y, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
