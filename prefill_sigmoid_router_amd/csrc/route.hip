// Router of the routed-MoE layer: sigmoid scoring with top-k selection.
//
// sglang PR #29509 analysis ("GLM-4.7-Flash on NPU"), section 2 "MoE TopK scoring
// function": the gate score is the sigmoid and the top-k is taken on it.  Readings
// this library fixes: key = x . Wr[e] (+ bias[e]) accumulated in fp64 so that the
// selection is reproducible; order = key descending, ties to the lower expert id;
// weights = sigmoid(key) of the k picks divided by their sum.
//
// Two kernels:
//   router_keys_kernel  -- fp64 dot products, one workgroup per (TM tokens x TE
//                          experts) tile, threads split H in 16-byte chunks (fully
//                          coalesced 4 KiB row segments per workgroup load).
//   router_topk_kernel  -- one workgroup per token: every expert's rank among the
//                          token's keys (key descending, ties to the lower id) by
//                          counting, picks = ranks below k; sigmoid and
//                          renormalisation in fp64.
#include "device_common.h"
#include "launchers.h"

namespace moe {

// One workgroup per (TM tokens x TE experts) tile.  Its 256 threads split H in 16-byte
// chunks (chunk c goes to thread c mod 256), PRE chunks per thread are requested before
// any arithmetic, and the per-thread fp64 partial sums meet in a fixed order: an xor
// butterfly inside each wave, then the four waves in ascending order through LDS.
template <int TM, int TE, int PRE>
__global__ __launch_bounds__(256) void router_keys_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wr,
                                                          int M, int H, int E,
                                                          double* __restrict__ keys) {
  __shared__ double part[4][TM][TE];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int e0 = blockIdx.x * TE;
  const int t0 = blockIdx.y * TM;

  double acc[TM][TE];
#pragma unroll
  for (int t = 0; t < TM; ++t)
#pragma unroll
    for (int e = 0; e < TE; ++e) acc[t][e] = 0.0;

  const int nchunk = H >> 3;  // 8 bf16 per 16-byte chunk
  const u32x4 z4 = u32x4{0, 0, 0, 0};
  for (int c0 = tid; c0 < nchunk; c0 += 256 * PRE) {
    u32x4 xr[PRE][TM], wv[PRE][TE];
#pragma unroll
    for (int p = 0; p < PRE; ++p) {
      const int c = c0 + 256 * p;
      const bool in = c < nchunk;
#pragma unroll
      for (int t = 0; t < TM; ++t)
        xr[p][t] = (in && t0 + t < M) ? ld16(x + (size_t)(t0 + t) * H + (size_t)c * 8) : z4;
#pragma unroll
      for (int e = 0; e < TE; ++e)
        wv[p][e] = (in && e0 + e < E) ? ld16(wr + (size_t)(e0 + e) * H + (size_t)c * 8) : z4;
    }
#pragma unroll
    for (int p = 0; p < PRE; ++p)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          double xd[TM], wd[TE];
#pragma unroll
          for (int t = 0; t < TM; ++t) xd[t] = (double)(half ? bf16hi(xr[p][t][q]) : bf16lo(xr[p][t][q]));
#pragma unroll
          for (int e = 0; e < TE; ++e) wd[e] = (double)(half ? bf16hi(wv[p][e][q]) : bf16lo(wv[p][e][q]));
#pragma unroll
          for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int e = 0; e < TE; ++e) acc[t][e] = fma(xd[t], wd[e], acc[t][e]);
        }
  }
#pragma unroll
  for (int t = 0; t < TM; ++t)
#pragma unroll
    for (int e = 0; e < TE; ++e) {
      const double s = wave_sum(acc[t][e]);
      if (lane == 0) part[wave][t][e] = s;
    }
  __syncthreads();
  if (tid < TM * TE) {
    const int t = tid / TE, e = tid % TE;
    if (t0 + t < M && e0 + e < E)
      keys[(size_t)(t0 + t) * E + e0 + e] =
          ((part[0][t][e] + part[1][t][e]) + part[2][t][e]) + part[3][t][e];
  }
}

constexpr int kTopkMaxE = 1024;
constexpr int kTopkThreads = 256;

// One workgroup per token.  Thread i owns experts i, i + 256, ... (SL of them).  The
// token's keys (logit + bias) sit in LDS; each owned expert's rank is the number of
// experts ahead of it -- a larger key, or an equal key with a lower id -- counted against
// every key through broadcast LDS reads, so ranks are a permutation of 0..E-1 and the
// experts with rank < k are the picks, already in output order.  No arg-max chains.
// The picks' sigmoids are summed in rank order (fixed) for the renormalisation.
template <int SL>
__global__ __launch_bounds__(kTopkThreads) void router_topk_kernel(const double* __restrict__ keys,
                                                                   const float* __restrict__ bias,
                                                                   int M, int E, int top_k,
                                                                   int32_t* __restrict__ ids,
                                                                   float* __restrict__ weights) {
  __shared__ double sk[kTopkMaxE];
  __shared__ double ssig[kTopkMaxE];
  const int t = blockIdx.x, tid = threadIdx.x;
  double mine[SL];
#pragma unroll
  for (int s = 0; s < SL; ++s) {
    const int e = tid + kTopkThreads * s;
    mine[s] = 0.0;
    if (e < E) {
      mine[s] = keys[(size_t)t * E + e] + (bias ? (double)bias[e] : 0.0);
      sk[e] = mine[s];
    }
  }
  __syncthreads();
  int rank[SL];
#pragma unroll
  for (int s = 0; s < SL; ++s) rank[s] = 0;
  for (int j = 0; j < E; ++j) {
    const double kj = sk[j];
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      const int e = tid + kTopkThreads * s;
      rank[s] += (kj > mine[s] || (kj == mine[s] && j < e)) ? 1 : 0;
    }
  }
#pragma unroll
  for (int s = 0; s < SL; ++s) {
    const int e = tid + kTopkThreads * s;
    if (e < E && rank[s] < top_k) {
      ids[(size_t)t * top_k + rank[s]] = e;
      ssig[rank[s]] = 1.0 / (1.0 + exp(-mine[s]));
    }
  }
  __syncthreads();
  if (tid < kWave) {
    double part = 0.0;
    for (int r = tid; r < top_k; r += kWave) part += ssig[r];
    const double total = wave_sum(part);
    for (int r = tid; r < top_k; r += kWave)
      weights[(size_t)t * top_k + r] = (float)(ssig[r] / total);
  }
}

template <int TM, int TE, int PRE>
static hipError_t launch_keys(const uint16_t* x, const uint16_t* wr, int M, int H, int E,
                              double* keys, hipStream_t s) {
  dim3 grid((E + TE - 1) / TE, (M + TM - 1) / TM);
  hipLaunchKernelGGL((router_keys_kernel<TM, TE, PRE>), grid, dim3(256), 0, s, x, wr, M, H, E, keys);
  return hipGetLastError();
}

template <int SL>
static hipError_t launch_topk(const double* keys, const float* bias, int M, int E, int k,
                              int32_t* ids, float* w, hipStream_t s) {
  hipLaunchKernelGGL((router_topk_kernel<SL>), dim3(M), dim3(kTopkThreads), 0, s, keys, bias, M, E,
                     k, ids, w);
  return hipGetLastError();
}

hipError_t launch_route(const uint16_t* x, const uint16_t* wr, const float* bias, int M, int H,
                        int E, int top_k, int32_t* ids, float* w, double* keys, hipStream_t s) {
  hipError_t err;
  if (M <= 16) err = launch_keys<2, 4, 4>(x, wr, M, H, E, keys, s);
  else if (M <= 256) err = launch_keys<4, 4, 2>(x, wr, M, H, E, keys, s);
  else err = launch_keys<4, 8, 1>(x, wr, M, H, E, keys, s);
  if (err != hipSuccess) return err;
  const int per_thread = (E + kTopkThreads - 1) / kTopkThreads;
  if (per_thread <= 1) return launch_topk<1>(keys, bias, M, E, top_k, ids, w, s);
  if (per_thread <= 2) return launch_topk<2>(keys, bias, M, E, top_k, ids, w, s);
  return launch_topk<4>(keys, bias, M, E, top_k, ids, w, s);
}

}  // namespace moe
