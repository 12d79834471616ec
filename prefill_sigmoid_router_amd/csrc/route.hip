// Router of the routed-MoE layer: sigmoid scoring with top-k selection.
//
// sglang PR #29509 analysis ("GLM-4.7-Flash on NPU"), section 2 "MoE TopK scoring
// function": the gate score is the sigmoid and the top-k is taken on it.  Readings
// this library fixes: key = x . Wr[e] (+ bias[e]) accumulated in fp64 so that the
// selection is reproducible; order = key descending, ties to the lower expert id;
// weights = sigmoid(key) of the k picks divided by their sum.
//
// Two kernels:
//   router_keys_kernel  -- fp64 dot products, one wave per (TM tokens x TEW experts)
//                          tile, lanes split H in 16-byte chunks (fully coalesced
//                          1 KiB row segments per wave load), xor-butterfly reduction.
//   router_topk_kernel  -- one wave per token: the E keys sit in registers
//                          (ceil(E/64) per lane), k rounds of a wave arg-max on
//                          (key, -id), then sigmoid and renormalisation in fp64.
#include "device_common.h"
#include "launchers.h"

namespace moe {

template <int TM, int TEW>
__global__ __launch_bounds__(256) void router_keys_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wr,
                                                          int M, int H, int E,
                                                          double* __restrict__ keys) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e0 = (blockIdx.x * 4 + wave) * TEW;
  const int t0 = blockIdx.y * TM;
  if (e0 >= E) return;  // wave-uniform; no block barrier below

  double acc[TM][TEW];
#pragma unroll
  for (int t = 0; t < TM; ++t)
#pragma unroll
    for (int e = 0; e < TEW; ++e) acc[t][e] = 0.0;

  const int nchunk = H >> 3;  // 8 bf16 per 16-byte chunk
  for (int c = lane; c < nchunk; c += kWave) {
    u32x4 xr[TM], wrv[TEW];
#pragma unroll
    for (int t = 0; t < TM; ++t)
      xr[t] = (t0 + t < M) ? ld16(x + (size_t)(t0 + t) * H + (size_t)c * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < TEW; ++e)
      wrv[e] = (e0 + e < E) ? ld16(wr + (size_t)(e0 + e) * H + (size_t)c * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        double xv[TM], wv[TEW];
#pragma unroll
        for (int t = 0; t < TM; ++t)
          xv[t] = (double)(half ? bf16hi(xr[t][q]) : bf16lo(xr[t][q]));
#pragma unroll
        for (int e = 0; e < TEW; ++e)
          wv[e] = (double)(half ? bf16hi(wrv[e][q]) : bf16lo(wrv[e][q]));
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
          for (int e = 0; e < TEW; ++e) acc[t][e] = fma(xv[t], wv[e], acc[t][e]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TM; ++t)
#pragma unroll
    for (int e = 0; e < TEW; ++e) {
      const double s = wave_sum(acc[t][e]);
      if (lane == 0 && t0 + t < M && e0 + e < E) keys[(size_t)(t0 + t) * E + e0 + e] = s;
    }
}

constexpr int kTopkMaxE = 1024;
constexpr int kTopkWaves = 4;

template <int SLOTS>
__global__ __launch_bounds__(256) void router_topk_kernel(const double* __restrict__ keys,
                                                          const float* __restrict__ bias,
                                                          int M, int E, int top_k,
                                                          int32_t* __restrict__ ids,
                                                          float* __restrict__ weights) {
  __shared__ double win_key[kTopkWaves][kTopkMaxE];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * kTopkWaves + wave;
  if (t >= M) return;  // wave-uniform; only this wave touches win_key[wave]

  double kv[SLOTS];
  uint32_t taken = 0;
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int e = lane + s * kWave;
    if (e < E) {
      kv[s] = keys[(size_t)t * E + e] + (bias ? (double)bias[e] : 0.0);
    } else {
      kv[s] = 0.0;
      taken |= 1u << s;
    }
  }

  for (int r = 0; r < top_k; ++r) {
    double bk = 0.0;
    int bi = 0x7fffffff;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const int e = lane + s * kWave;  // ascending in s: ties keep the lower id
      if (!((taken >> s) & 1u) && (bi == 0x7fffffff || kv[s] > bk)) {
        bk = kv[s];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const double ok = __shfl_xor(bk, off, kWave);
      const int oi = __shfl_xor(bi, off, kWave);
      const bool other_valid = oi != 0x7fffffff;
      const bool mine_valid = bi != 0x7fffffff;
      if (other_valid && (!mine_valid || ok > bk || (ok == bk && oi < bi))) {
        bk = ok;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == 0) {
      ids[(size_t)t * top_k + r] = bi;
      win_key[wave][r] = bk;
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  // sigmoid of the picks, renormalised; lanes own picks r = lane + 64 q
  double part = 0.0;
  for (int r = lane; r < top_k; r += kWave) part += 1.0 / (1.0 + exp(-win_key[wave][r]));
  const double total = wave_sum(part);
  for (int r = lane; r < top_k; r += kWave) {
    const double s = 1.0 / (1.0 + exp(-win_key[wave][r]));
    weights[(size_t)t * top_k + r] = (float)(s / total);
  }
}

template <int TM, int TEW>
static hipError_t launch_keys(const uint16_t* x, const uint16_t* wr, int M, int H, int E,
                              double* keys, hipStream_t s) {
  dim3 grid((E + 4 * TEW - 1) / (4 * TEW), (M + TM - 1) / TM);
  hipLaunchKernelGGL((router_keys_kernel<TM, TEW>), grid, dim3(256), 0, s, x, wr, M, H, E, keys);
  return hipGetLastError();
}

template <int SLOTS>
static hipError_t launch_topk(const double* keys, const float* bias, int M, int E, int k,
                              int32_t* ids, float* w, hipStream_t s) {
  dim3 grid((M + kTopkWaves - 1) / kTopkWaves);
  hipLaunchKernelGGL((router_topk_kernel<SLOTS>), grid, dim3(256), 0, s, keys, bias, M, E, k, ids, w);
  return hipGetLastError();
}

hipError_t launch_route(const uint16_t* x, const uint16_t* wr, const float* bias, int M, int H,
                        int E, int top_k, int32_t* ids, float* w, double* keys, hipStream_t s) {
  hipError_t err;
  if (M <= 16) err = launch_keys<2, 2>(x, wr, M, H, E, keys, s);
  else if (M <= 128) err = launch_keys<4, 4>(x, wr, M, H, E, keys, s);
  else err = launch_keys<8, 4>(x, wr, M, H, E, keys, s);
  if (err != hipSuccess) return err;
  const int slots = (E + kWave - 1) / kWave;
  if (slots <= 1) return launch_topk<1>(keys, bias, M, E, top_k, ids, w, s);
  if (slots <= 2) return launch_topk<2>(keys, bias, M, E, top_k, ids, w, s);
  if (slots <= 4) return launch_topk<4>(keys, bias, M, E, top_k, ids, w, s);
  if (slots <= 8) return launch_topk<8>(keys, bias, M, E, top_k, ids, w, s);
  return launch_topk<16>(keys, bias, M, E, top_k, ids, w, s);
}

}  // namespace moe
