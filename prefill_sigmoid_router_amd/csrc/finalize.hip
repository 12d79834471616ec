// Finalize step of the routed-MoE layer: weighted top-k combine, residual add, RMSNorm.
//
// FlashInfer PR #5701 analysis ("Kimi K3 H7168/K16 MNNVL CuTe DSL"), intro and section 3:
// the MoE finalize (combine of the top-k expert rows) is fused with the residual path
// and RMSNorm, with RMS_EPS = 1e-5 and WEIGHT_BIAS = 0 (weight used as is); section 2: a
// 7168-wide bf16 row is 896 packs of 16 bytes.  FlashInfer PR #4690 analysis
// ("MiniMax-H3 BF16 pre-attention"), section 1: RMSNorm = torch rms_norm over the hidden
// dim, eps inside the square root.  sglang PR #29509 analysis, "why it's good" 1:
// RMSNorm is memory-bound, so it is fused with its producer's consumer here.
//
// One workgroup of 1024 threads per token; each thread owns V groups of 4 hidden values,
// so z stays in registers between the sum of squares and the scaling.  The y rows of 8
// picks are requested together (all V groups), with the residual and norm weight in the
// first batch, so a token costs about k/8 memory round trips rather than k + 2.  All arithmetic is fp32 with a single bf16 rounding (RNE) at the
// store; the combine adds the picks in ascending j.
#include "device_common.h"
#include "launchers.h"

namespace moe {

constexpr int kFinThreads = 1024;
constexpr int kFinBatch = 8;

template <int V>
__global__ __launch_bounds__(kFinThreads) void finalize_kernel(
    const float* __restrict__ y, const float* __restrict__ topk_w,
    const uint16_t* __restrict__ residual, const uint16_t* __restrict__ norm_w, float eps, int H,
    int top_k, uint16_t* __restrict__ out, uint16_t* __restrict__ residual_out) {
  __shared__ float part[kFinThreads / kWave];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int ngroups = H >> 2;

  float4 m[V];
#pragma unroll
  for (int v = 0; v < V; ++v) m[v] = make_float4(0.f, 0.f, 0.f, 0.f);

  // residual and norm weight are requested with the first batch of y rows, so a token
  // costs ceil(k / 8) memory round trips in all
  const uint2* rr = reinterpret_cast<const uint2*>(residual + (size_t)t * H);
  const uint2* gw = reinterpret_cast<const uint2*>(norm_w);
  uint2 res[V], gv[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int c = tid + kFinThreads * v;
    res[v] = c < ngroups ? rr[c] : uint2{0u, 0u};
    gv[v] = c < ngroups ? gw[c] : uint2{0u, 0u};
  }

  const float* yt = y + (size_t)t * top_k * H;
  const float* wt = topk_w + (size_t)t * top_k;
  for (int j0 = 0; j0 < top_k; j0 += kFinBatch) {
    float4 a[kFinBatch][V];
#pragma unroll
    for (int u = 0; u < kFinBatch; ++u)
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int c = tid + kFinThreads * v;
        a[u][v] = (j0 + u < top_k && c < ngroups)
                      ? reinterpret_cast<const float4*>(yt + (size_t)(j0 + u) * H)[c]
                      : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
    for (int u = 0; u < kFinBatch; ++u) {
      if (j0 + u < top_k) {
        const float w = wt[j0 + u];
#pragma unroll
        for (int v = 0; v < V; ++v) {
          m[v].x = fmaf(w, a[u][v].x, m[v].x);
          m[v].y = fmaf(w, a[u][v].y, m[v].y);
          m[v].z = fmaf(w, a[u][v].z, m[v].z);
          m[v].w = fmaf(w, a[u][v].w, m[v].w);
        }
      }
    }
  }

  float ss = 0.f;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int c = tid + kFinThreads * v;
    if (c < ngroups) {
      const uint2 r = res[v];
      m[v].x += bf16lo(r.x);
      m[v].y += bf16hi(r.x);
      m[v].z += bf16lo(r.y);
      m[v].w += bf16hi(r.y);
      ss = fmaf(m[v].x, m[v].x, ss);
      ss = fmaf(m[v].y, m[v].y, ss);
      ss = fmaf(m[v].z, m[v].z, ss);
      ss = fmaf(m[v].w, m[v].w, ss);
    }
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  float total = 0.f;
#pragma unroll
  for (int w = 0; w < kFinThreads / kWave; ++w) total += part[w];
  const float inv = 1.0f / sqrtf(total / (float)H + eps);

  uint2* ot = reinterpret_cast<uint2*>(out + (size_t)t * H);
  uint2* rt = residual_out ? reinterpret_cast<uint2*>(residual_out + (size_t)t * H) : nullptr;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int c = tid + kFinThreads * v;
    if (c < ngroups) {
      const uint2 g = gv[v];
      uint2 o;
      o.x = pack_bf16x2(m[v].x * inv * bf16lo(g.x), m[v].y * inv * bf16hi(g.x));
      o.y = pack_bf16x2(m[v].z * inv * bf16lo(g.y), m[v].w * inv * bf16hi(g.y));
      ot[c] = o;
      if (rt) {
        uint2 zr;
        zr.x = pack_bf16x2(m[v].x, m[v].y);
        zr.y = pack_bf16x2(m[v].z, m[v].w);
        rt[c] = zr;
      }
    }
  }
}

template <int V>
static hipError_t launch_fin(const float* y, const float* w, const uint16_t* res, const uint16_t* g,
                             float eps, int M, int H, int k, uint16_t* out, uint16_t* rout,
                             hipStream_t s) {
  hipLaunchKernelGGL((finalize_kernel<V>), dim3(M), dim3(kFinThreads), 0, s, y, w, res, g, eps, H, k,
                     out, rout);
  return hipGetLastError();
}

hipError_t launch_finalize(const float* y, const float* topk_w, const uint16_t* residual,
                           const uint16_t* norm_w, float eps, int M, int H, int top_k,
                           uint16_t* out, uint16_t* residual_out, hipStream_t s) {
  const int per_thread = (H / 4 + kFinThreads - 1) / kFinThreads;
  if (per_thread <= 1) return launch_fin<1>(y, topk_w, residual, norm_w, eps, M, H, top_k, out, residual_out, s);
  if (per_thread <= 2) return launch_fin<2>(y, topk_w, residual, norm_w, eps, M, H, top_k, out, residual_out, s);
  return launch_fin<4>(y, topk_w, residual, norm_w, eps, M, H, top_k, out, residual_out, s);
}

}  // namespace moe
