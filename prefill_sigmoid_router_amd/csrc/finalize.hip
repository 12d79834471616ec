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
#include <type_traits>

#include "device_common.h"
#include "launchers.h"

namespace moe {

constexpr int kFinThreads = 1024;
constexpr int kFinBatch = 8;

// Values 4 c .. 4 c + 3 of a y row as fp32: fp32 rows (moe_finalize) or bf16 rows
// (moe_forward, whose down GEMMs round every pick but a token's first to bf16).
__device__ __forceinline__ float4 y4(const float* row, int c) {
  return reinterpret_cast<const float4*>(row)[c];
}
__device__ __forceinline__ float4 y4(const uint16_t* row, int c) {
  const uint2 v = reinterpret_cast<const uint2*>(row)[c];
  return make_float4(bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y));
}

template <int V, typename Y>
__global__ __launch_bounds__(kFinThreads) void finalize_kernel(
    const Y* __restrict__ y, const float* __restrict__ topk_w,
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

  // picks per batch: 8, or 4 with 4 groups per thread (1024 threads leave 128 registers each;
  // 8 x 4 float4 rows in flight would spill)
  constexpr int NB = V >= 4 ? kFinBatch / 2 : kFinBatch;
  const Y* yt = y + (size_t)t * top_k * H;
  const float* wt = topk_w + (size_t)t * top_k;
  for (int j0 = 0; j0 < top_k; j0 += NB) {
    float4 a[NB][V];
#pragma unroll
    for (int u = 0; u < NB; ++u)
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int c = tid + kFinThreads * v;
        a[u][v] = (j0 + u < top_k && c < ngroups) ? y4(yt + (size_t)(j0 + u) * H, c)
                                                  : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
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

template <int V, typename Y>
static hipError_t launch_fin(const Y* y, const float* w, const uint16_t* res, const uint16_t* g,
                             float eps, int M, int H, int k, uint16_t* out, uint16_t* rout,
                             hipStream_t s) {
  hipLaunchKernelGGL((finalize_kernel<V, Y>), dim3(M), dim3(kFinThreads), 0, s, y, w, res, g, eps,
                     H, k, out, rout);
  return hipGetLastError();
}

// moe_forward's y (each token's first pick in fp32 at row t of y0, the other picks in bf16
// at their rows of y) when H is a multiple of 8: each thread owns V groups of 8 hidden
// values, so every bf16 y request is 16 bytes per lane -- twice the bytes in flight of the
// 4-value groups above for the same number of requests.  Same fp32 arithmetic and
// combine order; the sum of squares is taken over 8-value groups.
template <int V>
__global__ __launch_bounds__(kFinThreads) void finalize_bf16_kernel(
    const uint16_t* __restrict__ y, const float* __restrict__ y0,
    const float* __restrict__ topk_w,
    const uint16_t* __restrict__ residual, const uint16_t* __restrict__ norm_w, float eps, int H,
    int top_k, uint16_t* __restrict__ out, uint16_t* __restrict__ residual_out) {
  __shared__ float part[kFinThreads / kWave];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int ngroups = H >> 3;

  float m[V][8];
#pragma unroll
  for (int v = 0; v < V; ++v)
#pragma unroll
    for (int e = 0; e < 8; ++e) m[v][e] = 0.f;

  // residual, norm weight and the first pick's fp32 row are requested with the first batch
  // of bf16 rows
  const uint4* rr = reinterpret_cast<const uint4*>(residual + (size_t)t * H);
  const uint4* gw = reinterpret_cast<const uint4*>(norm_w);
  const float4* f0 = reinterpret_cast<const float4*>(y0 + (size_t)t * H);
  uint4 res[V], gv[V];
  float4 first[V][2];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int c = tid + kFinThreads * v;
    res[v] = c < ngroups ? rr[c] : uint4{0u, 0u, 0u, 0u};
    gv[v] = c < ngroups ? gw[c] : uint4{0u, 0u, 0u, 0u};
    first[v][0] = c < ngroups ? f0[2 * c] : make_float4(0.f, 0.f, 0.f, 0.f);
    first[v][1] = c < ngroups ? f0[2 * c + 1] : make_float4(0.f, 0.f, 0.f, 0.f);
  }

  const uint16_t* yt = y + (size_t)t * top_k * H;
  const float* wt = topk_w + (size_t)t * top_k;
  {
    const float w = wt[0];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const float f[8] = {first[v][0].x, first[v][0].y, first[v][0].z, first[v][0].w,
                          first[v][1].x, first[v][1].y, first[v][1].z, first[v][1].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) m[v][e] = fmaf(w, f[e], m[v][e]);
    }
  }
  for (int j0 = 1; j0 < top_k; j0 += kFinBatch) {
    uint4 a[kFinBatch][V];
#pragma unroll
    for (int u = 0; u < kFinBatch; ++u)
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int c = tid + kFinThreads * v;
        a[u][v] = (j0 + u < top_k && c < ngroups)
                      ? reinterpret_cast<const uint4*>(yt + (size_t)(j0 + u) * H)[c]
                      : uint4{0u, 0u, 0u, 0u};
      }
#pragma unroll
    for (int u = 0; u < kFinBatch; ++u) {
      if (j0 + u < top_k) {
        const float w = wt[j0 + u];
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const uint32_t q[4] = {a[u][v].x, a[u][v].y, a[u][v].z, a[u][v].w};
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            m[v][2 * h] = fmaf(w, bf16lo(q[h]), m[v][2 * h]);
            m[v][2 * h + 1] = fmaf(w, bf16hi(q[h]), m[v][2 * h + 1]);
          }
        }
      }
    }
  }

  float ss = 0.f;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int c = tid + kFinThreads * v;
    if (c < ngroups) {
      const uint32_t r[4] = {res[v].x, res[v].y, res[v].z, res[v].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        m[v][2 * h] += bf16lo(r[h]);
        m[v][2 * h + 1] += bf16hi(r[h]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(m[v][e], m[v][e], ss);
    }
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  float total = 0.f;
#pragma unroll
  for (int w = 0; w < kFinThreads / kWave; ++w) total += part[w];
  const float inv = 1.0f / sqrtf(total / (float)H + eps);

  uint4* ot = reinterpret_cast<uint4*>(out + (size_t)t * H);
  uint4* rt = residual_out ? reinterpret_cast<uint4*>(residual_out + (size_t)t * H) : nullptr;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int c = tid + kFinThreads * v;
    if (c < ngroups) {
      const uint32_t g[4] = {gv[v].x, gv[v].y, gv[v].z, gv[v].w};
      uint32_t o[4], zr[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        o[h] = pack_bf16x2(m[v][2 * h] * inv * bf16lo(g[h]), m[v][2 * h + 1] * inv * bf16hi(g[h]));
        zr[h] = pack_bf16x2(m[v][2 * h], m[v][2 * h + 1]);
      }
      ot[c] = uint4{o[0], o[1], o[2], o[3]};
      if (rt) rt[c] = uint4{zr[0], zr[1], zr[2], zr[3]};
    }
  }
}

template <int V>
static hipError_t launch_fin_bf16(const uint16_t* y, const float* y0, const float* w,
                                  const uint16_t* res, const uint16_t* g, float eps, int M, int H,
                                  int k, uint16_t* out, uint16_t* rout, hipStream_t s) {
  hipLaunchKernelGGL((finalize_bf16_kernel<V>), dim3(M), dim3(kFinThreads), 0, s, y, y0, w, res,
                     g, eps, H, k, out, rout);
  return hipGetLastError();
}

template <typename Y>
static hipError_t launch_fin_rows(const Y* y, const float* topk_w, const uint16_t* residual,
                                  const uint16_t* norm_w, float eps, int M, int H, int top_k,
                                  uint16_t* out, uint16_t* residual_out, hipStream_t s) {
  const int per_thread = (H / 4 + kFinThreads - 1) / kFinThreads;
  if (per_thread <= 1) return launch_fin<1>(y, topk_w, residual, norm_w, eps, M, H, top_k, out, residual_out, s);
  if (per_thread <= 2) return launch_fin<2>(y, topk_w, residual, norm_w, eps, M, H, top_k, out, residual_out, s);
  return launch_fin<4>(y, topk_w, residual, norm_w, eps, M, H, top_k, out, residual_out, s);
}

hipError_t launch_finalize(const float* y, const float* topk_w, const uint16_t* residual,
                           const uint16_t* norm_w, float eps, int M, int H, int top_k,
                           uint16_t* out, uint16_t* residual_out, hipStream_t s) {
  return launch_fin_rows(y, topk_w, residual, norm_w, eps, M, H, top_k, out, residual_out, s);
}
hipError_t launch_finalize(const uint16_t* y, const float* y0, const float* topk_w,
                           const uint16_t* residual, const uint16_t* norm_w, float eps, int M,
                           int H, int top_k, uint16_t* out, uint16_t* residual_out,
                           hipStream_t s) {
  // every H the API accepts (a multiple of 8, at most 16384) fits one of the two
  if (H % 8 != 0 || H / 8 > 2 * kFinThreads) return hipErrorInvalidValue;
  if (H / 8 <= kFinThreads)
    return launch_fin_bf16<1>(y, y0, topk_w, residual, norm_w, eps, M, H, top_k, out,
                              residual_out, s);
  return launch_fin_bf16<2>(y, y0, topk_w, residual, norm_w, eps, M, H, top_k, out,
                            residual_out, s);
}


// Few tokens (fewer than CUs): one workgroup per token would read k rows of y through a
// single CU.  Instead, kernel 1 splits every row into slices of 1024 values over
// (slice, token) workgroups -- z = combine + residual for the slice, its sum of squares
// per slice -- and kernel 2 adds a token's slice sums in slice order and scales its z.
// Same fp32 arithmetic as finalize_kernel; only the order of the sum of squares differs.
constexpr int kFinSliceThreads = 256;
constexpr int kFinSlice = 4 * kFinSliceThreads;     // hidden values per slice

// Y = uint16_t: moe_forward's y, each token's first pick in fp32 at row t of y0, the others
// in bf16; Y = float: every pick in fp32 in y (y0 unused).
template <typename Y>
__global__ __launch_bounds__(kFinSliceThreads) void finalize_slice_kernel(
    const Y* __restrict__ y, const float* __restrict__ y0, const float* __restrict__ topk_w,
    const uint16_t* __restrict__ residual, int H, int top_k, float* __restrict__ z,
    float* __restrict__ slice_ss) {
  __shared__ float part[kFinSliceThreads / kWave];
  const int sl = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
  const int c = sl * kFinSliceThreads + tid;          // group of 4 hidden values
  const bool in = c < (H >> 2);
  const Y* yt = y + (size_t)t * top_k * H;
  const float* wt = topk_w + (size_t)t * top_k;
  float4 m = make_float4(0.f, 0.f, 0.f, 0.f);
  uint2 r = uint2{0u, 0u};
  if (in) r = reinterpret_cast<const uint2*>(residual + (size_t)t * H)[c];
  for (int j0 = 0; j0 < top_k; j0 += 16) {
    float4 a[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const bool split_first = std::is_same<Y, uint16_t>::value && u == 0 && j0 == 0;
      a[u] = !(in && j0 + u < top_k) ? make_float4(0.f, 0.f, 0.f, 0.f)
             : split_first ? reinterpret_cast<const float4*>(y0 + (size_t)t * H)[c]
                           : y4(yt + (size_t)(j0 + u) * H, c);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (j0 + u < top_k) {
        const float w = wt[j0 + u];
        m.x = fmaf(w, a[u].x, m.x);
        m.y = fmaf(w, a[u].y, m.y);
        m.z = fmaf(w, a[u].z, m.z);
        m.w = fmaf(w, a[u].w, m.w);
      }
    }
  }
  m.x += bf16lo(r.x);
  m.y += bf16hi(r.x);
  m.z += bf16lo(r.y);
  m.w += bf16hi(r.y);
  float ss = 0.f;
  if (in) {
    ss = fmaf(m.x, m.x, ss);
    ss = fmaf(m.y, m.y, ss);
    ss = fmaf(m.z, m.z, ss);
    ss = fmaf(m.w, m.w, ss);
    reinterpret_cast<float4*>(z + (size_t)t * H)[c] = m;
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  if (tid == 0) {
    float total = 0.f;
#pragma unroll
    for (int w = 0; w < kFinSliceThreads / kWave; ++w) total += part[w];
    slice_ss[(size_t)t * gridDim.x + sl] = total;
  }
}

__global__ __launch_bounds__(kFinSliceThreads) void finalize_scale_kernel(
    const float* __restrict__ z, const float* __restrict__ slice_ss,
    const uint16_t* __restrict__ norm_w, float eps, int H, uint16_t* __restrict__ out,
    uint16_t* __restrict__ residual_out) {
  const int sl = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
  const int c = sl * kFinSliceThreads + tid;
  if (c >= (H >> 2)) return;
  float total = 0.f;
  for (int s = 0; s < (int)gridDim.x; ++s) total += slice_ss[(size_t)t * gridDim.x + s];
  const float inv = 1.0f / sqrtf(total / (float)H + eps);
  const float4 m = reinterpret_cast<const float4*>(z + (size_t)t * H)[c];
  const uint2 g = reinterpret_cast<const uint2*>(norm_w)[c];
  uint2 o;
  o.x = pack_bf16x2(m.x * inv * bf16lo(g.x), m.y * inv * bf16hi(g.x));
  o.y = pack_bf16x2(m.z * inv * bf16lo(g.y), m.w * inv * bf16hi(g.y));
  reinterpret_cast<uint2*>(out + (size_t)t * H)[c] = o;
  if (residual_out) {
    uint2 zr;
    zr.x = pack_bf16x2(m.x, m.y);
    zr.y = pack_bf16x2(m.z, m.w);
    reinterpret_cast<uint2*>(residual_out + (size_t)t * H)[c] = zr;
  }
}

size_t finalize_slices_scratch_bytes(int M, int H) {
  const int slices = (H / 4 + kFinSliceThreads - 1) / kFinSliceThreads;
  return (size_t)M * H * sizeof(float) + (size_t)M * slices * sizeof(float);
}

template <typename Y>
static hipError_t launch_fin_slices(const Y* y, const float* y0, const float* topk_w,
                                    const uint16_t* residual, const uint16_t* norm_w, float eps,
                                    int M, int H, int top_k, uint16_t* out, uint16_t* residual_out,
                                    float* scratch, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int slices = (H / 4 + kFinSliceThreads - 1) / kFinSliceThreads;
  float* z = scratch;
  float* slice_ss = scratch + (size_t)M * H;
  hipLaunchKernelGGL((finalize_slice_kernel<Y>), dim3(slices, M), dim3(kFinSliceThreads), 0, s, y,
                     y0, topk_w, residual, H, top_k, z, slice_ss);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(finalize_scale_kernel, dim3(slices, M), dim3(kFinSliceThreads), 0, s, z,
                     slice_ss, norm_w, eps, H, out, residual_out);
  return hipGetLastError();
}

hipError_t launch_finalize_slices(const float* y, const float* topk_w, const uint16_t* residual,
                                  const uint16_t* norm_w, float eps, int M, int H, int top_k,
                                  uint16_t* out, uint16_t* residual_out, float* scratch,
                                  hipStream_t s) {
  return launch_fin_slices(y, nullptr, topk_w, residual, norm_w, eps, M, H, top_k, out,
                           residual_out, scratch, s);
}
hipError_t launch_finalize_slices(const uint16_t* y, const float* y0, const float* topk_w,
                                  const uint16_t* residual, const uint16_t* norm_w, float eps,
                                  int M, int H, int top_k, uint16_t* out, uint16_t* residual_out,
                                  float* scratch, hipStream_t s) {
  return launch_fin_slices(y, y0, topk_w, residual, norm_w, eps, M, H, top_k, out, residual_out,
                           scratch, s);
}

}  // namespace moe
