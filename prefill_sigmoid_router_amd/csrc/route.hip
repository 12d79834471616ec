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
#include <algorithm>

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
// Tokens from which the certified path (below) replaces the all-fp64 keys: from about
// 256 tokens its fp32 MFMA logits plus a few fp64 recomputes per token cost less than
// fp64 dot products for every (token, expert) pair.
#ifndef MOE_ROUTE_CERTIFIED_MIN
#define MOE_ROUTE_CERTIFIED_MIN 256
#endif
constexpr int kRouteCertifiedMinTokens = MOE_ROUTE_CERTIFIED_MIN;
constexpr int kSelChunks = 8;       // 16-byte chunks per lane in flight per candidate batch

// Number of entries of vals[0..n) ahead of (v, id): larger, or equal with a lower index.
// Eight LDS values are requested per step so the loop is not bound by LDS latency.
template <int SL>
__device__ __forceinline__ void count_ahead(const double* vals, int n, const double (&v)[SL],
                                            const int (&id)[SL], int (&rank)[SL]) {
#pragma unroll
  for (int s = 0; s < SL; ++s) rank[s] = 0;
  int j = 0;
  for (; j + 8 <= n; j += 8) {
    double b[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) b[u] = vals[j + u];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int s = 0; s < SL; ++s) rank[s] += (b[u] > v[s] || (b[u] == v[s] && j + u < id[s])) ? 1 : 0;
  }
  for (; j < n; ++j) {
    const double b = vals[j];
#pragma unroll
    for (int s = 0; s < SL; ++s) rank[s] += (b > v[s] || (b == v[s] && j < id[s])) ? 1 : 0;
  }
}

// Order-preserving 32-bit key of a lower bound lo of expert e: lo rounded toward -inf to
// fp32, mapped to an unsigned integer that orders like the value, its low 10 bits replaced
// by 1023 - e (keys are unique; equal truncated values order by ascending id).  Clearing
// those bits can only lower the value, and the k-th largest key decodes (key_floor) to a
// value at or below the k-th largest lo: a valid, slightly lower threshold for the
// candidate filter, found with integer compares instead of fp64 ones.
__device__ __forceinline__ uint32_t lo_key(double lo, int e) {
  const uint32_t b = __float_as_uint(__double2float_rd(lo));
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (ord & ~0x3FFu) | (uint32_t)(1023 - e);
}
__device__ __forceinline__ double key_floor(uint32_t key) {
  const uint32_t ord = key & ~0x3FFu;
  const uint32_t b = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
  const float f = __uint_as_float(b);
  return isfinite(f) ? (double)f : -INFINITY;   // non-finite bounds: every expert is a candidate
}

// rank[s] = number of keys in vals[0, n) greater than v[s] (sixteen LDS values per step)
template <int SL>
__device__ __forceinline__ void count_greater(const uint32_t* vals, int n, const uint32_t (&v)[SL],
                                              int (&rank)[SL]) {
#pragma unroll
  for (int s = 0; s < SL; ++s) rank[s] = 0;
  int j = 0;
  for (; j + 16 <= n; j += 16) {
    uint4 b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) b[u] = reinterpret_cast<const uint4*>(vals + j)[u];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int s = 0; s < SL; ++s)
        rank[s] += (b[u].x > v[s]) + (b[u].y > v[s]) + (b[u].z > v[s]) + (b[u].w > v[s]);
  }
  for (; j < n; ++j)
#pragma unroll
    for (int s = 0; s < SL; ++s) rank[s] += vals[j] > v[s] ? 1 : 0;
}

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
  int rank[SL], myid[SL];
#pragma unroll
  for (int s = 0; s < SL; ++s) myid[s] = tid + kTopkThreads * s;
  count_ahead<SL>(sk, E, mine, myid, rank);
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

// ---------------------------------------------------------------------------------------
// Certified fast path for many tokens.
//
// 1. router_logits_mfma_kernel: fp32 logits L = x . Wr^T on bf16 MFMA, together with
//    A = sum_h |x_h| |w_h| from the same fragments with the sign bits cleared, over P
//    contiguous parts of K (one partial result per part).  Products of two bf16 values
//    are exact in fp32, so the only error is the fp32 summation: a product passes at most
//    31 roundings inside its MFMA and one per later 32-wide K step of its part, n =
//    32 + ceil(Kpart / 32) in all.  With each rounding off by at most 2u (u = 2^-24, even
//    if the hardware truncates), |L_p - exact_p| <= n 2u A_p (1 + 2^-10) for n <= 1024,
//    and the computed A_p is within a factor (1 + 2^-10) of A_p.  The parts are added in
//    fp64.
// 2. router_select_kernel, one workgroup per token: with d = n 2^-23 A (1 + 2^-9) plus an
//    absolute floor for flushed subnormal products and the fp64 key rounding, lo = L + b
//    - d and hi = L + b + d, T at or below the k-th largest lo (found on 32-bit keys, see
//    lo_key).  An expert with hi < T has an exact key below at least k other exact keys,
//    so it cannot be picked; every other expert is a candidate.  The candidates' keys are recomputed as fp64 dot products and ranked
//    exactly as the fp64 path ranks them (key descending, ties to the lower id).
// ---------------------------------------------------------------------------------------
constexpr int kLgTokens = 32;               // tokens per workgroup
constexpr int kLgExperts = 64;              // experts per workgroup
constexpr int kLgKC = 64;                   // K values per chunk: one 128-byte line per row
constexpr int kLgStages = 4;
constexpr int kLgCopies = (kLgTokens + kLgExperts) / 8;   // 1 KiB copies per chunk
constexpr int kLgCPW = kLgCopies / 4;                     // per wave
constexpr int kLgMaxParts = 4;
static_assert(2 * kLgMaxParts * sizeof(float) <= kRouteScratchPerPair &&
              sizeof(double) <= kRouteScratchPerPair, "router scratch per (token, expert)");

template <int N>
__device__ __forceinline__ void lg_wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One workgroup per 64 experts x 32 tokens x one part of K.  The 96 rows of a 64-wide K
// chunk (experts first, then tokens) are copied global -> LDS with global_load_lds_dwordx4,
// 8 rows x one 128-byte line per copy, the 16-byte K chunks of a row XOR-swizzled
// (slot = chunk ^ row % 8 ^ (row / 8) % 2) so every MFMA fragment is one conflict-free
// ds_read_b128; a 4-chunk ring keeps 3 chunks in flight.  Wave w computes 16 tokens
// (half w % 2) x 32 experts (half w / 2).
__global__ __launch_bounds__(256) void router_logits_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int M, int H, int E,
    int kpart, float* __restrict__ logits, float* __restrict__ absdot) {
  __shared__ __align__(16) unsigned char lds[kLgStages * kLgCopies * 1024];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int e0 = blockIdx.x * kLgExperts;
  const int t0 = blockIdx.y * kLgTokens;
  const int part = blockIdx.z;
  const int kbeg = min(H, part * kpart), kend = min(H, kbeg + kpart);
  const int klen = kend - kbeg;

  const uint16_t* src[kLgCPW];
  bool on[kLgCPW];
  int qk[kLgCPW];
#pragma unroll
  for (int i = 0; i < kLgCPW; ++i) {
    const int f = wave * kLgCPW + i;
    const int r = 8 * f + (lane >> 3);
    qk[i] = (lane & 7) ^ (lane >> 3) ^ (f & 1);
    const uint16_t* row;
    if (r < kLgExperts) {
      on[i] = e0 + r < E;
      row = wr + (size_t)(on[i] ? e0 + r : 0) * H;
    } else {
      on[i] = t0 + r - kLgExperts < M;
      row = x + (size_t)(on[i] ? t0 + r - kLgExperts : 0) * H;
    }
    src[i] = row + kbeg + 8 * qk[i];
  }
  const int nch = (klen + kLgKC - 1) / kLgKC;
  const int ndma = klen / kLgKC;
  auto issue = [&](int c) {
    unsigned char* base = lds + (size_t)(c % kLgStages) * kLgCopies * 1024;
    if (c < ndma) {
#pragma unroll
      for (int i = 0; i < kLgCPW; ++i)
        __builtin_amdgcn_global_load_lds(
            (__attribute__((address_space(1))) void*)(src[i] + c * kLgKC),
            (__attribute__((address_space(3))) void*)(base + (wave * kLgCPW + i) * 1024), 16, 0, 0);
    } else {  // partial chunk: zero-filled through registers
#pragma unroll
      for (int i = 0; i < kLgCPW; ++i) {
        const int k = kbeg + c * kLgKC + 8 * qk[i];
        const u32x4 v = (on[i] && k + 8 <= kend) ? ld16(src[i] + c * kLgKC) : u32x4{0, 0, 0, 0};
        *reinterpret_cast<u32x4*>(base + (size_t)(wave * kLgCPW + i) * 1024 + lane * 16) = v;
      }
    }
  };
  const int frag_off = (li >> 3) * 1024 + (li & 7) * 128;
  auto frag = [&](int c, int t, int ks) -> u32x4 {
    const int q = (lg + 4 * ks) ^ (li & 7) ^ (li >> 3);
    return *reinterpret_cast<const u32x4*>(lds + (size_t)(c % kLgStages) * kLgCopies * 1024 +
                                           t * 2048 + frag_off + q * 16);
  };

  const u32x4 absmask = u32x4{0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu};
  const int ttile = kLgExperts / 16 + (wave & 1);   // token row tile in the stage
  const int etile = 2 * (wave >> 1);                // first of two expert row tiles
  f32x4 acc[2], aab[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) acc[j] = aab[j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int p = 0; p < kLgStages - 1; ++p)
    if (p < nch) issue(p);
  for (int c = 0; c < nch; ++c) {
    // this wave's whole chunks issued after c: min(2, ndma-1-c)
    const int after = c < ndma ? min(kLgStages - 2, ndma - 1 - c) : 0;
    if (after >= 2) lg_wait_vmcnt<2 * kLgCPW>();
    else if (after == 1) lg_wait_vmcnt<kLgCPW>();
    else lg_wait_vmcnt<0>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (c + kLgStages - 1 < nch) issue(c + kLgStages - 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4 xb = frag(c, ttile, ks);
      const u32x4 xa = xb & absmask;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 wa = frag(c, etile + j, ks);
        acc[j] = mfma16x16x32(wa, xb, acc[j]);
        aab[j] = mfma16x16x32(wa & absmask, xa, aab[j]);
      }
    }
  }
  // D rows 4*lg+q = experts of tile etile+j, column li = token
  const int t = t0 + 16 * (wave & 1) + li;
  if (t < M) {
    float* lrow = logits + ((size_t)part * M + t) * E;
    float* arow = absdot + ((size_t)part * M + t) * E;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = e0 + 16 * (etile + j) + 4 * lg;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (e + q < E) {
          lrow[e + q] = acc[j][q];
          arow[e + q] = aab[j][q];
        }
      }
    }
  }
}

template <int SL>
// At most 128 registers for E <= 512 (four workgroups per CU instead of three: the fp64
// recompute of the candidates is bound by L2 latency; measured at M=2048: 118 -> 110 us).
__global__ __launch_bounds__(kTopkThreads)
__attribute__((amdgpu_waves_per_eu(SL <= 2 ? 4 : 1))) void router_select_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, const float* __restrict__ bias,
    const float* __restrict__ logits, const float* __restrict__ absdot, int parts, int nround,
    int M, int H, int E, int top_k, int32_t* __restrict__ ids, float* __restrict__ weights) {
  // LDS sized by the launch: the token's x row, then per expert the lower bound, the
  // candidates' fp64 keys and ids, and the picks' sigmoids
  extern __shared__ __align__(16) unsigned char sel_lds[];
  u32x4* s_x = reinterpret_cast<u32x4*>(sel_lds);
  double* s_lo = reinterpret_cast<double*>(sel_lds + (size_t)H * 2);
  double* s_key = s_lo + E;     // fp64 keys of the candidates, by candidate slot
  double* s_sig = s_key + E;
  int* s_cand = reinterpret_cast<int*>(s_sig + E);   // expert id of each candidate slot
  __shared__ int s_wave_cnt[kTopkThreads / kWave];
  __shared__ double s_T;
  const int t = blockIdx.x, tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  for (int ch = tid; ch < (H >> 3); ch += kTopkThreads) s_x[ch] = ld16(x + (size_t)t * H + (size_t)ch * 8);

  const double rel = (double)nround * 0x1p-23 * (1.0 + 0x1p-9);
  uint32_t* s_k32 = reinterpret_cast<uint32_t*>(s_lo);   // 32-bit keys of the lower bounds
  double lo[SL], hi[SL];
  uint32_t mykey[SL];
#pragma unroll
  for (int s = 0; s < SL; ++s) {
    const int e = tid + kTopkThreads * s;
    lo[s] = hi[s] = 0.0;
    if (e < E) {
      double l = 0.0, a = 0.0;
      for (int p = 0; p < parts; ++p) {
        l += (double)logits[((size_t)p * M + t) * E + e];
        a += (double)absdot[((size_t)p * M + t) * E + e];
      }
      const double key = l + (bias ? (double)bias[e] : 0.0);
      const double d = a * rel + fabs(key) * 0x1p-50 + (double)H * 0x1p-126 + 1e-300;
      lo[s] = key - d;
      hi[s] = key + d;
    }
    mykey[s] = lo_key(lo[s], e);
    if (e < E) s_k32[e] = mykey[s];
  }
  __syncthreads();
  // T = the decoded top_k-th largest key: at or below the top_k-th largest lower bound
  int rank[SL];
  count_greater<SL>(s_k32, E, mykey, rank);
#pragma unroll
  for (int s = 0; s < SL; ++s)
    if (tid + kTopkThreads * s < E && rank[s] == top_k - 1) s_T = key_floor(mykey[s]);
  __syncthreads();
  const double T = s_T;

  // compact the candidates (hi >= T) in ascending expert order
  int ncand = 0;
#pragma unroll
  for (int s = 0; s < SL; ++s) {
    const int e = tid + kTopkThreads * s;
    const bool cand = e < E && hi[s] >= T;
    const uint64_t m = __ballot(cand);
    if (lane == 0) s_wave_cnt[wave] = __popcll(m);
    __syncthreads();
    int before = ncand;
    for (int w = 0; w < kTopkThreads / kWave; ++w) {
      if (w < wave) before += s_wave_cnt[w];
      ncand += s_wave_cnt[w];
    }
    if (cand) s_cand[before + __popcll(m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))))] = e;
    __syncthreads();
  }

  // fp64 keys of the candidates: wave w takes candidates w, w+4, ...; lane l takes the
  // 16-byte chunks l, l+64, ... of H (x from LDS).  A candidate's chunks are requested
  // together (kSelChunks per lane at a time) and the next candidate's first batch is in
  // flight while this one is summed; xor-butterfly reduction per candidate.
  const int nchunk = H >> 3;
  const int nwaves = kTopkThreads / kWave;
  u32x4 wv[2][kSelChunks];
  auto fetch = [&](int c, u32x4 (&dst)[kSelChunks], int base) {
    const uint16_t* wrow = wr + (size_t)s_cand[c] * H;
#pragma unroll
    for (int u = 0; u < kSelChunks; ++u) {
      const int ch = base + lane + u * kWave;
      dst[u] = ch < nchunk ? ld16(wrow + (size_t)ch * 8) : u32x4{0, 0, 0, 0};
    }
  };
  auto dot = [&](const u32x4 (&src)[kSelChunks], int base, double acc) {
#pragma unroll
    for (int u = 0; u < kSelChunks; ++u) {
      const int ch = base + lane + u * kWave;
      if (ch < nchunk) {
        const u32x4 xv = s_x[ch];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc = fma((double)bf16lo(xv[q]), (double)bf16lo(src[u][q]), acc);
          acc = fma((double)bf16hi(xv[q]), (double)bf16hi(src[u][q]), acc);
        }
      }
    }
    return acc;
  };
  if (wave < ncand) fetch(wave, wv[0], 0);
  for (int c = wave, it = 0; c < ncand; c += nwaves, ++it) {
    double acc = 0.0;
    for (int base = 0; base < nchunk; base += kSelChunks * kWave) {
      // batch (c, base) sits in wv[it & 1] ... keep the stage index static by branching
      const bool last_batch = base + kSelChunks * kWave >= nchunk;
      const int next_c = last_batch ? c + nwaves : c;
      const int next_base = last_batch ? 0 : base + kSelChunks * kWave;
      if ((it & 1) == 0) {
        if (next_c < ncand) fetch(next_c, wv[1], next_base);
        acc = dot(wv[0], base, acc);
      } else {
        if (next_c < ncand) fetch(next_c, wv[0], next_base);
        acc = dot(wv[1], base, acc);
      }
      it += last_batch ? 0 : 1;
    }
    acc = wave_sum(acc);
    if (lane == 0) s_key[c] = acc + (bias ? (double)bias[s_cand[c]] : 0.0);
  }
  __syncthreads();

  // rank the candidates exactly: key descending, ties to the lower id
  for (int c = tid; c < ncand; c += kTopkThreads) {
    const double kc = s_key[c];
    const int ec = s_cand[c];
    int r = 0;
    for (int j = 0; j < ncand; ++j) {
      const double kj = s_key[j];
      r += (kj > kc || (kj == kc && s_cand[j] < ec)) ? 1 : 0;
    }
    if (r < top_k) {
      ids[(size_t)t * top_k + r] = ec;
      s_sig[r] = 1.0 / (1.0 + exp(-kc));
    }
  }
  __syncthreads();
  if (tid < kWave) {
    double part = 0.0;
    for (int r = tid; r < top_k; r += kWave) part += s_sig[r];
    const double total = wave_sum(part);
    for (int r = tid; r < top_k; r += kWave)
      weights[(size_t)t * top_k + r] = (float)(s_sig[r] / total);
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
  const int per_thread = (E + kTopkThreads - 1) / kTopkThreads;
  if (M >= kRouteCertifiedMinTokens) {
    // K is cut into parts (whole 64-wide chunks) so that about 512 workgroups run; the
    // workspace holds parts x [M, E] fp32 logits, then parts x [M, E] fp32 |x|.|w|
    const int base = ((E + kLgExperts - 1) / kLgExperts) * ((M + kLgTokens - 1) / kLgTokens);
    const int parts = std::min(kLgMaxParts, std::max(1, (512 + base - 1) / base));
    const int chunks = (H + kLgKC - 1) / kLgKC;
    const int kpart = ((chunks + parts - 1) / parts) * kLgKC;
    const int nround = 32 + (kpart + 31) / 32;
    float* logits = reinterpret_cast<float*>(keys);
    float* absdot = logits + (size_t)parts * M * E;
    hipLaunchKernelGGL(router_logits_mfma_kernel,
                       dim3((E + kLgExperts - 1) / kLgExperts, (M + kLgTokens - 1) / kLgTokens, parts),
                       dim3(256), 0, s, x, wr, M, H, E, kpart, logits, absdot);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const size_t lds = (size_t)H * 2 + (size_t)E * (3 * sizeof(double) + sizeof(int));
#define MOE_SELECT(SLV)                                                                     \
  hipLaunchKernelGGL((router_select_kernel<SLV>), dim3(M), dim3(kTopkThreads), lds, s, x, wr, \
                     bias, logits, absdot, parts, nround, M, H, E, top_k, ids, w)
    if (per_thread <= 1) MOE_SELECT(1);
    else if (per_thread <= 2) MOE_SELECT(2);
    else MOE_SELECT(4);
#undef MOE_SELECT
    return hipGetLastError();
  }
  if (M <= 16) err = launch_keys<2, 4, 4>(x, wr, M, H, E, keys, s);
  else err = launch_keys<4, 4, 2>(x, wr, M, H, E, keys, s);
  if (err != hipSuccess) return err;
  if (per_thread <= 1) return launch_topk<1>(keys, bias, M, E, top_k, ids, w, s);
  if (per_thread <= 2) return launch_topk<2>(keys, bias, M, E, top_k, ids, w, s);
  return launch_topk<4>(keys, bias, M, E, top_k, ids, w, s);
}

}  // namespace moe
