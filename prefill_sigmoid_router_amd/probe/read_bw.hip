// Achievable HBM read bandwidth on this device, the measured ceiling the layer's
// weight-streaming kernels are compared with next to the 8 TB/s vendor figure.  Not part
// of the layer: a separate library (libmoe_probe.so) that only the benchmark loads.
//
// One fully coalesced pass over a buffer: each wave instruction reads 1 KiB contiguous,
// 8 loads in flight per lane, grid-stride over the buffer, loads marked nontemporal (the
// data is read once: 6.95 TB/s on MI355X against 6.26 TB/s with ordinary loads); the
// loaded words are folded with xor into one word per workgroup so the loads cannot be
// dropped.
//
// A second pass reads the W13 stack [E, 2I, K] the way the tiled up GEMMs stream it:
// whole 128-byte lines copied global -> LDS with nontemporal global_load_lds_dwordx4 (each
// copy 8 rows x one line), items of 256 rows (128 gate + 128 up; 32 KiB per chunk of 64 K
// values) or 128 rows (16 KiB per chunk), a ring of 3 to 5 chunks, 4-wave workgroups (one
// per CU with 256-row items, two or three with 128-row items) walking their XCD's share of
// the (expert, N tile) items.  Each wave waits for its own copies and a bare barrier
// publishes the chunk; every lane then folds one 16-byte LDS word per copy into its xor.
// It is the rate of that copy path with no arithmetic behind it.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
constexpr int kThreads = 256;
constexpr int kInFlight = 8;

__global__ __launch_bounds__(kThreads) void read_pass_kernel(const u32x4* __restrict__ p,
                                                             size_t n16, uint32_t* __restrict__ sink) {
  __shared__ uint32_t red[kThreads];
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * kThreads * kInFlight;
  for (size_t i = (size_t)blockIdx.x * kThreads * kInFlight + threadIdx.x; i < n16; i += stride) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const size_t j = i + (size_t)u * kThreads;
      v[u] = j < n16 ? __builtin_nontemporal_load(p + j) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

typedef __attribute__((address_space(1))) void global_void;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kLdsKC = 64;                     // K values per chunk: one line per row
constexpr int kLdsWaves = 4;

template <int N>
__device__ __forceinline__ void probe_wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int kLdsStages, int kLdsRows>
__global__ __launch_bounds__(64 * kLdsWaves) void read_lds_ring_kernel(
    const uint16_t* __restrict__ m, int E, int I, int K, uint32_t* __restrict__ sink) {
  constexpr int kLdsCopies = kLdsRows / 8;       // 1 KiB copies per chunk
  constexpr int kLdsCPW = kLdsCopies / kLdsWaves;
  __shared__ __align__(16) unsigned char lds[kLdsStages * kLdsCopies * 1024];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // items (expert e, N tile nt): rows nt*128 .. +127 of the first half of e's 2I rows and the
  // same rows of the second half; each XCD (workgroup p runs on XCD p % 8) takes a
  // contiguous share, N tile by N tile, like the tiled up GEMM's walk
  const int n_nt = I / (kLdsRows / 2);
  const int items = E * n_nt;
  const int per_xcd = (items + 7) / 8;
  const int first = (blockIdx.x % 8) * per_xcd;
  const int stride = gridDim.x / 8;
  const int nch = K / kLdsKC;
  uint32_t acc = 0;
  for (int slot = blockIdx.x / 8; slot < per_xcd && first + slot < items; slot += stride) {
    const int logical = first + slot;
    const int nt = logical / E, e = logical % E;
    const uint16_t* src[kLdsCPW];
#pragma unroll
    for (int i = 0; i < kLdsCPW; ++i) {
      const int f = wave * kLdsCPW + i;
      const int r = 8 * f + (lane >> 3);            // 0..255
      const int row = (r < kLdsRows / 2) ? nt * (kLdsRows / 2) + r : I + nt * (kLdsRows / 2) + r - kLdsRows / 2;
      src[i] = m + ((size_t)e * 2 * I + row) * K + 8 * (lane & 7);
    }
    auto issue = [&](int c) {
      unsigned char* base = lds + (size_t)(c % kLdsStages) * kLdsCopies * 1024;
#pragma unroll
      for (int i = 0; i < kLdsCPW; ++i)
        __builtin_amdgcn_global_load_lds((global_void*)(src[i] + c * kLdsKC),
                                         (lds_void*)(base + (wave * kLdsCPW + i) * 1024), 16, 0, 2);
    };
#pragma unroll
    for (int p = 0; p < kLdsStages - 1; ++p)
      if (p < nch) issue(p);
    for (int c = 0; c < nch; ++c) {
      // this wave's copies of chunk c are done once at most those of the chunks after it
      // (up to kLdsStages - 2 of them) are outstanding
      const int after = min(kLdsStages - 2, nch - 1 - c);
      if (after >= 3) probe_wait_vmcnt<3 * kLdsCPW>();
      else if (after == 2) probe_wait_vmcnt<2 * kLdsCPW>();
      else if (after == 1) probe_wait_vmcnt<kLdsCPW>();
      else probe_wait_vmcnt<0>();
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (c + kLdsStages - 1 < nch) issue(c + kLdsStages - 1);
      const unsigned char* base = lds + (size_t)(c % kLdsStages) * kLdsCopies * 1024;
#pragma unroll
      for (int i = 0; i < kLdsCPW; ++i) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(base + (wave * kLdsCPW + i) * 1024 + lane * 16);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
      }
    }
    __syncthreads();  // the next item's first copies reuse the ring
  }
  uint32_t* red = reinterpret_cast<uint32_t*>(lds);  // the ring is free after the last item
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 32 * kLdsWaves; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

}  // namespace

extern "C" {

// Workgroups of one pass; the sink must hold this many uint32.
int moe_probe_read_grid(void) { return 4096; }

// Reads a [E, 2I, K] bf16 weight stack (the W13 layout; I a multiple of rows / 2, K of 64,
// 16-byte aligned) once through the LDS ring on `stream`, in the item order of the tiled up
// GEMM: items of `rows` (256 or 128) weight rows, half gate and half up, an LDS ring of
// `stages` (3..5) chunks of rows x 128 bytes, and `grid` workgroups (a multiple of 8; with
// 128-row items two or three workgroups fit on a CU, so that more copies are in flight per
// CU); the sink must hold `grid` uint32.  Returns 0, -1 for invalid arguments, -4 for a
// launch failure.
int moe_probe_read_lds(const void* m, int E, int I, int K, int stages, int rows, int grid,
                       uint32_t* sink, hipStream_t stream) {
  if (m == nullptr || sink == nullptr || E <= 0 || I <= 0 || (rows != 256 && rows != 128) ||
      I % (rows / 2) != 0 || K <= 0 || K % kLdsKC != 0 || grid <= 0 || grid % 8 != 0 ||
      reinterpret_cast<uintptr_t>(m) % 16 != 0 || stages < 3 || stages > 5)
    return -1;
  const uint16_t* mm = static_cast<const uint16_t*>(m);
#define MOE_PROBE_LDS(S, R)                                                                      \
  hipLaunchKernelGGL((read_lds_ring_kernel<S, R>), dim3(grid), dim3(64 * kLdsWaves), 0, stream, \
                     mm, E, I, K, sink)
  if (rows == 256) {
    if (stages == 3) MOE_PROBE_LDS(3, 256);
    else if (stages == 4) MOE_PROBE_LDS(4, 256);
    else MOE_PROBE_LDS(5, 256);
  } else {
    if (stages == 3) MOE_PROBE_LDS(3, 128);
    else if (stages == 4) MOE_PROBE_LDS(4, 128);
    else MOE_PROBE_LDS(5, 128);
  }
#undef MOE_PROBE_LDS
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Reads `bytes` (a multiple of 16, 16-byte aligned device memory) once on `stream`.
// Returns 0, -1 for invalid arguments, -4 for a launch failure.
int moe_probe_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (buf == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0 ||
      reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return -1;
  hipLaunchKernelGGL(read_pass_kernel, dim3(moe_probe_read_grid()), dim3(kThreads), 0, stream,
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
