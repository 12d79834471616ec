// Achievable HBM read bandwidth on this device, the measured ceiling the layer's
// weight-streaming kernels are compared with next to the 8 TB/s vendor figure.  Not part
// of the layer: a separate library (libmoe_probe.so) that only the benchmark loads.
//
// One fully coalesced pass over a buffer: each wave instruction reads 1 KiB contiguous,
// 8 loads in flight per lane, grid-stride over the buffer, loads marked nontemporal (the
// data is read once: 6.95 TB/s on MI355X against 6.26 TB/s with ordinary loads); the
// loaded words are folded with xor into one word per workgroup so the loads cannot be
// dropped.
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

}  // namespace

extern "C" {

// Workgroups of one pass; the sink must hold this many uint32.
int moe_probe_read_grid(void) { return 4096; }

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
