// Align step of the routed-MoE layer: the expert-major token plan.
//
// FlashInfer PR #6511 analysis ("AlphaMoE NVFP4 kernels"), section 5: per-expert counts
// are scanned into a shared prefix array and each plan block finds its expert id by a
// binary search over that prefix; the fix on that page is the barrier between writing
// the prefix and searching it.  Section 6: the plan is the expert-major token order the
// up kernel consumes.
//
// One workgroup of 16 waves.  The flat ids are cut into 16 contiguous segments, one per
// wave, so the placement can be stable (ascending flat index inside each expert) without
// any ordering atomics:
//   1. per-wave histograms in LDS (atomic adds, whose order does not matter);
//   2. thread e sums its expert's 16 counts, pads to the block, and a block-wide
//      exclusive scan gives the prefix; each wave's cursor for expert e starts after the
//      entries of the lower waves;
//   -- barrier: prefix and cursors are complete before anyone reads them --
//   3. each wave walks its segment 64 entries at a time; lanes holding the same expert
//      find their rank among themselves with one ballot per id bit and write
//      cursor + rank; the highest lane of each group advances the cursor;
//   4. padding slots get the sentinel n; block b takes the expert found by a binary
//      search of b * block in the prefix.
// Optionally (for the grouped GEMMs of moe_forward) the kernel also lists the row tiles
// of height T that hold real entries: tile = {first plan row, real rows in it}, tiles
// never straddle two experts, listed expert by expert.
#include "device_common.h"
#include "launchers.h"

namespace moe {

constexpr int kAlignWaves = 16;
constexpr int kAlignThreads = kAlignWaves * kWave;
constexpr int kAlignMaxE = 1024;
constexpr int kAlignBatch = 8;   // ids per lane requested together

__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_total, int lane, int wave,
                                                    int* total_out) {
  int incl = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) wave_total[wave] = incl;
  __syncthreads();
  int base = 0, all = 0;
  for (int w = 0; w < kAlignWaves; ++w) {
    const int t = wave_total[w];
    if (w < wave) base += t;
    all += t;
  }
  *total_out = all;
  return base + incl - v;
}

__global__ __launch_bounds__(kAlignThreads) void align_kernel(
    const int32_t* __restrict__ ids, int n, int E, int block, int id_bits,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ num_padded, int tile_rows, int2* __restrict__ tiles,
    int32_t* __restrict__ num_tiles, int2* __restrict__ tile_groups) {
  __shared__ int32_t cnt[kAlignWaves][kAlignMaxE];  // count, then cursor, per (wave, expert)
  __shared__ int32_t prefix[kAlignMaxE + 1];
  __shared__ int32_t wave_total[kAlignWaves];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  for (int i = tid; i < kAlignWaves * kAlignMaxE; i += kAlignThreads) (&cnt[0][0])[i] = 0;
  __syncthreads();

  // segment of this wave, a multiple of 64 entries long
  const int seg = ((n + kAlignWaves - 1) / kAlignWaves + 63) & ~63;
  const int lo = min(n, wave * seg);
  const int hi = min(n, lo + seg);

  // 1. histogram (kAlignBatch ids requested before any is used: one memory round trip per
  // batch instead of per id)
  for (int b0 = lo; b0 < hi; b0 += kWave * kAlignBatch) {
    int ev[kAlignBatch];
#pragma unroll
    for (int u = 0; u < kAlignBatch; ++u) {
      const int i = b0 + kWave * u + lane;
      ev[u] = i < hi ? ids[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < kAlignBatch; ++u) {
      if (b0 + kWave * u >= hi) break;         // uniform: past this wave's segment
      if ((unsigned)ev[u] < (unsigned)E) atomicAdd(&cnt[wave][ev[u]], 1);
    }
  }
  __syncthreads();

  // 2. totals, padding, exclusive scan over experts (thread e owns expert e)
  int total = 0, padded = 0;
  if (tid < E) {
#pragma unroll
    for (int w = 0; w < kAlignWaves; ++w) total += cnt[w][tid];
    padded = (total + block - 1) / block * block;
  }
  int all_padded;
  const int excl = block_exclusive_scan(padded, wave_total, lane, wave, &all_padded);
  if (tid < E) {
    prefix[tid] = excl;
    int run = excl;
#pragma unroll
    for (int w = 0; w < kAlignWaves; ++w) {
      const int c = cnt[w][tid];
      cnt[w][tid] = run;
      run += c;
    }
    for (int r = excl + total; r < excl + padded; ++r) sorted_ids[r] = n;  // sentinel
  }
  if (tid == 0) {
    prefix[E] = all_padded;
    *num_padded = all_padded;
  }
  __syncthreads();  // prefix[] and the cursors are complete before they are read

  // 3. stable scatter
  const uint64_t lower_lanes = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int b0 = lo; b0 < hi; b0 += kWave * kAlignBatch) {
    int ev[kAlignBatch];
#pragma unroll
    for (int u = 0; u < kAlignBatch; ++u) {
      const int i = b0 + kWave * u + lane;
      ev[u] = i < hi ? ids[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < kAlignBatch; ++u) {   // in ascending flat index
      if (b0 + kWave * u >= hi) break;         // uniform: past this wave's segment
      const int i = b0 + kWave * u + lane;
      const int e = ev[u];
      const bool valid = (unsigned)e < (unsigned)E;
      uint64_t same = __ballot(valid);
      for (int b = 0; b < id_bits; ++b) {
        const bool bit = valid && ((e >> b) & 1);
        const uint64_t set = __ballot(bit);
        same &= bit ? set : ~set;
      }
      if (valid) {
        const int cursor = cnt[wave][e];
        sorted_ids[cursor + __popcll(same & lower_lanes)] = i;
        if ((same >> lane) == 1ull) cnt[wave][e] = cursor + __popcll(same);  // highest lane of the group
      }
    }
  }

  // 4. block -> expert: last e with prefix[e] <= b * block
  const int nblocks = prefix[E] / block;
  for (int b = tid; b < nblocks; b += kAlignThreads) {
    const int start = b * block;
    int l = 0, h = E;
    while (h - l > 1) {
      const int mid = (l + h) >> 1;
      if (prefix[mid] <= start) l = mid;
      else h = mid;
    }
    block_expert[b] = l;
  }

  // 5. optional list of row tiles holding real entries
  if (tiles != nullptr) {
    const int ntile_e = (tid < E) ? (total + tile_rows - 1) / tile_rows : 0;
    __syncthreads();  // wave_total is reused by the scan
    int all_tiles;
    const int first = block_exclusive_scan(ntile_e, wave_total, lane, wave, &all_tiles);
    if (tid < E) {
      for (int j = 0; j < ntile_e; ++j) {
        const int left = total - j * tile_rows;
        tiles[first + j] = make_int2(excl + j * tile_rows, left < tile_rows ? left : tile_rows);
        // optional: each tile's expert as {its first tile, its tile count}
        if (tile_groups != nullptr) tile_groups[first + j] = make_int2(first, ntile_e);
      }
    }
    if (tid == 0) *num_tiles = all_tiles;
  }
}

hipError_t launch_align(const int32_t* ids, int n, int E, int block, int32_t* sorted_ids,
                        int32_t* block_expert, int32_t* num_padded, int tile_rows, int2* tiles,
                        int32_t* num_tiles, hipStream_t s, int2* tile_groups) {
  int id_bits = 0;
  while ((1 << id_bits) < E) ++id_bits;
  hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kAlignThreads), 0, s, ids, n, E, block, id_bits,
                     sorted_ids, block_expert, num_padded, tile_rows, tiles, num_tiles,
                     tile_groups);
  return hipGetLastError();
}

}  // namespace moe
