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
// never straddle two experts, listed expert by expert (in id order, or -- with tile groups
// -- in a hot/cold-mixed order, step 5; the plan itself is always in id order).
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

  // 5. optional list of row tiles holding real entries.  With tile groups (the panel GEMMs,
  // which walk the list expert by expert in one contiguous share per XCD, so that the tiles
  // of an expert share its weight lines in one L2) the experts are listed hot and cold
  // mixed: ranked by count (descending, ties by id), dealt in a snake over 8 bins (ranks 0-7
  // to bins 0-7, 8-15 to bins 7-0, ...) and listed bin after bin, so that every share reads
  // about as many distinct weight bytes as the others (listed by id, the shares that hold
  // the hot experts fetch a few streams many times over while the cold shares fetch ten
  // times their bytes: measured M=2048 bf16 panels 5,383 -> 5,122 us per layer); without
  // tile groups in id order.
  if (tiles != nullptr) {
    __shared__ __align__(16) int32_t s_total[kAlignMaxE];
    __shared__ int32_t s_pos[kAlignMaxE];
    __shared__ int32_t s_multi;
    if (tid == 0) s_multi = 0;
    __syncthreads();
    if (tid < E) {
      s_total[tid] = total;
      if (total > tile_rows) s_multi = 1;   // some expert has several tiles
    } else if (tid < ((E + 3) & ~3)) {
      s_total[tid] = -1;                    // pads the last group of four
    }
    __syncthreads();  // totals complete; wave_total is reused by the scan
    int ep = tid;     // expert at list position tid
    // (with one tile per expert every share streams its experts' weights once: no reorder)
    if (tile_groups != nullptr && s_multi) {
      if (tid < E) {
        const int mine = s_total[tid];
        int rank = 0;
        const int4* t4 = reinterpret_cast<const int4*>(s_total);
        for (int q = 0; q < (E + 3) / 4; ++q) {
          const int4 o = t4[q];
          const int e = 4 * q;
          rank += (o.x > mine) || (o.x == mine && e < tid);
          rank += (o.y > mine) || (o.y == mine && e + 1 < tid);
          rank += (o.z > mine) || (o.z == mine && e + 2 < tid);
          rank += (o.w > mine) || (o.w == mine && e + 3 < tid);
        }
        const int round = rank / 8, r8 = rank % 8;
        const int bin = (round & 1) ? 7 - r8 : r8;
        // experts in bins 0 .. bin-1: two per whole block of 16 ranks, plus the partial block
        int before = 0;
        for (int b = 0; b < bin; ++b) before += E / 16 * 2 + (E % 16 > b) + (E % 16 > 15 - b);
        s_pos[before + round] = tid;   // one expert per bin and round, in rank order
      }
      __syncthreads();
      if (tid < E) ep = s_pos[tid];
    }
    const int tot_e = tid < E ? s_total[ep] : 0;
    const int ntile_e = (tid < E) ? (tot_e + tile_rows - 1) / tile_rows : 0;
    int all_tiles;
    const int first = block_exclusive_scan(ntile_e, wave_total, lane, wave, &all_tiles);
    if (tid < E) {
      const int base = prefix[ep];
      for (int j = 0; j < ntile_e; ++j) {
        const int left = tot_e - j * tile_rows;
        tiles[first + j] = make_int2(base + j * tile_rows, left < tile_rows ? left : tile_rows);
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
