// Grouped expert GEMMs of moe_forward (bf16 weights at every size, from decode to
// prefill; MXFP8 weights from 16 tokens per expert): LDS-tiled MFMA kernels fed by direct
// global -> LDS copies.
//
// AlphaMoE page (FlashInfer PR #6511 analysis), section 4: the up kernel of the large
// batch and prefill routes gathers a tile of tokens per expert; section 2: the down
// kernel streams W2 in deep K panels.  Trainium2 megakernel page, first paragraph,
// rule 1: keep the working set on chip -- the weight and token chunks in LDS are shared
// by all waves of a workgroup, and the M tiles of one expert run on one XCD at the same
// time so they share the weight stream through that XCD's L2.
//
// Workgroup tile: BM plan rows of one expert (a tile of the align kernel's list) x 64 WN
// weight rows (up: gate and up rows of 32 WN act columns; down: 64 WN output columns), K
// in chunks of 64.  Both operands are copied global -> LDS with global_load_lds_dwordx4,
// which lands lane l's 16 bytes at LDS base + 16 l.  One copy covers 8 rows x one whole
// 128-byte line each (a 16 rows x 64-byte pattern, two half lines per row, streams at a
// third of the rate when the lines come from L2), and inside a row the 16-byte K chunks
// are XOR-swizzled so that an MFMA fragment (16 rows x 32 K values) is one conflict-free
// ds_read_b128 per lane.  No registers stage the data.  An S-deep ring keeps S-1 chunks
// in flight; each wave waits for its own copies of chunk c with s_waitcnt vmcnt and a
// bare s_barrier publishes them (a fenced barrier would drain every copy in flight).
// Only a partial last K chunk goes through registers (zero-filled).  Waves form a
// WN x WM grid; each accumulates 4 weight tiles x BM/16/WM token tiles with
// v_mfma_f32_16x16x32_bf16.
//
// Work order: the hardware hands workgroup p to XCD p % 8.  Each XCD gets an equal,
// contiguous share of the live (tile, N tile) items (the tile count is read on the
// device), ordered N tile by N tile.  With 64-row tiles (few tokens per expert) the grid
// is one workgroup per CU, each walking its XCD's share, so that an item's epilogue stores
// drain while the next item's copies stream (a wave that ends waits for its stores first).
// The up GEMMs store act only for a tile's real rows: the down GEMM never reads the others.
//
// Besides that kernel: a self-routing up kernel that builds the plan itself (few ids, no
// align launch), a split-ring kernel with separate weight and token rings (two weight
// chunks in flight), and the MXFP8 kernels.
#include <type_traits>

#include "device_common.h"
#include "launchers.h"
#include "tiled_common.h"

namespace moe {

constexpr int kTileKC = 64;                     // K values per chunk: one 128-byte line per row
constexpr int kTileKS = kTileKC / 32;           // MFMA K steps per chunk

// Workgroup of WN x WM waves.  Weight rows: 64 * WN (4 row tiles of 16 per wave along
// WN); token rows: BM (BM / 16 / WM row tiles per wave along WM).  Each wave accumulates
// 4 weight tiles x MTW token tiles.
constexpr int kNT = 2;  // cache policy bits of a nontemporal load (gfx950)

template <int BM, int WN, int WM>
struct TiledCfg {
  static constexpr int THREADS = 64 * WN * WM;
  static constexpr int WT = 4 * WN;                          // weight row tiles per workgroup
  static constexpr int MT = BM / 16;                         // token row tiles per workgroup
  static constexpr int MTW = MT / WM;                        // token row tiles per wave
  static constexpr int FRAGS = (WT + MT) * 2;                // 1 KiB copies per chunk (8 rows each)
  static constexpr int FPW = FRAGS / (WN * WM);              // copies issued per wave
  static_assert(FRAGS % (WN * WM) == 0, "copies must split evenly over the waves");
  static_assert(MT % WM == 0, "token tiles must split evenly over the waves");
};

// Wait until only this wave's copies of the `after` chunks issued after the one needed
// are outstanding (FPW copies per chunk; after <= A).
template <int FPW, int A>
__device__ __forceinline__ void wait_chunks_after(int after) {
  if constexpr (A <= 0) {
    wait_vmcnt<0>();
  } else {
    if (after >= A) wait_vmcnt<A * FPW>();
    else wait_chunks_after<FPW, A - 1>(after);
  }
}

// One work item of the tiled GEMM: plan rows start..start+nlive-1 of expert e (row_ids[r] =
// the flat index of plan row start + r) against the weight rows of N tile `ntile`.
template <int BM, int WN, int WM, int S, bool UP, int WPOL>
__device__ __forceinline__ void tiled_gemm(
    unsigned char* __restrict__ lds, const uint16_t* __restrict__ tok_src,
    const uint16_t* __restrict__ w, const int32_t* row_ids, int start, int nlive, int e,
    int ntile, int K, int ncols, int I, int top_k, uint16_t* __restrict__ act,
    uint16_t* __restrict__ y, float* __restrict__ y0) {
  using C = TiledCfg<BM, WN, WM>;
  const int mt_active = (nlive + 15) >> 4;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int wn = wave % WN, wm = wave / WN;
  const int col0 = UP ? ntile * 32 * WN : ntile * 64 * WN;

  // Copy f of a chunk covers rows 8h..8h+7 (h = f % 2) of row tile f / 2 (weight tiles
  // first, then token tiles), one 128-byte line per row: lane l copies row 8h + l / 8, and
  // its 16 bytes land at LDS slot l % 8 of that row.  The slot holds K chunk
  // q = (l % 8) ^ (row % 8) ^ h of the row, an XOR swizzle that keeps the fragment reads
  // below free of bank conflicts.  Rows that hold no data point at a valid row (their
  // results are never stored).
  const uint16_t* src[C::FPW];
  bool src_on[C::FPW];
  int src_q[C::FPW];
  const size_t wexp = UP ? (size_t)e * 2 * I * K : (size_t)e * ncols * K;
#pragma unroll
  for (int i = 0; i < C::FPW; ++i) {
    const int f = wave * C::FPW + i;
    const int rt = f >> 1, h = f & 1;
    const int rr = 8 * h + (lane >> 3);           // row inside the 16-row tile
    src_q[i] = (lane & 7) ^ (lane >> 3) ^ h;
    const int koff = 8 * src_q[i];
    if (rt < C::WT) {
      int row;
      if (UP) row = (rt < C::WT / 2) ? col0 + rt * 16 + rr : I + col0 + (rt - C::WT / 2) * 16 + rr;
      else row = col0 + rt * 16 + rr;
      src_on[i] = UP || row < ncols;
      src[i] = w + wexp + (size_t)(src_on[i] ? row : 0) * K + koff;
    } else {
      const int r = 16 * (rt - C::WT) + rr;
      src_on[i] = r < nlive;
      const int prow = start + (src_on[i] ? r : 0);
      if (UP) {
        const int sid = src_on[i] ? row_ids[r] : 0;
        src[i] = tok_src + (size_t)(sid < 0 ? 0 : sid / top_k) * K + koff;
      } else {
        src[i] = tok_src + (size_t)prow * K + koff;
      }
    }
  }
  int wtile[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    wtile[j] = UP ? ((j < 2) ? 2 * wn + j : C::WT / 2 + 2 * wn + (j - 2)) : 4 * wn + j;

  const int nch = (K + kTileKC - 1) / kTileKC;
  const int ndma = K / kTileKC;  // whole chunks
  auto issue = [&](int c) {
    unsigned char* base = lds + (size_t)(c % S) * C::FRAGS * 1024;
    if (c < ndma) {
#pragma unroll
      for (int i = 0; i < C::FPW; ++i) {
        const int f = wave * C::FPW + i;
        // weight rows with the given cache policy (nontemporal when each weight is read by
        // one token tile), token rows with the default one
        if (f < 2 * C::WT)
          __builtin_amdgcn_global_load_lds((global_void*)(src[i] + c * kTileKC),
                                           (lds_void*)(base + f * 1024), 16, 0, WPOL);
        else
          __builtin_amdgcn_global_load_lds((global_void*)(src[i] + c * kTileKC),
                                           (lds_void*)(base + f * 1024), 16, 0, 0);
      }
    } else {  // partial chunk: zero-filled through registers
#pragma unroll
      for (int i = 0; i < C::FPW; ++i) {
        const int f = wave * C::FPW + i;
        const int k = c * kTileKC + 8 * src_q[i];
        const u32x4 v = (src_on[i] && k + 8 <= K) ? ld16(src[i] + c * kTileKC) : u32x4{0, 0, 0, 0};
        *reinterpret_cast<u32x4*>(base + (size_t)f * 1024 + lane * 16) = v;
      }
    }
  };
  // MFMA fragment (16 rows x 32 K values) ks of row tile t: lane (li, lg) reads row li,
  // K chunk lg + 4 ks, from its swizzled slot
  const int frag_off = (li >> 3) * 1024 + (li & 7) * 128;
  auto frag = [&](int c, int t, int ks) -> u32x4 {
    const int q = (lg + 4 * ks) ^ (li & 7) ^ (li >> 3);
    return *reinterpret_cast<const u32x4*>(lds + (size_t)(c % S) * C::FRAGS * 1024 + t * 2048 +
                                           frag_off + q * 16);
  };

  f32x4 acc[4][C::MTW];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int s = 0; s < C::MTW; ++s) acc[j][s] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int my_active = mt_active - wm * C::MTW;

  auto compute = [&](int c) {
    if (my_active <= 0) return;
#pragma unroll
    for (int ks = 0; ks < kTileKS; ++ks) {
      u32x4 wa[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) wa[j] = frag(c, wtile[j], ks);
#pragma unroll
      for (int s = 0; s < C::MTW; ++s) {
        if (s < my_active) {
          const u32x4 xb = frag(c, C::WT + wm * C::MTW + s, ks);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[j][s] = mfma16x16x32(wa[j], xb, acc[j][s]);
        }
      }
    }
  };

#pragma unroll
  for (int p = 0; p < S - 1; ++p)
    if (p < nch) issue(p);
  for (int c = 0; c < nch; ++c) {
    // this wave's whole chunks issued after c: min(S-2, ndma-1-c) (none once c reaches the
    // register-staged tail chunk, whose loads are complete when it is stored)
    const int after = c < ndma ? min(S - 2, ndma - 1 - c) : 0;
    wait_chunks_after<C::FPW, S - 2>(after);
    // chunk c landed for every wave (each waited for its own copies above) and chunk c-1
    // is fully consumed; a bare barrier, so the copies still in flight stay in flight
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (c + S - 1 < nch) issue(c + S - 1);
    compute(c);
  }

#pragma unroll
  for (int s = 0; s < C::MTW; ++s) {
    if (s >= my_active) continue;
    const int r = 16 * (wm * C::MTW + s) + li;
    if (UP && r < nlive) {  // padding rows of the tile are never read
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int n = col0 + wn * 32 + h * 16 + 4 * lg;
        float a[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) a[q] = silu_f32(acc[h][s][q]) * acc[2 + h][s][q];
        uint2 v;
        v.x = pack_bf16x2(a[0], a[1]);
        v.y = pack_bf16x2(a[2], a[3]);
        *reinterpret_cast<uint2*>(act + (size_t)(start + r) * I + n) = v;
      }
    } else if (!UP && r < nlive) {
      const YRow yr = y_row(row_ids[r], top_k, ncols);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = col0 + wn * 64 + j * 16 + 4 * lg;
        // plain stores: nontemporal stores of the 8-byte bf16 pieces drain slower (decode
        // finalize 13 -> 15 us, MXFP8 M=2048 down 1,803 -> 1,879 us)
        if (n < ncols)
          store_y4(y, y0, yr, n, acc[j][s][0], acc[j][s][1], acc[j][s][2], acc[j][s][3]);
      }
    }
  }
}

template <int BM, int WN, int WM, int S, bool UP, int WPOL>
__global__ __launch_bounds__(64 * WN * WM) void expert_tiled_kernel(
    const uint16_t* __restrict__ tok_src, const uint16_t* __restrict__ w,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ block_expert,
    const int2* __restrict__ tiles, const int32_t* __restrict__ num_tiles, int n_ntiles, int K,
    int ncols, int I, int top_k, int block, uint16_t* __restrict__ act, uint16_t* __restrict__ y,
    float* __restrict__ y0) {
  using C = TiledCfg<BM, WN, WM>;
  static_assert(S >= 2 && (S - 2) * C::FPW <= 63, "the copies in flight must fit the vmcnt counter");
  static_assert(S * C::FRAGS * 1024 <= 160 * 1024, "the ring must fit the LDS");
  __shared__ __align__(16) unsigned char lds[S * C::FRAGS * 1024];
  TiledWalk walk(*num_tiles, n_ntiles);
  int ntile, ti;
  while (walk.next(ntile, ti)) {
    const int2 tile = tiles[ti];
    const int start = tile.x, nlive = tile.y;
    const int e = block_expert[start / block];
    // In the up GEMM of a launch that keeps weights cached, an expert whose rows fit one
    // 128-row tile (the tiles before and after it in the list belong to other experts) has
    // its weights copied nontemporally: one item per N tile reads them, and cached they
    // would evict the lines the hot experts' tiles share (M=2048: up 3,707 -> 3,635 us,
    // layer 6,027 -> 5,962 us).
    bool single = false;
    if (UP && WPOL == 0 && BM == 128) {
      const bool first = ti == 0 || block_expert[tiles[ti - 1].x / block] != e;
      const bool last = ti + 1 >= walk.ntiles_live || block_expert[tiles[ti + 1].x / block] != e;
      single = first && last;
    }
    if (single)
      tiled_gemm<BM, WN, WM, S, UP, kNT>(lds, tok_src, w, sorted_ids + start, start, nlive, e,
                                         ntile, K, ncols, I, top_k, act, y, y0);
    else
      tiled_gemm<BM, WN, WM, S, UP, WPOL>(lds, tok_src, w, sorted_ids + start, start, nlive, e,
                                          ntile, K, ncols, I, top_k, act, y, y0);
    __syncthreads();  // the next item's first copies reuse the ring
  }
}

// Self-routing up GEMM (the align step fused into it, after the AlphaMoE page's section 6
// self-routing up kernels): no align launch.  Every workgroup rebuilds the plan's shape
// from the flat top-k ids in LDS -- per-expert counts, the exclusive scan of the counts
// padded to the block (plan offsets) and of the tile counts (tile list offsets) -- finds
// its tile by a binary search over the tile offsets, and collects the flat indices of its
// rows (the r-th occurrences of its expert, ascending) with one ballot per 64 ids.  The
// workgroups of N tile 0 also write the plan (sorted ids with the padding sentinel n,
// block -> expert, tile list, counts) exactly as the align kernel does, for the down GEMM
// and the caller.  For few ids only: every workgroup reads all of them.
template <int BM, int WN, int S, int WPOL>
__global__ __launch_bounds__(64 * WN) void expert_up_selfroute_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w13,
    const int32_t* __restrict__ ids, int n, int E, int block, int n_ntiles, int K, int I,
    int top_k, int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ num_padded, int2* __restrict__ tiles, int32_t* __restrict__ num_tiles,
    uint16_t* __restrict__ act) {
  using C = TiledCfg<BM, WN, 1>;
  constexpr int T = C::THREADS;
  constexpr int EPT = kSelfRouteMaxE / T;        // experts per thread in the scans
  static_assert(EPT * T == kSelfRouteMaxE, "the experts must split evenly over the threads");
  static_assert(S >= 2 && (S - 2) * C::FPW <= 63, "the copies in flight must fit the vmcnt counter");
  static_assert(S * C::FRAGS * 1024 +
                        (kSelfRouteMaxIds + 3 * kSelfRouteMaxE + 2 + BM + 2 * WN) * 4 <=
                    160 * 1024,
                "the ring and the plan must fit the LDS");
  __shared__ __align__(16) unsigned char lds[S * C::FRAGS * 1024];
  __shared__ int s_ids[kSelfRouteMaxIds];        // the flat ids
  __shared__ int s_cnt[kSelfRouteMaxE];          // per-expert counts
  __shared__ int s_pre[kSelfRouteMaxE + 1];      // plan offsets
  __shared__ int s_tpre[kSelfRouteMaxE + 1];     // tile list offsets
  __shared__ int s_rows[BM];                     // flat index of each row of the current tile
  __shared__ int s_wsum[2][WN];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += T) s_cnt[e] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += T) {
    const int e = ids[i];
    s_ids[i] = e;
    if ((unsigned)e < (unsigned)E) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  // thread t owns experts EPT t .. EPT t + EPT - 1: its padded rows and tiles, scanned
  int pad_sum = 0, tile_sum = 0;
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int e = EPT * tid + k;
    const int c = e < E ? s_cnt[e] : 0;
    pad_sum += (c + block - 1) / block * block;
    tile_sum += (c + BM - 1) / BM;
  }
  int p_inc = pad_sum, t_inc = tile_sum;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int pa = __shfl_up(p_inc, off, kWave), ta = __shfl_up(t_inc, off, kWave);
    if (lane >= off) {
      p_inc += pa;
      t_inc += ta;
    }
  }
  if (lane == kWave - 1) {
    s_wsum[0][wave] = p_inc;
    s_wsum[1][wave] = t_inc;
  }
  __syncthreads();
  int p_ex = p_inc - pad_sum, t_ex = t_inc - tile_sum;
  for (int wv = 0; wv < wave; ++wv) {
    p_ex += s_wsum[0][wv];
    t_ex += s_wsum[1][wv];
  }
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int e = EPT * tid + k;
    if (e < E) {
      const int c = s_cnt[e];
      s_pre[e] = p_ex;
      s_tpre[e] = t_ex;
      p_ex += (c + block - 1) / block * block;
      t_ex += (c + BM - 1) / BM;
    }
  }
  if (tid == T - 1) {  // the totals: this thread's running sums cover every expert
    s_pre[E] = p_ex;
    s_tpre[E] = t_ex;
  }
  __syncthreads();  // offsets complete before anyone searches them
  const int ntiles_live = s_tpre[E];
  if (blockIdx.x == 0 && tid == 0) {
    *num_padded = s_pre[E];
    *num_tiles = ntiles_live;
  }
  TiledWalk walk(ntiles_live, n_ntiles);
  int ntile, ti;
  while (walk.next(ntile, ti)) {
    // expert of tile ti: the last e with s_tpre[e] <= ti
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_tpre[mid] <= ti) lo = mid;
      else hi = mid;
    }
    const int e = lo;
    const int m = ti - s_tpre[e];
    const int cnt = s_cnt[e];
    const int start = s_pre[e] + m * BM;
    const int nlive = min(BM, cnt - m * BM);
    if (wave == 0) {  // occurrences m BM .. m BM + nlive - 1 of e, in ascending flat index
      const uint64_t lower = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
      const int r_lo = m * BM, r_hi = r_lo + nlive;
      int base = 0;
      for (int b0 = 0; b0 < n && base < r_hi; b0 += kWave) {
        const int i = b0 + lane;
        const bool hit = i < n && s_ids[i] == e;
        const uint64_t bal = __ballot(hit);
        const int r = base + __popcll(bal & lower);
        if (hit && r >= r_lo && r < r_hi) s_rows[r - r_lo] = i;
        base += __popcll(bal);
      }
    }
    __syncthreads();
    if (ntile == 0) {  // the plan of this tile (and of the rest of e's segment)
      for (int r = tid; r < nlive; r += T) sorted_ids[start + r] = s_rows[r];
      const int seg_end = s_pre[e + 1];
      if (m == (cnt + BM - 1) / BM - 1)
        for (int r = s_pre[e] + cnt + tid; r < seg_end; r += T) sorted_ids[r] = n;  // sentinel
      if (m == 0)
        for (int b = s_pre[e] / block + tid; b < seg_end / block; b += T) block_expert[b] = e;
      if (tid == 0) tiles[ti] = make_int2(start, nlive);
    }
    tiled_gemm<BM, WN, 1, S, true, WPOL>(lds, x, w13, s_rows, start, nlive, e, ntile, K, I, I,
                                         top_k, act, nullptr, nullptr);
    __syncthreads();  // s_rows and the ring are reused by the next item
  }
}

// Variant for weights that several token tiles share (many tokens per expert): the same
// 128 plan rows x 512 weight rows per workgroup, 8 waves, copy pattern, swizzle and work
// order as expert_tiled_kernel<128, 8, 1, 2, ...>, but with separate two-stage rings for
// the weight rows (2 x 64 KiB) and the token rows (2 x 16 KiB).  Each wave reads its
// weight fragments of chunk c (4 row tiles x 2 K steps, 32 registers) right after the
// chunk lands; once every wave has, the weight stage takes chunk c + 2 while chunk c is
// computed (token fragments still come from LDS), and the token stage takes chunk c + 2
// after the MFMAs.  Two weight chunks are thus in flight instead of one: measured with
// the MFMAs taken out at M=2048, the up GEMM's copies take 3.50 ms with one chunk in
// flight and 3.11 ms with two or three (the HBM read rate of ordinary loads).  Whole K
// chunks only (K % 64 == 0).
template <int BM, bool UP, int WPOL>
__global__ __launch_bounds__(512) void expert_tiled_reg_kernel(
    const uint16_t* __restrict__ tok_src, const uint16_t* __restrict__ w,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ block_expert,
    const int2* __restrict__ tiles, const int32_t* __restrict__ num_tiles, int n_ntiles, int K,
    int ncols, int I, int top_k, int block, uint16_t* __restrict__ act, uint16_t* __restrict__ y,
    float* __restrict__ y0) {
  constexpr int NW = 8;                          // waves
  constexpr int WT = 32;                         // weight row tiles (512 rows)
  constexpr int MT = BM / 16;                    // token row tiles
  constexpr int WCPW = WT * 2 / NW;              // weight copies (1 KiB) per wave per chunk
  constexpr int TCPW = MT * 2 / NW;              // token copies per wave per chunk
  constexpr int WSTAGE = WT * 2048, TSTAGE = MT * 2048;
  static_assert(WCPW + TCPW <= 63, "one chunk's copies must fit the vmcnt counter");
  static_assert(WCPW * NW == WT * 2 && TCPW * NW == MT * 2,
                "copies must split evenly over the waves");
  __shared__ __align__(16) unsigned char lds[2 * WSTAGE + 2 * TSTAGE];
  unsigned char* const wlds = lds;
  unsigned char* const tlds = lds + 2 * WSTAGE;

  TiledWalk walk(*num_tiles, n_ntiles);
  int ntile, ti;
  while (walk.next(ntile, ti)) {
    const int2 tile = tiles[ti];
    const int start = tile.x, nlive = tile.y;
    const int mt_active = (nlive + 15) >> 4;
    const int e = block_expert[start / block];

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int col0 = UP ? ntile * 256 : ntile * 512;

    // copy f of a ring: rows 8h..8h+7 (h = f % 2) of row tile f / 2; lane l copies 16 bytes of
    // row 8h + l / 8 into slot l % 8, holding K chunk (l % 8) ^ (row % 8) ^ h of the row.
    // Weight tiles 0..31 (up: gate rows in 0..15, up rows in 16..31), token tiles 0..7.
    const int rr = lane >> 3;
    const uint16_t* wsrc[WCPW];
    const uint16_t* tsrc[TCPW];
    const size_t wexp = UP ? (size_t)e * 2 * I * K : (size_t)e * ncols * K;
#pragma unroll
    for (int i = 0; i < WCPW; ++i) {
      const int f = wave * WCPW + i;
      const int rt = f >> 1, h = f & 1;
      const int koff = 8 * ((lane & 7) ^ rr ^ h);
      int row;
      if (UP)
        row = (rt < WT / 2) ? col0 + rt * 16 + 8 * h + rr
                            : I + col0 + (rt - WT / 2) * 16 + 8 * h + rr;
      else row = col0 + rt * 16 + 8 * h + rr;
      const bool on = UP || row < ncols;
      wsrc[i] = w + wexp + (size_t)(on ? row : 0) * K + koff;
    }
#pragma unroll
    for (int i = 0; i < TCPW; ++i) {
      const int f = wave * TCPW + i;
      const int rt = f >> 1, h = f & 1;
      const int koff = 8 * ((lane & 7) ^ rr ^ h);
      const int r = 16 * rt + 8 * h + rr;
      const bool on = r < nlive;
      const int prow = start + (on ? r : 0);
      if (UP) {
        const int sid = on ? sorted_ids[prow] : 0;
        tsrc[i] = tok_src + (size_t)(sid < 0 ? 0 : sid / top_k) * K + koff;
      } else {
        tsrc[i] = tok_src + (size_t)prow * K + koff;
      }
    }
    // this wave's weight tiles: up -- gate tiles 2w, 2w+1 and the up tiles of the same act
    // columns; down -- tiles 4w..4w+3
    int wtile[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      wtile[j] = UP ? ((j < 2) ? 2 * wave + j : WT / 2 + 2 * wave + j - 2) : 4 * wave + j;

    const int nch = K / kTileKC;
    auto issue_w = [&](int c) {
      unsigned char* base = wlds + (size_t)(c & 1) * WSTAGE;
#pragma unroll
      for (int i = 0; i < WCPW; ++i)
        __builtin_amdgcn_global_load_lds((global_void*)(wsrc[i] + c * kTileKC),
                                         (lds_void*)(base + (wave * WCPW + i) * 1024), 16, 0, WPOL);
    };
    auto issue_t = [&](int c) {
      unsigned char* base = tlds + (size_t)(c & 1) * TSTAGE;
#pragma unroll
      for (int i = 0; i < TCPW; ++i)
        __builtin_amdgcn_global_load_lds((global_void*)(tsrc[i] + c * kTileKC),
                                         (lds_void*)(base + (wave * TCPW + i) * 1024), 16, 0, 0);
    };
    // MFMA fragment (16 rows x 32 K values) ks of the row tile at `tbase`: lane (li, lg)
    // reads row li, K chunk lg + 4 ks, from its swizzled slot
    const int frag_off = (li >> 3) * 1024 + (li & 7) * 128;
    auto frag = [&](const unsigned char* tbase, int ks) -> u32x4 {
      const int q = (lg + 4 * ks) ^ (li & 7) ^ (li >> 3);
      return *reinterpret_cast<const u32x4*>(tbase + frag_off + q * 16);
    };

    f32x4 acc[4][MT];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int s = 0; s < MT; ++s) acc[j][s] = f32x4{0.f, 0.f, 0.f, 0.f};

    issue_w(0);
    issue_t(0);
    if (nch > 1) {
      issue_w(1);
      issue_t(1);
    }
    for (int c = 0; c < nch; ++c) {
      // this wave's copies of chunk c are done (those of c + 1 may be in flight) ...
      if (c + 1 < nch) wait_vmcnt<WCPW + TCPW>();
      else wait_vmcnt<0>();
      // ... and every wave's
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      const unsigned char* wb = wlds + (size_t)(c & 1) * WSTAGE;
      const unsigned char* tb = tlds + (size_t)(c & 1) * TSTAGE;
      u32x4 wa[kTileKS][4];
#pragma unroll
      for (int ks = 0; ks < kTileKS; ++ks)
#pragma unroll
        for (int j = 0; j < 4; ++j) wa[ks][j] = frag(wb + wtile[j] * 2048, ks);
      // every wave holds its weight fragments of chunk c: the weight stage takes chunk c + 2
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (c + 2 < nch) issue_w(c + 2);
#pragma unroll
      for (int ks = 0; ks < kTileKS; ++ks)
#pragma unroll
        for (int s = 0; s < MT; ++s)
          if (s < mt_active) {
            const u32x4 xb = frag(tb + s * 2048, ks);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j][s] = mfma16x16x32(wa[ks][j], xb, acc[j][s]);
          }
      // every wave has read its token fragments of chunk c: the token stage takes c + 2
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (c + 2 < nch) issue_t(c + 2);
    }

#pragma unroll
    for (int s = 0; s < MT; ++s) {
      if (s >= mt_active) continue;
      const int r = 16 * s + li;
      if (UP && r < nlive) {  // padding rows of the tile are never read
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int n = col0 + 32 * wave + 16 * h + 4 * lg;
          float a[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) a[q] = silu_f32(acc[h][s][q]) * acc[2 + h][s][q];
          uint2 v;
          v.x = pack_bf16x2(a[0], a[1]);
          v.y = pack_bf16x2(a[2], a[3]);
          *reinterpret_cast<uint2*>(act + (size_t)(start + r) * I + n) = v;
        }
      } else if (!UP && r < nlive) {
        const YRow yr = y_row(sorted_ids[start + r], top_k, ncols);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = col0 + 64 * wave + 16 * j + 4 * lg;
          if (n < ncols)
            store_y4(y, y0, yr, n, acc[j][s][0], acc[j][s][1], acc[j][s][2], acc[j][s][3]);
        }
      }
    }
    __syncthreads();  // the next item's first copies reuse the rings
  }
}

// MXFP8 weights (E4M3 codes, one E8M0 scale byte per 32 values along K) in the tiled
// kernels; moe_forward_mx runs it for the up GEMM from 64 tokens per expert, where the
// 128-row tiles of a hot expert share its codes (its other GEMMs copy the codes into LDS,
// expert_mx_decode.hip).  Same workgroup tile, work order, LDS ring layout and MFMA loop as
// expert_tiled_kernel; the weight part of a ring stage is filled from the codes instead of
// by copies: each thread loads PIECES pieces of 16 codes (4 lanes cover a row's 64 codes
// of a chunk: 16 rows x 64 bytes per wave load), dequantizes them exactly to bf16 with
// the block's scale (v_cvt_scalef32_pk_bf16_fp8) and writes them into the swizzled slots
// with ds_write_b128.  The scales of 4 chunks of a row come with one 8-byte load.  Token
// rows still arrive by global_load_lds.  Per chunk c: wait for the token copies of c and
// barrier, then dequantize the codes of c + 1 (loaded while c - 1 was computed) into the
// other stage, copy the token rows of c + 1 there, load the codes of c + 2, and compute c.
template <int BM, int WN, int WM, bool UP>
__global__ __launch_bounds__(64 * WN * WM) void expert_tiled_mx_kernel(
    const uint16_t* __restrict__ tok_src, const uint8_t* __restrict__ wc,
    const uint8_t* __restrict__ ws, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int2* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, int n_ntiles, int K, int ncols, int I, int top_k,
    int block, uint16_t* __restrict__ act, float* __restrict__ y) {
  using C = TiledCfg<BM, WN, WM>;
  constexpr int S = 2;
  constexpr int TCOPIES = 2 * C::MT;                    // 1 KiB token copies per chunk
  static_assert(TCOPIES % (WN * WM) == 0, "token copies must split evenly over the waves");
  constexpr int TPW = TCOPIES / (WN * WM);
  constexpr int PIECES = 16 * C::WT * 4 / C::THREADS;   // 16-code pieces per thread per chunk
  static_assert(PIECES * C::THREADS == 16 * C::WT * 4, "code pieces must split evenly");
  static_assert(S * C::FRAGS * 1024 <= 160 * 1024, "the ring must fit the LDS");
  __shared__ __align__(16) unsigned char lds[S * C::FRAGS * 1024];

  const int ntiles_live = *num_tiles;
  const int live_items = ntiles_live * n_ntiles;
  const int per_xcd = (live_items + kXcds - 1) / kXcds;
  const int slot = blockIdx.x / kXcds;
  if (slot >= per_xcd) return;
  const int logical = (blockIdx.x % kXcds) * per_xcd + slot;
  if (logical >= live_items) return;
  const int ntile = logical / ntiles_live;
  const int ti = logical % ntiles_live;
  const int2 tile = tiles[ti];
  const int start = tile.x, nlive = tile.y;
  const int mt_active = (nlive + 15) >> 4;
  const int e = block_expert[start / block];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int wn = wave % WN, wm = wave / WN;
  const int col0 = UP ? ntile * 32 * WN : ntile * 64 * WN;
  const int rows_e = UP ? 2 * I : ncols;                // weight rows per expert

  // code pieces: piece id = tid + THREADS * i is row R = id / 4 of the workgroup's weight
  // rows (row tile R / 16, weight tiles as in expert_tiled_kernel), K values 16 (id % 4)
  // .. + 16 of the chunk = the two 8-value slots q = 2 (id % 4) and q + 1
  const uint8_t* wsrc[PIECES];
  const uint8_t* ssrc[PIECES];
  int wdst[PIECES][2];
  int sbyte[PIECES];                                     // scale byte of a chunk: 2 (c % 4) + this
#pragma unroll
  for (int i = 0; i < PIECES; ++i) {
    const int id = tid + C::THREADS * i;
    const int R = id >> 2, p = id & 3;
    const int t = R >> 4, rr = R & 15;
    int row;
    if (UP) row = (t < C::WT / 2) ? col0 + t * 16 + rr : I + col0 + (t - C::WT / 2) * 16 + rr;
    else row = col0 + t * 16 + rr;
    if (!UP && row >= ncols) row = 0;                    // rows past H: never stored
    const size_t grow = (size_t)e * rows_e + row;
    wsrc[i] = wc + grow * K + 16 * p;
    ssrc[i] = ws + grow * (K / 32);
    sbyte[i] = p >> 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int q = 2 * p + h;
      wdst[i][h] = t * 2048 + (rr >> 3) * 1024 + (rr & 7) * 128 + ((q ^ (rr & 7) ^ (rr >> 3)) * 16);
    }
  }
  // token copies: copy f = 2 WT + wave * TPW + i as in expert_tiled_kernel
  const uint16_t* tsrc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int f = 2 * C::WT + wave * TPW + i;
    const int rt = f >> 1, h = f & 1;
    const int rr = 8 * h + (lane >> 3);
    const int koff = 8 * ((lane & 7) ^ (lane >> 3) ^ h);
    const int r = 16 * (rt - C::WT) + rr;
    const bool on = r < nlive;
    const int prow = start + (on ? r : 0);
    if (UP) {
      const int sid = on ? sorted_ids[prow] : 0;
      tsrc[i] = tok_src + (size_t)(sid < 0 ? 0 : sid / top_k) * K + koff;
    } else {
      tsrc[i] = tok_src + (size_t)prow * K + koff;
    }
  }
  int wtile[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    wtile[j] = UP ? ((j < 2) ? 2 * wn + j : C::WT / 2 + 2 * wn + (j - 2)) : 4 * wn + j;

  const int nch = K / kTileKC;                           // K is a multiple of 256
  u32x4 codes[PIECES];
  uint2 scl[PIECES];
  auto load = [&](int c) {                               // codes of chunk c (+ scales of its 4)
#pragma unroll
    for (int i = 0; i < PIECES; ++i) codes[i] = ld16(wsrc[i] + c * kTileKC);
    if ((c & 3) == 0) {
#pragma unroll
      for (int i = 0; i < PIECES; ++i) scl[i] = *reinterpret_cast<const uint2*>(ssrc[i] + 2 * c);
    }
  };
  auto put = [&](int c, int stage) {                     // dequantized codes of chunk c
    unsigned char* base = lds + (size_t)stage * C::FRAGS * 1024;
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
      const int b = 2 * (c & 3) + sbyte[i];
      const uint32_t word = b < 4 ? scl[i].x : scl[i].y;
      u32x4 lo, hi;
      mx_dequant16(codes[i], (word >> (8 * (b & 3))) & 0xFFu, lo, hi);
      *reinterpret_cast<u32x4*>(base + wdst[i][0]) = lo;
      *reinterpret_cast<u32x4*>(base + wdst[i][1]) = hi;
    }
  };
  auto copy_tokens = [&](int c, int stage) {
    unsigned char* base = lds + (size_t)stage * C::FRAGS * 1024;
#pragma unroll
    for (int i = 0; i < TPW; ++i)
      __builtin_amdgcn_global_load_lds((global_void*)(tsrc[i] + c * kTileKC),
                                       (lds_void*)(base + (2 * C::WT + wave * TPW + i) * 1024),
                                       16, 0, 0);
  };
  const int frag_off = (li >> 3) * 1024 + (li & 7) * 128;
  auto frag = [&](int stage, int t, int ks) -> u32x4 {
    const int q = (lg + 4 * ks) ^ (li & 7) ^ (li >> 3);
    return *reinterpret_cast<const u32x4*>(lds + (size_t)stage * C::FRAGS * 1024 + t * 2048 +
                                           frag_off + q * 16);
  };

  f32x4 acc[4][C::MTW];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int s = 0; s < C::MTW; ++s) acc[j][s] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int my_active = mt_active - wm * C::MTW;

  auto compute = [&](int stage) {
    if (my_active <= 0) return;
#pragma unroll
    for (int ks = 0; ks < kTileKS; ++ks) {
      u32x4 wa[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) wa[j] = frag(stage, wtile[j], ks);
#pragma unroll
      for (int s = 0; s < C::MTW; ++s) {
        if (s < my_active) {
          const u32x4 xb = frag(stage, C::WT + wm * C::MTW + s, ks);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[j][s] = mfma16x16x32(wa[j], xb, acc[j][s]);
        }
      }
    }
  };

  // The codes of a chunk are dequantized before the token copies of the same chunk are
  // issued, so waiting for the codes never waits for those copies.
  load(0);
  put(0, 0);
  copy_tokens(0, 0);
  if (nch > 1) load(1);
  for (int c = 0; c < nch; ++c) {
    // this wave's token copies of chunk c and the codes of c + 1 (needed right after the
    // barrier) have landed; after the barrier chunk c is in LDS for every wave and chunk
    // c - 1 is fully consumed
    wait_vmcnt<0>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (c + 1 < nch) {
      put(c + 1, (c + 1) & 1);
      copy_tokens(c + 1, (c + 1) & 1);
      if (c + 2 < nch) load(c + 2);
    }
    compute(c & 1);
  }

#pragma unroll
  for (int s = 0; s < C::MTW; ++s) {
    if (s >= my_active) continue;
    const int r = 16 * (wm * C::MTW + s) + li;
    if (UP) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int n = col0 + wn * 32 + h * 16 + 4 * lg;
        float a[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) a[q] = silu_f32(acc[h][s][q]) * acc[2 + h][s][q];
        uint2 v;
        v.x = pack_bf16x2(a[0], a[1]);
        v.y = pack_bf16x2(a[2], a[3]);
        *reinterpret_cast<uint2*>(act + (size_t)(start + r) * I + n) = v;
      }
    } else if (r < nlive) {
      const int dst = sorted_ids[start + r];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = col0 + wn * 64 + j * 16 + 4 * lg;
        if (n < ncols)
          *reinterpret_cast<float4*>(y + (size_t)dst * ncols + n) =
              make_float4(acc[j][s][0], acc[j][s][1], acc[j][s][2], acc[j][s][3]);
      }
    }
  }
}

template <int BM, int WN, int WM, int S, bool UP, int WPOL>
static hipError_t launch_tiled(const uint16_t* src, const uint16_t* w, const int32_t* sorted_ids,
                               const int32_t* block_expert, const int2* tiles,
                               const int32_t* num_tiles, int max_tiles, int K, int ncols, int I,
                               int top_k, int block, uint16_t* act, uint16_t* y, float* y0,
                               hipStream_t s) {
  const int per_ntile = UP ? 32 * WN : 64 * WN;
  if (UP && I % per_ntile != 0) return hipErrorInvalidValue;
  const int n_ntiles = (ncols + per_ntile - 1) / per_ntile;
  // 64-row tiles (few tokens per expert) walk several items per workgroup; 128-row tiles
  // take one each (measured: walking costs 1-2 % at M=512 and M=2048)
  const long items = (long)max_tiles * n_ntiles;
  const long grid = BM == 64 ? walk_grid(items, S * TiledCfg<BM, WN, WM>::FRAGS * 1024)
                             : (items + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL((expert_tiled_kernel<BM, WN, WM, S, UP, WPOL>), dim3((unsigned)grid),
                     dim3(TiledCfg<BM, WN, WM>::THREADS), 0, s, src, w, sorted_ids, block_expert,
                     tiles, num_tiles, n_ntiles, K, ncols, I, top_k, block, act, y, y0);
  return hipGetLastError();
}

template <int BM, bool UP, int WPOL>
static hipError_t launch_tiled_reg(const uint16_t* src, const uint16_t* w,
                                   const int32_t* sorted_ids, const int32_t* block_expert,
                                   const int2* tiles, const int32_t* num_tiles, int max_tiles,
                                   int K, int ncols, int I, int top_k, int block, uint16_t* act,
                                   uint16_t* y, float* y0, hipStream_t s) {
  const int per_ntile = UP ? 256 : 512;
  if (K % kTileKC != 0 || (UP && I % per_ntile != 0)) return hipErrorInvalidValue;
  const int n_ntiles = (ncols + per_ntile - 1) / per_ntile;
  const long items = (long)max_tiles * n_ntiles;
  const long grid = (items + kXcds - 1) / kXcds * kXcds;  // one item per workgroup
  hipLaunchKernelGGL((expert_tiled_reg_kernel<BM, UP, WPOL>), dim3((unsigned)grid), dim3(512), 0, s,
                     src, w, sorted_ids, block_expert, tiles, num_tiles, n_ntiles, K, ncols, I,
                     top_k, block, act, y, y0);
  return hipGetLastError();
}

// Configurations, measured on MI355X at H=7168, E=256, k=16, I=2048 (two interleaved runs
// each).  Weights every token tile of an expert shares (many tokens per expert, M=2048):
// 8 waves x 512 weight rows, one workgroup per CU, default cache policy -- nontemporal
// copies cost 3 % there, 4 waves x 256 rows with a 3-chunk ring 3.5 %; the down GEMM runs
// the split-ring kernel (2,150 -> 2,075 us), the up GEMM the one-ring kernel (the split
// ring is 0.6 % slower there).  Weights read by one token tile (few tokens per expert):
// the weight copies are nontemporal (a plain read pass streams 6.95 TB/s that way against
// 6.26 TB/s).  With 64-row tiles (M=8, M=128) the up GEMM runs 4 waves x 256 weight rows
// with a 3-chunk ring (two chunks in flight): decode M=8 up 1,027 -> 925 us against the
// streaming kernels, M=128 2,458 -> 2,181 us; the down GEMM 8 waves x 512 rows (M=8:
// 499 -> 459 us; the split ring loses 2 % there).  With 128-row tiles (M=512) both GEMMs
// run the split-ring kernel: up 2,549 -> 2,428 us, down 1,455 -> 1,400 us.
constexpr int kTileWN = 8;
constexpr int kTileStages = 2;

int tiled_up_columns() { return 32 * kTileWN; }

hipError_t launch_expert_up_selfroute(const uint16_t* x, const uint16_t* w13, const int32_t* ids,
                                      int M, int H, int E, int I, int top_k, int block,
                                      int32_t* sorted_ids, int32_t* block_expert,
                                      int32_t* num_padded, int2* tiles, int32_t* num_tiles,
                                      uint16_t* act, hipStream_t s) {
  constexpr int BM = 64, WN = 4;
  const int n = M * top_k;
  const int per_ntile = 32 * WN;
  if (n > kSelfRouteMaxIds || E > kSelfRouteMaxE || I % per_ntile != 0) return hipErrorInvalidValue;
  const int n_ntiles = I / per_ntile;
  const long grid = walk_grid((long)tile_capacity(n, E, BM) * n_ntiles, 160 * 1024);
  hipLaunchKernelGGL((expert_up_selfroute_kernel<BM, WN, 3, kNT>), dim3((unsigned)grid),
                     dim3(TiledCfg<BM, WN, 1>::THREADS), 0, s, x, w13, ids, n, E, block,
                     n_ntiles, H, I, top_k, sorted_ids, block_expert, num_padded, tiles,
                     num_tiles, act);
  return hipGetLastError();
}


hipError_t launch_expert_up_tiled(const uint16_t* x, const uint16_t* w13, const int32_t* sorted_ids,
                                  const int32_t* block_expert, const int2* tiles,
                                  const int32_t* num_tiles, int max_tiles, int tile_rows,
                                  bool stream_weights, int M, int H, int I, int top_k, int block,
                                  uint16_t* act, hipStream_t s) {
  (void)M;
#define MOE_UP(BM, WN, S, POL)                                                                   \
  return launch_tiled<BM, WN, 1, S, true, POL>(x, w13, sorted_ids, block_expert, tiles,         \
                                               num_tiles, max_tiles, H, I, I, top_k, block, act, \
                                               nullptr, nullptr, s)
  if (tile_rows == 64) {
    if (stream_weights) MOE_UP(64, 4, 3, kNT);
    MOE_UP(64, kTileWN, kTileStages, 0);
  }
  if (tile_rows == 128) {
    if (stream_weights && H % kTileKC == 0)
      return launch_tiled_reg<128, true, kNT>(x, w13, sorted_ids, block_expert, tiles, num_tiles,
                                              max_tiles, H, I, I, top_k, block, act, nullptr,
                                              nullptr, s);
    if (stream_weights) MOE_UP(128, 4, 3, kNT);
    MOE_UP(128, kTileWN, kTileStages, 0);
  }
#undef MOE_UP
  return hipErrorInvalidValue;
}

hipError_t launch_expert_down_tiled(const uint16_t* act, const uint16_t* w2,
                                    const int32_t* sorted_ids, const int32_t* block_expert,
                                    const int2* tiles, const int32_t* num_tiles, int max_tiles,
                                    int tile_rows, bool stream_weights, int M, int H, int I,
                                    int top_k, int block, uint16_t* y, float* y0,
                                    hipStream_t s) {
  (void)M;
#define MOE_DOWN(BM, POL)                                                                       \
  return launch_tiled<BM, kTileWN, 1, kTileStages, false, POL>(act, w2, sorted_ids, block_expert, \
                                                               tiles, num_tiles, max_tiles, I, H, \
                                                               I, top_k, block, nullptr, y, y0, s)
  if (tile_rows == 64) {
    if (stream_weights) MOE_DOWN(64, kNT);
    MOE_DOWN(64, 0);
  }
  if (tile_rows == 128) {
    if (I % kTileKC == 0) {
      if (stream_weights)
        return launch_tiled_reg<128, false, kNT>(act, w2, sorted_ids, block_expert, tiles,
                                                 num_tiles, max_tiles, I, H, I, top_k, block,
                                                 nullptr, y, y0, s);
      return launch_tiled_reg<128, false, 0>(act, w2, sorted_ids, block_expert, tiles, num_tiles,
                                             max_tiles, I, H, I, top_k, block, nullptr, y, y0, s);
    }
    if (stream_weights) MOE_DOWN(128, kNT);
    MOE_DOWN(128, 0);
  }
#undef MOE_DOWN
  return hipErrorInvalidValue;
}

template <int BM, bool UP>
static hipError_t launch_tiled_mx(const uint16_t* src, const uint8_t* wc, const uint8_t* ws,
                                  const int32_t* sorted_ids, const int32_t* block_expert,
                                  const int2* tiles, const int32_t* num_tiles, int max_tiles, int K,
                                  int ncols, int I, int top_k, int block, uint16_t* act, float* y,
                                  hipStream_t s) {
  const int per_ntile = UP ? 32 * kTileWN : 64 * kTileWN;
  if (K % 256 != 0 || (UP && I % per_ntile != 0) || (uintptr_t)ws % 8 != 0)
    return hipErrorInvalidValue;
  const int n_ntiles = (ncols + per_ntile - 1) / per_ntile;
  const long total = (long)max_tiles * n_ntiles;
  const long grid = (total + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL((expert_tiled_mx_kernel<BM, kTileWN, 1, UP>), dim3((unsigned)grid),
                     dim3(TiledCfg<BM, kTileWN, 1>::THREADS), 0, s, src, wc, ws, sorted_ids,
                     block_expert, tiles, num_tiles, n_ntiles, K, ncols, I, top_k, block, act, y);
  return hipGetLastError();
}

hipError_t launch_expert_up_tiled_mx(const uint16_t* x, const uint8_t* w13c, const uint8_t* w13s,
                                     const int32_t* sorted_ids, const int32_t* block_expert,
                                     const int2* tiles, const int32_t* num_tiles, int max_tiles,
                                     int tile_rows, int M, int H, int I, int top_k, int block,
                                     uint16_t* act, hipStream_t s) {
  (void)M;
  if (tile_rows == 128)
    return launch_tiled_mx<128, true>(x, w13c, w13s, sorted_ids, block_expert, tiles, num_tiles,
                                      max_tiles, H, I, I, top_k, block, act, nullptr, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
