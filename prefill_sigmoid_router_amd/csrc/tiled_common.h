// Work distribution and copy helpers shared by the LDS-tiled grouped GEMMs (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace moe {

constexpr int kXcds = 8;  // MI355X: 8 XCDs; the hardware hands workgroup p to XCD p % 8

typedef __attribute__((address_space(1))) void global_void;
typedef __attribute__((address_space(3))) void lds_void;

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Work items (tile ti, N tile ntile), live_items = ntiles_live * n_ntiles of them, walked by
// a grid of any multiple of 8 workgroups: each XCD takes an equal contiguous share of the
// items, N tile by N tile, and its workgroups step through that share with a stride of
// their count (the count of live tiles is read on the device).  A grid as large as the items gives
// one item per workgroup; the launchers use one workgroup per CU instead, so a workgroup's
// epilogue stores drain while its next item's first copies are in flight (a wave that ends
// waits for its outstanding stores, holding the CU's LDS meanwhile).
struct TiledWalk {
  int ntiles_live, live, per_xcd, first, slot, stride;
  __device__ TiledWalk(int ntl, int n_ntiles)
      : ntiles_live(ntl), live(ntl * n_ntiles), per_xcd((live + kXcds - 1) / kXcds),
        first((blockIdx.x % kXcds) * per_xcd), slot(blockIdx.x / kXcds),
        stride(gridDim.x / kXcds) {}
  // this workgroup's next item; false once its share is done
  __device__ bool next(int& ntile, int& ti) {
    if (slot >= per_xcd) return false;
    const int logical = first + slot;
    if (logical >= live) return false;
    slot += stride;
    ntile = logical / ntiles_live;
    ti = logical % ntiles_live;
    return true;
  }
};

// Grid of the item-walking kernels: at most as many workgroups as fit on the device at once
// (the CU count times the workgroups one CU's 160 KiB of LDS holds, a multiple of the 8
// XCDs), and no more than the items need.
inline long walk_grid(long items, size_t lds_bytes) {
  const long all = (items + kXcds - 1) / kXcds * kXcds;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < kXcds)
    return all;
  const long per_cu = lds_bytes > 0 ? (long)((160 * 1024) / lds_bytes) : 1;
  const long resident = (long)cus * (per_cu > 0 ? per_cu : 1) / kXcds * kXcds;
  return all < resident ? all : resident;
}

}  // namespace moe
