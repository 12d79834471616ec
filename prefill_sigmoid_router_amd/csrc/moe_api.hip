// C ABI of the routed-MoE layer (declared in include/moe.h): host-side validation,
// workspace carve-up and stream-ordered launches.  Nothing here allocates device memory
// or synchronises the host.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/moe.h"
#include "launchers.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxE = 1024;
constexpr int kMaxH = 16384;

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool sizes_ok(int32_t M, int32_t H, int32_t E, int32_t I, int32_t top_k) {
  if (M < 0 || E < 1 || E > kMaxE || top_k < 1 || top_k > E) return false;
  if (H < 8 || H > kMaxH || H % 8 != 0) return false;
  if (I < 16 || I % 16 != 0) return false;
  if ((int64_t)M * top_k >= ((int64_t)1 << 31)) return false;
  return true;
}

bool gemm_block_ok(int32_t block) {
  return block == 16 || block == 32 || block == 64 || block == 128;
}

size_t capacity_of(int32_t M, int32_t top_k, int32_t E, int32_t block) {
  const int64_t n = (int64_t)M * top_k;
  const int64_t touched = n < E ? n : E;
  const int64_t cap = n + touched * (block - 1);
  return (size_t)round_up((size_t)cap, (size_t)block);
}

// Workspace layout of moe_forward; every region starts on a 256-byte boundary.
struct Layout {
  size_t keys, ids, w, sorted, bexp, npad, tiles, groups, ntiles, act, y, y0, fin, total;
  int max_tiles;
};

Layout layout_of(int32_t M, int32_t H, int32_t E, int32_t I, int32_t top_k, int32_t block) {
  Layout L;
  const size_t n = (size_t)M * top_k;
  const size_t cap = capacity_of(M, top_k, E, block);
  size_t off = 0;
  L.keys = off;   off += round_up((size_t)M * E * moe::kRouteScratchPerPair, kAlign);
  L.ids = off;    off += round_up(n * sizeof(int32_t), kAlign);
  L.w = off;      off += round_up(n * sizeof(float), kAlign);
  L.sorted = off; off += round_up(cap * sizeof(int32_t), kAlign);
  L.bexp = off;   off += round_up((cap / block) * sizeof(int32_t), kAlign);
  L.npad = off;   off += kAlign;
  L.max_tiles = moe::tile_capacity((int)n, E, 16);
  L.tiles = off;  off += round_up((size_t)L.max_tiles * sizeof(int2), kAlign);
  L.groups = off; off += round_up((size_t)L.max_tiles * sizeof(int2), kAlign);  // expert of each tile
  L.ntiles = off; off += kAlign;
  L.act = off;    off += round_up(cap * (size_t)I * sizeof(uint16_t), kAlign);
  L.y = off;      off += round_up(n * (size_t)H * sizeof(uint16_t), kAlign);  // bf16 y
  L.y0 = off;     off += round_up((size_t)M * H * sizeof(float), kAlign);     // first picks
  L.fin = off;    // z and per-slice sums of the sliced finalize (few tokens only)
  if (M < moe::kFinSlicesMaxTokens) off += round_up(moe::finalize_slices_scratch_bytes(M, H), kAlign);
  L.total = off;
  return L;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }



// Grouped-GEMM kernels by expected tokens per expert (M * top_k / E), the M-range
// dispatch pattern of the FlashInfer MNNVL finalize presets (thresholds measured on
// MI355X at H=7168, I=2048, E=256).  Returns the token-tile height: 64 or 128 for the
// LDS-tiled kernels, 16 for the weight-streaming kernels, 32 for the MXFP8 kernels of few
// tokens per expert.  bf16 weights use the tiled kernels at every size (with nontemporal
// weight copies they beat the streaming kernels even at decode: M=8 layer 1,551 -> 1,405
// us); the streaming kernels serve I that is not a multiple of 256.  MXFP8 weights run the
// kernels that copy the codes into LDS and dequantize them into the MFMA operands -- 32-row
// tiles below 16 tokens per expert (M=8 layer 867 -> 773-790 us, M=128 2,528 -> 1,900 us
// against the streaming MXFP8 kernels they replaced), 64-row tiles up to 63 (M=512 3,399 ->
// 2,790 us against the kernels that dequantize into the LDS tiles; 2,987 with 128-row
// tiles), 128-row tiles from 64 (M=2048: 64-row tiles 7 % slower) -- and there the up GEMM
// runs the dequantize-into-LDS kernel, 2 % faster when the tiles of a hot expert share its
// codes (M=2048 up 3,368 against 3,445 us).
int gemm_tile_rows(int32_t M, int32_t E, int32_t top_k, int32_t I, bool mx) {
  if (I % moe::tiled_up_columns() != 0) return 16;
  const int64_t per_expert = (int64_t)M * top_k / E;
  if (mx) return per_expert < 16 ? moe::kMxDecodeTileRows : per_expert < 64 ? 64 : 128;
  if (per_expert < 32) return 64;
  return 128;
}

// Self-routing (align fused into the up GEMM, bf16 weights): 64-row tiles with streamed
// weights and at most this many flat ids (measured: -3 us per layer at 128 ids, +16 us at
// 2048).
constexpr int kSelfRouteIds = 256;
static_assert(kSelfRouteIds <= moe::kSelfRouteMaxIds, "self-routing id limit");

// Token-tile height of the fragment GEMMs on panels, by weight format (16 bf16, 8 MXFP8,
// 4 MXFP4).  Narrow weights make a hot expert's extra tiles cheap in weight bytes, so the
// MX formats take 64-row tiles (less padding) below 64 tokens per expert (measured: MXFP4
// at M=512 2,326 -> 1,800 us per layer, MXFP8 2,775 -> 2,588 us) and 128-row tiles from 64,
// where the up GEMM's per-expert cache policy favours them (M=2048: MXFP8 4,428 -> 4,180 us,
// MXFP4 3,471 -> 3,268 us); bf16 keeps gemm_tile_rows.
int panel_tile_rows(int32_t M, int32_t E, int32_t top_k, int32_t I, int bits) {
  const int64_t per_expert = (int64_t)M * top_k / E;
  if (bits == 4 || bits == 8) return per_expert < 64 ? 64 : 128;
  return gemm_tile_rows(M, E, top_k, I, false);
}

bool stream_weights(int32_t M, int32_t E, int32_t top_k, int trows) {
  return (int64_t)M * top_k / E < trows / 2;
}

bool self_routes(int32_t M, int32_t E, int32_t top_k, int32_t I) {
  const int trows = gemm_tile_rows(M, E, top_k, I, false);
  return trows == moe::kSelfRouteTileRows && stream_weights(M, E, top_k, trows) &&
         (int64_t)M * top_k <= kSelfRouteIds && I % 128 == 0;
}

}  // namespace

extern "C" {

const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument (size, pointer, alignment or scalar out of range)";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration (no kernel built for it)";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch or event call failed";
    default: return "unknown status";
  }
}

int moe_abi_version(void) { return 108; }

size_t moe_align_capacity(int32_t M, int32_t top_k, int32_t E, int32_t block) {
  if (M < 0 || top_k < 1 || E < 1 || block < 1) return 0;
  if ((int64_t)M * top_k >= ((int64_t)1 << 31)) return 0;
  return capacity_of(M, top_k, E, block);
}

size_t moe_route_workspace_bytes(int32_t M, int32_t E) {
  if (M < 0 || E < 1 || E > kMaxE) return 0;
  return round_up((size_t)M * E * moe::kRouteScratchPerPair, kAlign) + kAlign;
}

int32_t moe_gemm_tile_rows(int32_t M, int32_t E, int32_t top_k, int32_t I) {
  if (M < 0 || E < 1 || E > kMaxE || top_k < 1 || top_k > E || I < 16 || I % 16 != 0) return 0;
  return gemm_tile_rows(M, E, top_k, I, false);
}

int32_t moe_gemm_tile_rows_mx(int32_t M, int32_t E, int32_t top_k, int32_t I) {
  if (M < 0 || E < 1 || E > kMaxE || top_k < 1 || top_k > E || I < 256 || I % 256 != 0) return 0;
  return gemm_tile_rows(M, E, top_k, I, true);
}

int32_t moe_gemm_tile_rows_panels(int32_t M, int32_t E, int32_t top_k, int32_t I,
                                  int32_t weight_bits) {
  if (M < 0 || E < 1 || E > kMaxE || top_k < 1 || top_k > E || I < 256 || I % 256 != 0) return 0;
  if (weight_bits != 16 && weight_bits != 8 && weight_bits != 4) return 0;
  return panel_tile_rows(M, E, top_k, I, weight_bits);
}

int32_t moe_forward_self_routes(int32_t M, int32_t E, int32_t top_k, int32_t I) {
  if (M < 0 || E < 1 || E > kMaxE || top_k < 1 || top_k > E || I < 16 || I % 16 != 0) return 0;
  return self_routes(M, E, top_k, I) ? 1 : 0;
}

size_t moe_workspace_bytes(int32_t M, int32_t H, int32_t E, int32_t I, int32_t top_k,
                           int32_t block) {
  if (!sizes_ok(M, H, E, I, top_k) || !gemm_block_ok(block)) return 0;
  return layout_of(M, H, E, I, top_k, block).total;
}

int moe_route(const uint16_t* x, const uint16_t* router_w, const float* router_bias,
              int32_t M, int32_t H, int32_t E, int32_t top_k, int32_t* topk_ids, float* topk_w,
              void* workspace, size_t workspace_bytes, moe_stream_t stream) {
  if (M < 0 || E < 1 || E > kMaxE || top_k < 1 || top_k > E || H < 8 || H > kMaxH ||
      H % 8 != 0 || (int64_t)M * top_k >= ((int64_t)1 << 31))
    return MOE_ERR_INVALID_ARG;
  if (M == 0) return MOE_OK;
  if (!x || !router_w || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(router_w, 16) || !aligned(topk_ids, 4) || !aligned(topk_w, 4) ||
      (router_bias && !aligned(router_bias, 4)))
    return MOE_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, 16) || workspace_bytes < moe_route_workspace_bytes(M, E))
    return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_route(x, router_w, router_bias, M, H, E, top_k, topk_ids, topk_w,
                                      static_cast<double*>(workspace), (hipStream_t)stream));
}

int moe_align(const int32_t* topk_ids, int32_t M, int32_t top_k, int32_t E, int32_t block,
              int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
              moe_stream_t stream) {
  if (M < 0 || top_k < 1 || E < 1 || E > kMaxE || block < 1 ||
      (int64_t)M * top_k >= ((int64_t)1 << 31))
    return MOE_ERR_INVALID_ARG;
  if (!topk_ids || !sorted_ids || !block_expert || !num_padded) return MOE_ERR_INVALID_ARG;
  if (!aligned(topk_ids, 4) || !aligned(sorted_ids, 4) || !aligned(block_expert, 4) ||
      !aligned(num_padded, 4))
    return MOE_ERR_INVALID_ARG;
  if (capacity_of(M, top_k, E, block) >= ((size_t)1 << 31)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_align(topk_ids, M * top_k, E, block, sorted_ids, block_expert,
                                      num_padded, 16, nullptr, nullptr, (hipStream_t)stream));
}

int moe_expert_up(const uint16_t* x, const uint16_t* w13, const int32_t* sorted_ids,
                  const int32_t* block_expert, const int32_t* num_padded, int32_t M, int32_t H,
                  int32_t E, int32_t I, int32_t top_k, int32_t block, int32_t capacity,
                  uint16_t* act, moe_stream_t stream) {
  if (!sizes_ok(M, H, E, I, top_k)) return MOE_ERR_INVALID_ARG;
  if (!gemm_block_ok(block)) return MOE_ERR_UNSUPPORTED;
  if (capacity < 0 || capacity % block != 0 ||
      (size_t)capacity < capacity_of(M, top_k, E, block))
    return MOE_ERR_INVALID_ARG;
  if (M == 0) return MOE_OK;
  if (!x || !w13 || !sorted_ids || !block_expert || !num_padded || !act) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w13, 16) || !aligned(act, 16)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_expert_up(x, w13, sorted_ids, block_expert, num_padded, nullptr,
                                          nullptr, capacity / 16, M, H, I, top_k, block, act,
                                          (hipStream_t)stream));
}

int moe_expert_down(const uint16_t* act, const uint16_t* w2, const int32_t* sorted_ids,
                    const int32_t* block_expert, const int32_t* num_padded, int32_t M, int32_t H,
                    int32_t E, int32_t I, int32_t top_k, int32_t block, int32_t capacity,
                    float* y, moe_stream_t stream) {
  if (!sizes_ok(M, H, E, I, top_k)) return MOE_ERR_INVALID_ARG;
  if (!gemm_block_ok(block)) return MOE_ERR_UNSUPPORTED;
  if (capacity < 0 || capacity % block != 0 ||
      (size_t)capacity < capacity_of(M, top_k, E, block))
    return MOE_ERR_INVALID_ARG;
  if (M == 0) return MOE_OK;
  if (!act || !w2 || !sorted_ids || !block_expert || !num_padded || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned(act, 16) || !aligned(w2, 16) || !aligned(y, 16)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_expert_down(act, w2, sorted_ids, block_expert, num_padded, nullptr,
                                            nullptr, capacity / 16, M, H, I, top_k, block, y,
                                            (hipStream_t)stream));
}

int moe_finalize(const float* y, const float* topk_w, const uint16_t* residual,
                 const uint16_t* norm_w, float eps, int32_t M, int32_t H, int32_t top_k,
                 uint16_t* out, uint16_t* residual_out, moe_stream_t stream) {
  if (M < 0 || top_k < 1 || H < 8 || H > kMaxH || H % 8 != 0 || !(eps > 0.0f) || !isfinite(eps) ||
      (int64_t)M * top_k >= ((int64_t)1 << 31))
    return MOE_ERR_INVALID_ARG;
  if (M == 0) return MOE_OK;
  if (!y || !topk_w || !residual || !norm_w || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned(y, 16) || !aligned(residual, 16) || !aligned(norm_w, 16) || !aligned(out, 16) ||
      (residual_out && !aligned(residual_out, 16)) || !aligned(topk_w, 4))
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_finalize(y, topk_w, residual, norm_w, eps, M, H, top_k, out,
                                         residual_out, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Scratch of moe_forward_noalloc, for callers that cannot allocate: one static array per
// GPU the library runs on (each device holds its own copy until the process ends).  In host
// code `scratch` names a host-side stand-in, never a device address: the device address of
// each GPU's copy comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is handed to kernels.
__device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The current device's scratch address (MOE_ERR_HIP if the device or the symbol lookup fails).
int device_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::call_once(g_scratch_once[dev], [dev] {
    g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr) return MOE_ERR_HIP;
  *ptr = g_scratch_ptr[dev];
  return MOE_OK;
}

// Expert weights of one call: bf16 (w13, w2) or MXFP8 (codes and scale bytes).
struct ExpertWeights {
  const uint16_t* w13 = nullptr;
  const uint16_t* w2 = nullptr;
  const uint8_t* w13c = nullptr;
  const uint8_t* w13s = nullptr;
  const uint8_t* w2c = nullptr;
  const uint8_t* w2s = nullptr;
  bool prepared = false;  // w13 / w2 hold the fragment panels of moe_prepare_weights
  bool fp4 = false;       // w13c / w13s / w2c / w2s hold the MXFP4 panels of moe_mx4_quantize
  bool fp8p = false;      // ... the MXFP8 panels of moe_mx_prepare_weights
  bool mx() const { return w13c != nullptr && !fp4 && !fp8p; }     // natural MXFP8
  bool panels() const { return prepared || fp4 || fp8p; }
};

int forward_impl(const uint16_t* x, const uint16_t* router_w, const float* router_bias,
                 const ExpertWeights& W, const uint16_t* residual, const uint16_t* norm_w,
                 float eps, int32_t M, int32_t H, int32_t E, int32_t I, int32_t top_k,
                 int32_t block, uint16_t* out, uint16_t* residual_out, int32_t* topk_ids_out,
                 float* topk_w_out, int32_t* sorted_ids_out, int32_t* block_expert_out,
                 int32_t* num_padded_out, void* workspace, size_t workspace_bytes,
                 const moe_event_t* stage_events, moe_stream_t stream) {
  if (!sizes_ok(M, H, E, I, top_k) || !(eps > 0.0f) || !isfinite(eps)) return MOE_ERR_INVALID_ARG;
  if (!gemm_block_ok(block)) return MOE_ERR_UNSUPPORTED;
  if (W.mx() && (H % 256 != 0 || I % 256 != 0)) return MOE_ERR_UNSUPPORTED;
  if (W.panels() && (H % 64 != 0 || I % 256 != 0)) return MOE_ERR_UNSUPPORTED;
  if (M == 0) return MOE_OK;
  const bool w_ok =
      (W.fp4 || W.fp8p)
          ? (W.w13c && W.w13s && W.w2c && W.w2s && aligned(W.w13c, 16) && aligned(W.w2c, 16) &&
             aligned(W.w13s, 4) && aligned(W.w2s, 4))
      : W.mx() ? (W.w13c && W.w13s && W.w2c && W.w2s && aligned(W.w13c, 16) &&
                  aligned(W.w2c, 16) && aligned(W.w13s, 8) && aligned(W.w2s, 8))
               : (W.w13 && W.w2 && aligned(W.w13, 16) && aligned(W.w2, 16));
  if (!x || !router_w || !w_ok || !residual || !norm_w || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(router_w, 16) || !aligned(residual, 16) ||
      !aligned(norm_w, 16) || !aligned(out, 16) ||
      (residual_out && !aligned(residual_out, 16)) || (router_bias && !aligned(router_bias, 4)) ||
      (topk_ids_out && !aligned(topk_ids_out, 4)) || (topk_w_out && !aligned(topk_w_out, 4)) ||
      (sorted_ids_out && !aligned(sorted_ids_out, 4)) ||
      (block_expert_out && !aligned(block_expert_out, 4)) ||
      (num_padded_out && !aligned(num_padded_out, 4)))
    return MOE_ERR_INVALID_ARG;
  const size_t cap = capacity_of(M, top_k, E, block);
  if (cap >= ((size_t)1 << 31)) return MOE_ERR_INVALID_ARG;
  const Layout L = layout_of(M, H, E, I, top_k, block);
  if (!workspace || !aligned(workspace, kAlign) || workspace_bytes < L.total) return MOE_ERR_WORKSPACE;

  char* ws = static_cast<char*>(workspace);
  double* keys = reinterpret_cast<double*>(ws + L.keys);
  int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(ws + L.ids);
  float* w = topk_w_out ? topk_w_out : reinterpret_cast<float*>(ws + L.w);
  int32_t* sorted = sorted_ids_out ? sorted_ids_out : reinterpret_cast<int32_t*>(ws + L.sorted);
  int32_t* bexp = block_expert_out ? block_expert_out : reinterpret_cast<int32_t*>(ws + L.bexp);
  int32_t* npad = num_padded_out ? num_padded_out : reinterpret_cast<int32_t*>(ws + L.npad);
  int2* tiles = reinterpret_cast<int2*>(ws + L.tiles);
  int2* groups = reinterpret_cast<int2*>(ws + L.groups);
  int32_t* ntiles = reinterpret_cast<int32_t*>(ws + L.ntiles);
  uint16_t* act = reinterpret_cast<uint16_t*>(ws + L.act);
  uint16_t* y = reinterpret_cast<uint16_t*>(ws + L.y);
  float* y0 = reinterpret_cast<float*>(ws + L.y0);
  hipStream_t s = (hipStream_t)stream;

  auto mark = [&](int i) -> bool {
    return !stage_events || hipEventRecord((hipEvent_t)stage_events[i], s) == hipSuccess;
  };
  if (!mark(0)) return MOE_ERR_HIP;
  if (moe::launch_route(x, router_w, router_bias, M, H, E, top_k, ids, w, keys, s) != hipSuccess)
    return MOE_ERR_HIP;
  if (!mark(1)) return MOE_ERR_HIP;
  const int trows = W.panels() ? panel_tile_rows(M, E, top_k, I, W.fp4 ? 4 : W.fp8p ? 8 : 16)
                                : gemm_tile_rows(M, E, top_k, I, W.mx());
  // about one token tile per expert: each weight is read once, copied nontemporally
  // (measured: M=8/128/512 gain, M=2048 -- many tiles of a hot expert share its weights
  // through the L2 -- loses 3 %)
  const bool stream_w = stream_weights(M, E, top_k, trows);
  const int max_tiles = moe::tile_capacity(M * top_k, E, trows);
  // few ids: the up GEMM builds the plan itself (no align launch)
  const bool self_route = !W.mx() && !W.panels() && self_routes(M, E, top_k, I);
  if (!self_route &&
      moe::launch_align(ids, M * top_k, E, block, sorted, bexp, npad, trows, tiles, ntiles, s,
                        W.panels() ? groups : nullptr) != hipSuccess)
    return MOE_ERR_HIP;
  if (!mark(2)) return MOE_ERR_HIP;
  hipError_t up_err;
  if (W.fp4 || W.fp8p)
    up_err = moe::launch_expert_up_frag_mx(x, W.w13c, W.w13s, W.fp4, sorted, bexp, tiles, groups,
                                           ntiles, max_tiles, trows, stream_w, H, I, top_k, block,
                                           act, s);
  else if (W.prepared)
    up_err = moe::launch_expert_up_frag(x, W.w13, sorted, bexp, tiles, groups, ntiles, max_tiles,
                                        trows, stream_w, H, I, top_k, block, act, s);
  else if (self_route)
    up_err = moe::launch_expert_up_selfroute(x, W.w13, ids, M, H, E, I, top_k, block, sorted, bexp,
                                             npad, tiles, ntiles, act, s);
  else if (W.mx() && trows <= 64)
    up_err = moe::launch_expert_up_mx_lds(x, W.w13c, W.w13s, sorted, bexp, tiles, ntiles,
                                          max_tiles, trows, stream_w, H, I, top_k, block, act, s);
  else if (W.mx())
    up_err = moe::launch_expert_up_tiled_mx(x, W.w13c, W.w13s, sorted, bexp, tiles, ntiles,
                                            max_tiles, trows, M, H, I, top_k, block, act, s);
  else if (trows == 16)
    up_err = moe::launch_expert_up(x, W.w13, sorted, bexp, npad, tiles, ntiles, max_tiles, M, H, I,
                                   top_k, block, act, s);
  else
    up_err = moe::launch_expert_up_tiled(x, W.w13, sorted, bexp, tiles, ntiles, max_tiles, trows,
                                         stream_w, M, H, I, top_k, block, act, s);
  if (up_err != hipSuccess) return MOE_ERR_HIP;
  if (!mark(3)) return MOE_ERR_HIP;
  hipError_t down_err;
  if (W.fp4 || W.fp8p)
    down_err = moe::launch_expert_down_frag_mx(act, W.w2c, W.w2s, W.fp4, sorted, bexp, tiles,
                                               groups, ntiles, max_tiles, trows, stream_w, H, I,
                                               top_k, block, y, y0, s);
  else if (W.prepared)
    down_err = moe::launch_expert_down_frag(act, W.w2, sorted, bexp, tiles, groups, ntiles,
                                            max_tiles, trows, stream_w, H, I, top_k, block, y, y0,
                                            s);
  else if (W.mx())
    down_err = moe::launch_expert_down_mx_lds(act, W.w2c, W.w2s, sorted, bexp, tiles, ntiles,
                                              max_tiles, trows, stream_w, H, I, top_k, block, y,
                                              y0, s);
  else if (trows == 16)
    down_err = moe::launch_expert_down(act, W.w2, sorted, bexp, npad, tiles, ntiles, max_tiles, M,
                                       H, I, top_k, block, y, y0, s);
  else
    down_err = moe::launch_expert_down_tiled(act, W.w2, sorted, bexp, tiles, ntiles, max_tiles,
                                             trows, stream_w, M, H, I, top_k, block, y, y0, s);
  if (down_err != hipSuccess) return MOE_ERR_HIP;
  if (!mark(4)) return MOE_ERR_HIP;
  const hipError_t fin_err =
      M < moe::kFinSlicesMaxTokens
          ? moe::launch_finalize_slices(y, y0, w, residual, norm_w, eps, M, H, top_k, out,
                                        residual_out, reinterpret_cast<float*>(ws + L.fin), s)
          : moe::launch_finalize(y, y0, w, residual, norm_w, eps, M, H, top_k, out, residual_out,
                                 s);
  if (fin_err != hipSuccess) return MOE_ERR_HIP;
  if (!mark(5)) return MOE_ERR_HIP;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward(const uint16_t* x, const uint16_t* router_w, const float* router_bias,
                const uint16_t* w13, const uint16_t* w2, const uint16_t* residual,
                const uint16_t* norm_w, float eps, int32_t M, int32_t H, int32_t E, int32_t I,
                int32_t top_k, int32_t block, uint16_t* out, uint16_t* residual_out,
                int32_t* topk_ids_out, float* topk_w_out, int32_t* sorted_ids_out,
                int32_t* block_expert_out, int32_t* num_padded_out, void* workspace,
                size_t workspace_bytes, const moe_event_t* stage_events, moe_stream_t stream) {
  ExpertWeights W;
  W.w13 = w13;
  W.w2 = w2;
  return forward_impl(x, router_w, router_bias, W, residual, norm_w, eps, M, H, E, I, top_k, block,
                      out, residual_out, topk_ids_out, topk_w_out, sorted_ids_out,
                      block_expert_out, num_padded_out, workspace, workspace_bytes, stage_events,
                      stream);
}

int moe_forward_mx(const uint16_t* x, const uint16_t* router_w, const float* router_bias,
                   const uint8_t* w13_codes, const uint8_t* w13_scales, const uint8_t* w2_codes,
                   const uint8_t* w2_scales, const uint16_t* residual, const uint16_t* norm_w,
                   float eps, int32_t M, int32_t H, int32_t E, int32_t I, int32_t top_k,
                   int32_t block, uint16_t* out, uint16_t* residual_out, int32_t* topk_ids_out,
                   float* topk_w_out, int32_t* sorted_ids_out, int32_t* block_expert_out,
                   int32_t* num_padded_out, void* workspace, size_t workspace_bytes,
                   const moe_event_t* stage_events, moe_stream_t stream) {
  ExpertWeights W;
  W.w13c = w13_codes;
  W.w13s = w13_scales;
  W.w2c = w2_codes;
  W.w2s = w2_scales;
  if (!w13_codes) return MOE_ERR_INVALID_ARG;
  return forward_impl(x, router_w, router_bias, W, residual, norm_w, eps, M, H, E, I, top_k, block,
                      out, residual_out, topk_ids_out, topk_w_out, sorted_ids_out,
                      block_expert_out, num_padded_out, workspace, workspace_bytes, stage_events,
                      stream);
}

size_t moe_prepared_w13_bytes(int32_t E, int32_t H, int32_t I) {
  if (E < 1 || E > kMaxE || H < 64 || H > kMaxH || H % 64 != 0 || I < 256 || I % 256 != 0) return 0;
  return moe::frag_w13_elems(E, H, I) * sizeof(uint16_t);
}

size_t moe_prepared_w2_bytes(int32_t E, int32_t H, int32_t I) {
  if (E < 1 || E > kMaxE || H < 64 || H > kMaxH || H % 64 != 0 || I < 256 || I % 256 != 0) return 0;
  return moe::frag_w2_elems(E, H, I) * sizeof(uint16_t);
}

int moe_prepare_weights(const uint16_t* w13, const uint16_t* w2, int32_t E, int32_t H, int32_t I,
                        uint16_t* w13_prepared, uint16_t* w2_prepared, moe_stream_t stream) {
  if (E < 1 || E > kMaxE || H < 8 || H > kMaxH || H % 8 != 0 || I < 16 || I % 16 != 0)
    return MOE_ERR_INVALID_ARG;
  if (H % 64 != 0 || I % 256 != 0) return MOE_ERR_UNSUPPORTED;
  if ((w13 == nullptr) != (w13_prepared == nullptr) || (w2 == nullptr) != (w2_prepared == nullptr))
    return MOE_ERR_INVALID_ARG;
  if ((w13 && (!aligned(w13, 16) || !aligned(w13_prepared, 16))) ||
      (w2 && (!aligned(w2, 16) || !aligned(w2_prepared, 16))))
    return MOE_ERR_INVALID_ARG;
  if (!w13 && !w2) return MOE_OK;
  return hip_status(moe::launch_prepare_weights(w13, w2, E, H, I, w13_prepared, w2_prepared,
                                                (hipStream_t)stream));
}

int moe_forward_prepared(const uint16_t* x, const uint16_t* router_w, const float* router_bias,
                         const uint16_t* w13_prepared, const uint16_t* w2_prepared,
                         const uint16_t* residual, const uint16_t* norm_w, float eps, int32_t M,
                         int32_t H, int32_t E, int32_t I, int32_t top_k, int32_t block,
                         uint16_t* out, uint16_t* residual_out, int32_t* topk_ids_out,
                         float* topk_w_out, int32_t* sorted_ids_out, int32_t* block_expert_out,
                         int32_t* num_padded_out, void* workspace, size_t workspace_bytes,
                         const moe_event_t* stage_events, moe_stream_t stream) {
  ExpertWeights W;
  W.w13 = w13_prepared;
  W.w2 = w2_prepared;
  W.prepared = true;
  return forward_impl(x, router_w, router_bias, W, residual, norm_w, eps, M, H, E, I, top_k, block,
                      out, residual_out, topk_ids_out, topk_w_out, sorted_ids_out,
                      block_expert_out, num_padded_out, workspace, workspace_bytes, stage_events,
                      stream);
}

int moe_mx4_weight_bytes(int32_t E, int32_t H, int32_t I, size_t* w13_codes, size_t* w13_scales,
                         size_t* w2_codes, size_t* w2_scales) {
  if (E < 1 || E > kMaxE || H < 8 || H > kMaxH || H % 8 != 0 || I < 16 || I % 16 != 0)
    return MOE_ERR_INVALID_ARG;
  if (H % 64 != 0 || I % 256 != 0) return MOE_ERR_UNSUPPORTED;
  if (w13_codes) *w13_codes = moe::mx4_codes_bytes(E, H, I, true);
  if (w13_scales) *w13_scales = moe::mx4_scales_bytes(E, H, I, true);
  if (w2_codes) *w2_codes = moe::mx4_codes_bytes(E, H, I, false);
  if (w2_scales) *w2_scales = moe::mx4_scales_bytes(E, H, I, false);
  return MOE_OK;
}

int moe_mx4_quantize(const uint16_t* w13, const uint16_t* w2, int32_t E, int32_t H, int32_t I,
                     uint8_t* w13_codes, uint8_t* w13_scales, uint8_t* w2_codes,
                     uint8_t* w2_scales, moe_stream_t stream) {
  const int st = moe_mx4_weight_bytes(E, H, I, nullptr, nullptr, nullptr, nullptr);
  if (st != MOE_OK) return st;
  if ((w13 == nullptr) != (w13_codes == nullptr) || (w13 == nullptr) != (w13_scales == nullptr) ||
      (w2 == nullptr) != (w2_codes == nullptr) || (w2 == nullptr) != (w2_scales == nullptr))
    return MOE_ERR_INVALID_ARG;
  if ((w13 && (!aligned(w13, 16) || !aligned(w13_codes, 16) || !aligned(w13_scales, 4))) ||
      (w2 && (!aligned(w2, 16) || !aligned(w2_codes, 16) || !aligned(w2_scales, 4))))
    return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (w13 && moe::launch_mx4_quantize(w13, true, E, H, I, w13_codes, w13_scales, s) != hipSuccess)
    return MOE_ERR_HIP;
  if (w2 && moe::launch_mx4_quantize(w2, false, E, H, I, w2_codes, w2_scales, s) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

int moe_mx4_dequantize(const uint8_t* codes, const uint8_t* scales, int32_t which, int32_t E,
                       int32_t H, int32_t I, uint16_t* w, moe_stream_t stream) {
  const int st = moe_mx4_weight_bytes(E, H, I, nullptr, nullptr, nullptr, nullptr);
  if (st != MOE_OK) return st;
  if ((which != 13 && which != 2) || !codes || !scales || !w || !aligned(codes, 16) ||
      !aligned(scales, 4) || !aligned(w, 16))
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_mx4_dequantize(codes, scales, which == 13, E, H, I, w,
                                               (hipStream_t)stream));
}

int moe_forward_mx4(const uint16_t* x, const uint16_t* router_w, const float* router_bias,
                    const uint8_t* w13_codes, const uint8_t* w13_scales, const uint8_t* w2_codes,
                    const uint8_t* w2_scales, const uint16_t* residual, const uint16_t* norm_w,
                    float eps, int32_t M, int32_t H, int32_t E, int32_t I, int32_t top_k,
                    int32_t block, uint16_t* out, uint16_t* residual_out, int32_t* topk_ids_out,
                    float* topk_w_out, int32_t* sorted_ids_out, int32_t* block_expert_out,
                    int32_t* num_padded_out, void* workspace, size_t workspace_bytes,
                    const moe_event_t* stage_events, moe_stream_t stream) {
  ExpertWeights W;
  W.w13c = w13_codes;
  W.w13s = w13_scales;
  W.w2c = w2_codes;
  W.w2s = w2_scales;
  W.fp4 = true;
  if (!w13_codes) return MOE_ERR_INVALID_ARG;
  return forward_impl(x, router_w, router_bias, W, residual, norm_w, eps, M, H, E, I, top_k, block,
                      out, residual_out, topk_ids_out, topk_w_out, sorted_ids_out,
                      block_expert_out, num_padded_out, workspace, workspace_bytes, stage_events,
                      stream);
}

int moe_mx_prepared_bytes(int32_t E, int32_t H, int32_t I, size_t* w13_codes,
                          size_t* w13_scales, size_t* w2_codes, size_t* w2_scales) {
  if (E < 1 || E > kMaxE || H < 8 || H > kMaxH || H % 8 != 0 || I < 16 || I % 16 != 0)
    return MOE_ERR_INVALID_ARG;
  if (H % 64 != 0 || I % 256 != 0) return MOE_ERR_UNSUPPORTED;
  if (w13_codes) *w13_codes = moe::mx8_codes_bytes(E, H, I, true);
  if (w13_scales) *w13_scales = moe::mx4_scales_bytes(E, H, I, true);
  if (w2_codes) *w2_codes = moe::mx8_codes_bytes(E, H, I, false);
  if (w2_scales) *w2_scales = moe::mx4_scales_bytes(E, H, I, false);
  return MOE_OK;
}

int moe_mx_prepare_weights(const uint8_t* w13_codes, const uint8_t* w13_scales,
                           const uint8_t* w2_codes, const uint8_t* w2_scales, int32_t E,
                           int32_t H, int32_t I, uint8_t* w13_codes_p, uint8_t* w13_scales_p,
                           uint8_t* w2_codes_p, uint8_t* w2_scales_p, moe_stream_t stream) {
  const int st = moe_mx_prepared_bytes(E, H, I, nullptr, nullptr, nullptr, nullptr);
  if (st != MOE_OK) return st;
  const bool a13 = w13_codes != nullptr, a2 = w2_codes != nullptr;
  if (a13 != (w13_scales != nullptr) || a13 != (w13_codes_p != nullptr) ||
      a13 != (w13_scales_p != nullptr) || a2 != (w2_scales != nullptr) ||
      a2 != (w2_codes_p != nullptr) || a2 != (w2_scales_p != nullptr))
    return MOE_ERR_INVALID_ARG;
  if ((a13 && (!aligned(w13_codes, 16) || !aligned(w13_codes_p, 16) || !aligned(w13_scales_p, 4))) ||
      (a2 && (!aligned(w2_codes, 16) || !aligned(w2_codes_p, 16) || !aligned(w2_scales_p, 4))))
    return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (a13 && moe::launch_mx8_prepare(w13_codes, w13_scales, true, E, H, I, w13_codes_p,
                                     w13_scales_p, s) != hipSuccess)
    return MOE_ERR_HIP;
  if (a2 && moe::launch_mx8_prepare(w2_codes, w2_scales, false, E, H, I, w2_codes_p, w2_scales_p,
                                    s) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

int moe_forward_mx_prepared(const uint16_t* x, const uint16_t* router_w, const float* router_bias,
                            const uint8_t* w13_codes_p, const uint8_t* w13_scales_p,
                            const uint8_t* w2_codes_p, const uint8_t* w2_scales_p,
                            const uint16_t* residual, const uint16_t* norm_w, float eps, int32_t M,
                            int32_t H, int32_t E, int32_t I, int32_t top_k, int32_t block,
                            uint16_t* out, uint16_t* residual_out, int32_t* topk_ids_out,
                            float* topk_w_out, int32_t* sorted_ids_out, int32_t* block_expert_out,
                            int32_t* num_padded_out, void* workspace, size_t workspace_bytes,
                            const moe_event_t* stage_events, moe_stream_t stream) {
  ExpertWeights W;
  W.w13c = w13_codes_p;
  W.w13s = w13_scales_p;
  W.w2c = w2_codes_p;
  W.w2s = w2_scales_p;
  W.fp8p = true;
  if (!w13_codes_p) return MOE_ERR_INVALID_ARG;
  return forward_impl(x, router_w, router_bias, W, residual, norm_w, eps, M, H, E, I, top_k, block,
                      out, residual_out, topk_ids_out, topk_w_out, sorted_ids_out,
                      block_expert_out, num_padded_out, workspace, workspace_bytes, stage_events,
                      stream);
}

int moe_forward_noalloc(const uint16_t* x, const uint16_t* router_w, const float* router_bias,
                        const uint16_t* w13, const uint16_t* w2, const uint16_t* residual,
                        const uint16_t* norm_w, float eps, int32_t M, int32_t H, int32_t E,
                        int32_t I, int32_t top_k, int32_t block, uint16_t* out,
                        uint16_t* residual_out, int32_t* topk_ids_out, float* topk_w_out,
                        int32_t* sorted_ids_out, int32_t* block_expert_out,
                        int32_t* num_padded_out, moe_stream_t stream) {
  if (!sizes_ok(M, H, E, I, top_k) || !(eps > 0.0f) || !isfinite(eps)) return MOE_ERR_INVALID_ARG;
  if (!gemm_block_ok(block)) return MOE_ERR_UNSUPPORTED;
  if (M == 0) return MOE_OK;
  // the sizes' workspace must fit the static scratch: checked before anything runs
  const Layout L = layout_of(M, H, E, I, top_k, block);
  if (L.total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  const int st = device_scratch(&ws);
  if (st != MOE_OK) return st;
  ExpertWeights W;
  W.w13 = w13;
  W.w2 = w2;
  return forward_impl(x, router_w, router_bias, W, residual, norm_w, eps, M, H, E, I, top_k, block,
                      out, residual_out, topk_ids_out, topk_w_out, sorted_ids_out,
                      block_expert_out, num_padded_out, ws, MOE_NOALLOC_SCRATCH_BYTES, nullptr,
                      stream);
}

int moe_mx_quantize(const uint16_t* w, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                    moe_stream_t stream) {
  if (rows < 0 || K < 32 || K % 32 != 0 || rows > ((int64_t)1 << 40) / K) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (!w || !codes || !scales || !aligned(w, 16) || !aligned(codes, 16)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_mx_quantize(w, rows, K, codes, scales, (hipStream_t)stream));
}

int moe_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t K,
                      uint16_t* w, moe_stream_t stream) {
  if (rows < 0 || K < 32 || K % 32 != 0 || rows > ((int64_t)1 << 40) / K) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (!w || !codes || !scales || !aligned(w, 16) || !aligned(codes, 16)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_mx_dequantize(codes, scales, rows, K, w, (hipStream_t)stream));
}

}  // extern "C"
