// Internal launchers of the routed-MoE kernels (host side, C++ linkage).  The C ABI in
// moe_api.hip validates arguments and then calls these; each returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Router: top-k ids / renormalised sigmoid weights.  `keys` is scratch of
// kRouteScratchPerPair bytes per (token, expert): fp64 keys below the many-token
// threshold, fp32 partial logits and |x|.|w| sums above it.
constexpr int kRouteScratchPerPair = 32;
hipError_t launch_route(const uint16_t* x, const uint16_t* wr, const float* bias, int M, int H,
                        int E, int top_k, int32_t* ids, float* w, double* keys, hipStream_t s);

// Expert-major plan of the flat ids [n]; sentinel = n.  When `tiles` is not null the
// kernel also lists the row tiles of height tile_rows holding real entries
// ({first plan row, real rows}) and their count; at most tile_capacity(n, E, tile_rows).
// When `tile_groups` is not null too, entry t holds the expert of tile t as {its first
// tile, its number of tiles} (tiles of one expert are consecutive).
hipError_t launch_align(const int32_t* ids, int n, int E, int block, int32_t* sorted_ids,
                        int32_t* block_expert, int32_t* num_padded, int tile_rows, int2* tiles,
                        int32_t* num_tiles, hipStream_t s, int2* tile_groups = nullptr);

inline int tile_capacity(int n, int E, int tile_rows) {
  return (n + tile_rows - 1) / tile_rows + (n < E ? n : E);
}

// Grouped up-GEMM + SwiGLU over the plan: act [capacity, I] bf16.  Work items are the
// 16-row tiles of `tiles` (at most max_tiles of them), or, with tiles == nullptr, the
// max_tiles consecutive 16-row slices of the plan.
hipError_t launch_expert_up(const uint16_t* x, const uint16_t* w13, const int32_t* sorted_ids,
                            const int32_t* block_expert, const int32_t* num_padded,
                            const int2* tiles, const int32_t* num_tiles, int max_tiles, int M,
                            int H, int I, int top_k, int block, uint16_t* act, hipStream_t s);

// Grouped down-GEMM over the plan: y [M*top_k, H] in fp32 (moe_expert_down), or, for
// moe_forward (like every down GEMM of its other paths), each token's first pick in fp32 at
// row t of y0 [M, H] and the other picks in bf16 at their rows of y (see y_row).  Work
// items as for the up GEMM.
hipError_t launch_expert_down(const uint16_t* act, const uint16_t* w2, const int32_t* sorted_ids,
                              const int32_t* block_expert, const int32_t* num_padded,
                              const int2* tiles, const int32_t* num_tiles, int max_tiles, int M,
                              int H, int I, int top_k, int block, float* y, hipStream_t s);
hipError_t launch_expert_down(const uint16_t* act, const uint16_t* w2, const int32_t* sorted_ids,
                              const int32_t* block_expert, const int32_t* num_padded,
                              const int2* tiles, const int32_t* num_tiles, int max_tiles, int M,
                              int H, int I, int top_k, int block, uint16_t* y, float* y0,
                              hipStream_t s);

// LDS-tiled variants for plans whose experts carry many tokens: work items are the tiles
// of height tile_rows (64 or 128) of `tiles`.  The up variant needs I to be a multiple of
// tiled_up_columns().
int tiled_up_columns();
// stream_weights: each expert's weights are read by about one token tile, so they are
// copied nontemporally (and the up GEMM uses its streaming configuration).
hipError_t launch_expert_up_tiled(const uint16_t* x, const uint16_t* w13, const int32_t* sorted_ids,
                                  const int32_t* block_expert, const int2* tiles,
                                  const int32_t* num_tiles, int max_tiles, int tile_rows,
                                  bool stream_weights, int M, int H, int I, int top_k, int block,
                                  uint16_t* act, hipStream_t s);
hipError_t launch_expert_down_tiled(const uint16_t* act, const uint16_t* w2,
                                    const int32_t* sorted_ids, const int32_t* block_expert,
                                    const int2* tiles, const int32_t* num_tiles, int max_tiles,
                                    int tile_rows, bool stream_weights, int M, int H, int I,
                                    int top_k, int block, uint16_t* y, float* y0,
                                    hipStream_t s);

// Self-routing variant of the tiled up GEMM for few ids (the align step fused into it):
// from the flat ids [M * top_k] it writes the same plan and tile list (tile height 64) as
// launch_align, and act as launch_expert_up_tiled with streamed weights.  Needs
// M * top_k <= kSelfRouteMaxIds, E <= kSelfRouteMaxE and I a multiple of 128.
constexpr int kSelfRouteMaxIds = 2048;
constexpr int kSelfRouteMaxE = 1024;
constexpr int kSelfRouteTileRows = 64;
hipError_t launch_expert_up_selfroute(const uint16_t* x, const uint16_t* w13, const int32_t* ids,
                                      int M, int H, int E, int I, int top_k, int block,
                                      int32_t* sorted_ids, int32_t* block_expert,
                                      int32_t* num_padded, int2* tiles, int32_t* num_tiles,
                                      uint16_t* act, hipStream_t s);

// The LDS-tiled up GEMM on MXFP8 weights (codes dequantized into the LDS tiles; tile_rows
// 128); H a multiple of 256, scales 8-byte aligned.
hipError_t launch_expert_up_tiled_mx(const uint16_t* x, const uint8_t* w13c, const uint8_t* w13s,
                                     const int32_t* sorted_ids, const int32_t* block_expert,
                                     const int2* tiles, const int32_t* num_tiles, int max_tiles,
                                     int tile_rows, int M, int H, int I, int top_k, int block,
                                     uint16_t* act, hipStream_t s);

// MXFP8 GEMMs with the codes copied whole lines at a time into LDS and dequantized from
// there into the MFMA operands; work items are the tiles of height tile_rows (32, 64 or
// 128) of `tiles`; stream_weights: copy the codes nontemporally (each expert's weights are
// read by about one token tile).  H and I multiples of 128, scales 4-byte aligned.
// moe_forward_mx uses them below 16 tokens per expert, at tile height kMxDecodeTileRows.
constexpr int kMxDecodeTileRows = 32;
hipError_t launch_expert_up_mx_lds(const uint16_t* x, const uint8_t* w13c, const uint8_t* w13s,
                                   const int32_t* sorted_ids, const int32_t* block_expert,
                                   const int2* tiles, const int32_t* num_tiles, int max_tiles,
                                   int tile_rows, bool stream_weights, int H, int I, int top_k,
                                   int block, uint16_t* act, hipStream_t s);
hipError_t launch_expert_down_mx_lds(const uint16_t* act, const uint8_t* w2c, const uint8_t* w2s,
                                     const int32_t* sorted_ids, const int32_t* block_expert,
                                     const int2* tiles, const int32_t* num_tiles, int max_tiles,
                                     int tile_rows, bool stream_weights, int H, int I, int top_k,
                                     int block, uint16_t* y, float* y0, hipStream_t s);

// MXFP8 weights (E4M3 codes, one E8M0 scale byte per 32 values along K): quantize bf16
// [rows, K] (K % 32 == 0) and dequantize back to bf16.
hipError_t launch_mx_quantize(const uint16_t* w, int64_t rows, int K, uint8_t* codes,
                              uint8_t* scales, hipStream_t s);
hipError_t launch_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int K,
                                uint16_t* w, hipStream_t s);

// Prepared ("fragment panel") expert weights: the natural stacks W13 [E, 2I, H] and
// W2 [E, H, I] re-laid-out once so that each wave of the GEMMs below streams its weight
// fragments as contiguous 1 KiB loads (H % 64 == 0, I % 256 == 0).  Element counts of the
// prepared stacks, the preparation, and the grouped GEMMs on them (tile_rows 64 or 128).
size_t frag_w13_elems(int E, int H, int I);
size_t frag_w2_elems(int E, int H, int I);
hipError_t launch_prepare_weights(const uint16_t* w13, const uint16_t* w2, int E, int H, int I,
                                  uint16_t* w13p, uint16_t* w2p, hipStream_t s);
// Work items (tile, N tile) walk expert by expert (tile_groups of launch_align).
hipError_t launch_expert_up_frag(const uint16_t* x, const uint16_t* w13p, const int32_t* sorted_ids,
                                 const int32_t* block_expert, const int2* tiles,
                                 const int2* tile_groups, const int32_t* num_tiles, int max_tiles,
                                 int tile_rows, bool stream_weights, int H, int I, int top_k,
                                 int block, uint16_t* act, hipStream_t s);
hipError_t launch_expert_down_frag(const uint16_t* act, const uint16_t* w2p,
                                   const int32_t* sorted_ids, const int32_t* block_expert,
                                   const int2* tiles, const int2* tile_groups,
                                   const int32_t* num_tiles, int max_tiles, int tile_rows,
                                   bool stream_weights, int H, int I, int top_k, int block,
                                   uint16_t* y, float* y0, hipStream_t s);

// MXFP4 expert weights in the same panel order (E2M1 codes, 4 bytes per lane and tile; E8M0
// scale bytes per 32-value block): sizes, quantization from / dequantization to the natural
// stacks (w13 true: W13 [E, 2I, H], false: W2 [E, H, I]), and the grouped GEMMs on them.
size_t mx4_codes_bytes(int E, int H, int I, bool w13);
size_t mx4_scales_bytes(int E, int H, int I, bool w13);
hipError_t launch_mx4_quantize(const uint16_t* w, bool w13, int E, int H, int I, uint8_t* codes,
                               uint8_t* scales, hipStream_t s);
hipError_t launch_mx4_dequantize(const uint8_t* codes, const uint8_t* scales, bool w13, int E,
                                 int H, int I, uint16_t* w, hipStream_t s);
// MXFP8 expert weights in the panel order (E4M3 codes, 8 bytes per lane and tile; scale
// bytes as for MXFP4), re-laid-out from the natural MXFP8 stacks of launch_mx_quantize
// (codes [rows, K], scale bytes [rows, K/32]); scale panels are mx4_scales_bytes long.
size_t mx8_codes_bytes(int E, int H, int I, bool w13);
hipError_t launch_mx8_prepare(const uint8_t* codes, const uint8_t* scales, bool w13, int E, int H,
                              int I, uint8_t* pcodes, uint8_t* pscales, hipStream_t s);
// The grouped GEMMs on MXFP4 (fp4) or MXFP8 panels.
hipError_t launch_expert_up_frag_mx(const uint16_t* x, const uint8_t* w13c, const uint8_t* w13s,
                                   bool fp4, const int32_t* sorted_ids,
                                   const int32_t* block_expert, const int2* tiles,
                                   const int2* tile_groups, const int32_t* num_tiles,
                                   int max_tiles, int tile_rows, bool stream_weights, int H, int I,
                                   int top_k, int block, uint16_t* act, hipStream_t s);
hipError_t launch_expert_down_frag_mx(const uint16_t* act, const uint8_t* w2c, const uint8_t* w2s,
                                     bool fp4, const int32_t* sorted_ids,
                                     const int32_t* block_expert, const int2* tiles,
                                     const int2* tile_groups, const int32_t* num_tiles,
                                     int max_tiles, int tile_rows, bool stream_weights, int H,
                                     int I, int top_k, int block, uint16_t* y, float* y0,
                                     hipStream_t s);

// Weighted top-k combine + residual add + RMSNorm over fp32 rows of y, or over moe_forward's
// split rows (first picks in fp32 in y0, the others in bf16 in y).
hipError_t launch_finalize(const float* y, const float* topk_w, const uint16_t* residual,
                           const uint16_t* norm_w, float eps, int M, int H, int top_k,
                           uint16_t* out, uint16_t* residual_out, hipStream_t s);
hipError_t launch_finalize(const uint16_t* y, const float* y0, const float* topk_w,
                           const uint16_t* residual, const uint16_t* norm_w, float eps, int M,
                           int H, int top_k, uint16_t* out, uint16_t* residual_out,
                           hipStream_t s);
// The same step for fewer tokens than CUs: rows split into slices over (slice, token)
// workgroups, then a second kernel scales; scratch of finalize_slices_scratch_bytes.
constexpr int kFinSlicesMaxTokens = 256;
size_t finalize_slices_scratch_bytes(int M, int H);
hipError_t launch_finalize_slices(const float* y, const float* topk_w, const uint16_t* residual,
                                  const uint16_t* norm_w, float eps, int M, int H, int top_k,
                                  uint16_t* out, uint16_t* residual_out, float* scratch,
                                  hipStream_t s);
hipError_t launch_finalize_slices(const uint16_t* y, const float* y0, const float* topk_w,
                                  const uint16_t* residual, const uint16_t* norm_w, float eps,
                                  int M, int H, int top_k, uint16_t* out, uint16_t* residual_out,
                                  float* scratch, hipStream_t s);

}  // namespace moe
