/*
 * moe.h -- C ABI of the MI355X (gfx950) routed Mixture-of-Experts layer.
 *
 * One call of moe_forward runs the routed-MoE layer of an LLM decode/prefill step on
 * one GPU, in five stream-ordered kernels (four for at most 256 flat ids on bf16 weights,
 * where the up-GEMM kernel builds the plan itself -- the self-routing up kernels of the
 * AlphaMoE page, section 6 -- and writes the same plan the align kernel would):
 *
 *   1. router: key[t,e] = sum_h x[t,h] * Wr[e,h] (+ bias[e]), accumulated in fp64;
 *      top-k by (key descending, expert id ascending); weights = sigmoid(key) of the
 *      k picks renormalised to sum 1.
 *      (sglang PR #29509 analysis, "GLM-4.7-Flash on NPU", section 2 "MoE TopK
 *      scoring function": sigmoid scoring fused with the top-k.)
 *   2. align: an expert-major token plan built from a histogram and a prefix scan,
 *      padded to the GEMM block, with a block -> expert map.
 *      (FlashInfer PR #6511 analysis, "AlphaMoE NVFP4 kernels", section 5
 *      "moe_align_block_size_kernel synchronisation" and section 6 "self-routing up
 *      kernels".)
 *   3. grouped up-GEMM with SwiGLU: act = silu(x W13[e,0:I]^T) * (x W13[e,I:2I]^T).
 *   4. grouped down-GEMM: y = act W2[e]^T, one row per (token, pick).
 *      (AlphaMoE page, sections 1-4: up kernels, down kernels, token-tile gather.)
 *   5. finalize: m = sum_j w[t,j] y[t*k+j]; z = m + residual; out = RMSNorm(z) * g.
 *      (FlashInfer PR #5701 analysis, "Kimi K3 H7168/K16 MNNVL", intro and section 3:
 *      MoE finalize followed by RMSNorm with RMS_EPS = 1e-5 and no weight offset;
 *      FlashInfer PR #4690 analysis, "MiniMax-H3 BF16 pre-attention", section 1: the
 *      RMSNorm is torch's rms_norm, eps inside the square root.)
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library keeps no
 *     reference to them after the call returns and allocates no device memory; all
 *     scratch lives in a caller-provided workspace.
 *   - bf16 values are passed as uint16_t bit patterns.  Layouts are row-major with the
 *     last dimension contiguous.  Every device pointer must be 16-byte aligned.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null stream).
 *     No entry point synchronises the host, so a call can be captured in a graph.
 *   - Arguments are validated on the host before anything is launched.  Errors are
 *     returned as status codes (never abort); on error nothing has been launched,
 *     except MOE_ERR_HIP, which reports a failed launch.
 *   - Sizes: 1 <= top_k <= E <= 1024, H % 8 == 0 and 8 <= H <= 16384, I % 16 == 0 and
 *     I >= 16, M >= 0 (M == 0 is a successful no-op), M * top_k < 2^31.  (moe_forward_mx
 *     needs H and I to be multiples of 256.)
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* moe_stream_t; /* hipStream_t */
typedef void* moe_event_t;  /* hipEvent_t  */

enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* a size, pointer or scalar is outside its documented range */
  MOE_ERR_UNSUPPORTED = -2, /* valid but not built (e.g. a block size with no kernel) */
  MOE_ERR_WORKSPACE = -3,   /* workspace pointer NULL or smaller than required */
  MOE_ERR_HIP = -4          /* a HIP launch or event call failed */
};

/* Human-readable text of a status code.  Never NULL; static storage. */
const char* moe_strerror(int status);

/* ABI version of this header (major * 100 + minor): 108. */
int moe_abi_version(void);

/*
 * Entries the align plan may need: M*top_k real entries plus at most block-1 padding
 * slots for each touched expert (at most min(E, M*top_k) experts), rounded up to a
 * whole block.  sorted_ids needs this many int32; block_expert needs capacity/block.
 * Returns 0 for invalid sizes.
 */
size_t moe_align_capacity(int32_t M, int32_t top_k, int32_t E, int32_t block);

/*
 * Workspace bytes moe_route needs: router scratch of 32 bytes per (token, expert) (fp64
 * keys, or fp32 partial logits and |x|.|w| sums for many tokens).  0 for invalid sizes.
 */
size_t moe_route_workspace_bytes(int32_t M, int32_t E);

/*
 * Workspace bytes moe_forward needs for these sizes: routing ids/weights, the plan,
 * the router keys, the bf16 SwiGLU activations [capacity, I] and the per-pick
 * down-projection rows (bf16 [M*top_k, H], each token's first pick -- its largest routing
 * weight -- in fp32 [M, H] instead).  0 for invalid sizes.
 */
size_t moe_workspace_bytes(int32_t M, int32_t H, int32_t E, int32_t I, int32_t top_k,
                           int32_t block);

/*
 * Token-tile height moe_forward uses for its grouped GEMMs at these sizes: 64 or 128
 * select the LDS-tiled MFMA kernels (64 below 32 expected tokens per expert M * top_k / E,
 * 128 from there), 16 the weight-streaming kernels, used when I is not a multiple of the
 * tiled kernels' 256 act columns.  Below half a tile of tokens per expert the tiled
 * kernels copy the weights nontemporally.  Host-only; 0 for invalid sizes.
 */
int32_t moe_gemm_tile_rows(int32_t M, int32_t E, int32_t top_k, int32_t I);
/* The same for moe_forward_mx (MXFP8 weights; I a multiple of 256, else 0): 32 below 16
 * expected tokens per expert, 64 below 64, then 128.  Its GEMMs copy the codes into LDS and
 * dequantize them into the MFMA operands, except the up GEMM at 128-row tiles, which
 * dequantizes them into the LDS tiles of the tiled kernel. */
int32_t moe_gemm_tile_rows_mx(int32_t M, int32_t E, int32_t top_k, int32_t I);
/* The same for the entry points on fragment panels: weight_bits 16 (moe_forward_prepared)
 * follows moe_gemm_tile_rows; 8 (moe_forward_mx_prepared) and 4 (moe_forward_mx4) give 64
 * below 64 expected tokens per expert, then 128.  Host-only; 0 for
 * invalid sizes, I not a multiple of 256, or another weight_bits. */
int32_t moe_gemm_tile_rows_panels(int32_t M, int32_t E, int32_t top_k, int32_t I,
                                  int32_t weight_bits);
/* 1 when moe_forward (bf16 weights) builds the plan inside its up-GEMM kernel for these
 * sizes -- the self-routing up kernels of the AlphaMoE page (FlashInfer PR #6511 analysis),
 * section 6: 64-row tiles, weights copied nontemporally, at most 256 flat ids M * top_k --
 * and so runs no align kernel; 0 when it runs the align kernel, and for invalid sizes.
 * Host-only. */
int32_t moe_forward_self_routes(int32_t M, int32_t E, int32_t top_k, int32_t I);

/*
 * Router (step 1).
 *   x          [M, H] bf16        hidden states
 *   router_w   [E, H] bf16        gate weight
 *   router_bias[E]    fp32 or NULL additive bias, used for selection and in the sigmoid
 *   topk_ids   [M, top_k] int32   out: expert ids, key descending, ties to the lower id
 *   topk_w     [M, top_k] fp32    out: sigmoid(key) renormalised over the k picks
 *   workspace  >= moe_route_workspace_bytes(M, E) bytes of device memory
 */
int moe_route(const uint16_t* x, const uint16_t* router_w, const float* router_bias,
              int32_t M, int32_t H, int32_t E, int32_t top_k,
              int32_t* topk_ids, float* topk_w,
              void* workspace, size_t workspace_bytes, moe_stream_t stream);

/*
 * Align (step 2).  Flat index i = t * top_k + j of topk_ids [M, top_k].
 *   sorted_ids  [moe_align_capacity] int32 out: expert-major plan; inside an expert the
 *               flat indices ascend; each expert's run is padded with the sentinel
 *               M*top_k up to a multiple of `block`.  Entries past num_padded are
 *               left unwritten.
 *   block_expert[capacity/block] int32 out: expert of each plan block (first
 *               num_padded/block entries written).
 *   num_padded  [1] int32 out: total plan length (a multiple of block).
 * Ids outside [0, E) are skipped (never placed).  Any block >= 1 is accepted.
 */
int moe_align(const int32_t* topk_ids, int32_t M, int32_t top_k, int32_t E, int32_t block,
              int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
              moe_stream_t stream);

/*
 * Grouped up-GEMM with SwiGLU (step 3) over an align plan.
 *   act [capacity, I] bf16 out: for every plan row r inside the 16-row groups that hold
 *   at least one real entry, act[r] = silu(x[t] W13[e,0:I]^T) * (x[t] W13[e,I:2I]^T)
 *   with t = sorted_ids[r] / top_k (rows holding the sentinel get 0).  Other rows are
 *   left unwritten.  block must be 16, 32, 64 or 128.
 */
int moe_expert_up(const uint16_t* x, const uint16_t* w13, const int32_t* sorted_ids,
                  const int32_t* block_expert, const int32_t* num_padded,
                  int32_t M, int32_t H, int32_t E, int32_t I, int32_t top_k, int32_t block,
                  int32_t capacity, uint16_t* act, moe_stream_t stream);

/*
 * Grouped down-GEMM (step 4).
 *   y [M*top_k, H] fp32 out: y[i] = act[r] W2[e]^T for every plan row r holding a real
 *   flat index i = sorted_ids[r].
 */
int moe_expert_down(const uint16_t* act, const uint16_t* w2, const int32_t* sorted_ids,
                    const int32_t* block_expert, const int32_t* num_padded,
                    int32_t M, int32_t H, int32_t E, int32_t I, int32_t top_k,
                    int32_t block, int32_t capacity, float* y, moe_stream_t stream);

/*
 * Finalize (step 5).
 *   y [M*top_k, H] fp32, topk_w [M, top_k] fp32, residual [M, H] bf16, norm_w [H] bf16.
 *   z = sum_j topk_w[t,j] * y[t*top_k + j] (j ascending, fp32) + residual[t]
 *   out[t] = bf16(z * (mean(z^2) + eps)^(-1/2) * norm_w); residual_out[t] = bf16(z)
 *   when residual_out is not NULL.  eps > 0.
 */
int moe_finalize(const float* y, const float* topk_w, const uint16_t* residual,
                 const uint16_t* norm_w, float eps, int32_t M, int32_t H, int32_t top_k,
                 uint16_t* out, uint16_t* residual_out, moe_stream_t stream);

/*
 * The whole layer: steps 1-5 on one stream.
 *   Required: x, router_w, w13 [E, 2I, H], w2 [E, H, I], residual, norm_w, out,
 *   workspace.  Optional (NULL allowed): router_bias, residual_out, and the exported
 *   intermediates topk_ids_out [M, top_k], topk_w_out [M, top_k], sorted_ids_out
 *   [capacity], block_expert_out [capacity/block], num_padded_out [1]; when given,
 *   the step writes there instead of the workspace.
 *   block must be 16, 32, 64 or 128.
 *   stage_events: NULL, or 6 hipEvent_t recorded on `stream` before step 1 and after
 *   each of the five steps (for per-step timing; with a self-routing up GEMM, events 1
 *   and 2 enclose no kernel).
 */
int moe_forward(const uint16_t* x, const uint16_t* router_w, const float* router_bias,
                const uint16_t* w13, const uint16_t* w2,
                const uint16_t* residual, const uint16_t* norm_w, float eps,
                int32_t M, int32_t H, int32_t E, int32_t I, int32_t top_k, int32_t block,
                uint16_t* out, uint16_t* residual_out,
                int32_t* topk_ids_out, float* topk_w_out,
                int32_t* sorted_ids_out, int32_t* block_expert_out, int32_t* num_padded_out,
                void* workspace, size_t workspace_bytes,
                const moe_event_t* stage_events, moe_stream_t stream);

/*
 * Prepared expert weights: the offline weight re-layout of the AlphaMoE page (FlashInfer
 * PR #6511 analysis, section 2, where the down kernel streams W2 from panels prepared once).
 * moe_prepare_weights re-lays the natural stacks W13 [E, 2I, H] and W2 [E, H, I] out once
 * into "fragment panels": for every expert and N tile of the grouped GEMMs (256 act columns
 * = 512 W13 rows, gate and up rows interleaved; 512 W2 rows), each of the GEMM's 8 waves
 * finds the MFMA operand fragments of its 64 weight rows for consecutive 32-wide K steps in
 * one contiguous stream, so every weight load is 1 KiB of contiguous memory that lands
 * directly in registers.  Layout (bf16, last index fastest):
 *   W13p [E][I/256][8][H/32][4][64][8]: tile j of wave w, N tile n holds rows
 *        n*256 + 32w + 16j + l%16 (j < 2, gate) or I + n*256 + 32w + 16(j-2) + l%16 (up)
 *        for lane l, K values 32 s + 8 (l / 16) + v of step s;
 *   W2p  [E][ceil(H/512)][8][I/32][4][64][8]: rows n*512 + 64w + 16j + l%16 (zero past H).
 * Needs H % 64 == 0 and I % 256 == 0 (MOE_ERR_UNSUPPORTED otherwise; the *_bytes queries
 * return 0).  The caller allocates the prepared stacks (moe_prepared_w13_bytes /
 * moe_prepared_w2_bytes bytes); either pair (w13, w13_prepared) or (w2, w2_prepared) may be
 * NULL to prepare only the other.  Asynchronous on `stream`; allocates nothing.
 *
 * moe_forward_prepared is moe_forward on the prepared stacks, with the same arguments,
 * workspace and results (it always runs the align kernel: the self-routing up kernel reads
 * the natural layout).
 */
size_t moe_prepared_w13_bytes(int32_t E, int32_t H, int32_t I);
size_t moe_prepared_w2_bytes(int32_t E, int32_t H, int32_t I);
int moe_prepare_weights(const uint16_t* w13, const uint16_t* w2, int32_t E, int32_t H, int32_t I,
                        uint16_t* w13_prepared, uint16_t* w2_prepared, moe_stream_t stream);
int moe_forward_prepared(const uint16_t* x, const uint16_t* router_w, const float* router_bias,
                         const uint16_t* w13_prepared, const uint16_t* w2_prepared,
                         const uint16_t* residual, const uint16_t* norm_w, float eps,
                         int32_t M, int32_t H, int32_t E, int32_t I, int32_t top_k, int32_t block,
                         uint16_t* out, uint16_t* residual_out,
                         int32_t* topk_ids_out, float* topk_w_out,
                         int32_t* sorted_ids_out, int32_t* block_expert_out, int32_t* num_padded_out,
                         void* workspace, size_t workspace_bytes,
                         const moe_event_t* stage_events, moe_stream_t stream);

/*
 * MXFP4 expert weights: the 4-bit format of the OCP Microscaling (MX) v1.0 specification --
 * E2M1 elements (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) with one E8M0 scale byte
 * b = s + 127 per 32 consecutive values of a row along K, s = floor(log2(max |v|)) - 2 (a
 * run of zeros gets b = 0); each value becomes the E2M1 code of v / 2^s, rounded to nearest
 * even and clamped to +-6.  The AlphaMoE page (FlashInfer PR #6511 analysis, intro and
 * section 1) streams 4-bit block-scaled expert weights (NVFP4) to cut a decode step's bytes;
 * MXFP4 is the OCP format with MXFP8's block and scale.  Only W13 and W2 are quantized.
 *
 * The codes are stored in the prepared panel order of moe_prepare_weights (H % 64 == 0 and
 * I % 256 == 0, else MOE_ERR_UNSUPPORTED): for expert e, N tile n, wave w and K step s (one
 * 32-value block), lane l holds the 8 values of its tile j as 4 code bytes (value 2b in the
 * low nibble of byte b), the 4 tiles' bytes together, and the step's scale bytes follow as
 * [16 rows][4 tiles]:
 *   W13 codes [E][I/256][8][H/32][64][4][4], W13 scales [E][I/256][8][H/32][16][4]
 *   W2  codes [E][ceil(H/512)][8][I/32][64][4][4], W2 scales [E][ceil(H/512)][8][I/32][16][4]
 * with tile j of lane l holding row n*256 + 32w + 16(j%2) + l%16 (+ I for j >= 2) of W13 and
 * row n*512 + 64w + 16j + l%16 of W2 (codes and scales 0 past H), K values 32 s + 8(l/16) + v.
 *
 * moe_mx4_weight_bytes: the four buffer sizes (any pointer may be NULL).
 * moe_mx4_quantize:     natural bf16 W13 [E, 2I, H] and/or W2 [E, H, I] -> codes and scales
 *                       (a (w, codes, scales) triple may be all NULL to skip that stack).
 * moe_mx4_dequantize:   codes + scales of W13 (which = 13) or W2 (which = 2) -> the natural
 *                       bf16 stack, with the conversion the GEMMs use (exact).
 * moe_forward_mx4:      moe_forward on MXFP4 weights (the layer on the dequantized weights;
 *                       always runs the align kernel).
 * Codes 16-byte and scales 4-byte aligned; asynchronous on `stream`; nothing is allocated.
 */
int moe_mx4_weight_bytes(int32_t E, int32_t H, int32_t I, size_t* w13_codes, size_t* w13_scales,
                         size_t* w2_codes, size_t* w2_scales);
int moe_mx4_quantize(const uint16_t* w13, const uint16_t* w2, int32_t E, int32_t H, int32_t I,
                     uint8_t* w13_codes, uint8_t* w13_scales, uint8_t* w2_codes,
                     uint8_t* w2_scales, moe_stream_t stream);
int moe_mx4_dequantize(const uint8_t* codes, const uint8_t* scales, int32_t which, int32_t E,
                       int32_t H, int32_t I, uint16_t* w, moe_stream_t stream);
int moe_forward_mx4(const uint16_t* x, const uint16_t* router_w, const float* router_bias,
                    const uint8_t* w13_codes, const uint8_t* w13_scales,
                    const uint8_t* w2_codes, const uint8_t* w2_scales,
                    const uint16_t* residual, const uint16_t* norm_w, float eps,
                    int32_t M, int32_t H, int32_t E, int32_t I, int32_t top_k, int32_t block,
                    uint16_t* out, uint16_t* residual_out,
                    int32_t* topk_ids_out, float* topk_w_out,
                    int32_t* sorted_ids_out, int32_t* block_expert_out, int32_t* num_padded_out,
                    void* workspace, size_t workspace_bytes,
                    const moe_event_t* stage_events, moe_stream_t stream);

/*
 * MXFP8 expert weights in the prepared panel order, for the fragment GEMMs of
 * moe_forward_prepared (the offline re-layout of the AlphaMoE page, FlashInfer PR #6511
 * analysis, section 2, applied to the MXFP8 codes of moe_mx_quantize).  The input is the
 * natural MXFP8 format of moe_mx_quantize / moe_forward_mx: W13 codes [E, 2I, H] with scale
 * bytes [E, 2I, H/32], W2 codes [E, H, I] with scale bytes [E, H, I/32].  The output is a
 * byte permutation of it (nothing is re-quantized): for expert e, N tile n, wave w and K step
 * s (one 32-value block), two 1 KiB halves, half h holding, for lane l, the 8 codes of tile
 * 2h then the 8 codes of tile 2h + 1 (value v in byte v); the step's scale bytes follow as
 * [16 rows][4 tiles], as in the MXFP4 panels:
 *   W13 codes [E][I/256][8][H/32][2][64][2][8], W13 scales [E][I/256][8][H/32][16][4]
 *   W2  codes [E][ceil(H/512)][8][I/32][2][64][2][8], W2 scales [E][ceil(H/512)][8][I/32][16][4]
 * with the rows and K values of the MXFP4 panels (codes and scale bytes 0 past H).
 * Needs H % 64 == 0 and I % 256 == 0 (MOE_ERR_UNSUPPORTED otherwise).
 *
 * moe_mx_prepared_bytes:   the four buffer sizes (any pointer may be NULL).
 * moe_mx_prepare_weights:  natural codes + scales -> panels, for W13 and/or W2 (the four
 *                          pointers of a stack all NULL to skip it); natural and panel codes
 *                          16-byte aligned, panel scales 4-byte aligned.
 * moe_forward_mx_prepared: moe_forward_mx on the panels (same arguments, workspace and
 *                          results; always runs the align kernel).
 * Asynchronous on `stream`; nothing is allocated.
 */
int moe_mx_prepared_bytes(int32_t E, int32_t H, int32_t I, size_t* w13_codes,
                          size_t* w13_scales, size_t* w2_codes, size_t* w2_scales);
int moe_mx_prepare_weights(const uint8_t* w13_codes, const uint8_t* w13_scales,
                           const uint8_t* w2_codes, const uint8_t* w2_scales,
                           int32_t E, int32_t H, int32_t I,
                           uint8_t* w13_codes_p, uint8_t* w13_scales_p,
                           uint8_t* w2_codes_p, uint8_t* w2_scales_p, moe_stream_t stream);
int moe_forward_mx_prepared(const uint16_t* x, const uint16_t* router_w, const float* router_bias,
                            const uint8_t* w13_codes_p, const uint8_t* w13_scales_p,
                            const uint8_t* w2_codes_p, const uint8_t* w2_scales_p,
                            const uint16_t* residual, const uint16_t* norm_w, float eps,
                            int32_t M, int32_t H, int32_t E, int32_t I, int32_t top_k,
                            int32_t block, uint16_t* out, uint16_t* residual_out,
                            int32_t* topk_ids_out, float* topk_w_out,
                            int32_t* sorted_ids_out, int32_t* block_expert_out,
                            int32_t* num_padded_out, void* workspace, size_t workspace_bytes,
                            const moe_event_t* stage_events, moe_stream_t stream);

/*
 * moe_forward for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same five steps and outputs as
 * moe_forward, with the workspace taken from a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on until the process
 * ends.  It allocates nothing and takes no workspace or stage events.  Sizes whose
 * moe_workspace_bytes exceed MOE_NOALLOC_SCRATCH_BYTES return MOE_ERR_WORKSPACE before
 * anything is launched (the real-shape layer, H=7168, E=256, top_k=16, I=2048, fits up to
 * 142 tokens with block 16, 14 with block 64).  Every call on a GPU shares that GPU's array,
 * which keeps the last call's contents (nothing in it needs to start at zero): calls that
 * overlap on one GPU -- on different streams, or from different host threads -- race and
 * must be ordered by the caller.  The first call on a device looks up that device's array
 * address (hipGetSymbolAddress) with the device current; a failed lookup is MOE_ERR_HIP.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_forward_noalloc(const uint16_t* x, const uint16_t* router_w, const float* router_bias,
                        const uint16_t* w13, const uint16_t* w2,
                        const uint16_t* residual, const uint16_t* norm_w, float eps,
                        int32_t M, int32_t H, int32_t E, int32_t I, int32_t top_k, int32_t block,
                        uint16_t* out, uint16_t* residual_out,
                        int32_t* topk_ids_out, float* topk_w_out,
                        int32_t* sorted_ids_out, int32_t* block_expert_out,
                        int32_t* num_padded_out, moe_stream_t stream);

/*
 * MXFP8 expert weights.  The AlphaMoE page (FlashInfer PR #6511 analysis, section 1)
 * streams block-scaled narrow expert weights to cut the bytes of a decode step and gives
 * no recipe; the one here is the OCP Microscaling (MX) v1.0 conversion with FP8 E4M3
 * elements: each run of 32 consecutive values of a row (along K) gets one E8M0 scale
 * byte b = s + 127 with s = floor(log2(max |v|)) - 8 (a run of zeros gets b = 0), and
 * each value becomes the E4M3 code of v / 2^s, rounded to nearest even and clamped to
 * +-448.  Dequantized values code * 2^s are exact bf16 numbers.  Only the expert weights
 * are quantized; activations stay bf16.
 *
 * moe_mx_quantize:   w [rows, K] bf16 -> codes [rows, K] uint8 and scales
 *                    [rows, K / 32] uint8.  K a multiple of 32; w and codes 16-byte
 *                    aligned.  Values must be finite.  W13 [E, 2I, H] is rows = E * 2I,
 *                    K = H; W2 [E, H, I] is rows = E * H, K = I.
 * moe_mx_dequantize: the inverse map back to bf16 [rows, K], with the same conversion
 *                    the MXFP8 GEMMs use.
 * Both return MOE_ERR_INVALID_ARG for bad sizes or pointers; rows = 0 is a no-op.
 */
int moe_mx_quantize(const uint16_t* w, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                    moe_stream_t stream);
int moe_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t K,
                      uint16_t* w, moe_stream_t stream);

/*
 * moe_forward with MXFP8 expert weights: w13_codes [E, 2I, H] + w13_scales [E, 2I, H/32],
 * w2_codes [E, H, I] + w2_scales [E, H, I/32] (as written by moe_mx_quantize) in place of
 * w13 and w2; every other argument, the workspace and the outputs are those of
 * moe_forward.  The result is the layer on the dequantized weights.  H and I must be
 * multiples of 256 (MOE_ERR_UNSUPPORTED otherwise); codes 16-byte and scales 8-byte
 * aligned (MOE_ERR_INVALID_ARG otherwise).  The GEMMs copy the codes into LDS and
 * dequantize them from there into the MFMA operands; the up GEMM from 64 tokens per expert
 * (128-row tiles) dequantizes them into the LDS tiles of the tiled kernel instead
 * (moe_gemm_tile_rows_mx).
 */
int moe_forward_mx(const uint16_t* x, const uint16_t* router_w, const float* router_bias,
                   const uint8_t* w13_codes, const uint8_t* w13_scales,
                   const uint8_t* w2_codes, const uint8_t* w2_scales,
                   const uint16_t* residual, const uint16_t* norm_w, float eps,
                   int32_t M, int32_t H, int32_t E, int32_t I, int32_t top_k, int32_t block,
                   uint16_t* out, uint16_t* residual_out,
                   int32_t* topk_ids_out, float* topk_w_out,
                   int32_t* sorted_ids_out, int32_t* block_expert_out, int32_t* num_padded_out,
                   void* workspace, size_t workspace_bytes,
                   const moe_event_t* stage_events, moe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
