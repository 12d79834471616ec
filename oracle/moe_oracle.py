"""CPU oracle for one routed-MoE layer: sigmoid router + top-k, expert-major token plan,
grouped up-GEMM with SwiGLU, grouped down-GEMM, and the fused finalize (weighted top-k
combine, residual add, RMSNorm).

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the benchmark's CPU
baseline leg may import this module.  The product path (the HIP library and its Python
binding) never calls it, and it shares no code with that path: no kernels, headers,
helpers or constants.

Plain, slow and meant to be read against the pages.  All floating point is float64
(the pages fix no precision; the Trainium2 megakernel page's accuracy paragraph checks
against a high-precision reference).  bf16 inputs arrive as uint16 bit patterns and are
decoded here exactly.

Sources (page title, then the section):
  [SIG]   sglang PR #29509 analysis, "GLM-4.7-Flash on NPU: fused Triton kernels",
          section 2 "MoE TopK scoring function": the gate score is the sigmoid
          (norm_type fixed to 1), followed by the fused top-k.
  [ALIGN] FlashInfer PR #6511 analysis, "AlphaMoE NVFP4 kernels", section 5
          "moe_align_block_size_kernel synchronisation": per-expert counts are scanned
          into a shared prefix array, and each block finds its expert id by a binary
          search over that prefix; section 6 "self-routing up kernels": the plan is an
          expert-major token plan consumed by the up kernel; the route chain is
          up -> down -> finalize.
  [RMS]   FlashInfer PR #4690 analysis, "MiniMax-H3 BF16 pre-attention", section 1
          "segmented baseline": RMSNorm is torch's rms_norm over the hidden dim with a
          weight and eps (eps inside the square root).
  [FIN]   FlashInfer PR #5701 analysis, "Kimi K3 H7168/K16 MNNVL CuTe DSL", intro and
          section 3: the MoE finalize (top-k combine) is followed by the residual path
          and RMSNorm; the benchmark uses RMS_EPS = 1e-5 and WEIGHT_BIAS = 0.0 (the norm
          weight is used as is, no 1 + g offset).

Readings where the pages are silent (each is listed in the design notes):
  * key[t, e] = sum_h x[t, h] * Wr[e, h] + bias[e]; the bias (optional) is additive and
    is used both for the selection and inside the sigmoid.
  * Top-k order: descending key, ties to the lower expert index.
  * Weights: s = sigmoid(key) of the k picks, renormalised to sum 1; no scaling factor.
  * W13[e] rows [0, I) are the gate projection, rows [I, 2I) the up projection;
    act = silu(gate) * up, silu(z) = z * sigmoid(z).
  * The combine weight multiplies after the down projection.
  * Plan: experts in ascending id; inside an expert, flat indices i = t * k + j in
    ascending order; padding slots hold M * k; ids outside [0, E) are skipped.
  * Finalize: m = sum_j w[t, j] * y[t*k + j] (j ascending); z = m + residual;
    out = z * (mean(z^2) + eps)^(-1/2) * g; the updated residual z is also returned.

Every function here is pinned by tests that do not reuse its code (brute force, exact
summation, closed forms, library special cases and invariants).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_to_f64", "router_keys", "route", "align_capacity", "align", "expert_swiglu",
    "expert_down", "finalize", "forward", "forward_tokens",
]


# ----------------------------------------------------------------------------------------
# bf16 decode
# ----------------------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns: a bf16 is the upper 16 bits of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------------
# Router: sigmoid scoring and top-k  [SIG]
# ----------------------------------------------------------------------------------------
def router_keys(x_bits, router_w_bits, router_bias=None) -> np.ndarray:
    """key[t, e] = sum_h x[t, h] * Wr[e, h] (+ bias[e]), in float64.  Shape [M, E]."""
    x = bf16_to_f64(x_bits)
    wr = bf16_to_f64(router_w_bits)
    keys = x @ wr.T
    if router_bias is not None:
        keys = keys + np.asarray(router_bias, dtype=np.float32).astype(np.float64)[None, :]
    return keys


def route(x_bits, router_w_bits, router_bias, top_k: int):
    """Sigmoid router with top-k selection and renormalised weights.

    Returns (topk_ids [M, k] int32, topk_w [M, k] float64, keys [M, E] float64).
    Selection: the k largest keys, ordered by (key descending, expert id ascending).
    Weights: s = 1 / (1 + exp(-key)) for the k picks, w = s / sum(s).
    """
    keys = router_keys(x_bits, router_w_bits, router_bias)
    M, E = keys.shape
    if not (1 <= top_k <= E):
        raise ValueError("top_k must be in [1, E]")
    ids = np.empty((M, top_k), dtype=np.int32)
    w = np.empty((M, top_k), dtype=np.float64)
    expert_index = np.arange(E)
    for t in range(M):
        # lexsort: last key is primary -> sort by -key, then by expert index
        order = np.lexsort((expert_index, -keys[t]))
        pick = order[:top_k]
        s = 1.0 / (1.0 + np.exp(-keys[t, pick]))
        ids[t] = pick
        w[t] = s / s.sum()
    return ids, w, keys


# ----------------------------------------------------------------------------------------
# Align: expert-major token plan padded to the GEMM block  [ALIGN]
# ----------------------------------------------------------------------------------------
def align_capacity(M: int, top_k: int, E: int, block: int) -> int:
    """Entries the plan may need: every touched expert pads at most block-1 slots, and at
    most min(E, M*k) experts are touched; rounded up to a whole block."""
    n = M * top_k
    cap = n + min(E, n) * (block - 1)
    return ((cap + block - 1) // block) * block


def align(topk_ids, E: int, block: int):
    """Build the plan from the flat top-k ids (flat index i = t * top_k + j).

    Returns (sorted_ids [num_padded] int32, block_expert [num_padded // block] int32,
    num_padded int, counts [E] int64, offsets [E + 1] int64).

    Steps, in the order the align kernel on the AlphaMoE page takes them:
      1. histogram: count[e] = number of flat entries equal to e (ids outside [0, E) skipped)
      2. pad each count up to a multiple of the block
      3. exclusive prefix scan of the padded counts -> offsets; num_padded = offsets[E]
      4. place each flat index at offsets[e] + (its rank among the entries of e, in
         ascending flat order); unfilled slots get the sentinel M * k
      5. each block b finds its expert by a binary search of b * block in the prefix
    """
    flat = np.asarray(topk_ids, dtype=np.int64).ravel()
    n = flat.size
    if block < 1:
        raise ValueError("block must be >= 1")
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E).astype(np.int64)
    padded = ((counts + block - 1) // block) * block
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    num_padded = int(offsets[E])

    sorted_ids = np.full(num_padded, n, dtype=np.int32)
    fill = offsets[:E].copy()
    for i in range(n):                      # ascending flat index -> stable placement
        e = flat[i]
        if 0 <= e < E:
            sorted_ids[fill[e]] = i
            fill[e] += 1

    nblocks = num_padded // block
    starts = np.arange(nblocks, dtype=np.int64) * block
    # expert e owns [offsets[e], offsets[e+1]); empty experts own nothing, so the last
    # prefix entry <= start (side="right" - 1) is the owner.
    block_expert = (np.searchsorted(offsets, starts, side="right") - 1).astype(np.int32)
    return sorted_ids, block_expert, num_padded, counts, offsets


# ----------------------------------------------------------------------------------------
# Experts
# ----------------------------------------------------------------------------------------
def _silu(z):
    return z / (1.0 + np.exp(-z))


def expert_swiglu(x_rows, w13_e, I: int) -> np.ndarray:
    """act = silu(x . W13[e, 0:I]^T) * (x . W13[e, I:2I]^T); x_rows [r, H] f64, w13_e bits."""
    w = bf16_to_f64(w13_e)
    gate = x_rows @ w[:I].T
    up = x_rows @ w[I:2 * I].T
    return _silu(gate) * up


def expert_down(act, w2_e) -> np.ndarray:
    """y = act . W2[e]^T; act [r, I] f64, w2_e bits [H, I]."""
    return act @ bf16_to_f64(w2_e).T


# ----------------------------------------------------------------------------------------
# Finalize: weighted top-k combine, residual add, RMSNorm  [FIN] [RMS]
# ----------------------------------------------------------------------------------------
def finalize(y, topk_w, residual_bits, norm_w_bits, eps: float):
    """y [M*k, H] f64 rows at flat index t*k + j; returns (out [M,H] f64, z [M,H] f64)."""
    w = np.asarray(topk_w, dtype=np.float64)
    M, k = w.shape
    H = y.shape[1]
    m = np.zeros((M, H), dtype=np.float64)
    for j in range(k):                      # j ascending
        m += w[:, j:j + 1] * y[j::k][:M]
    z = m + bf16_to_f64(residual_bits)
    ms = np.mean(z * z, axis=1, keepdims=True)
    out = z / np.sqrt(ms + float(eps)) * bf16_to_f64(norm_w_bits)[None, :]
    return out, z


# ----------------------------------------------------------------------------------------
# Whole layer
# ----------------------------------------------------------------------------------------
def forward(x_bits, router_w_bits, router_bias, w13, w2, residual_bits, norm_w_bits,
            eps: float, top_k: int, block: int):
    """The layer in the pages' order: route -> align -> up+SwiGLU -> down -> finalize.

    w13 / w2 are indexable by expert (item e: uint16 bits [2I, H] / [H, I]).
    Returns a dict with topk_ids, topk_w, keys, sorted_ids, block_expert, num_padded,
    counts, act (per plan row; zero rows at padding), y [M*k, H], out, residual_out.
    """
    x = bf16_to_f64(x_bits)
    M, H = x.shape
    E = np.asarray(router_w_bits).shape[0]
    ids, w, keys = route(x_bits, router_w_bits, router_bias, top_k)
    sorted_ids, block_expert, num_padded, counts, offsets = align(ids, E, block)
    n = M * top_k
    I = None
    y = np.zeros((n, H), dtype=np.float64)
    act_rows = {}
    for b in range(num_padded // block):    # plan blocks, expert-major
        e = int(block_expert[b])
        rows = sorted_ids[b * block:(b + 1) * block]
        live = rows[rows < n]
        if live.size == 0:
            continue
        w13_e = w13[e]
        if I is None:
            I = np.asarray(w13_e).shape[0] // 2
        tokens = live // top_k
        act = expert_swiglu(x[tokens], w13_e, I)
        y[live] = expert_down(act, w2[e])
        for r, a in zip(live, act):
            act_rows[int(r)] = a
    out, z = finalize(y, w, residual_bits, norm_w_bits, eps)
    return {
        "topk_ids": ids, "topk_w": w, "keys": keys, "sorted_ids": sorted_ids,
        "block_expert": block_expert, "num_padded": num_padded, "counts": counts,
        "offsets": offsets, "act_rows": act_rows, "y": y, "out": out, "residual_out": z,
    }


def forward_tokens(tokens, x_bits, router_w_bits, router_bias, w13, w2, residual_bits,
                   norm_w_bits, eps: float, top_k: int):
    """The layer's output for a subset of tokens, token by token (no plan).

    A token's output depends only on its own row of x and residual (routing is per
    token), so this equals rows `tokens` of `forward`.  Each needed expert is decoded
    once.  Returns (out [len(tokens), H], z, topk_ids, topk_w).
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    xb = np.asarray(x_bits)[tokens]
    ids, w, _ = route(xb, router_w_bits, router_bias, top_k)
    x = bf16_to_f64(xb)
    S, H = x.shape
    y = np.zeros((S * top_k, H), dtype=np.float64)
    needed = sorted(set(int(e) for e in ids.ravel()))
    for e in needed:
        sel = np.argwhere(ids == e)         # (sample row, slot)
        w13_e = w13[e]
        I = np.asarray(w13_e).shape[0] // 2
        act = expert_swiglu(x[sel[:, 0]], w13_e, I)
        y[sel[:, 0] * top_k + sel[:, 1]] = expert_down(act, w2[e])
    out, z = finalize(y, w, np.asarray(residual_bits)[tokens], norm_w_bits, eps)
    return out, z, ids, w
