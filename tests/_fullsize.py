"""Full-size parity helpers: token samples and one streamed oracle pass over the experts.

The real-shape layer (E=256, H=7168, I=2048) holds 22.5 GB of bf16 expert weights, so the
oracle cannot decode them all at once.  Instead the sampled tokens of every workload are
gathered per expert, and each expert is fetched and decoded once for all of them:
act = oracle.expert_swiglu, y = oracle.expert_down for the (workload, token, pick) rows
that chose it.  The combine, residual add and RMSNorm then run through oracle.finalize per
workload.  Nothing here computes the layer by itself: it only routes rows to the oracle's
functions and collects the results -- and, for the allowance of the layer's bf16 act (see
round_act_bf16), feeds the oracle's down projection act rounded the way the layer stores it.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import moe_oracle as orc


def sample_tokens(ids, n_min: int = 256, all_up_to: int = 128, seed: int = 0) -> np.ndarray:
    """Tokens to compare against the oracle.

    Every token when M <= all_up_to.  Otherwise: token 0 and token M - 1; for every
    expert, the first and the last token that picked it (so every expert's first and last
    token tile of the grouped GEMMs holds a checked row); then seeded uniform picks until
    at least n_min tokens are chosen.
    """
    ids = np.asarray(ids)
    M = ids.shape[0]
    if M <= all_up_to:
        return np.arange(M)
    chosen = {0, M - 1}
    for e in np.unique(ids):
        rows = np.nonzero((ids == e).any(axis=1))[0]
        chosen.add(int(rows[0]))
        chosen.add(int(rows[-1]))
    rng = np.random.default_rng(seed)
    while len(chosen) < min(n_min, M):
        chosen.add(int(rng.integers(M)))
    return np.array(sorted(chosen))


def round_act_bf16(act):
    """act as the layer keeps it between its two GEMMs: float32, then bf16 (nearest even)."""
    u = np.asarray(act, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def stream_expert_rows(jobs, w13_of, w2_of, I: int, threads: int = 0, act_bf16: bool = False):
    """y rows of every job through the oracle, expert by expert.

    jobs: {name: (x_rows [S, H] f64, ids [S, k] int)} -- the sampled tokens' hidden rows and
    their routed experts.  w13_of(e) / w2_of(e) return expert e's bf16 bit patterns
    ([2I, H] / [H, I]).  Returns {name: y [S * k, H] f64} with row s * k + j = the down
    projection of pick j of sample s; with act_bf16, also the same rows from act rounded by
    round_act_bf16 (a second dict), in the same pass over the experts.
    """
    rows_of = {}
    for name, (x, ids) in jobs.items():
        S, k = ids.shape
        for s in range(S):
            for j in range(k):
                rows_of.setdefault(int(ids[s, j]), []).append((name, s, j))
    ys = {name: np.zeros((ids.shape[0] * ids.shape[1], x.shape[1])) for name, (x, ids) in jobs.items()}
    ys7 = {name: np.zeros_like(y) for name, y in ys.items()} if act_bf16 else None

    def one(e):
        rows = rows_of[e]
        xr = np.stack([jobs[name][0][s] for name, s, _ in rows])
        act = orc.expert_swiglu(xr, w13_of(e), I)
        w2 = w2_of(e)
        y7 = orc.expert_down(round_act_bf16(act), w2) if act_bf16 else None
        return e, orc.expert_down(act, w2), y7

    cpus = len(os.sched_getaffinity(0))
    n = threads or max(1, min(16, cpus))
    try:
        from threadpoolctl import threadpool_limits
        limits = threadpool_limits(limits=max(1, cpus // n))
    except ImportError:     # threadpoolctl missing: BLAS keeps its own thread count
        limits = None
    try:
        with ThreadPoolExecutor(max_workers=n) as ex:
            for done, (e, y, y7) in enumerate(ex.map(one, sorted(rows_of)), 1):
                for r, (name, s, j) in enumerate(rows_of[e]):
                    k = jobs[name][1].shape[1]
                    ys[name][s * k + j] = y[r]
                    if act_bf16:
                        ys7[name][s * k + j] = y7[r]
                if done % 64 == 0 or done == len(rows_of):
                    print(f"  oracle: {done} of {len(rows_of)} experts", flush=True)
    finally:
        if limits is not None:
            limits.restore_original_limits()
    return (ys, ys7) if act_bf16 else ys
