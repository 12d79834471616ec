"""The parity bar of the layer's bf16 outputs (out, residual_out) against the oracle.

Element-wise |gpu - oracle| <= max(2e-2, one bf16 unit in the last place of the oracle
value), and relative L2 error <= 1e-2 over the compared values.  Below 4 in magnitude the
element-wise bound is 2e-2 (a bf16 number there is at most 2^-7 from the value it rounds).
From 4 on, a bf16 output's own rounding is already up to 2^-6 = 0.0156 (2^-5 from 8 on),
and act, rounded to bf16 before the down GEMM as the layer's readings fix, adds up to about
0.01 more at the tail when one pick carries a token's whole weight; there the bound is one
unit in the last place: half of it for the output's rounding, half for the arithmetic.
A check may add an element-wise allowance `extra` to that bound: the full-size tests allow
residual_out (z, not normalized) the difference that act rounded to bf16, as the layer keeps
it, makes to the oracle's z -- under a routing that puts a token's whole weight on one pick
that difference alone reaches 1e-2 at the tail.
"""
import numpy as np

MAX_ABS = 2e-2
REL_L2 = 1e-2


def bf16_ulp(v):
    """Spacing of bf16 numbers at |v| (8 significant bits): 2^(floor(log2 |v|) - 7)."""
    a = np.maximum(np.abs(np.asarray(v, dtype=np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(np.int64) - 7)


def abs_bound(ref):
    return np.maximum(MAX_ABS, bf16_ulp(ref))


def check_close(got_bf16, ref, what, extra=None):
    """got_bf16: a torch bf16 (or float) tensor; ref: the oracle's float64 values; extra: an
    element-wise allowance added to the bound (None: none)."""
    g = got_bf16.float().cpu().numpy().astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - ref)
    bound = abs_bound(ref) if extra is None else abs_bound(ref) + np.abs(extra)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert (err <= bound).all(), (f"{what}: error {err[worst]:.4e} at {worst} (|oracle| "
                                  f"{abs(ref[worst]):.3f}, bound {bound[worst]:.3e}); "
                                  f"max-abs {err.max():.4e}")
    rel = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30)
    assert rel <= REL_L2, f"{what}: rel-L2 {rel:.4e}"
    return err.max(), rel
