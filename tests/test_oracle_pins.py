"""Pins of the CPU oracle against facts that do not come from the oracle itself:
exact summation, brute force on tiny inputs, hand-worked plans, closed forms, torch
library routines for the special cases the layer reduces to, and invariants.

Each test names the kind of mistake it is there to catch.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import moe_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32_to_bf16_bits(a):
    """Round-to-nearest-even float32 -> bf16 bits (test-side helper, via torch)."""
    t = torch.as_tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _rand_bits(rng, shape, std=1.0, mean=0.0):
    return _f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * std + mean)


def _bits_to_fraction(b):
    """Exact rational value of one bf16 pattern from its fields (sign, exponent, mantissa)."""
    b = int(b)
    sign = -1 if b >> 15 else 1
    exp = (b >> 7) & 0xFF
    man = b & 0x7F
    assert exp != 0xFF
    if exp == 0:
        return sign * Fraction(man, 1 << 7) * Fraction(2) ** (-126)
    return sign * (1 + Fraction(man, 1 << 7)) * Fraction(2) ** (exp - 127)


# ---------------------------------------------------------------------------------------
# bf16 decode: the IEEE binary32 upper-half definition (catches a wrong shift / sign)
# ---------------------------------------------------------------------------------------
def test_bf16_decode_known_patterns():
    pats = np.array([0x3F80, 0xC000, 0x3E00, 0x0001, 0x8000, 0x7F7F, 0x3FC0, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 0.125, 2.0 ** -133, -0.0, (2 - 2 ** -7) * 2.0 ** 127, 1.5, 3.140625]
    got = orc.bf16_to_f64(pats)
    assert got.dtype == np.float64
    for g, w in zip(got, want):
        assert g == w
    assert math.copysign(1.0, got[4]) == -1.0


def test_bf16_decode_matches_field_arithmetic():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 0x7F80, size=2000, dtype=np.int64).astype(np.uint16)
    bits[::2] |= np.uint16(0x8000)
    got = orc.bf16_to_f64(bits)
    for b, g in zip(bits, got):
        assert Fraction(g) == _bits_to_fraction(b)


# ---------------------------------------------------------------------------------------
# Router keys: correctly rounded exact sum (math.fsum) of the exact bf16 products
# (catches a dropped term, a transposed operand, a dropped or mis-signed bias)
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("with_bias", [False, True])
def test_router_keys_vs_exact_sum(with_bias):
    rng = np.random.default_rng(11)
    M, H, E = 5, 96, 7
    xb = _rand_bits(rng, (M, H))
    wb = _rand_bits(rng, (E, H), std=0.02)
    bias = (rng.standard_normal(E) * 0.3).astype(np.float32) if with_bias else None
    keys = orc.router_keys(xb, wb, bias)
    assert keys.shape == (M, E)
    for t in range(M):
        for e in range(E):
            prods = [float(_bits_to_fraction(xb[t, h]) * _bits_to_fraction(wb[e, h])) for h in range(H)]
            exact = math.fsum(prods)
            if with_bias:
                exact = math.fsum([exact, float(bias[e])])
            bound = (H + 2) * 2.0 ** -53 * math.fsum(abs(p) for p in prods) + 2.0 ** -52 * abs(exact)
            assert abs(keys[t, e] - exact) <= bound, (t, e)


# ---------------------------------------------------------------------------------------
# Top-k: brute-force selection by repeated maximum (catches reversed order, wrong tie rule,
# off-by-one in k)
# ---------------------------------------------------------------------------------------
def _brute_topk(keys_row, k):
    remaining = list(range(len(keys_row)))
    picks = []
    for _ in range(k):
        best = remaining[0]
        for e in remaining[1:]:
            if keys_row[e] > keys_row[best]:   # strict: earlier (lower) index wins ties
                best = e
        picks.append(best)
        remaining.remove(best)
    return picks


@pytest.mark.parametrize("E,k", [(8, 2), (16, 5), (64, 16), (3, 3), (5, 1)])
def test_topk_vs_bruteforce(E, k):
    rng = np.random.default_rng(E * 100 + k)
    M, H = 6, 32
    xb = _rand_bits(rng, (M, H))
    wb = _rand_bits(rng, (E, H), std=0.02)
    ids, w, keys = orc.route(xb, wb, None, k)
    assert ids.dtype == np.int32 and ids.shape == (M, k)
    for t in range(M):
        assert list(ids[t]) == _brute_topk(list(keys[t]), k)
        chosen = set(ids[t].tolist())
        assert len(chosen) == k
        lo = min(keys[t, e] for e in chosen)
        assert all(keys[t, e] <= lo for e in range(E) if e not in chosen)


def test_topk_exact_ties_hand_worked():
    # x = 0 makes every logit exactly 0, so key = bias.  bias = [0.5, 1.0, 0.5, 1.0, 0.25]
    # with k = 3: the two 1.0 keys (experts 1, 3) come first, lower id first; the 0.5 tie
    # between experts 0 and 2 at the cut goes to expert 0.
    xb = np.zeros((1, 8), dtype=np.uint16)
    wb = _rand_bits(np.random.default_rng(0), (5, 8))
    bias = np.array([0.5, 1.0, 0.5, 1.0, 0.25], dtype=np.float32)
    ids, w, _ = orc.route(xb, wb, bias, 3)
    assert ids.tolist() == [[1, 3, 0]]


def test_topk_ties_from_duplicated_router_rows():
    rng = np.random.default_rng(3)
    H, E = 64, 12
    xb = _rand_bits(rng, (4, H))
    wb = _rand_bits(rng, (E, H), std=0.02)
    wb[9] = wb[2]            # experts 2 and 9 always tie
    wb[7] = wb[2]            # and 7
    ids, w, keys = orc.route(xb, wb, None, E)   # full order
    for t in range(4):
        order = ids[t].tolist()
        assert order.index(2) < order.index(7) < order.index(9)
        assert order.index(9) == order.index(2) + 2


# ---------------------------------------------------------------------------------------
# Weights: closed forms of the renormalised sigmoid (catches a sign error in the sigmoid,
# softmax instead of sigmoid, missing renormalisation)
# ---------------------------------------------------------------------------------------
def test_weights_closed_form_symmetric_pair():
    # keys +2 and -2: sigmoid(a) + sigmoid(-a) = 1, so the renormalised weights equal the
    # raw scores: sigmoid(2) = (1 + tanh(1)) / 2.
    xb = np.zeros((1, 4), dtype=np.uint16)
    wb = np.zeros((2, 4), dtype=np.uint16)
    ids, w, _ = orc.route(xb, wb, np.array([-2.0, 2.0], dtype=np.float32), 2)
    assert ids.tolist() == [[1, 0]]
    s = 0.5 * (1.0 + math.tanh(1.0))
    assert abs(w[0, 0] - s) < 1e-15 and abs(w[0, 1] - (1.0 - s)) < 1e-15


def test_weights_closed_form_three_quarters_and_half():
    # keys ln 3 and 0: sigmoid(ln 3) = 3/4, sigmoid(0) = 1/2 -> weights 0.6 and 0.4
    # (bias is fp32, so ln 3 carries a relative error of about 3e-8).
    xb = np.zeros((1, 4), dtype=np.uint16)
    wb = np.zeros((3, 4), dtype=np.uint16)
    bias = np.array([0.0, math.log(3.0), -5.0], dtype=np.float32)
    ids, w, _ = orc.route(xb, wb, bias, 2)
    assert ids.tolist() == [[1, 0]]
    assert abs(w[0, 0] - 0.6) < 1e-7 and abs(w[0, 1] - 0.4) < 1e-7


def test_weights_invariants_random():
    rng = np.random.default_rng(21)
    xb = _rand_bits(rng, (32, 128))
    wb = _rand_bits(rng, (64, 128), std=0.02)
    bias = (-0.9 * np.log(np.arange(64) + 1.0)).astype(np.float32)
    ids, w, keys = orc.route(xb, wb, bias, 16)
    assert np.all(np.abs(w.sum(axis=1) - 1.0) < 1e-12)
    assert np.all((w > 0) & (w < 1))
    # descending key order implies non-increasing weights
    assert np.all(np.diff(w, axis=1) <= 0)


# ---------------------------------------------------------------------------------------
# Align: hand-worked plans, brute force, invariants (catches unstable placement, wrong
# padding, an exclusive/inclusive scan mix-up, a wrong block->expert search)
# ---------------------------------------------------------------------------------------
def test_align_hand_worked_golden():
    with open(os.path.join(GOLDEN, "align_hand.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        sorted_ids, block_expert, num_padded, counts, offsets = orc.align(
            np.array(c["topk_ids"]), c["E"], c["block"])
        assert counts.tolist() == c["counts"], c["name"]
        assert num_padded == c["num_padded"], c["name"]
        assert sorted_ids.tolist() == c["sorted_ids"], c["name"]
        assert block_expert.tolist() == c["block_expert"], c["name"]


def _brute_plan(flat, E, block):
    groups = {e: [] for e in range(E)}
    for i, e in enumerate(flat):
        if 0 <= e < E:
            groups[e].append(i)
    plan, owners = [], []
    for e in range(E):
        g = groups[e]
        padded = g + [len(flat)] * ((-len(g)) % block)
        plan += padded
        owners += [e] * (len(padded) // block)
    return plan, owners


def _check_plan_invariants(flat, E, block, sorted_ids, block_expert, num_padded, counts):
    n = len(flat)
    valid = [i for i in range(n) if 0 <= flat[i] < E]
    assert num_padded % block == 0
    real = [int(v) for v in sorted_ids if v != n]
    assert sorted(real) == valid                      # every valid flat index exactly once
    assert all(c % block == 0 for c in ((counts + block - 1) // block * block))
    assert (sorted_ids == n).sum() == num_padded - len(valid)
    assert len(valid) <= num_padded <= len(valid) + int((counts > 0).sum()) * (block - 1)
    assert np.all(np.diff(block_expert) >= 0)
    for b, e in enumerate(block_expert):
        rows = sorted_ids[b * block:(b + 1) * block]
        assert all(flat[r] == e for r in rows if r != n)
    assert num_padded <= orc.align_capacity(len(flat) // 1, 1, E, block)


@pytest.mark.parametrize("M,k,E,block", [(7, 2, 8, 16), (33, 4, 16, 4), (128, 16, 256, 64),
                                         (64, 8, 64, 1), (40, 16, 256, 16), (9, 3, 5, 128)])
def test_align_vs_bruteforce(M, k, E, block):
    rng = np.random.default_rng(M * 7 + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(M)]).astype(np.int32)
    sorted_ids, block_expert, num_padded, counts, offsets = orc.align(ids, E, block)
    plan, owners = _brute_plan(ids.ravel().tolist(), E, block)
    assert sorted_ids.tolist() == plan
    assert block_expert.tolist() == owners
    assert num_padded == len(plan)
    assert num_padded <= orc.align_capacity(M, k, E, block)
    _check_plan_invariants(ids.ravel().tolist(), E, block, sorted_ids, block_expert, num_padded, counts)
    # every token appears exactly k times
    tok = [int(v) // k for v in sorted_ids if v != M * k]
    assert np.all(np.bincount(tok, minlength=M) == k)


@pytest.mark.parametrize("case", ["one_expert", "all_distinct", "empty", "out_of_range", "skewed"])
def test_align_adversarial(case):
    rng = np.random.default_rng(1)
    E, block = 32, 16
    if case == "one_expert":
        flat = np.full(200, 5)
    elif case == "all_distinct":
        flat = np.arange(E)
    elif case == "empty":
        flat = np.zeros(0, dtype=np.int64)
    elif case == "out_of_range":
        flat = rng.integers(-3, E + 3, size=300)
    else:
        flat = np.minimum(rng.zipf(1.3, size=500) - 1, E - 1)
    sorted_ids, block_expert, num_padded, counts, offsets = orc.align(flat, E, block)
    plan, owners = _brute_plan(flat.tolist(), E, block)
    assert sorted_ids.tolist() == plan and block_expert.tolist() == owners
    _check_plan_invariants(flat.tolist(), E, block, sorted_ids, block_expert, num_padded, counts)


def test_align_capacity_is_an_upper_bound_and_tight():
    # tight: every token on its own expert with count 1 -> each pads block - 1
    M, k, E, block = 16, 1, 64, 8
    ids = np.arange(M).reshape(M, 1)
    _, _, num_padded, _, _ = orc.align(ids, E, block)
    assert num_padded == orc.align_capacity(M, k, E, block) == M * block


# ---------------------------------------------------------------------------------------
# Experts and the whole layer: special cases that reduce to torch library routines
# (catches a gate/up swap, transposed weights, a missing residual, a wrong eps placement)
# ---------------------------------------------------------------------------------------
def _to_t(bits):
    return torch.from_numpy(orc.bf16_to_f64(bits))


def test_single_expert_reduces_to_swiglu_mlp_and_rms_norm():
    rng = np.random.default_rng(2)
    M, H, I = 6, 64, 48
    xb = _rand_bits(rng, (M, H))
    rb = _rand_bits(rng, (M, H))
    gb = _rand_bits(rng, (H,), std=0.05, mean=1.0)
    wr = _rand_bits(rng, (1, H), std=0.02)
    w13 = _rand_bits(rng, (1, 2 * I, H), std=0.1)
    w2 = _rand_bits(rng, (1, H, I), std=0.1)
    eps = 1e-5
    res = orc.forward(xb, wr, None, w13, w2, rb, gb, eps, top_k=1, block=4)
    assert res["topk_ids"].tolist() == [[0]] * M
    assert np.all(res["topk_w"] == 1.0)
    x, W13, W2 = _to_t(xb), _to_t(w13[0]), _to_t(w2[0])
    act = F.silu(F.linear(x, W13[:I])) * F.linear(x, W13[I:])
    z = F.linear(act, W2) + _to_t(rb)
    ref = F.rms_norm(z, (H,), _to_t(gb), eps)
    np.testing.assert_allclose(res["out"], ref.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(res["residual_out"], z.numpy(), rtol=1e-12, atol=1e-12)


def test_identical_experts_make_routing_irrelevant():
    rng = np.random.default_rng(4)
    M, H, E, I, k = 5, 32, 6, 16, 3
    xb = _rand_bits(rng, (M, H))
    rb = _rand_bits(rng, (M, H))
    gb = _rand_bits(rng, (H,), std=0.05, mean=1.0)
    one13 = _rand_bits(rng, (2 * I, H), std=0.1)
    one2 = _rand_bits(rng, (H, I), std=0.1)
    w13 = np.stack([one13] * E)
    w2 = np.stack([one2] * E)
    outs = []
    for seed in (10, 20):
        wr = _rand_bits(np.random.default_rng(seed), (E, H), std=0.5)
        outs.append(orc.forward(xb, wr, None, w13, w2, rb, gb, 1e-5, k, 2)["out"])
    x = _to_t(xb)
    act = F.silu(F.linear(x, _to_t(one13[:I]))) * F.linear(x, _to_t(one13[I:]))
    ref = F.rms_norm(F.linear(act, _to_t(one2)) + _to_t(rb), (H,), _to_t(gb), 1e-5).numpy()
    for o in outs:
        np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_zero_down_projection_gives_rms_norm_of_residual():
    rng = np.random.default_rng(6)
    M, H, E, I, k = 4, 40, 5, 8, 2
    xb = _rand_bits(rng, (M, H))
    rb = _rand_bits(rng, (M, H))
    gb = _rand_bits(rng, (H,), std=0.05, mean=1.0)
    wr = _rand_bits(rng, (E, H), std=0.02)
    w13 = _rand_bits(rng, (E, 2 * I, H), std=0.1)
    w2 = np.zeros((E, H, I), dtype=np.uint16)
    res = orc.forward(xb, wr, None, w13, w2, rb, gb, 1e-5, k, 4)
    ref = F.rms_norm(_to_t(rb), (H,), _to_t(gb), 1e-5).numpy()
    np.testing.assert_allclose(res["out"], ref, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------------------
# Finalize: closed form and invariants (catches eps outside the root, a missing weight)
# ---------------------------------------------------------------------------------------
def test_finalize_constant_vector_closed_form():
    H, eps = 64, 1e-5
    y = np.zeros((2, H))
    w = np.array([[0.7, 0.3]])
    rb = np.full((1, H), 0x4000, dtype=np.uint16)      # residual = 2.0 everywhere
    gb = np.full(H, 0x3F80, dtype=np.uint16)           # g = 1
    out, z = orc.finalize(y, w, rb, gb, eps)
    assert np.all(z == 2.0)
    np.testing.assert_allclose(out, 2.0 / math.sqrt(4.0 + eps), rtol=1e-15)


def test_finalize_rms_invariant_and_combine_weights():
    rng = np.random.default_rng(8)
    M, k, H, eps = 3, 4, 50, 1e-5
    y = rng.standard_normal((M * k, H))
    w = rng.random((M, k))
    w /= w.sum(axis=1, keepdims=True)
    rb = _rand_bits(rng, (M, H))
    gb = _rand_bits(rng, (H,), std=0.05, mean=1.0)
    out, z = orc.finalize(y, w, rb, gb, eps)
    # combine by exact rationals, one entry at a time (different arithmetic)
    for t in range(M):
        for h in (0, H // 2, H - 1):
            m = sum(Fraction(w[t, j]) * Fraction(y[t * k + j, h]) for j in range(k))
            assert abs(float(m + _bits_to_fraction(rb[t, h])) - z[t, h]) < 1e-14
    g = orc.bf16_to_f64(gb)
    ms = np.mean(z * z, axis=1)
    np.testing.assert_allclose(np.mean((out / g) ** 2, axis=1), ms / (ms + eps), rtol=1e-13)


# ---------------------------------------------------------------------------------------
# Whole layer: dense-masked brute force with exact sums, no plan (catches any gather or
# scatter index slip in the plan-based forward)
# ---------------------------------------------------------------------------------------
def _dense_bruteforce(xb, wr, bias, w13, w2, rb, gb, eps, k):
    M, H = xb.shape
    E = wr.shape[0]
    I = w13.shape[1] // 2
    fx = lambda b: float(_bits_to_fraction(b))  # noqa: E731
    X = [[fx(v) for v in row] for row in xb]
    out = np.zeros((M, H))
    for t in range(M):
        keys = [math.fsum(X[t][h] * fx(wr[e, h]) for h in range(H)) + (float(bias[e]) if bias is not None else 0.0)
                for e in range(E)]
        picks = _brute_topk(keys, k)
        s = {e: 1.0 / (1.0 + math.exp(-keys[e])) for e in picks}
        tot = math.fsum(s.values())
        m = [0.0] * H
        for e in range(E):                   # every expert, masked by the selection
            if e not in s:
                continue
            wgt = s[e] / tot
            gate = [math.fsum(X[t][h] * fx(w13[e, n, h]) for h in range(H)) for n in range(I)]
            up = [math.fsum(X[t][h] * fx(w13[e, I + n, h]) for h in range(H)) for n in range(I)]
            act = [g_ / (1.0 + math.exp(-g_)) * u_ for g_, u_ in zip(gate, up)]
            for h in range(H):
                m[h] += wgt * math.fsum(act[n] * fx(w2[e, h, n]) for n in range(I))
        z = [m[h] + fx(rb[t, h]) for h in range(H)]
        inv = 1.0 / math.sqrt(math.fsum(v * v for v in z) / H + eps)
        out[t] = [z[h] * inv * fx(gb[h]) for h in range(H)]
    return out


@pytest.mark.parametrize("with_bias", [False, True])
def test_forward_vs_dense_bruteforce(with_bias):
    rng = np.random.default_rng(12 + with_bias)
    M, H, E, I, k, block = 5, 12, 6, 8, 2, 4
    xb = _rand_bits(rng, (M, H))
    wr = _rand_bits(rng, (E, H), std=0.3)
    bias = (-0.9 * np.log(np.arange(E) + 1.0)).astype(np.float32) if with_bias else None
    w13 = _rand_bits(rng, (E, 2 * I, H), std=0.3)
    w2 = _rand_bits(rng, (E, H, I), std=0.3)
    rb = _rand_bits(rng, (M, H))
    gb = _rand_bits(rng, (H,), std=0.05, mean=1.0)
    res = orc.forward(xb, wr, bias, w13, w2, rb, gb, 1e-5, k, block)
    ref = _dense_bruteforce(xb, wr, bias, w13, w2, rb, gb, 1e-5, k)
    np.testing.assert_allclose(res["out"], ref, rtol=1e-11, atol=1e-11)


def test_forward_tokens_matches_forward_rows():
    rng = np.random.default_rng(13)
    M, H, E, I, k, block = 9, 32, 8, 16, 3, 4
    xb = _rand_bits(rng, (M, H))
    wr = _rand_bits(rng, (E, H), std=0.1)
    w13 = _rand_bits(rng, (E, 2 * I, H), std=0.1)
    w2 = _rand_bits(rng, (E, H, I), std=0.1)
    rb = _rand_bits(rng, (M, H))
    gb = _rand_bits(rng, (H,), std=0.05, mean=1.0)
    full = orc.forward(xb, wr, None, w13, w2, rb, gb, 1e-5, k, block)
    sample = [7, 0, 4]
    out, z, ids, w = orc.forward_tokens(sample, xb, wr, None, w13, w2, rb, gb, 1e-5, k)
    np.testing.assert_allclose(out, full["out"][sample], rtol=1e-13, atol=1e-13)
    assert ids.tolist() == full["topk_ids"][sample].tolist()


def test_forward_empty_batch():
    rng = np.random.default_rng(14)
    H, E, I = 16, 4, 8
    res = orc.forward(np.zeros((0, H), np.uint16), _rand_bits(rng, (E, H)), None,
                      _rand_bits(rng, (E, 2 * I, H)), _rand_bits(rng, (E, H, I)),
                      np.zeros((0, H), np.uint16), _rand_bits(rng, (H,)), 1e-5, 2, 4)
    assert res["out"].shape == (0, H) and res["num_padded"] == 0
