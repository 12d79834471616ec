"""GPU parity of the MXFP8 panels (moe_mx_prepare_weights, moe_forward_mx_prepared) through
the C ABI.

The panels are a byte permutation of the natural MXFP8 stacks: the test maps natural codes
and scale bytes to the panel order on the host (from the definition in include/moe.h) and
compares every byte.  The layer on the panels is checked against the oracle layer run on the
oracle's own dequantized MXFP8 weights (routing and plan bit-exact, outputs max-abs 2e-2 and
relative-L2 1e-2), on small layers and at full size (every token at M=8 and M=128, at least
256 stratified tokens at M=512 and M=2048).
"""
import functools

import numpy as np
import pytest
import torch

import _bars as bars
import _fullsize as fs
import moe_inputs as mi
from oracle import moe_oracle as orc
from oracle import mx_oracle as mxo

pytestmark = pytest.mark.gpu

bits = mi.bf16_bits


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def B(dev):
    from prefill_sigmoid_router_amd import binding
    binding.load_library()
    return binding


# ---------------------------------------------------------------------------------------
# Host map of natural MXFP8 stacks to the panel order (include/moe.h)
# ---------------------------------------------------------------------------------------
@functools.lru_cache(maxsize=4)
def _panel_index(which, H, I):
    """Natural (row, K) of every panel code byte and (row, block) of every panel scale byte,
    in panel order; rows past the stack are marked by `ok` / `sok` False."""
    if which == 13:
        nnt, K, rows = I // 256, H, 2 * I
    else:
        nnt, K, rows = (H + 511) // 512, I, H
    steps = K // 32
    a = lambda m: np.arange(m, dtype=np.int32)  # noqa: E731
    # codes: [n][w][s][half][lane][tile in half][8]
    n, w, s, h, lane, t, v = np.meshgrid(a(nnt), a(8), a(steps), a(2), a(64), a(2), a(8),
                                         indexing="ij", sparse=True)
    j = 2 * h + t
    if which == 13:
        row = n * 256 + 32 * w + 16 * (j % 2) + lane % 16 + np.where(j >= 2, I, 0)
    else:
        row = n * 512 + 64 * w + 16 * j + lane % 16
    k = 32 * s + 8 * (lane // 16) + v
    row, k = np.broadcast_arrays(row, k)
    row, k = row.reshape(-1), k.reshape(-1)
    ok = row < rows
    # scales: [n][w][s][16 rows][4 tiles]
    n2, w2, s2, r2, j2 = np.meshgrid(a(nnt), a(8), a(steps), a(16), a(4), indexing="ij",
                                     sparse=True)
    if which == 13:
        srow = n2 * 256 + 32 * w2 + 16 * (j2 % 2) + r2 + np.where(j2 >= 2, I, 0)
    else:
        srow = n2 * 512 + 64 * w2 + 16 * j2 + r2
    srow, sblk = np.broadcast_arrays(srow, s2)
    srow, sblk = srow.reshape(-1), sblk.reshape(-1)
    sok = srow < rows
    return row[ok], k[ok], ok, srow[sok], sblk[sok], sok


def natural_to_panels(codes, scales, which, E, H, I):
    """Panel codes and scale bytes (flat uint8) from natural codes [E, rows, K] and scale
    bytes [E, rows, K/32]."""
    row, k, ok, srow, sblk, sok = _panel_index(which, H, I)
    pc = np.zeros((E, ok.size), dtype=np.uint8)
    pc[:, ok] = codes[:, row, k]
    ps = np.zeros((E, sok.size), dtype=np.uint8)
    ps[:, sok] = scales[:, srow, sblk]
    return pc.reshape(-1), ps.reshape(-1)


def _prepare(B, c13, s13, c2, s2, E, H, I, dev):
    n = B.moe_mx_prepared_bytes(E, H, I)
    bufs = [torch.full((nb,), 0x5A, dtype=torch.uint8, device=dev) for nb in n]
    B.moe_mx_prepare_weights(c13, s13, c2, s2, E, H, I, *bufs)
    torch.cuda.synchronize()
    return bufs


PREP_SHAPES = [(3, 128, 256), (2, 640, 512)]   # (E, H, I); H = 640: a partial W2 panel


@pytest.mark.parametrize("shape", PREP_SHAPES, ids=lambda s: f"E{s[0]}_H{s[1]}_I{s[2]}")
def test_prepare_permutation_bit_exact(B, dev, shape):
    """Arbitrary code and scale bytes: every panel byte is the natural byte the layout names
    (zero past H)."""
    E, H, I = shape
    rng = np.random.default_rng(E * H + I)
    nat = {13: (rng.integers(0, 256, (E, 2 * I, H), dtype=np.uint8),
                rng.integers(0, 256, (E, 2 * I, H // 32), dtype=np.uint8)),
           2: (rng.integers(0, 256, (E, H, I), dtype=np.uint8),
               rng.integers(0, 256, (E, H, I // 32), dtype=np.uint8))}
    t = {k: tuple(torch.from_numpy(a).to(dev) for a in v) for k, v in nat.items()}
    p = _prepare(B, t[13][0], t[13][1], t[2][0], t[2][1], E, H, I, dev)
    for which, (pc, ps) in ((13, (p[0], p[1])), (2, (p[2], p[3]))):
        want_c, want_s = natural_to_panels(*nat[which], which, E, H, I)
        assert np.array_equal(pc.cpu().numpy(), want_c), which
        assert np.array_equal(ps.cpu().numpy(), want_s), which


def test_prepare_rejects_unsupported_widths(B, dev):
    with pytest.raises(B.MoeError) as ei:
        B.moe_mx_prepared_bytes(4, 96, 256)      # H % 64 != 0
    assert ei.value.status == -2
    with pytest.raises(B.MoeError) as ei:
        B.moe_mx_prepared_bytes(4, 128, 128)     # I % 256 != 0
    assert ei.value.status == -2


# ---------------------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------------------
# MXFP8 panel tiles: 64 rows below 64 expected tokens per expert (nontemporal weights below
# 32), 128 rows from there
SMALL = {
    # 64-row tiles, nontemporal weights; 4-wave workgroups on half N tiles
    "mxp_tiles64": mi.LayerConfig("mxp_tiles64", M=64, H=320, E=16, top_k=4, I=256, block=16),
    # 64-row tiles, default cache policy, Zipf routing
    "mxp_tiles64_zipf": mi.LayerConfig("mxp_tiles64_zipf", M=100, H=448, E=8, top_k=4,
                                       I=256, block=32, zipf_s=1.0),
    # 128-row tiles of a hot expert sharing its weights, a partial W2 panel (H = 640)
    "mxp_tiles128_shared": mi.LayerConfig("mxp_tiles128_shared", M=300, H=640, E=8, top_k=4,
                                          I=512, block=64, zipf_s=1.0),
    "mxp_one_token": mi.LayerConfig("mxp_one_token", M=1, H=256, E=32, top_k=8, I=256, block=16),
}


def _run(B, L, dev, p):
    cfg = L["cfg"]
    M, H, E, I, k, blk = L["M"], cfg.H, cfg.E, cfg.I, cfg.top_k, cfg.block
    cap = B.moe_align_capacity(M, k, E, blk)
    r = {
        "out": torch.full((M, H), float("nan"), dtype=torch.bfloat16, device=dev),
        "rout": torch.full((M, H), float("nan"), dtype=torch.bfloat16, device=dev),
        "ids": torch.full((M, k), -7, dtype=torch.int32, device=dev),
        "sorted": torch.full((cap,), -7, dtype=torch.int32, device=dev),
        "npad": torch.full((1,), -7, dtype=torch.int32, device=dev),
    }
    ws = torch.empty(B.moe_workspace_bytes(M, H, E, I, k, blk), dtype=torch.uint8, device=dev)
    B.moe_forward_mx_prepared(L["x"], L["router_w"], L["router_bias"], *p, I, L["residual"],
                              L["norm_w"], L["eps"], k, blk, r["out"], ws, residual_out=r["rout"],
                              topk_ids_out=r["ids"], sorted_ids_out=r["sorted"],
                              num_padded_out=r["npad"])
    torch.cuda.synchronize()
    return r


_check_close = bars.check_close


def _bias_np(L):
    return None if L["router_bias"] is None else L["router_bias"].cpu().numpy()


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_mx_prepared_small(B, dev, name):
    """Natural codes from the oracle's MXFP8 conversion, re-laid-out on the device."""
    cfg = SMALL[name]
    print(f"forward_mx_prepared parity {name}", flush=True)
    L = mi.make_layer(cfg, device=dev, seed=5)
    c13, s13 = mxo.mx_quantize(bits(L["w13"]))
    c2, s2 = mxo.mx_quantize(bits(L["w2"]))
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    p = _prepare(B, up(c13), up(s13), up(c2), up(s2), cfg.E, cfg.H, cfg.I, dev)
    r = _run(B, L, dev, p)
    ref = orc.forward(bits(L["x"]), bits(L["router_w"]), _bias_np(L),
                      mxo.mx_dequantize_bf16_bits(c13, s13), mxo.mx_dequantize_bf16_bits(c2, s2),
                      bits(L["residual"]), bits(L["norm_w"]), L["eps"], cfg.top_k, cfg.block)
    assert np.array_equal(r["ids"].cpu().numpy(), ref["topk_ids"])
    n_pad = int(r["npad"].item())
    assert n_pad == ref["num_padded"]
    assert np.array_equal(r["sorted"].cpu().numpy()[:n_pad], ref["sorted_ids"])
    _check_close(r["out"], ref["out"], name)
    _check_close(r["rout"], ref["residual_out"], name + " residual_out")


FULL = ["decode_m8", "batch_m128", "batch_m512", "prefill_m2048", "prefill_m8192",
        "skew_m512"]


@pytest.fixture(scope="module")
def mxp_full(B, dev):
    cfg = mi.CONFIGS["decode_m8"]
    E, H, I = cfg.E, cfg.H, cfg.I
    print("generating full-size expert weights, their MXFP8 codes and panels", flush=True)
    L = mi.make_layer(cfg, device=dev, seed=0)
    weights = {k: L[k] for k in ("w13", "w2", "router_w", "norm_w")}
    nat = []
    for name in ("w13", "w2"):
        w = weights[name]
        c = torch.empty(tuple(w.shape), dtype=torch.uint8, device=dev)
        sc = torch.empty(tuple(w.shape[:-1]) + (w.shape[-1] // 32,), dtype=torch.uint8,
                         device=dev)
        B.moe_mx_quantize(w, c, sc)
        nat += [c, sc]
    p = _prepare(B, *nat, E, H, I, dev)
    # natural codes of a few real-shape experts against the oracle, and their panels against
    # the host map of those codes, byte for byte
    n = B.moe_mx_prepared_bytes(E, H, I)
    per = [nb // E for nb in n]
    for e in (0, 131, 255):
        rc, rs = mxo.mx_quantize_lut(bits(weights["w13"][e]))
        assert np.array_equal(nat[0][e].cpu().numpy(), rc), e
        assert np.array_equal(nat[1][e].cpu().numpy(), rs), e
        want_c, want_s = natural_to_panels(rc[None], rs[None], 13, 1, H, I)
        assert np.array_equal(p[0][e * per[0]:(e + 1) * per[0]].cpu().numpy(), want_c), e
        assert np.array_equal(p[1][e * per[1]:(e + 1) * per[1]].cpu().numpy(), want_s), e
        rc2, rs2 = mxo.mx_quantize_lut(bits(weights["w2"][e]))
        want_c, want_s = natural_to_panels(rc2[None], rs2[None], 2, 1, H, I)
        assert np.array_equal(p[2][e * per[2]:(e + 1) * per[2]].cpu().numpy(), want_c), e
        assert np.array_equal(p[3][e * per[3]:(e + 1) * per[3]].cpu().numpy(), want_s), e
    del nat
    torch.cuda.empty_cache()
    runs = {}
    for name in FULL:
        c = mi.CONFIGS[name]
        print(f"forward_mx_prepared full-size {name} M={c.M}", flush=True)
        Lw = mi.make_layer(c, device=dev, seed=0, with_experts=False)
        Lw.update(weights)
        r = _run(B, Lw, dev, p)
        runs[name] = {
            "cfg": c, "eps": Lw["eps"], "x": bits(Lw["x"]), "residual": bits(Lw["residual"]),
            "bias": _bias_np(Lw), "router_w": bits(Lw["router_w"]), "norm_w": bits(Lw["norm_w"]),
            "ids": r["ids"].cpu().numpy(), "sorted": r["sorted"].cpu().numpy(),
            "npad": int(r["npad"].item()),
            "out": r["out"].float().cpu().numpy().astype(np.float64),
            "rout": r["rout"].float().cpu().numpy().astype(np.float64),
        }
        del r, Lw
    del p
    torch.cuda.empty_cache()
    return weights, runs


@pytest.mark.parametrize("name", FULL)
def test_forward_mx_prepared_full_size_plan(mxp_full, name):
    _, runs = mxp_full
    run = runs[name]
    cfg = run["cfg"]
    ref_ids, _, _ = orc.route(run["x"], run["router_w"], run["bias"], cfg.top_k)
    assert np.array_equal(run["ids"], ref_ids)
    sorted_ids, _, n_pad, _, _ = orc.align(ref_ids, cfg.E, cfg.block)
    assert run["npad"] == n_pad
    assert np.array_equal(run["sorted"][:n_pad], sorted_ids)
    assert np.isfinite(run["out"]).all()


@pytest.fixture(scope="module")
def mxp_full_oracle(mxp_full):
    weights, runs = mxp_full
    jobs, meta = {}, {}
    for name, run in runs.items():
        cfg = run["cfg"]
        ref_ids, ref_w, _ = orc.route(run["x"], run["router_w"], run["bias"], cfg.top_k)
        sample = fs.sample_tokens(ref_ids, n_min=256, all_up_to=128, seed=cfg.M + 11)
        jobs[name] = (orc.bf16_to_f64(run["x"][sample]), ref_ids[sample])
        meta[name] = (sample, ref_w[sample])
    w13 = lambda e: mxo.mx_roundtrip_bf16_bits_lut(bits(weights["w13"][int(e)]))  # noqa: E731
    w2 = lambda e: mxo.mx_roundtrip_bf16_bits_lut(bits(weights["w2"][int(e)]))    # noqa: E731
    ys, ys7 = fs.stream_expert_rows(jobs, w13, w2, mi.CONFIGS["decode_m8"].I, act_bf16=True)
    res = {}
    for name, run in runs.items():
        sample, w = meta[name]
        out, z = orc.finalize(ys[name], w, run["residual"][sample], run["norm_w"], run["eps"])
        z7 = orc.finalize(ys7[name], w, run["residual"][sample], run["norm_w"], run["eps"])[1]
        res[name] = (sample, out, z, z7)
    return res


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", FULL)
def test_forward_mx_prepared_full_size_against_oracle(mxp_full, mxp_full_oracle, name):
    _, runs = mxp_full
    run = runs[name]
    sample, out, z, z7 = mxp_full_oracle[name]
    if run["cfg"].M <= 128:
        assert len(sample) == run["cfg"].M
    else:
        assert len(sample) >= 256 and sample[-1] == run["cfg"].M - 1
    print(f"{name}: {len(sample)} tokens against the oracle", flush=True)
    _check_close(torch.from_numpy(run["out"][sample]), out, f"{name} mxfp8 panels out")
    _check_close(torch.from_numpy(run["rout"][sample]), z, f"{name} mxfp8 panels residual_out",
                 extra=z7 - z)
