"""GPU parity of the MXFP4 expert weights (moe_mx4_quantize, moe_mx4_dequantize,
moe_forward_mx4) through the C ABI, against the CPU oracle.

The device stores the codes in the prepared panel order that include/moe.h defines; the tests
map the panels back to natural [rows, K] codes and scale bytes on the host (from that
definition) and compare them with the oracle's MXFP4 conversion bit for bit.  The layer on
MXFP4 weights is checked against the oracle layer run on the oracle's own dequantized weights
(routing and plan bit-exact, outputs max-abs 2e-2 and relative-L2 1e-2).
"""
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
# Host map of the panel order (include/moe.h) back to natural [rows, K]
# ---------------------------------------------------------------------------------------
def _panel_rows_k(which, H, I):
    """Row and first K value of every (n, w, s, lane, tile) of the panels, and the scale
    rows of every (n, w, s, r, tile)."""
    if which == 13:
        nnt, K = I // 256, H
    else:
        nnt, K = (H + 511) // 512, I
    n, w, s, lane, j = np.meshgrid(np.arange(nnt), np.arange(8), np.arange(K // 32),
                                   np.arange(64), np.arange(4), indexing="ij")
    if which == 13:
        row = n * 256 + 32 * w + 16 * (j % 2) + lane % 16 + np.where(j >= 2, I, 0)
    else:
        row = n * 512 + 64 * w + 16 * j + lane % 16
    k0 = 32 * s + 8 * (lane // 16)
    n2, w2, s2, r2, j2 = np.meshgrid(np.arange(nnt), np.arange(8), np.arange(K // 32),
                                     np.arange(16), np.arange(4), indexing="ij")
    if which == 13:
        srow = n2 * 256 + 32 * w2 + 16 * (j2 % 2) + r2 + np.where(j2 >= 2, I, 0)
    else:
        srow = n2 * 512 + 64 * w2 + 16 * j2 + r2
    return row, k0, srow, s2


def panels_to_natural(codes, scales, which, E, H, I):
    """(codes [E, 2I or H, K] one code per byte, scale bytes [E, rows, K/32]) from panels."""
    rows_n = 2 * I if which == 13 else H
    K = H if which == 13 else I
    row, k0, srow, sblk = _panel_rows_k(which, H, I)
    c = np.asarray(codes).reshape((E,) + row.shape + (4,))
    sc = np.asarray(scales).reshape((E,) + srow.shape)
    out_c = np.zeros((E, rows_n, K), dtype=np.uint8)
    out_s = np.zeros((E, rows_n, K // 32), dtype=np.uint8)
    ok = row < rows_n
    for b in range(4):
        out_c[:, row[ok], k0[ok] + 2 * b] = c[..., b][:, ok] & 0xF
        out_c[:, row[ok], k0[ok] + 2 * b + 1] = c[..., b][:, ok] >> 4
    sok = srow < rows_n
    out_s[:, srow[sok], sblk[sok]] = sc[:, sok]
    # rows past H in the W2 panels hold zero codes and scale bytes
    if which == 2:
        assert np.all(c[:, ~ok] == 0) and np.all(sc[:, ~sok] == 0)
    return out_c, out_s


def _quantize(B, w13, w2, dev):
    E, two_i, H = w13.shape
    I = two_i // 2
    n = B.moe_mx4_weight_bytes(E, H, I)
    bufs = [torch.full((nb,), 0x5A, dtype=torch.uint8, device=dev) for nb in n]
    B.moe_mx4_quantize(w13, w2, *bufs)
    torch.cuda.synchronize()
    return bufs


# ---------------------------------------------------------------------------------------
# Conversion
# ---------------------------------------------------------------------------------------
def test_dequantize_every_code_byte_at_several_scales(B, dev):
    """Every code byte (two E2M1 values) at scale bytes from 2^-100 to 2^20, through the
    conversion the GEMMs use, against the format."""
    E, H, I = 1, 64, 256
    n = B.moe_mx4_weight_bytes(E, H, I)
    codes_np = np.resize(np.arange(256, dtype=np.uint8), n[0])
    scales_np = np.resize(np.array([27, 100, 120, 125, 127, 130, 147], dtype=np.uint8), n[1])
    w = torch.full((E, 2 * I, H), float("nan"), dtype=torch.bfloat16, device=dev)
    B.moe_mx4_dequantize(torch.from_numpy(codes_np).to(dev), torch.from_numpy(scales_np).to(dev),
                         13, E, H, I, w)
    torch.cuda.synchronize()
    nat_c, nat_s = panels_to_natural(codes_np, scales_np, 13, E, H, I)
    want = mxo.mx4_dequantize_bf16_bits(nat_c, nat_s)
    assert np.array_equal(bits(w), want)


QUANT_SHAPES = [(3, 128, 256), (2, 640, 512)]   # (E, H, I); H = 640: a partial W2 panel


@pytest.mark.parametrize("shape", QUANT_SHAPES, ids=lambda s: f"E{s[0]}_H{s[1]}_I{s[2]}")
def test_quantize_bit_exact(B, dev, shape):
    E, H, I = shape
    rng = np.random.default_rng(E * H)
    v13 = rng.normal(0, 0.02, (E, 2 * I, H)) * np.exp2(rng.integers(-8, 8, (E, 2 * I, 1)))
    v2 = rng.normal(0, 1, (E, H, I))
    # ties between E2M1 neighbours after scaling, zero blocks, values that clamp to 6
    mags = mxo.e2m1_decode(np.arange(8))
    mids = (mags[1:] + mags[:-1]) / 2
    v13[0, 0, :7] = mids
    v13[0, 0, 7] = 6.0
    v13[0, 1, :32] = 0.0
    v13[0, 2, :32] = -mids.max()
    v2[0, 3, 5] = 1.875
    w13_bits = (v13.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w2_bits = (v2.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w13 = torch.from_numpy(w13_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    w2 = torch.from_numpy(w2_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    q13, s13, q2, s2 = _quantize(B, w13, w2, dev)
    for which, q, sc, wb in ((13, q13, s13, w13_bits), (2, q2, s2, w2_bits)):
        nat_c, nat_s = panels_to_natural(q.cpu().numpy(), sc.cpu().numpy(), which, E, H, I)
        ref_c, ref_s = mxo.mx4_quantize(wb)
        assert np.array_equal(nat_s, ref_s), which
        assert np.array_equal(nat_c, ref_c), which
    # and back: the device dequantization equals the oracle's
    w_back = torch.empty_like(w13)
    B.moe_mx4_dequantize(q13, s13, 13, E, H, I, w_back)
    torch.cuda.synchronize()
    c, sc = mxo.mx4_quantize(w13_bits)
    assert np.array_equal(bits(w_back), mxo.mx4_dequantize_bf16_bits(c, sc))


# ---------------------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------------------
# MXFP4 tiles: 64 rows below 64 expected tokens per expert (nontemporal weights below 32),
# 128 rows from there
MX4_SMALL = {
    "mx4_tiles64_stream": mi.LayerConfig("mx4_tiles64_stream", M=64, H=320, E=16, top_k=4,
                                         I=256, block=16),
    "mx4_tiles64_zipf": mi.LayerConfig("mx4_tiles64_zipf", M=100, H=448, E=8, top_k=4,
                                       I=256, block=32, zipf_s=1.0),
    "mx4_tiles64_shared": mi.LayerConfig("mx4_tiles64_shared", M=120, H=640, E=8, top_k=4,
                                         I=512, block=64, zipf_s=1.0),
    "mx4_tiles128": mi.LayerConfig("mx4_tiles128", M=600, H=384, E=8, top_k=4, I=256,
                                   block=64, zipf_s=1.0),
    "mx4_one_token": mi.LayerConfig("mx4_one_token", M=1, H=256, E=32, top_k=8, I=256, block=16),
}


def _run(B, L, dev, q):
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
    B.moe_forward_mx4(L["x"], L["router_w"], L["router_bias"], *q, I, L["residual"], L["norm_w"],
                      L["eps"], k, blk, r["out"], ws, residual_out=r["rout"], topk_ids_out=r["ids"],
                      sorted_ids_out=r["sorted"], num_padded_out=r["npad"])
    torch.cuda.synchronize()
    return r


_check_close = bars.check_close


def _bias_np(L):
    return None if L["router_bias"] is None else L["router_bias"].cpu().numpy()


@pytest.mark.parametrize("name", list(MX4_SMALL))
def test_forward_mx4_small(B, dev, name):
    cfg = MX4_SMALL[name]
    print(f"forward_mx4 parity {name}", flush=True)
    L = mi.make_layer(cfg, device=dev, seed=5)
    q = _quantize(B, L["w13"], L["w2"], dev)
    r = _run(B, L, dev, q)
    c13, s13 = mxo.mx4_quantize(bits(L["w13"]))
    c2, s2 = mxo.mx4_quantize(bits(L["w2"]))
    ref = orc.forward(bits(L["x"]), bits(L["router_w"]), _bias_np(L),
                      mxo.mx4_dequantize_bf16_bits(c13, s13), mxo.mx4_dequantize_bf16_bits(c2, s2),
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
def mx4_full(B, dev):
    cfg = mi.CONFIGS["decode_m8"]
    print("generating full-size expert weights and their MXFP4 panels", flush=True)
    L = mi.make_layer(cfg, device=dev, seed=0)
    weights = {k: L[k] for k in ("w13", "w2", "router_w", "norm_w")}
    q = _quantize(B, L["w13"], L["w2"], dev)
    runs = {}
    for name in FULL:
        c = mi.CONFIGS[name]
        print(f"forward_mx4 full-size {name} M={c.M}", flush=True)
        Lw = mi.make_layer(c, device=dev, seed=0, with_experts=False)
        Lw.update(weights)
        r = _run(B, Lw, dev, q)
        runs[name] = {
            "cfg": c, "eps": Lw["eps"], "x": bits(Lw["x"]), "residual": bits(Lw["residual"]),
            "bias": _bias_np(Lw), "router_w": bits(Lw["router_w"]), "norm_w": bits(Lw["norm_w"]),
            "ids": r["ids"].cpu().numpy(), "sorted": r["sorted"].cpu().numpy(),
            "npad": int(r["npad"].item()),
            "out": r["out"].float().cpu().numpy().astype(np.float64),
            "rout": r["rout"].float().cpu().numpy().astype(np.float64),
        }
        del r, Lw
    # codes of a few real-shape experts bit for bit (host map of the panels of expert e)
    E, H, I = cfg.E, cfg.H, cfg.I
    n = B.moe_mx4_weight_bytes(E, H, I)
    per = [nb // E for nb in n]
    for e in (0, 97, 255):
        nat_c, nat_s = panels_to_natural(q[0][e * per[0]:(e + 1) * per[0]].cpu().numpy(),
                                         q[1][e * per[1]:(e + 1) * per[1]].cpu().numpy(), 13, 1, H, I)
        rc, rs = mxo.mx4_quantize_lut(bits(weights["w13"][e]))
        assert np.array_equal(nat_c[0], rc) and np.array_equal(nat_s[0], rs), e
    del q
    torch.cuda.empty_cache()
    return weights, runs


@pytest.mark.parametrize("name", FULL)
def test_forward_mx4_full_size_plan(mx4_full, name):
    _, runs = mx4_full
    run = runs[name]
    cfg = run["cfg"]
    ref_ids, _, _ = orc.route(run["x"], run["router_w"], run["bias"], cfg.top_k)
    assert np.array_equal(run["ids"], ref_ids)
    sorted_ids, _, n_pad, _, _ = orc.align(ref_ids, cfg.E, cfg.block)
    assert run["npad"] == n_pad
    assert np.array_equal(run["sorted"][:n_pad], sorted_ids)
    assert np.isfinite(run["out"]).all()


@pytest.fixture(scope="module")
def mx4_full_oracle(mx4_full):
    weights, runs = mx4_full
    jobs, meta = {}, {}
    for name, run in runs.items():
        cfg = run["cfg"]
        ref_ids, ref_w, _ = orc.route(run["x"], run["router_w"], run["bias"], cfg.top_k)
        sample = fs.sample_tokens(ref_ids, n_min=256, all_up_to=128, seed=cfg.M + 3)
        jobs[name] = (orc.bf16_to_f64(run["x"][sample]), ref_ids[sample])
        meta[name] = (sample, ref_w[sample])
    w13 = lambda e: mxo.mx4_roundtrip_bf16_bits_lut(bits(weights["w13"][int(e)]))  # noqa: E731
    w2 = lambda e: mxo.mx4_roundtrip_bf16_bits_lut(bits(weights["w2"][int(e)]))    # noqa: E731
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
def test_forward_mx4_full_size_against_oracle(mx4_full, mx4_full_oracle, name):
    _, runs = mx4_full
    run = runs[name]
    sample, out, z, z7 = mx4_full_oracle[name]
    if run["cfg"].M <= 128:
        assert len(sample) == run["cfg"].M
    else:
        assert len(sample) >= 256 and sample[-1] == run["cfg"].M - 1
    print(f"{name}: {len(sample)} tokens against the oracle", flush=True)
    _check_close(torch.from_numpy(run["out"][sample]), out, f"{name} mx4 out")
    _check_close(torch.from_numpy(run["rout"][sample]), z, f"{name} mx4 residual_out",
                 extra=z7 - z)
