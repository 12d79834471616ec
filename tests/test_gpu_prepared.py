"""GPU parity of the prepared-weights path (moe_prepare_weights + moe_forward_prepared)
through the C ABI.

The preparation is a pure re-layout: it is checked bit for bit against a host re-layout
written from the layout definition in include/moe.h.  moe_forward_prepared is checked
against the oracle to the bf16 bar (routing and plan bit-exact, outputs max-abs 2e-2 and
relative-L2 1e-2) and, since its GEMMs add the same MFMA products in the same K order as
moe_forward's, bit for bit against moe_forward on the natural weights.
"""
import numpy as np
import pytest
import torch

import _bars as bars
import _fullsize as fs
import moe_inputs as mi
from oracle import moe_oracle as orc

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


def _host_w13_panels(w13_bits, I):
    """W13p [E][I/256][8][H/32][4][64][8] from the definition: tile j of wave w, N tile n,
    lane l holds row n*256 + 32w + 16(j%2) + l%16 of the gate half (j < 2) or the up half
    (j >= 2), K values 32 s + 8 (l // 16) + v."""
    E, _, H = w13_bits.shape
    out = np.empty((E, I // 256, 8, H // 32, 4, 64, 8), dtype=np.uint16)
    lanes = np.arange(64)
    for n in range(I // 256):
        for w in range(8):
            for j in range(4):
                rows = n * 256 + 32 * w + 16 * (j % 2) + lanes % 16 + (0 if j < 2 else I)
                for s in range(H // 32):
                    ks = 32 * s + 8 * (lanes // 16)
                    idx = ks[:, None] + np.arange(8)[None, :]
                    out[:, n, w, s, j] = w13_bits[:, rows[:, None], idx]
    return out


def _host_w2_panels(w2_bits):
    """W2p [E][ceil(H/512)][8][I/32][4][64][8]: rows n*512 + 64w + 16j + l%16 (zero past H)."""
    E, H, I = w2_bits.shape
    nt = (H + 511) // 512
    out = np.zeros((E, nt, 8, I // 32, 4, 64, 8), dtype=np.uint16)
    lanes = np.arange(64)
    for n in range(nt):
        for w in range(8):
            for j in range(4):
                rows = n * 512 + 64 * w + 16 * j + lanes % 16
                for s in range(I // 32):
                    ks = 32 * s + 8 * (lanes // 16)
                    idx = ks[:, None] + np.arange(8)[None, :]
                    ok = rows < H
                    out[:, n, w, s, j][:, ok] = w2_bits[:, rows[ok][:, None], idx[ok]]
    return out


def _prepare(B, w13, w2, dev):
    E, two_i, H = w13.shape
    I = two_i // 2
    p13 = torch.full((B.moe_prepared_w13_bytes(E, H, I) // 2,), float("nan"), dtype=torch.bfloat16,
                     device=dev)
    p2 = torch.full((B.moe_prepared_w2_bytes(E, H, I) // 2,), float("nan"), dtype=torch.bfloat16,
                    device=dev)
    B.moe_prepare_weights(w13, w2, p13, p2)
    torch.cuda.synchronize()
    return p13, p2


def test_prepare_layout_bit_exact(B, dev):
    """W13 with two N tiles, W2 with H = 640 (a partial second panel, zero rows past H)."""
    cfg = mi.LayerConfig("prep_layout", M=1, H=640, E=3, top_k=1, I=512, block=16)
    L = mi.make_layer(cfg, device=dev, seed=7)
    p13, p2 = _prepare(B, L["w13"], L["w2"], dev)
    want13 = _host_w13_panels(bits(L["w13"]), cfg.I)
    want2 = _host_w2_panels(bits(L["w2"]))
    assert np.array_equal(bits(p13), want13.ravel())
    assert np.array_equal(bits(p2), want2.ravel())


# 64-row tiles with streamed weights (16 tokens per expert), 128-row tiles with streamed
# weights (50 per expert), 128-row tiles whose weights several tiles share (150 per expert,
# hot experts over several tiles, partial last tiles), and a partial down N tile (H = 640)
PREP_SMALL = {
    "prep64_stream": mi.LayerConfig("prep64_stream", M=64, H=320, E=16, top_k=4, I=256, block=16),
    "prep128_stream": mi.LayerConfig("prep128_stream", M=100, H=448, E=8, top_k=4, I=256,
                                     block=32, zipf_s=1.0),
    "prep128_shared": mi.LayerConfig("prep128_shared", M=300, H=640, E=8, top_k=4, I=512,
                                     block=64, zipf_s=1.0),
    "prep_one_token": mi.LayerConfig("prep_one_token", M=1, H=256, E=32, top_k=8, I=256,
                                     block=16),
}


def _run(B, L, dev, prepared=None):
    cfg = L["cfg"]
    M, H, E, I, k, blk = L["M"], cfg.H, cfg.E, cfg.I, cfg.top_k, cfg.block
    cap = B.moe_align_capacity(M, k, E, blk)
    r = {
        "out": torch.full((M, H), float("nan"), dtype=torch.bfloat16, device=dev),
        "rout": torch.full((M, H), float("nan"), dtype=torch.bfloat16, device=dev),
        "ids": torch.full((M, k), -7, dtype=torch.int32, device=dev),
        "w": torch.full((M, k), float("nan"), dtype=torch.float32, device=dev),
        "sorted": torch.full((cap,), -7, dtype=torch.int32, device=dev),
        "bexp": torch.full((cap // blk,), -7, dtype=torch.int32, device=dev),
        "npad": torch.full((1,), -7, dtype=torch.int32, device=dev),
    }
    ws = torch.empty(B.moe_workspace_bytes(M, H, E, I, k, blk), dtype=torch.uint8, device=dev)
    kw = dict(residual_out=r["rout"], topk_ids_out=r["ids"], topk_w_out=r["w"],
              sorted_ids_out=r["sorted"], block_expert_out=r["bexp"], num_padded_out=r["npad"])
    if prepared is None:
        B.moe_forward(L["x"], L["router_w"], L["router_bias"], L["w13"], L["w2"], L["residual"],
                      L["norm_w"], L["eps"], k, blk, r["out"], ws, **kw)
    else:
        B.moe_forward_prepared(L["x"], L["router_w"], L["router_bias"], prepared[0], prepared[1],
                               I, L["residual"], L["norm_w"], L["eps"], k, blk, r["out"], ws, **kw)
    torch.cuda.synchronize()
    return r


_check_close = bars.check_close


def _bias_np(L):
    return None if L["router_bias"] is None else L["router_bias"].cpu().numpy()


@pytest.mark.parametrize("name", list(PREP_SMALL))
def test_forward_prepared_small(B, dev, name):
    cfg = PREP_SMALL[name]
    rows = B.moe_gemm_tile_rows(cfg.M, cfg.E, cfg.top_k, cfg.I)
    print(f"forward_prepared parity {name} (token tile {rows})", flush=True)
    L = mi.make_layer(cfg, device=dev, seed=3)
    prepared = _prepare(B, L["w13"], L["w2"], dev)
    r = _run(B, L, dev, prepared)
    ref = orc.forward(bits(L["x"]), bits(L["router_w"]), _bias_np(L), bits(L["w13"]), bits(L["w2"]),
                      bits(L["residual"]), bits(L["norm_w"]), L["eps"], cfg.top_k, cfg.block)
    assert np.array_equal(r["ids"].cpu().numpy(), ref["topk_ids"])
    n_pad = int(r["npad"].item())
    assert n_pad == ref["num_padded"]
    assert np.array_equal(r["sorted"].cpu().numpy()[:n_pad], ref["sorted_ids"])
    assert np.array_equal(r["bexp"].cpu().numpy()[:n_pad // cfg.block], ref["block_expert"])
    _check_close(r["out"], ref["out"], name)
    _check_close(r["rout"], ref["residual_out"], name + " residual_out")
    nat = _run(B, L, dev)
    assert torch.equal(nat["out"].view(torch.int16), r["out"].view(torch.int16)), name
    assert torch.equal(nat["rout"].view(torch.int16), r["rout"].view(torch.int16)), name


def test_prepared_rejects_unsupported_widths(B, dev):
    assert B.moe_prepared_w13_bytes(8, 200, 256) == 0          # H % 64 != 0
    assert B.moe_prepared_w2_bytes(8, 256, 192) == 0           # I % 256 != 0
    w13 = torch.zeros((2, 384, 256), dtype=torch.bfloat16, device=dev)
    w2 = torch.zeros((2, 256, 192), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        B.moe_prepare_weights(w13, w2, torch.empty_like(w13), torch.empty_like(w2))


# ---------------------------------------------------------------------------------------
# Real shape: every workload, bit for bit against the natural path, sampled tokens against
# the oracle
# ---------------------------------------------------------------------------------------
FULL = ["decode_m8", "batch_m128", "batch_m512", "prefill_m2048", "prefill_m8192",
        "skew_m512"]


@pytest.fixture(scope="module")
def prep_full(B, dev):
    cfg = mi.CONFIGS["decode_m8"]
    print("generating full-size expert weights and their prepared panels", flush=True)
    L = mi.make_layer(cfg, device=dev, seed=0)
    weights = {k: L[k] for k in ("w13", "w2", "router_w", "norm_w")}
    p13, p2 = _prepare(B, L["w13"], L["w2"], dev)
    runs = {}
    for name in FULL:
        c = mi.CONFIGS[name]
        print(f"forward_prepared full-size {name} M={c.M}", flush=True)
        Lw = mi.make_layer(c, device=dev, seed=0, with_experts=False)
        Lw.update(weights)
        rp = _run(B, Lw, dev, (p13, p2))
        rn = _run(B, Lw, dev)
        runs[name] = {
            "cfg": c, "eps": Lw["eps"], "x": bits(Lw["x"]), "residual": bits(Lw["residual"]),
            "bias": _bias_np(Lw), "router_w": bits(Lw["router_w"]), "norm_w": bits(Lw["norm_w"]),
            "ids": rp["ids"].cpu().numpy(), "sorted": rp["sorted"].cpu().numpy(),
            "npad": int(rp["npad"].item()),
            "same_as_natural": (torch.equal(rp["out"].view(torch.int16), rn["out"].view(torch.int16))
                                and torch.equal(rp["rout"].view(torch.int16),
                                                rn["rout"].view(torch.int16))),
            "out": rp["out"].float().cpu().numpy().astype(np.float64),
            "rout": rp["rout"].float().cpu().numpy().astype(np.float64),
        }
        del rp, rn, Lw
    del p13, p2
    torch.cuda.empty_cache()
    return weights, runs


@pytest.mark.parametrize("name", FULL)
def test_forward_prepared_full_size_plan_and_natural(prep_full, name):
    _, runs = prep_full
    run = runs[name]
    cfg = run["cfg"]
    ref_ids, _, _ = orc.route(run["x"], run["router_w"], run["bias"], cfg.top_k)
    assert np.array_equal(run["ids"], ref_ids)
    sorted_ids, _, n_pad, _, _ = orc.align(ref_ids, cfg.E, cfg.block)
    assert run["npad"] == n_pad
    assert np.array_equal(run["sorted"][:n_pad], sorted_ids)
    assert run["same_as_natural"], f"{name}: prepared and natural outputs differ"


@pytest.fixture(scope="module")
def prep_full_oracle(prep_full):
    weights, runs = prep_full
    jobs, meta = {}, {}
    for name, run in runs.items():
        cfg = run["cfg"]
        ref_ids, ref_w, _ = orc.route(run["x"], run["router_w"], run["bias"], cfg.top_k)
        sample = fs.sample_tokens(ref_ids, n_min=256, all_up_to=128, seed=cfg.M + 2)
        jobs[name] = (orc.bf16_to_f64(run["x"][sample]), ref_ids[sample])
        meta[name] = (sample, ref_w[sample])
    w13 = mi.DeviceExpertsAsBits(weights["w13"])
    w2 = mi.DeviceExpertsAsBits(weights["w2"])
    ys, ys7 = fs.stream_expert_rows(jobs, w13.__getitem__, w2.__getitem__,
                                    mi.CONFIGS["decode_m8"].I, act_bf16=True)
    res = {}
    for name, run in runs.items():
        sample, w = meta[name]
        out, z = orc.finalize(ys[name], w, run["residual"][sample], run["norm_w"], run["eps"])
        z7 = orc.finalize(ys7[name], w, run["residual"][sample], run["norm_w"], run["eps"])[1]
        res[name] = (sample, out, z, z7)
    return res


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", FULL)
def test_forward_prepared_full_size_against_oracle(prep_full, prep_full_oracle, name):
    _, runs = prep_full
    run = runs[name]
    sample, out, z, z7 = prep_full_oracle[name]
    print(f"{name}: {len(sample)} tokens against the oracle", flush=True)
    _check_close(torch.from_numpy(run["out"][sample]), out, f"{name} prepared out")
    _check_close(torch.from_numpy(run["rout"][sample]), z, f"{name} prepared residual_out",
                 extra=z7 - z)
