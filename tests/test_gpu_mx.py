"""GPU parity of the MXFP8 expert weights (through the C ABI) against the CPU oracle.

Bar: the device's E4M3 codes and E8M0 scale bytes equal the oracle's bit for bit; its
dequantization to bf16 equals the oracle's exact values bit for bit; moe_forward_mx
equals the oracle layer run on the oracle's own dequantized weights to the bf16 bar
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


def _quantize(B, w, dev):
    K = w.shape[-1]
    codes = torch.full(tuple(w.shape), 0x5A, dtype=torch.uint8, device=dev)
    scales = torch.full(tuple(w.shape[:-1]) + (K // 32,), 0xA5, dtype=torch.uint8, device=dev)
    B.moe_mx_quantize(w, codes, scales)
    torch.cuda.synchronize()
    return codes, scales


def test_dequantize_every_code_at_several_scales(B, dev):
    """The conversion the MXFP8 GEMMs use, for all 254 finite codes, against the format."""
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    codes_np = np.resize(finite, (6, 256)).astype(np.uint8)      # 254 codes + 2 repeats per row
    scales_np = np.array([[10] * 8, [60] * 8, [119] * 8, [127] * 8, [150] * 8, [246] * 8],
                         dtype=np.uint8)
    codes = torch.from_numpy(codes_np).to(dev)
    scales = torch.from_numpy(scales_np).to(dev)
    w = torch.full((6, 256), float("nan"), dtype=torch.bfloat16, device=dev)
    B.moe_mx_dequantize(codes, scales, w)
    torch.cuda.synchronize()
    want = mxo.mx_dequantize_bf16_bits(codes_np, scales_np)
    assert np.array_equal(bits(w), want)


@pytest.mark.parametrize("case", ["normal", "wide", "ties_and_zeros", "full_row"])
def test_quantize_bit_exact(B, dev, case):
    rng = np.random.default_rng(7)
    if case == "normal":
        v = rng.normal(0, 0.02, (64, 512))
    elif case == "wide":      # blocks whose magnitudes span many binades
        v = rng.normal(0, 1, (32, 256)) * np.exp2(rng.integers(-20, 20, (32, 256)))
    elif case == "ties_and_zeros":
        # values that land exactly between E4M3 neighbours after scaling, zero blocks,
        # negative zeros and block maxima that clamp to 448
        pos = mxo.e4m3_decode(np.arange(0x00, 0x7F, dtype=np.uint8))
        mids = (pos[1:] + pos[:-1]) / 2
        v = np.zeros((8, 256))
        v[0, :125] = mids[:125] / 256.0
        v[0, 200] = 1.0                                   # sets s = -8 for its block
        v[1, :125] = -mids[:125] / 256.0 * 8
        v[2, 32:64] = -0.0
        v[3, 5] = 1.875
        v[4] = rng.normal(0, 1e-30, 256)
        v[5, ::7] = 3.0
    else:                     # a whole W13 row of the decode shape
        v = rng.normal(0, 0.02, (4, 7168))
    w_bits = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w = torch.from_numpy(w_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    codes, scales = _quantize(B, w, dev)
    ref_codes, ref_scales = mxo.mx_quantize(w_bits)
    assert np.array_equal(scales.cpu().numpy(), ref_scales), case
    assert np.array_equal(codes.cpu().numpy(), ref_codes), case


def _mx_weights(B, L, dev):
    w13c, w13s = _quantize(B, L["w13"], dev)
    w2c, w2s = _quantize(B, L["w2"], dev)
    return w13c, w13s, w2c, w2s


def _run_forward_mx(B, L, dev, mx):
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
    B.moe_forward_mx(L["x"], L["router_w"], L["router_bias"], *mx, L["residual"], L["norm_w"],
                     L["eps"], k, blk, r["out"], ws, residual_out=r["rout"], topk_ids_out=r["ids"],
                     topk_w_out=r["w"], sorted_ids_out=r["sorted"], block_expert_out=r["bexp"],
                     num_padded_out=r["npad"])
    torch.cuda.synchronize()
    return r


_check_close = bars.check_close


def _bias_np(L):
    return None if L["router_bias"] is None else L["router_bias"].cpu().numpy()


# expected tokens per expert M * top_k / E, with the kernels that copy the codes into LDS:
# below 16 32-row tiles (mx_tiny 1, mx_mid 4.6, mx_one_token 0.1, mx_dec_partial 10,
# mx_dec_groups 6), 16..63 64-row tiles (mx_tiles64 24 with nontemporal code copies,
# mx_tiles64_shared 50 without), from 64 128-row tiles, where the up GEMM dequantizes into
# the LDS tiles of the tiled kernel (mx_many 150)
SMALL_MX = {
    "mx_tiny": mi.LayerConfig("mx_tiny", M=4, H=256, E=8, top_k=2, I=512, block=16),
    "mx_mid": mi.LayerConfig("mx_mid", M=37, H=1024, E=32, top_k=4, I=256, block=16),
    # H=768: three 256-value K groups over four waves (one wave streams none)
    "mx_tiles64": mi.LayerConfig("mx_tiles64", M=48, H=512, E=8, top_k=4, I=256, block=32,
                                 zipf_s=1.0),
    "mx_many": mi.LayerConfig("mx_many", M=300, H=768, E=8, top_k=4, I=512, block=64,
                              zipf_s=1.0),
    # I=256: one K group, so one down K half is empty
    "mx_one_token": mi.LayerConfig("mx_one_token", M=1, H=512, E=64, top_k=8, I=256, block=16),
    "mx_tiles64_shared": mi.LayerConfig("mx_tiles64_shared", M=200, H=512, E=8, top_k=2,
                                        I=256, block=64, zipf_s=1.0),
    # 32-row tiles: H=768 is 6 K chunks of 128 with 24 scale bytes per row (one partial
    # group of 8 chunks), and Zipf routing gives the hot expert more than 16 rows (both
    # token row tiles of its tile live)
    "mx_dec_partial": mi.LayerConfig("mx_dec_partial", M=40, H=768, E=8, top_k=2, I=256,
                                     block=16, zipf_s=1.0),
    # H=1280: 10 K chunks, a whole scale group then a partial one (8 of 32 bytes)
    "mx_dec_groups": mi.LayerConfig("mx_dec_groups", M=24, H=1280, E=16, top_k=4, I=512,
                                    block=32),
}


@pytest.mark.parametrize("name", list(SMALL_MX))
def test_forward_mx_small(B, dev, name):
    cfg = SMALL_MX[name]
    print(f"forward_mx parity {name}", flush=True)
    L = mi.make_layer(cfg, device=dev, seed=5)
    mx = _mx_weights(B, L, dev)
    r = _run_forward_mx(B, L, dev, mx)
    ref_w13c, ref_w13s = mxo.mx_quantize(bits(L["w13"]))
    ref_w2c, ref_w2s = mxo.mx_quantize(bits(L["w2"]))
    assert np.array_equal(mx[0].cpu().numpy(), ref_w13c) and np.array_equal(mx[1].cpu().numpy(), ref_w13s)
    assert np.array_equal(mx[2].cpu().numpy(), ref_w2c) and np.array_equal(mx[3].cpu().numpy(), ref_w2s)
    ref = orc.forward(bits(L["x"]), bits(L["router_w"]), _bias_np(L),
                      mxo.mx_dequantize_bf16_bits(ref_w13c, ref_w13s),
                      mxo.mx_dequantize_bf16_bits(ref_w2c, ref_w2s),
                      bits(L["residual"]), bits(L["norm_w"]), L["eps"], cfg.top_k, cfg.block)
    assert np.array_equal(r["ids"].cpu().numpy(), ref["topk_ids"])
    n_pad = int(r["npad"].item())
    assert n_pad == ref["num_padded"]
    assert np.array_equal(r["sorted"].cpu().numpy()[:n_pad], ref["sorted_ids"])
    _check_close(r["out"], ref["out"], name)
    _check_close(r["rout"], ref["residual_out"], name + " residual_out")


def test_forward_mx_rejects_unsupported_widths(B, dev):
    cfg = mi.LayerConfig("mx_bad", M=4, H=208, E=8, top_k=2, I=256, block=16)
    L = mi.make_layer(cfg, device=dev, seed=5)
    w13c = torch.zeros((8, 512, 208), dtype=torch.uint8, device=dev)
    w13s = torch.zeros((8, 512, 6), dtype=torch.uint8, device=dev)
    w2c = torch.zeros((8, 208, 256), dtype=torch.uint8, device=dev)
    w2s = torch.zeros((8, 208, 8), dtype=torch.uint8, device=dev)
    out = torch.empty((4, 208), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(B.moe_workspace_bytes(4, 208, 8, 256, 2, 16), dtype=torch.uint8, device=dev)
    with pytest.raises(B.MoeError) as ei:
        B.moe_forward_mx(L["x"], L["router_w"], None, w13c, w13s, w2c, w2s, L["residual"],
                         L["norm_w"], L["eps"], 2, 16, out, ws)
    assert ei.value.status == -2


MX_FULL = ["decode_m8", "batch_m128", "batch_m512", "prefill_m2048", "prefill_m8192",
           "skew_m512"]


@pytest.fixture(scope="module")
def mx_full(B, dev):
    """The real-shape expert weights (E=256, H=7168, I=2048) and their MXFP8 codes."""
    L = mi.make_layer(mi.CONFIGS["decode_m8"], device=dev, seed=0)
    weights = {k: L[k] for k in ("w13", "w2", "router_w", "norm_w")}
    return weights, _mx_weights(B, L, dev)


@pytest.fixture(scope="module")
def mx_full_runs(B, dev, mx_full):
    """The four real-shape workloads through moe_forward_mx, results on the host."""
    weights, mx = mx_full
    runs = {}
    for name in MX_FULL:
        cfg = mi.CONFIGS[name]
        print(f"forward_mx full-size {name} M={cfg.M}", flush=True)
        L = mi.make_layer(cfg, device=dev, seed=0, with_experts=False)
        L.update(weights)
        r = _run_forward_mx(B, L, dev, mx)
        runs[name] = {
            "cfg": cfg, "eps": L["eps"], "x": bits(L["x"]), "residual": bits(L["residual"]),
            "bias": _bias_np(L), "router_w": bits(L["router_w"]), "norm_w": bits(L["norm_w"]),
            "ids": r["ids"].cpu().numpy(), "sorted": r["sorted"].cpu().numpy(),
            "npad": int(r["npad"].item()),
            "out": r["out"].float().cpu().numpy().astype(np.float64),
            "rout": r["rout"].float().cpu().numpy().astype(np.float64),
        }
        del r, L
        torch.cuda.empty_cache()
    return runs


@pytest.mark.parametrize("name", MX_FULL)
def test_forward_mx_full_size_routing_and_plan(mx_full_runs, name):
    """32-row tiles of LDS codes at M=8 and M=128, 64-row tiles at M=512 (Zipf), 128-row tiles
    at M=2048: routing and plan bit-exact for every token, every output row finite."""
    run = mx_full_runs[name]
    cfg = run["cfg"]
    ref_ids, _, _ = orc.route(run["x"], run["router_w"], run["bias"], cfg.top_k)
    assert np.array_equal(run["ids"], ref_ids)
    sorted_ids, _, n_pad, _, _ = orc.align(ref_ids, cfg.E, cfg.block)
    assert run["npad"] == n_pad
    assert np.array_equal(run["sorted"][:n_pad], sorted_ids)
    assert np.isfinite(run["out"]).all() and np.isfinite(run["rout"]).all()


def test_mx_full_size_codes_bit_exact(mx_full):
    """The device quantizer on real-shape experts (every 17th expert and the last): codes
    and scale bytes equal the oracle's."""
    weights, mx = mx_full
    for e in list(range(0, 256, 17)) + [255]:
        c, sc = mxo.mx_quantize_lut(bits(weights["w13"][e]))
        assert np.array_equal(mx[0][e].cpu().numpy(), c) and np.array_equal(mx[1][e].cpu().numpy(), sc), e
        c, sc = mxo.mx_quantize_lut(bits(weights["w2"][e]))
        assert np.array_equal(mx[2][e].cpu().numpy(), c) and np.array_equal(mx[3][e].cpu().numpy(), sc), e


@pytest.fixture(scope="module")
def mx_full_oracle(mx_full_runs, mx_full):
    """The oracle on the sampled tokens of all four workloads, on the oracle's own
    dequantized MXFP8 weights, in one pass over the experts."""
    weights, _ = mx_full
    jobs, meta = {}, {}
    for name, run in mx_full_runs.items():
        cfg = run["cfg"]
        ref_ids, ref_w, _ = orc.route(run["x"], run["router_w"], run["bias"], cfg.top_k)
        sample = fs.sample_tokens(ref_ids, n_min=256, all_up_to=128, seed=cfg.M + 1)
        jobs[name] = (orc.bf16_to_f64(run["x"][sample]), ref_ids[sample])
        meta[name] = (sample, ref_w[sample])
    print(f"oracle pass over the MXFP8 experts for {sum(len(m[0]) for m in meta.values())} "
          "tokens", flush=True)
    w13 = lambda e: mxo.mx_roundtrip_bf16_bits_lut(bits(weights["w13"][int(e)]))  # noqa: E731
    w2 = lambda e: mxo.mx_roundtrip_bf16_bits_lut(bits(weights["w2"][int(e)]))    # noqa: E731
    ys, ys7 = fs.stream_expert_rows(jobs, w13, w2, mi.CONFIGS["decode_m8"].I, act_bf16=True)
    res = {}
    for name, run in mx_full_runs.items():
        sample, w = meta[name]
        out, z = orc.finalize(ys[name], w, run["residual"][sample], run["norm_w"], run["eps"])
        z7 = orc.finalize(ys7[name], w, run["residual"][sample], run["norm_w"], run["eps"])[1]
        res[name] = (sample, out, z, z7)
    return res


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", MX_FULL)
def test_forward_mx_full_size_against_oracle(mx_full_runs, mx_full_oracle, name):
    """Sampled tokens against the oracle layer on the oracle's dequantized weights: all 8
    tokens at decode; from M=128 at least 256 tokens (all 128 at M=128) including token M-1
    and, for every expert, the first and the last token that picked it."""
    run = mx_full_runs[name]
    cfg = run["cfg"]
    sample, out, z, z7 = mx_full_oracle[name]
    if cfg.M <= 128:
        assert len(sample) == cfg.M
    else:
        assert len(sample) >= 256 and sample[-1] == cfg.M - 1
        ids = run["ids"]
        for e in np.unique(ids):
            rows = np.nonzero((ids == e).any(axis=1))[0]
            assert rows[-1] in sample and rows[0] in sample
    print(f"{name}: {len(sample)} tokens against the oracle", flush=True)
    _check_close(torch.from_numpy(run["out"][sample]), out, f"{name} mx out")
    _check_close(torch.from_numpy(run["rout"][sample]), z, f"{name} mx residual_out",
                 extra=z7 - z)


@pytest.mark.parametrize("name", ["mx_tiny", "mx_many"])
def test_forward_mx_graph_replay(B, dev, name):
    """moe_forward_mx captured in a HIP graph (32-row tiles of LDS codes for mx_tiny, 128-row tiles
    for mx_many): each replay, with new inputs copied in and eager work between replays,
    equals bit for bit an eager call on the same inputs on a side stream."""
    cfg = SMALL_MX[name]
    print(f"forward_mx graph replay {name}", flush=True)
    L = mi.make_layer(cfg, device=dev, seed=4)
    mx = _mx_weights(B, L, dev)
    M, H, E, I, k, blk = L["M"], cfg.H, cfg.E, cfg.I, cfg.top_k, cfg.block
    nws = B.moe_workspace_bytes(M, H, E, I, k, blk)

    def buffers():
        return (torch.empty((M, H), dtype=torch.bfloat16, device=dev),
                torch.empty(nws, dtype=torch.uint8, device=dev))

    def call(x, out, ws):
        B.moe_forward_mx(x, L["router_w"], L["router_bias"], *mx, L["residual"], L["norm_w"],
                         L["eps"], k, blk, out, ws)

    x_static = L["x"].clone()
    out_g, ws_g = buffers()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(x_static, out_g, ws_g)
    side = torch.cuda.Stream()
    gen = torch.Generator(device=dev)
    gen.manual_seed(12)
    for rep in range(3):
        xr = torch.randn((M, H), generator=gen, device=dev).to(torch.bfloat16)
        x_static.copy_(xr)
        graph.replay()
        out_e, ws_e = buffers()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call(xr, out_e, ws_e)
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), (name, rep)
        torch.randn(1 << 20, device=dev).sum().item()
