"""GPU parity of the whole layer on seeded random shapes (bf16, MXFP8, and the fragment
panels of bf16, MXFP8 and MXFP4 experts), through the C ABI, against the CPU oracle: routing
and plan bit-exact, outputs to the bf16 bar (max-abs 2e-2, relative-L2 1e-2).  The shapes
mix token counts that land on every GEMM path (16-row streaming, 32-row MXFP8 LDS codes,
64- and 128-row LDS tiles, 64- and 128-row panel tiles), K tails, partial N tiles, single
and many experts, every block size and both routing recipes."""
import numpy as np
import pytest
import torch

import _bars as bars
import moe_inputs as mi
from oracle import moe_oracle as orc
from oracle import mx_oracle as mxo

pytestmark = pytest.mark.gpu

bits = mi.bf16_bits


def _random_configs(seed, n, mx, panels=False):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 3, 8, 16, 40]))
        k = int(rng.integers(1, min(E, 8) + 1))
        if panels:
            # panel entry points: H a multiple of 64 (a partial last 512-row W2 N tile when
            # H % 512 != 0), I a multiple of 256
            H = 64 * int(rng.integers(1, 13))
            I = 256 * int(rng.integers(1, 3))
        elif mx:
            H = 256 * int(rng.integers(1, 4))
            I = 256 * int(rng.integers(1, 3))
        else:
            H = 16 * int(rng.integers(2, 49))
            # the tiled kernels need I to be a multiple of 256
            I = 256 * int(rng.integers(1, 3)) if rng.random() < 0.6 else 64 * int(rng.integers(1, 9))
        # token counts around the GEMM path thresholds (expected tokens per expert M*k/E)
        per_expert = float(rng.choice([0.5, 3, 6, 20, 40, 70] + ([300] if panels else [])))
        M = int(max(1, min(400 if panels else 200, round(per_expert * E / k))))
        block = int(rng.choice([16, 32, 64, 128]))
        zipf = None if rng.random() < 0.5 else 1.0
        tag = "panel" if panels else ("mx" if mx else "bf16")
        name = f"{tag}{i}_M{M}_H{H}_E{E}_k{k}_I{I}_B{block}{'_zipf' if zipf else ''}"
        out.append(mi.LayerConfig(name, M=M, H=H, E=E, top_k=k, I=I, block=block, zipf_s=zipf))
    return out


BF16_CASES = _random_configs(2024, 8, mx=False)
MX_CASES = _random_configs(2025, 5, mx=True)
PANEL_CASES = _random_configs(2026, 6, mx=False, panels=True) + [
    # many tokens per expert: 128-row tiles for every format
    mi.LayerConfig("panel_many_M400_H320_E3_k2_I256_B64", M=400, H=320, E=3, top_k=2, I=256,
                   block=64),
    # 128-row tiles for every format (150 tokens per expert), a partial W2 N tile (H = 448)
    mi.LayerConfig("panel_mid_M300_H448_E4_k2_I512_B32_zipf", M=300, H=448, E=4, top_k=2,
                   I=512, block=32, zipf_s=1.0),
]


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


def _buffers(B, cfg, M, dev):
    k, blk = cfg.top_k, cfg.block
    cap = B.moe_align_capacity(M, k, cfg.E, blk)
    return {
        "out": torch.full((M, cfg.H), float("nan"), dtype=torch.bfloat16, device=dev),
        "rout": torch.full((M, cfg.H), float("nan"), dtype=torch.bfloat16, device=dev),
        "ids": torch.full((M, k), -7, dtype=torch.int32, device=dev),
        "w": torch.full((M, k), float("nan"), dtype=torch.float32, device=dev),
        "sorted": torch.full((cap,), -7, dtype=torch.int32, device=dev),
        "bexp": torch.full((cap // blk,), -7, dtype=torch.int32, device=dev),
        "npad": torch.full((1,), -7, dtype=torch.int32, device=dev),
    }


def _kwargs(r):
    return dict(residual_out=r["rout"], topk_ids_out=r["ids"], topk_w_out=r["w"],
                sorted_ids_out=r["sorted"], block_expert_out=r["bexp"], num_padded_out=r["npad"])


def _check(r, ref, cfg, name):
    assert np.array_equal(r["ids"].cpu().numpy(), ref["topk_ids"]), name
    np.testing.assert_allclose(r["w"].cpu().numpy(), ref["topk_w"], rtol=0, atol=1e-6)
    n_pad = int(r["npad"].item())
    assert n_pad == ref["num_padded"], name
    assert np.array_equal(r["sorted"].cpu().numpy()[:n_pad], ref["sorted_ids"]), name
    assert np.array_equal(r["bexp"].cpu().numpy()[:n_pad // cfg.block], ref["block_expert"]), name
    for key, want in (("out", ref["out"]), ("rout", ref["residual_out"])):
        bars.check_close(r[key], want, f"{name} {key}")


def _bias(L):
    return None if L["router_bias"] is None else L["router_bias"].cpu().numpy()


@pytest.mark.parametrize("cfg", BF16_CASES, ids=[c.name for c in BF16_CASES])
def test_forward_random_shape(B, dev, cfg):
    print(f"random-shape forward {cfg.name} (GEMM token tile "
          f"{B.moe_gemm_tile_rows(cfg.M, cfg.E, cfg.top_k, cfg.I)})", flush=True)
    L = mi.make_layer(cfg, device=dev, seed=9)
    r = _buffers(B, cfg, L["M"], dev)
    ws = torch.empty(B.moe_workspace_bytes(L["M"], cfg.H, cfg.E, cfg.I, cfg.top_k, cfg.block),
                     dtype=torch.uint8, device=dev)
    B.moe_forward(L["x"], L["router_w"], L["router_bias"], L["w13"], L["w2"], L["residual"],
                  L["norm_w"], L["eps"], cfg.top_k, cfg.block, r["out"], ws, **_kwargs(r))
    torch.cuda.synchronize()
    ref = orc.forward(bits(L["x"]), bits(L["router_w"]), _bias(L), bits(L["w13"]), bits(L["w2"]),
                      bits(L["residual"]), bits(L["norm_w"]), L["eps"], cfg.top_k, cfg.block)
    _check(r, ref, cfg, cfg.name)


@pytest.mark.parametrize("cfg", MX_CASES, ids=[c.name for c in MX_CASES])
def test_forward_mx_random_shape(B, dev, cfg):
    print(f"random-shape forward_mx {cfg.name} (GEMM token tile "
          f"{B.moe_gemm_tile_rows_mx(cfg.M, cfg.E, cfg.top_k, cfg.I)})", flush=True)
    L = mi.make_layer(cfg, device=dev, seed=9)
    mx = []
    for name in ("w13", "w2"):
        w = L[name]
        c = torch.empty(tuple(w.shape), dtype=torch.uint8, device=dev)
        s = torch.empty(tuple(w.shape[:-1]) + (w.shape[-1] // 32,), dtype=torch.uint8, device=dev)
        B.moe_mx_quantize(w, c, s)
        mx += [c, s]
    r = _buffers(B, cfg, L["M"], dev)
    ws = torch.empty(B.moe_workspace_bytes(L["M"], cfg.H, cfg.E, cfg.I, cfg.top_k, cfg.block),
                     dtype=torch.uint8, device=dev)
    B.moe_forward_mx(L["x"], L["router_w"], L["router_bias"], *mx, L["residual"], L["norm_w"],
                     L["eps"], cfg.top_k, cfg.block, r["out"], ws, **_kwargs(r))
    torch.cuda.synchronize()
    w13c, w13s = mxo.mx_quantize(bits(L["w13"]))
    w2c, w2s = mxo.mx_quantize(bits(L["w2"]))
    assert np.array_equal(mx[0].cpu().numpy(), w13c) and np.array_equal(mx[3].cpu().numpy(), w2s)
    ref = orc.forward(bits(L["x"]), bits(L["router_w"]), _bias(L),
                      mxo.mx_dequantize_bf16_bits(w13c, w13s), mxo.mx_dequantize_bf16_bits(w2c, w2s),
                      bits(L["residual"]), bits(L["norm_w"]), L["eps"], cfg.top_k, cfg.block)
    _check(r, ref, cfg, cfg.name)


@pytest.mark.parametrize("cfg", PANEL_CASES, ids=[c.name for c in PANEL_CASES])
def test_forward_panels_random_shape(B, dev, cfg):
    """The same layer through moe_forward_prepared (bf16 panels, bit-identical to
    moe_forward), moe_forward_mx_prepared (MXFP8 panels of the oracle-checked natural codes)
    and moe_forward_mx4 (MXFP4 panels), each against the oracle on its own weights."""
    M, E, k, I = cfg.M, cfg.E, cfg.top_k, cfg.I
    print(f"random-shape panels {cfg.name} (tiles bf16 "
          f"{B.moe_gemm_tile_rows_panels(M, E, k, I, 16)}, MXFP8 "
          f"{B.moe_gemm_tile_rows_panels(M, E, k, I, 8)}, MXFP4 "
          f"{B.moe_gemm_tile_rows_panels(M, E, k, I, 4)})", flush=True)
    L = mi.make_layer(cfg, device=dev, seed=9)
    H = cfg.H
    ws = torch.empty(B.moe_workspace_bytes(L["M"], H, E, I, k, cfg.block), dtype=torch.uint8,
                     device=dev)
    x, rw, bias = L["x"], L["router_w"], L["router_bias"]
    common = (L["residual"], L["norm_w"], L["eps"], k, cfg.block)
    # bf16 panels: the natural layer, bit for bit
    p13 = torch.empty(B.moe_prepared_w13_bytes(E, H, I) // 2, dtype=torch.bfloat16, device=dev)
    p2 = torch.empty(B.moe_prepared_w2_bytes(E, H, I) // 2, dtype=torch.bfloat16, device=dev)
    B.moe_prepare_weights(L["w13"], L["w2"], p13, p2)
    rp = _buffers(B, cfg, L["M"], dev)
    B.moe_forward_prepared(x, rw, bias, p13, p2, I, *common, rp["out"], ws, **_kwargs(rp))
    rn = _buffers(B, cfg, L["M"], dev)
    B.moe_forward(x, rw, bias, L["w13"], L["w2"], *common, rn["out"], ws, **_kwargs(rn))
    torch.cuda.synchronize()
    ref = orc.forward(bits(x), bits(rw), _bias(L), bits(L["w13"]), bits(L["w2"]),
                      bits(L["residual"]), bits(L["norm_w"]), L["eps"], k, cfg.block)
    _check(rp, ref, cfg, cfg.name + " bf16 panels")
    assert torch.equal(rp["out"].view(torch.int16), rn["out"].view(torch.int16)), cfg.name
    del p13, p2
    # MXFP8 panels from the oracle's natural codes
    c13, s13 = mxo.mx_quantize(bits(L["w13"]))
    c2, s2 = mxo.mx_quantize(bits(L["w2"]))
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    q8 = [torch.empty(n, dtype=torch.uint8, device=dev) for n in B.moe_mx_prepared_bytes(E, H, I)]
    B.moe_mx_prepare_weights(up(c13), up(s13), up(c2), up(s2), E, H, I, *q8)
    r8 = _buffers(B, cfg, L["M"], dev)
    B.moe_forward_mx_prepared(x, rw, bias, *q8, I, *common, r8["out"], ws, **_kwargs(r8))
    torch.cuda.synchronize()
    ref8 = orc.forward(bits(x), bits(rw), _bias(L), mxo.mx_dequantize_bf16_bits(c13, s13),
                       mxo.mx_dequantize_bf16_bits(c2, s2), bits(L["residual"]),
                       bits(L["norm_w"]), L["eps"], k, cfg.block)
    _check(r8, ref8, cfg, cfg.name + " MXFP8 panels")
    # MXFP4 panels, quantized on the device (bit-exact against the oracle elsewhere)
    q4 = [torch.empty(n, dtype=torch.uint8, device=dev) for n in B.moe_mx4_weight_bytes(E, H, I)]
    B.moe_mx4_quantize(L["w13"], L["w2"], *q4)
    r4 = _buffers(B, cfg, L["M"], dev)
    B.moe_forward_mx4(x, rw, bias, *q4, I, *common, r4["out"], ws, **_kwargs(r4))
    torch.cuda.synchronize()
    d13, e13 = mxo.mx4_quantize(bits(L["w13"]))
    d2, e2 = mxo.mx4_quantize(bits(L["w2"]))
    ref4 = orc.forward(bits(x), bits(rw), _bias(L), mxo.mx4_dequantize_bf16_bits(d13, e13),
                       mxo.mx4_dequantize_bf16_bits(d2, e2), bits(L["residual"]),
                       bits(L["norm_w"]), L["eps"], k, cfg.block)
    _check(r4, ref4, cfg, cfg.name + " MXFP4")
