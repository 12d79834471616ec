"""The fragment-panel entry points (moe_forward_prepared, moe_forward_mx_prepared,
moe_forward_mx4) captured in a HIP graph: every replay, with new inputs copied in and eager
work between replays, equals bit for bit an eager call on the same inputs made on a second
stream into separate buffers.  The panels' own parity against the oracle is in
test_gpu_prepared.py, test_gpu_mx_prepared.py and test_gpu_mx4.py."""
import pytest
import torch

import moe_inputs as mi

pytestmark = pytest.mark.gpu

CASES = {
    # 64-row tiles, nontemporal weights, 4-wave workgroups on half N tiles
    "tiles64": mi.LayerConfig("graph_tiles64", M=64, H=320, E=16, top_k=4, I=256, block=16),
    # 128-row tiles of a hot expert sharing its weights (Zipf routing), partial W2 panel
    "tiles128": mi.LayerConfig("graph_tiles128", M=600, H=640, E=8, top_k=4, I=256, block=64,
                               zipf_s=1.0),
}


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


def _panels(B, fmt, L, dev):
    """The entry point's weight arguments: bf16 panels, MXFP8 panels or MXFP4 panels."""
    cfg = L["cfg"]
    E, H, I = cfg.E, cfg.H, cfg.I
    if fmt == "bf16":
        p13 = torch.empty(B.moe_prepared_w13_bytes(E, H, I) // 2, dtype=torch.bfloat16, device=dev)
        p2 = torch.empty(B.moe_prepared_w2_bytes(E, H, I) // 2, dtype=torch.bfloat16, device=dev)
        B.moe_prepare_weights(L["w13"], L["w2"], p13, p2)
        return [p13, p2]
    if fmt == "mx4":
        q = [torch.empty(n, dtype=torch.uint8, device=dev) for n in B.moe_mx4_weight_bytes(E, H, I)]
        B.moe_mx4_quantize(L["w13"], L["w2"], *q)
        return q
    nat = []
    for name in ("w13", "w2"):
        w = L[name]
        c = torch.empty(tuple(w.shape), dtype=torch.uint8, device=dev)
        sc = torch.empty(tuple(w.shape[:-1]) + (w.shape[-1] // 32,), dtype=torch.uint8, device=dev)
        B.moe_mx_quantize(w, c, sc)
        nat += [c, sc]
    p = [torch.empty(n, dtype=torch.uint8, device=dev) for n in B.moe_mx_prepared_bytes(E, H, I)]
    B.moe_mx_prepare_weights(*nat, E, H, I, *p)
    return p


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("fmt", ["bf16", "mx8", "mx4"])
def test_panel_forward_graph_replay(B, dev, fmt, case):
    cfg = CASES[case]
    bits = 16 if fmt == "bf16" else 8 if fmt == "mx8" else 4
    rows = B.moe_gemm_tile_rows_panels(cfg.M, cfg.E, cfg.top_k, cfg.I, bits)
    print(f"panel graph replay {fmt} {case} (token tile {rows})", flush=True)
    assert rows == (64 if case == "tiles64" else 128)
    L = mi.make_layer(cfg, device=dev, seed=6)
    w = _panels(B, fmt, L, dev)
    torch.cuda.synchronize()
    M, H, E, I, k, blk = L["M"], cfg.H, cfg.E, cfg.I, cfg.top_k, cfg.block
    nws = B.moe_workspace_bytes(M, H, E, I, k, blk)
    fwd = {"bf16": B.moe_forward_prepared, "mx8": B.moe_forward_mx_prepared,
           "mx4": B.moe_forward_mx4}[fmt]

    def buffers():
        return (torch.full((M, H), float("nan"), dtype=torch.bfloat16, device=dev),
                torch.full((M, H), float("nan"), dtype=torch.bfloat16, device=dev),
                torch.full((M, k), -7, dtype=torch.int32, device=dev),
                torch.empty(nws, dtype=torch.uint8, device=dev))

    def call(x, bufs):
        out, rout, ids, ws = bufs
        fwd(x, L["router_w"], L["router_bias"], *w, I, L["residual"], L["norm_w"], L["eps"], k,
            blk, out, ws, residual_out=rout, topk_ids_out=ids)

    x_static = L["x"].clone()
    bufs_g = buffers()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(x_static, bufs_g)
    side = torch.cuda.Stream()
    gen = torch.Generator(device=dev)
    gen.manual_seed(13)
    for rep in range(3):
        xr = torch.randn((M, H), generator=gen, device=dev).to(torch.bfloat16)
        x_static.copy_(xr)
        graph.replay()
        bufs_e = buffers()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call(xr, bufs_e)
        torch.cuda.synchronize()
        assert torch.equal(bufs_g[2], bufs_e[2]), (fmt, case, rep)
        for i in (0, 1):
            assert not torch.isnan(bufs_g[i].float()).any(), (fmt, case, rep, i)
            assert torch.equal(bufs_g[i].view(torch.int16), bufs_e[i].view(torch.int16)), \
                (fmt, case, rep, i)
        # unrelated eager work between replays
        torch.randn(1 << 20, device=dev).sum().item()
