"""moe_forward_noalloc (the library's static per-GPU scratch, for callers that cannot
allocate) against moe_forward with a caller workspace, through the C ABI: the two share
every kernel, so routing, plan and outputs must be identical bit for bit -- on two calls in
a row, the second with a smaller input, so the second call runs over the first call's
leftovers in the shared scratch.  Sizes past the scratch are refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import moe_inputs as mi

pytestmark = pytest.mark.gpu


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


# (layer, token count of the first call, token count of the second call)
SEQUENCES = [
    # 64-row tiled GEMMs with the self-routing up kernel (at most 256 flat ids)
    (mi.LayerConfig("noalloc_tiled", M=40, H=336, E=16, top_k=4, I=512, block=16, zipf_s=1.0), 40, 13),
    # the align kernel and 128-row tiles, then a call small enough to self-route
    (mi.LayerConfig("noalloc_many", M=300, H=256, E=8, top_k=4, I=256, block=64, zipf_s=1.0), 300, 30),
    # weight-streaming kernels (I not a multiple of 256) and the sliced finalize
    (mi.LayerConfig("noalloc_stream", M=37, H=1024, E=32, top_k=4, I=192, block=16), 37, 5),
]


def _call(B, L, dev, noalloc):
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
    kw = dict(residual_out=r["rout"], topk_ids_out=r["ids"], topk_w_out=r["w"],
              sorted_ids_out=r["sorted"], block_expert_out=r["bexp"], num_padded_out=r["npad"])
    args = (L["x"], L["router_w"], L["router_bias"], L["w13"], L["w2"], L["residual"],
            L["norm_w"], L["eps"], k, blk, r["out"])
    if noalloc:
        B.moe_forward_noalloc(*args, **kw)
    else:
        ws = torch.empty(B.moe_workspace_bytes(M, H, E, I, k, blk), dtype=torch.uint8, device=dev)
        B.moe_forward(*args, ws, **kw)
    torch.cuda.synchronize()
    return r


def _same(a, b, what):
    n = int(a["npad"].item())
    assert n == int(b["npad"].item()), what
    for key in ("ids", "w"):
        assert torch.equal(a[key], b[key]), (what, key)
    for key in ("out", "rout"):
        assert torch.equal(a[key].view(torch.int16), b[key].view(torch.int16)), (what, key)
    assert torch.equal(a["sorted"][:n], b["sorted"][:n]), what
    blk = a["sorted"].numel() // a["bexp"].numel()
    assert torch.equal(a["bexp"][:n // blk], b["bexp"][:n // blk]), what


@pytest.mark.parametrize("seq", SEQUENCES, ids=lambda s: s[0].name)
def test_noalloc_equals_workspace_call_twice_in_a_row(B, dev, seq):
    cfg, m1, m2 = seq
    assert m2 < m1
    for call, M in enumerate((m1, m2)):
        print(f"noalloc {cfg.name} call {call} M={M}", flush=True)
        assert B.moe_workspace_bytes(M, cfg.H, cfg.E, cfg.I, cfg.top_k, cfg.block) <= B.NOALLOC_SCRATCH_BYTES
        L = mi.make_layer(cfg, device=dev, seed=call, M=M)
        a = _call(B, L, dev, noalloc=True)
        b = _call(B, L, dev, noalloc=False)
        assert np.isfinite(a["out"].float().cpu().numpy()).all()
        _same(a, b, f"{cfg.name} call {call}")


def test_noalloc_refuses_sizes_past_the_scratch(B, dev):
    """The real-shape layer with block 64 fits the scratch up to 14 tokens; 15 do not: the
    call fails with MOE_ERR_WORKSPACE on the host, before any launch (pointers are never
    dereferenced)."""
    lib = B.load_library()
    p = ctypes.c_void_p
    fits = B.moe_workspace_bytes(14, 7168, 256, 2048, 16, 64) <= B.NOALLOC_SCRATCH_BYTES
    past = B.moe_workspace_bytes(15, 7168, 256, 2048, 16, 64) > B.NOALLOC_SCRATCH_BYTES
    assert fits and past
    st = lib.moe_forward_noalloc(p(256), p(256), None, p(256), p(256), p(256), p(256), 1e-5, 15,
                                 7168, 256, 2048, 16, 64, p(256), None, None, None, None, None,
                                 None, None)
    assert st == -3
    assert lib.moe_forward_noalloc(None, None, None, None, None, None, None, 1e-5, 0, 7168, 256,
                                   2048, 16, 64, None, None, None, None, None, None, None,
                                   None) == 0
