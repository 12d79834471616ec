"""CPU checks of the C ABI: the library builds, loads, exports every function that
include/moe.h declares, and rejects invalid arguments on the host before launching
anything (no compute call runs here: these paths return before any HIP call)."""
import ctypes
import os
import re
import subprocess

import pytest

from oracle import moe_oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def B():
    from prefill_sigmoid_router_amd import binding, build
    if not os.path.exists(binding.library_path()):
        build.build()
    binding.load_library()
    return binding


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(moe_[a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_documented_entry_points():
    names = _declared_functions()
    for want in ("moe_route", "moe_align", "moe_forward", "moe_expert_up", "moe_expert_down",
                 "moe_finalize", "moe_workspace_bytes", "moe_align_capacity", "moe_strerror",
                 "moe_route_workspace_bytes", "moe_abi_version"):
        assert want in names


def test_library_exports_every_declared_symbol(B):
    out = subprocess.run(["nm", "-D", "--defined-only", B.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(B.load_library(), name)
    assert set(B.EXPORTED_SYMBOLS) == set(_declared_functions())


def test_library_links_no_torch(B):
    out = subprocess.run(["ldd", B.library_path()], capture_output=True, text=True).stdout
    # library names only: the load addresses ldd prints are hex and can spell "c10"
    names = [line.split()[0] for line in out.splitlines() if line.strip()]
    assert names and not any("torch" in n or n.startswith("libc10") for n in names), names


def test_strerror_and_version(B):
    assert B.moe_abi_version() == 108
    for s in (0, -1, -2, -3, -4, 17):
        assert isinstance(B.moe_strerror(s), str) and B.moe_strerror(s)


@pytest.mark.parametrize("M,k,E,block", [(4, 2, 8, 16), (8, 16, 256, 16), (128, 16, 256, 64),
                                         (512, 16, 256, 64), (2048, 16, 256, 64), (1, 1, 1, 1),
                                         (3, 5, 7, 3), (0, 4, 8, 16)])
def test_align_capacity_agrees_with_oracle(B, M, k, E, block):
    assert B.moe_align_capacity(M, k, E, block) == orc.align_capacity(M, k, E, block)


def test_workspace_bytes_cover_the_buffers(B):
    M, H, E, I, k, blk = 2048, 7168, 256, 2048, 16, 64
    cap = B.moe_align_capacity(M, k, E, blk)
    tiles16 = (M * k + 15) // 16 + min(E, M * k)      # 16-row tiles of real entries, at most
    # tiles and their expert groups: 2 x tiles16 int2; y: bf16 rows of every pick and the
    # fp32 rows of each token's first pick
    need = (M * E * 32 + 2 * M * k * 4 + cap * 4 + cap // blk * 4 + 4 + 2 * tiles16 * 8 + 4
            + cap * I * 2 + M * k * H * 2 + M * H * 4)
    got = B.moe_workspace_bytes(M, H, E, I, k, blk)
    assert need <= got <= need + 10 * 256
    assert B.moe_workspace_bytes(M, H, E, I, k, 48) == 0          # no kernel for block 48
    assert B.moe_workspace_bytes(M, 7164, E, I, k, blk) == 0      # H % 8 != 0
    assert B.moe_workspace_bytes(M, 7160, E, 2032, k, blk) > 0   # H % 8 == 0, I % 16 == 0
    assert B.moe_workspace_bytes(M, H, E, 2044, k, blk) == 0      # I % 16 != 0
    assert B.moe_workspace_bytes(M, H, 2000, I, k, blk) == 0      # E > 1024
    assert B.moe_route_workspace_bytes(M, E) >= M * E * 32


def _fwd(lib, **kw):
    args = dict(x=256, rw=256, bias=None, w13=256, w2=256, res=256, g=256, eps=1e-5, M=4, H=256,
                E=8, I=512, k=2, block=16, out=256, rout=None, ids=None, w=None, sid=None, bexp=None, npad=None,
                ws=256, wsb=1 << 40, ev=None)
    args.update(kw)
    p = lambda v: None if v is None else ctypes.c_void_p(v)  # noqa: E731
    return lib.moe_forward(p(args["x"]), p(args["rw"]), p(args["bias"]), p(args["w13"]),
                           p(args["w2"]), p(args["res"]), p(args["g"]), args["eps"], args["M"],
                           args["H"], args["E"], args["I"], args["k"], args["block"], p(args["out"]),
                           p(args["rout"]), p(args["ids"]), p(args["w"]), p(args["sid"]),
                           p(args["bexp"]), p(args["npad"]), p(args["ws"]), args["wsb"], args["ev"],
                           None)


@pytest.mark.parametrize("bad,code", [
    (dict(M=-1), -1), (dict(k=0), -1), (dict(k=9), -1), (dict(E=1025, k=2), -1),
    (dict(H=250), -1), (dict(H=4), -1), (dict(I=100), -1), (dict(I=8), -1), (dict(eps=0.0), -1), (dict(eps=float("nan")), -1),
    (dict(block=48), -2), (dict(block=8), -2), (dict(x=None), -1), (dict(out=None), -1),
    (dict(w13=None), -1), (dict(x=9), -1), (dict(ws=None), -3), (dict(wsb=16), -3),
    (dict(ws=64), -3),
])
def test_forward_rejects_invalid_arguments_on_the_host(B, bad, code):
    assert _fwd(B.load_library(), **bad) == code


def test_forward_zero_tokens_is_a_noop(B):
    assert _fwd(B.load_library(), M=0, x=None, res=None, out=None, ws=None, wsb=0) == 0


def test_route_align_finalize_validation(B):
    lib = B.load_library()
    p = ctypes.c_void_p
    # route: top_k > E, H % 8, workspace too small
    assert lib.moe_route(p(16), p(16), None, 4, 256, 8, 9, p(16), p(16), p(256), 1 << 30, None) == -1
    assert lib.moe_route(p(16), p(16), None, 4, 204, 8, 2, p(16), p(16), p(256), 1 << 30, None) == -1
    assert lib.moe_route(p(16), p(16), None, 4, 256, 8, 2, p(16), p(16), p(256), 8, None) == -3
    assert lib.moe_route(None, p(16), None, 4, 256, 8, 2, p(16), p(16), p(256), 1 << 30, None) == -1
    assert lib.moe_route(None, None, None, 0, 256, 8, 2, None, None, None, 0, None) == 0
    # align: block 0, E too large, null output
    assert lib.moe_align(p(16), 4, 2, 8, 0, p(16), p(16), p(16), None) == -1
    assert lib.moe_align(p(16), 4, 2, 1025, 16, p(16), p(16), p(16), None) == -1
    assert lib.moe_align(p(16), 4, 2, 8, 16, None, p(16), p(16), None) == -1
    assert lib.moe_align(p(16), 4, 2, 8, 16, p(16), p(16), p(18), None) == -1   # misaligned
    # finalize: eps <= 0, H % 8, null y
    assert lib.moe_finalize(p(16), p(16), p(16), p(16), 0.0, 4, 256, 2, p(16), None, None) == -1
    assert lib.moe_finalize(p(16), p(16), p(16), p(16), 1e-5, 4, 250, 2, p(16), None, None) == -1
    assert lib.moe_finalize(None, p(16), p(16), p(16), 1e-5, 4, 256, 2, p(16), None, None) == -1
    # expert GEMMs: capacity too small, unsupported block
    assert lib.moe_expert_up(p(16), p(16), p(16), p(16), p(16), 4, 256, 8, 512, 2, 16, 16, p(16), None) == -1
    assert lib.moe_expert_up(p(16), p(16), p(16), p(16), p(16), 4, 256, 8, 512, 2, 24, 240, p(16), None) == -2
    assert lib.moe_expert_down(p(16), p(16), p(16), p(16), p(16), 4, 256, 8, 512, 2, 16, 16, p(16), None) == -1


def test_forward_self_routes_for_few_ids(B):
    # the up GEMM builds the plan itself for 64-row tiles with streamed weights and at most
    # 256 flat ids; otherwise the align kernel runs
    assert B.moe_forward_self_routes(8, 256, 16, 2048)
    assert B.moe_forward_self_routes(1, 256, 16, 2048)
    assert B.moe_forward_self_routes(16, 256, 16, 2048)        # 256 ids
    assert not B.moe_forward_self_routes(17, 256, 16, 2048)    # 272 ids
    assert not B.moe_forward_self_routes(128, 256, 16, 2048)
    assert not B.moe_forward_self_routes(2048, 256, 16, 2048)  # 128-row tiles
    assert not B.moe_forward_self_routes(8, 256, 16, 192)      # streaming kernels (16 rows)
    assert B.moe_forward_self_routes(40, 16, 4, 512)           # 160 ids, 10 per expert
    assert not B.moe_forward_self_routes(8, 0, 1, 2048)
    assert not B.moe_forward_self_routes(-1, 256, 16, 2048)


def test_gemm_tile_rows_follows_tokens_per_expert(B):
    # bf16: expected tokens per expert M * top_k / E < 32 -> 64-row tiles, else 128-row
    # tiles; I not a multiple of 256 -> the 16-row streaming kernels
    assert B.moe_gemm_tile_rows(8, 256, 16, 2048) == 64
    assert B.moe_gemm_tile_rows(1, 256, 16, 2048) == 64
    assert B.moe_gemm_tile_rows(63, 256, 16, 2048) == 64
    assert B.moe_gemm_tile_rows(64, 256, 16, 2048) == 64
    assert B.moe_gemm_tile_rows(128, 256, 16, 2048) == 64
    assert B.moe_gemm_tile_rows(512, 256, 16, 2048) == 128
    assert B.moe_gemm_tile_rows(2048, 256, 16, 2048) == 128
    assert B.moe_gemm_tile_rows(2048, 256, 16, 192) == 16
    assert B.moe_gemm_tile_rows(2048, 256, 16, 100) == 0
    assert B.moe_gemm_tile_rows(2048, 256, 16, 48) == 16        # I % 16 == 0: streaming kernels
    assert B.moe_gemm_tile_rows(8, 0, 1, 2048) == 0
    assert B.moe_gemm_tile_rows(-1, 256, 16, 2048) == 0
    # MXFP8 weights: 32-row tiles of LDS codes below 16 tokens per expert, I a multiple of 256
    assert B.moe_gemm_tile_rows_mx(8, 256, 16, 2048) == 32
    assert B.moe_gemm_tile_rows_mx(128, 256, 16, 2048) == 32
    assert B.moe_gemm_tile_rows_mx(255, 256, 16, 2048) == 32
    assert B.moe_gemm_tile_rows_mx(256, 256, 16, 2048) == 64
    assert B.moe_gemm_tile_rows_mx(512, 256, 16, 2048) == 64
    assert B.moe_gemm_tile_rows_mx(1023, 256, 16, 2048) == 64
    assert B.moe_gemm_tile_rows_mx(1024, 256, 16, 2048) == 128
    assert B.moe_gemm_tile_rows_mx(2048, 256, 16, 2048) == 128
    assert B.moe_gemm_tile_rows_mx(2048, 256, 16, 384) == 0
    # fragment panels: bf16 as moe_forward; MXFP8 64-row tiles below 64 tokens per expert;
    # MXFP4 below 256
    for M in (1, 8, 128, 512, 2048):
        assert B.moe_gemm_tile_rows_panels(M, 256, 16, 2048, 16) == B.moe_gemm_tile_rows(M, 256, 16, 2048)
    assert B.moe_gemm_tile_rows_panels(512, 256, 16, 2048, 8) == 64
    assert B.moe_gemm_tile_rows_panels(1023, 256, 16, 2048, 8) == 64
    assert B.moe_gemm_tile_rows_panels(1024, 256, 16, 2048, 8) == 128
    assert B.moe_gemm_tile_rows_panels(512, 256, 16, 2048, 4) == 64
    assert B.moe_gemm_tile_rows_panels(1023, 256, 16, 2048, 4) == 64
    assert B.moe_gemm_tile_rows_panels(1024, 256, 16, 2048, 4) == 128
    assert B.moe_gemm_tile_rows_panels(2048, 256, 16, 2048, 4) == 128
    assert B.moe_gemm_tile_rows_panels(2048, 256, 16, 2048, 6) == 0
    assert B.moe_gemm_tile_rows_panels(2048, 256, 16, 384, 4) == 0


def test_read_probe_library_is_built_apart_from_the_layer(B):
    probe = os.path.join(os.path.dirname(B.library_path()), "libmoe_probe.so")
    out = subprocess.run(["nm", "-D", "--defined-only", probe], capture_output=True, text=True,
                         check=True).stdout
    names = set(line.split()[-1] for line in out.splitlines() if line.strip())
    assert {"moe_probe_read", "moe_probe_read_grid"} <= names
    layer = subprocess.run(["nm", "-D", "--defined-only", B.library_path()], capture_output=True,
                           text=True, check=True).stdout
    assert "moe_probe_read" not in layer


def test_mx_entry_points_validate_on_the_host(B):
    lib = B.load_library()
    p = ctypes.c_void_p
    # quantize / dequantize: K not a multiple of 32, null or misaligned pointers, rows 0
    assert lib.moe_mx_quantize(p(256), 4, 48, p(256), p(256), None) == -1
    assert lib.moe_mx_quantize(None, 4, 64, p(256), p(256), None) == -1
    assert lib.moe_mx_quantize(p(258), 4, 64, p(256), p(256), None) == -1
    assert lib.moe_mx_quantize(p(256), -1, 64, p(256), p(256), None) == -1
    assert lib.moe_mx_quantize(None, 0, 64, None, None, None) == 0
    assert lib.moe_mx_dequantize(p(256), p(256), 4, 16, p(256), None) == -1
    assert lib.moe_mx_dequantize(p(256), None, 4, 64, p(256), None) == -1
    assert lib.moe_mx_dequantize(None, None, 0, 64, None, None) == 0

    def fwd_mx(H=256, I=512, w13c=256, w13s=256, w2s=256, M=4):
        return lib.moe_forward_mx(p(256), p(256), None, None if w13c is None else p(w13c),
                                  p(w13s), p(256), p(w2s), p(256), p(256), 1e-5, M, H, 8, I, 2, 16,
                                  p(256), None, None, None, None, None, None, p(256), 1 << 40, None,
                                  None)
    assert fwd_mx(H=208) == -2             # H % 256 != 0
    assert fwd_mx(H=384) == -2             # H % 256 != 0
    assert fwd_mx(I=192) == -2             # I % 256 != 0
    assert fwd_mx(I=384) == -2             # I % 256 != 0
    assert fwd_mx(w13c=None) == -1
    assert fwd_mx(w13s=260) == -1          # scales must be 8-byte aligned
    assert fwd_mx(w2s=252) == -1
    assert fwd_mx(H=250) == -1             # H % 8 != 0 fails the shared size checks first
    assert fwd_mx(H=200) == -2             # H % 8 == 0 but not a multiple of 256


def test_size_contract_is_h_mod_8_and_i_mod_16(B):
    """The boundary accepts H % 8 == 0 (8 <= H <= 16384) and I % 16 == 0 (I >= 16): shapes
    with I not a multiple of 256 run the 16-row weight-streaming kernels."""
    for H, I, ok in [(8, 16, True), (200, 48, True), (264, 256, True), (16384, 64, True),
                     (4, 16, False), (12, 16, False), (16392, 16, False), (200, 8, False),
                     (200, 40, False)]:
        assert (B.moe_workspace_bytes(4, H, 8, I, 2, 16) > 0) == ok, (H, I)
    assert B.moe_gemm_tile_rows(64, 8, 2, 48) == 16
    assert B.moe_gemm_tile_rows(64, 8, 2, 256) == 64


def test_panel_entry_points_validate_on_the_host(B):
    """moe_prepare_weights / moe_forward_prepared, the MXFP4 and the MXFP8-panel entry points:
    sizes outside H % 64 == 0 and I % 256 == 0 are MOE_ERR_UNSUPPORTED, null, unpaired or
    misaligned pointers MOE_ERR_INVALID_ARG, before any launch."""
    lib = B.load_library()
    p = ctypes.c_void_p
    sz = ctypes.c_size_t
    # sizes of the panels
    assert lib.moe_prepared_w13_bytes(256, 7168, 2048) == 256 * 4096 * 7168 * 2
    assert lib.moe_prepared_w2_bytes(256, 7168, 2048) == 256 * 7168 * 2048 * 2
    assert lib.moe_prepared_w2_bytes(2, 640, 512) == 2 * 1024 * 512 * 2     # whole 512-row N tiles
    assert lib.moe_prepared_w13_bytes(4, 96, 256) == 0
    assert lib.moe_prepared_w13_bytes(4, 128, 128) == 0
    out = [sz(7) for _ in range(4)]
    assert lib.moe_mx4_weight_bytes(256, 7168, 2048, *[ctypes.byref(o) for o in out]) == 0
    assert [o.value for o in out] == [256 * 4096 * 7168 // 2, 256 * 4096 * 7168 // 32,
                                      256 * 7168 * 2048 // 2, 256 * 7168 * 2048 // 32]
    assert lib.moe_mx_prepared_bytes(256, 7168, 2048, *[ctypes.byref(o) for o in out]) == 0
    assert [o.value for o in out] == [256 * 4096 * 7168, 256 * 4096 * 7168 // 32,
                                      256 * 7168 * 2048, 256 * 7168 * 2048 // 32]
    for fn in (lib.moe_mx4_weight_bytes, lib.moe_mx_prepared_bytes):
        assert fn(4, 96, 256, None, None, None, None) == -2
        assert fn(4, 128, 128, None, None, None, None) == -2
        assert fn(4, 100, 256, None, None, None, None) == -1       # H % 8 != 0
        assert fn(0, 128, 256, None, None, None, None) == -1
    # re-layout and quantization: unpaired or misaligned pointers
    assert lib.moe_prepare_weights(p(256), None, 2, 128, 256, None, None, None) == -1
    assert lib.moe_prepare_weights(p(258), None, 2, 128, 256, p(256), None, None) == -1
    assert lib.moe_prepare_weights(p(256), None, 2, 96, 256, p(256), None, None) == -2
    assert lib.moe_mx4_quantize(p(256), None, 2, 128, 256, p(256), None, None, None, None) == -1
    assert lib.moe_mx4_quantize(p(256), None, 2, 128, 256, p(256), p(258), None, None, None) == -1
    assert lib.moe_mx4_dequantize(p(256), p(256), 7, 2, 128, 256, p(256), None) == -1
    assert lib.moe_mx_prepare_weights(p(256), p(256), None, None, 2, 128, 256, p(256), None, None,
                                      None, None) == -1
    assert lib.moe_mx_prepare_weights(p(256), p(256), None, None, 2, 128, 256, p(256), p(258),
                                      None, None, None) == -1
    assert lib.moe_mx_prepare_weights(None, None, None, None, 2, 128, 128, None, None, None, None,
                                      None) == -2

    # the forward passes on panels: unsupported widths, null weights, misaligned scales
    def fwd(fn, H=256, I=512, c13=256, s13=256, s2=256, M=4, eps=1e-5):
        return fn(p(256), p(256), None, None if c13 is None else p(c13), p(s13), p(256), p(s2),
                  p(256), p(256), eps, M, H, 8, I, 2, 16, p(256), None, None, None, None, None,
                  None, p(256), 1 << 40, None, None)
    for fn in (lib.moe_forward_mx4, lib.moe_forward_mx_prepared):
        assert fwd(fn, H=96) == -2
        assert fwd(fn, I=128) == -2
        assert fwd(fn, H=100) == -1
        assert fwd(fn, c13=None) == -1
        assert fwd(fn, s13=258) == -1                # scale panels 4-byte aligned
        assert fwd(fn, s2=254) == -1
        assert fwd(fn, eps=0.0) == -1
        assert fwd(fn, M=0) == 0                      # no tokens: nothing to do
    def fwd_prep(H=256, I=512, w13=256, M=4):
        return lib.moe_forward_prepared(p(256), p(256), None, None if w13 is None else p(w13),
                                        p(256), p(256), p(256), 1e-5, M, H, 8, I, 2, 16, p(256),
                                        None, None, None, None, None, None, p(256), 1 << 40, None,
                                        None)
    assert fwd_prep(H=96) == -2
    assert fwd_prep(I=128) == -2
    assert fwd_prep(w13=None) == -1
    assert fwd_prep(w13=264) == -1                    # 16-byte aligned panels
    assert fwd_prep(M=0) == 0
