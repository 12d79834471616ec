"""Host logic of bench.py (CPU): the algorithmic byte and flop counts behind every roofline
figure, the refusal of more than one GPU, and the rules by which a counter record under
profiles/ is used or ignored."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import moe_inputs as mi  # noqa: E402

REAL = mi.CONFIGS["decode_m8"]           # H=7168, E=256, k=16, I=2048


def test_real_shape_sizes():
    # per-expert weight bytes of the real shape: W13 [2I, H] and W2 [H, I] in bf16
    assert 2 * REAL.I * REAL.H * 2 == 58_720_256
    assert REAL.H * REAL.I * 2 == 29_360_128


@pytest.mark.parametrize("M,touched", [(8, 103), (8, 106), (128, 256), (2048, 256)])
def test_layer_bytes_is_weights_router_rows_and_norm(M, touched):
    expect = touched * 88_080_384 + 3_670_016 + 3 * M * 7168 * 2 + 2 * 7168
    assert bench.layer_bytes(REAL, M, touched) == expect


def test_layer_bytes_all_experts_at_m2048():
    # all 256 experts resident and read once: 22.64 GB, 2.83 ms at 8 TB/s
    b = bench.layer_bytes(REAL, 2048, 256)
    assert b == 22_548_578_304 + 3_670_016 + 3 * 2048 * 7168 * 2 + 14_336
    assert abs(b / 8e12 * 1e6 - 2830) < 1


def test_narrow_weight_bytes():
    # MXFP8: one code byte plus one scale byte per 32 values; MXFP4: half a byte plus one
    # scale byte per 32 values; the router, rows and norm weight stay bf16
    rest = 3_670_016 + 3 * 8 * 7168 * 2 + 2 * 7168
    vals = 3 * 2048 * 7168
    assert bench.layer_bytes(REAL, 8, 100, "mx8") == 100 * (vals + vals // 32) + rest
    assert bench.layer_bytes(REAL, 8, 100, "mx4") == 100 * (vals // 2 + vals // 32) + rest


def test_up_and_down_bytes():
    M, t = 8, 106
    assert bench.up_bytes(REAL, M, t) == t * 58_720_256 + M * 7168 * 2 + M * 16 * 2048 * 2
    assert bench.down_bytes(REAL, M, t) == t * 29_360_128 + M * 16 * (2048 + 7168) * 2
    # the two GEMMs' weights are the layer's expert bytes
    assert (bench.up_bytes(REAL, M, t) - M * 7168 * 2 - M * 16 * 2048 * 2
            + bench.down_bytes(REAL, M, t) - M * 16 * (2048 + 7168) * 2) == t * 88_080_384


def test_flops():
    M = 2048
    assert bench.up_flops(REAL, M) == 4 * M * 16 * 7168 * 2048
    assert bench.down_flops(REAL, M) == 2 * M * 16 * 2048 * 7168
    assert bench.layer_flops(REAL, M) == (2 * M * 256 * 7168 + bench.up_flops(REAL, M)
                                          + bench.down_flops(REAL, M))
    # prefill M=2048: 2.89 TFLOP, 1.16 ms at the 2.5 PFLOP/s dense bf16 peak
    assert abs(bench.layer_flops(REAL, M) / 2.5e15 * 1e6 - 1158) < 1


def test_roofline_object():
    res = {"up_gbs": 6880.0, "up_bytes": 6_224_986_112, "up_us": 905.0, "up_tflops": 8.3,
           "down_gbs": 6790.0, "down_tflops": 8.2}
    prof = {"traffic_gbs": 6901.7, "traffic_bytes_per_launch": 6_226_223_231,
            "mfma_busy_frac": 0.0445}
    r = bench.roofline(res, "k", 6800.0, prof)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["frac"] == round(6880.0 / 8000.0, 4)
    assert r["traffic"] == 6901.7 and r["mfma_busy_frac_counter"] == 0.0445
    assert r["frac_of_measured_read"] == round(6880.0 / 6800.0, 4)
    r = bench.roofline(res, "k", None, None)
    assert r["traffic"] is None and "mfma_busy_frac_counter" not in r
    assert "measured_read_peak" not in r


def test_tile_rows_parse():
    assert bench._tile_rows("moe::expert_frag_kernel<128, true, 0, 2, 8>") == 128
    assert bench._tile_rows("expert_mx_decode_kernel<true> (32-row tiles)") == 32
    assert bench._tile_rows("expert_tiled (64-row tiles, up)") == 64
    assert bench._tile_rows("expert_up_stream_kernel") is None


def _record(tmp_path, **over):
    src = "expert_frag.hip"
    rec = {"kernel": "moe::expert_frag_kernel<128, true, 0, 2, 8> (grid 2097152)",
           "workload": "prefill_m2048", "source_file": src,
           "source_sha256_16": bench.source_hash(
               os.path.join(ROOT, "prefill_sigmoid_router_amd", "csrc", src)),
           "traffic_gbs": 3031.6}
    rec.update(over)
    (tmp_path / "rec.json").write_text(json.dumps(rec))


def test_load_profile_rules(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    kernel = "expert_frag_kernel<128, ...> (MXFP4 panels)"
    _record(tmp_path)
    assert bench.load_profile("rec.json", "prefill_m2048", kernel)["traffic_gbs"] == 3031.6
    # another workload, another tile height, a changed source, a missing source or file
    assert bench.load_profile("rec.json", "batch_m512", kernel) is None
    assert bench.load_profile("rec.json", "prefill_m2048", "expert_frag_kernel<64, ...>") is None
    _record(tmp_path, source_sha256_16="0" * 16)
    assert bench.load_profile("rec.json", "prefill_m2048", kernel) is None
    _record(tmp_path, source_file="no_such_file.hip")
    assert bench.load_profile("rec.json", "prefill_m2048", kernel) is None
    assert bench.load_profile("missing.json", "prefill_m2048", kernel) is None


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    msg = json.loads(p.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]
