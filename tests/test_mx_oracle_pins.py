"""Pins of the MXFP8 weight oracle (oracle/mx_oracle.py) against the format definitions:
E4M3 values printed from the field layout, a brute-force nearest-value encoder, tie and
saturation cases, and hand-worked MX blocks.  CPU only."""
import numpy as np

from oracle import mx_oracle as mx


def _bf16(values):
    f = np.asarray(values, dtype=np.float32).view(np.uint32)
    assert np.all((f & 0xFFFF) == 0), "test value not exact in bf16"
    return (f >> 16).astype(np.uint16)


def test_e4m3_decode_known_codes():
    known = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
             0x38: 1.0, 0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x70: 128.0, 0x78: 256.0,
             0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for code, val in known.items():
        assert mx.e4m3_decode(np.uint8(code)) == val, hex(code)
    assert np.isnan(mx.e4m3_decode(np.uint8(0x7F))) and np.isnan(mx.e4m3_decode(np.uint8(0xFF)))
    assert mx.e4m3_decode(np.uint8(0x80)) == 0.0


def test_e4m3_decode_monotone_and_symmetric():
    pos = mx.e4m3_decode(np.arange(0x00, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    neg = mx.e4m3_decode(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg, -pos)
    # spacing doubles every 8 codes above the subnormals
    assert np.allclose(np.diff(pos[8:])[::8][1:] / np.diff(pos[8:])[::8][:-1], 2.0)


def test_e4m3_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F and c != 0x80], dtype=np.uint8)
    assert np.array_equal(mx.e4m3_encode(mx.e4m3_decode(codes)), codes)


def _brute_encode(v):
    codes = np.arange(0x00, 0x7F, dtype=np.uint8)
    vals = mx.e4m3_decode(codes)
    out = []
    for x in np.atleast_1d(v):
        a = min(abs(float(x)), 448.0)
        d = np.abs(vals - a)
        best = np.flatnonzero(d == d.min())
        c = int(codes[best[0]] if len(best) == 1 else codes[best[best % 2 == 0][0]])
        if x < 0 and c != 0:
            c |= 0x80
        out.append(c)
    return np.array(out, dtype=np.uint8)


def test_e4m3_encode_matches_brute_force_nearest():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.normal(0, 30, 2000), rng.normal(0, 0.01, 500),
                        rng.uniform(-500, 500, 500)])
    # every midpoint between neighbouring codes is a tie
    pos = mx.e4m3_decode(np.arange(0x00, 0x7F, dtype=np.uint8))
    mids = (pos[1:] + pos[:-1]) / 2
    v = np.concatenate([v, mids, -mids])
    assert np.array_equal(mx.e4m3_encode(v), _brute_encode(v))


def test_e4m3_encode_ties_and_saturation():
    assert mx.e4m3_encode(1.0 + 1.0 / 16) == 0x38      # between 1 (m=0) and 1.125 -> even
    assert mx.e4m3_encode(1.0 + 3.0 / 16) == 0x3A      # between 1.125 and 1.25 -> m=2
    assert mx.e4m3_encode(2.0 ** -10) == 0x00          # half of the smallest subnormal
    assert mx.e4m3_encode(3 * 2.0 ** -10) == 0x02      # between m=1 and m=2 subnormals
    assert mx.e4m3_encode(449.0) == 0x7E
    assert mx.e4m3_encode(1e6) == 0x7E
    assert mx.e4m3_encode(-1e6) == 0xFE
    assert mx.e4m3_encode(-0.0) == 0x00


def test_mx_block_worked_examples():
    # amax = 1.0: s = 0 - 8, scale byte 119; 1.0 * 2^8 = 256 -> 0x78, 0.5 -> 128 -> 0x70
    row = np.zeros(32, dtype=np.float32)
    row[0], row[5], row[31] = 1.0, 0.5, -0.25
    codes, scales = mx.mx_quantize(_bf16(row))
    assert scales.tolist() == [119]
    assert codes[0] == 0x78 and codes[5] == 0x70 and codes[31] == 0xE8
    assert np.all(codes[[i for i in range(32) if i not in (0, 5, 31)]] == 0)
    assert np.array_equal(mx.mx_dequantize(codes, scales), row.astype(np.float64))
    # amax = 1.875: floor(log2) = 0, so 1.875 * 256 = 480 > 448 is clamped to 448 (1.75)
    row2 = np.zeros(32, dtype=np.float32)
    row2[3] = 1.875
    codes2, scales2 = mx.mx_quantize(_bf16(row2))
    assert scales2.tolist() == [119] and codes2[3] == 0x7E
    assert mx.mx_dequantize(codes2, scales2)[3] == 1.75
    # a block of zeros: scale byte 0, zero elements; two blocks per row are independent
    row3 = np.zeros(64, dtype=np.float32)
    row3[40] = 3.0                                   # floor(log2 3) = 1 -> s = -7
    codes3, scales3 = mx.mx_quantize(_bf16(row3))
    assert scales3.tolist() == [0, 120]
    assert np.all(codes3[:32] == 0) and mx.e4m3_decode(codes3[40]) == 3.0 * 128


def test_mx_quantization_error_bound_and_exact_bf16():
    rng = np.random.default_rng(1)
    w = (rng.normal(0, 0.02, (6, 256))).astype(np.float32)
    w_bits = (w.view(np.uint32) >> 16).astype(np.uint16)        # truncate to bf16 bits
    wv = (w_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    codes, scales = mx.mx_quantize(w_bits)
    deq = mx.mx_dequantize(codes, scales)
    s = np.repeat(scales.astype(np.float64) - 127.0, 32, axis=-1)
    # no clamping below 448 * 2^s: the error is at most half a grid step at |w|
    step = np.exp2(np.maximum(np.floor(np.log2(np.maximum(np.abs(wv) / np.exp2(s), 2.0 ** -6))), -6) - 3 + s)
    unclamped = np.abs(wv) <= 448 * np.exp2(s)
    assert np.all(np.abs(deq - wv)[unclamped] <= step[unclamped] / 2)
    # values in E4M3's normal range keep 3 mantissa bits: relative error <= 2^-4
    normal = unclamped & (np.abs(wv) >= 2.0 ** -6 * np.exp2(s))
    assert np.all(np.abs(deq - wv)[normal] <= np.abs(wv)[normal] * 2.0 ** -4)
    # values above 448 * 2^s (only a block's largest can be) come back as +-448 * 2^s
    assert np.array_equal(np.abs(deq)[~unclamped], (448 * np.exp2(s))[~unclamped])
    # dequantized values are exact bf16 numbers
    bits = mx.mx_dequantize_bf16_bits(codes, scales)
    back = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(back, deq)
