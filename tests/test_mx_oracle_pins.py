"""Pins of the MXFP8 weight oracle (oracle/mx_oracle.py) against the format definitions:
E4M3 values printed from the field layout, a brute-force nearest-value encoder, tie and
saturation cases, and hand-worked MX blocks.  CPU only."""
import numpy as np
import pytest

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


def _trunc_bf16(values):
    """bf16 bit patterns of values, truncated (any pattern will do for these pins)."""
    return (np.asarray(values, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _lut_cases():
    """bf16 bit patterns [rows, K] covering the conversion's branches: several magnitudes,
    blocks spanning many binades, midpoints between E4M3 neighbours (ties), maxima that clamp
    to 448, zero and negative-zero blocks, and bf16 subnormals."""
    rng = np.random.default_rng(11)
    cases = []
    for sd in (0.02, 1.0, 1e-6, 3e4):
        cases.append(_trunc_bf16(rng.normal(0, sd, (16, 256))))
    wide = rng.normal(0, 1, (16, 256)) * np.exp2(rng.integers(-30, 30, (16, 256)))
    cases.append(_trunc_bf16(wide))
    pos = mx.e4m3_decode(np.arange(0x00, 0x7F, dtype=np.uint8))
    mids = (pos[1:] + pos[:-1]) / 2
    t = np.zeros((4, 256), dtype=np.float32)
    t[0, :125] = mids[:125] / 256.0
    t[0, 200] = 1.0
    t[1, :125] = -mids[:125] / 256.0 * 8
    t[2, 32:64] = -0.0
    t[3, 5] = 1.875
    cases.append(_trunc_bf16(t))
    sub = np.zeros((2, 64), dtype=np.uint16)
    sub[0, :32] = np.arange(1, 33, dtype=np.uint16)             # bf16 subnormals only
    sub[1, :32] = 0x8000                                        # negative zeros
    sub[1, 32:] = np.arange(0x0080, 0x00A0, dtype=np.uint16)    # smallest normals
    cases.append(sub)
    return cases


def test_lut_quantize_equals_the_definition():
    """The tabulated conversion (used to convert whole expert stacks) against mx_quantize."""
    for w in _lut_cases():
        c0, s0 = mx.mx_quantize(w)
        c1, s1 = mx.mx_quantize_lut(w, rows_per_pass=5)
        assert np.array_equal(s0, s1)
        assert np.array_equal(c0, c1)


def test_lut_roundtrip_equals_the_definition():
    # (dequantized values of bf16 inputs are always bf16 numbers: the E4M3 grid below a block's
    # scale never gets finer than the bf16 values it rounds, so the subnormal case is exact too)
    for w in _lut_cases():
        c0, s0 = mx.mx_quantize(w)
        assert np.array_equal(mx.mx_roundtrip_bf16_bits_lut(w), mx.mx_dequantize_bf16_bits(c0, s0))


# ---------------------------------------------------------------------------------------
# MXFP4 (E2M1 elements, the same E8M0 block scale)
# ---------------------------------------------------------------------------------------
def test_e2m1_decode_known_codes():
    """All 16 codes from the field layout: S.EE.M, exponent bias 1, field 0 subnormal."""
    want = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert mx.e2m1_decode(np.arange(8)).tolist() == want
    assert mx.e2m1_decode(np.arange(8, 16)).tolist() == [-v for v in want]
    assert mx.E2M1_MAX == 6.0


def _brute_encode4(v):
    """Nearest of the 8 magnitudes; a tie goes to the neighbour with mantissa bit 0."""
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    out = []
    for x in np.atleast_1d(v):
        a = min(abs(float(x)), 6.0)
        d = np.abs(mags - a)
        best = np.flatnonzero(d == d.min())
        c = int(best[0] if len(best) == 1 else best[best % 2 == 0][0])
        if x < 0 and c != 0:
            c |= 0x8
        out.append(c)
    return np.array(out, dtype=np.uint8)


def test_e2m1_encode_matches_brute_force_nearest():
    rng = np.random.default_rng(4)
    mags = mx.e2m1_decode(np.arange(8))
    mids = (mags[1:] + mags[:-1]) / 2            # every midpoint is a tie
    v = np.concatenate([rng.normal(0, 2, 3000), rng.uniform(-9, 9, 1000), mids, -mids,
                        mags, -mags, [6.5, 7.0, 1e9, -1e9, -0.0]])
    assert np.array_equal(mx.e2m1_encode(v), _brute_encode4(v))


def test_e2m1_ties_and_saturation():
    assert mx.e2m1_encode(0.25) == 0x0        # 0 and 0.5: to 0 (mantissa 0)
    assert mx.e2m1_encode(0.75) == 0x2        # 0.5 and 1: to 1
    assert mx.e2m1_encode(1.25) == 0x2        # 1 and 1.5: to 1
    assert mx.e2m1_encode(1.75) == 0x4        # 1.5 and 2: to 2
    assert mx.e2m1_encode(2.5) == 0x4         # 2 and 3: to 2
    assert mx.e2m1_encode(3.5) == 0x6         # 3 and 4: to 4
    assert mx.e2m1_encode(5.0) == 0x6         # 4 and 6: to 4
    assert mx.e2m1_encode(5.5) == 0x7
    assert mx.e2m1_encode(100.0) == 0x7 and mx.e2m1_encode(-100.0) == 0xF
    assert mx.e2m1_encode(-0.2) == 0x0        # rounds to zero: +0


def test_mx4_block_worked_examples():
    # amax 6: floor(log2 6) = 2 -> s = 0, scale byte 127; elements as they are
    row = np.zeros(32, dtype=np.float32)
    row[[0, 1, 2, 3]] = [6.0, -1.5, 0.5, 2.5]
    codes, scales = mx.mx4_quantize(_bf16(row))
    assert scales.tolist() == [127]
    assert codes[:4].tolist() == [0x7, 0xB, 0x1, 0x4]           # 2.5 ties to 2
    # amax 1: s = -2 (byte 125), elements scaled by 4: 1 -> 4, 0.25 -> 1, 0.125 -> 0.5
    row2 = np.zeros(32, dtype=np.float32)
    row2[[5, 6, 7]] = [1.0, 0.25, -0.125]
    codes2, scales2 = mx.mx4_quantize(_bf16(row2))
    assert scales2.tolist() == [125] and codes2[[5, 6, 7]].tolist() == [0x6, 0x2, 0x9]
    # amax 1.875: s = -2, 1.875 * 4 = 7.5 clamps to 6 -> dequantized 1.5
    row3 = np.zeros(32, dtype=np.float32)
    row3[9] = 1.875
    codes3, scales3 = mx.mx4_quantize(_bf16(row3))
    assert codes3[9] == 0x7 and mx.mx4_dequantize(codes3, scales3)[9] == 1.5
    # a zero block: scale byte 0, zero codes; blocks of one row are independent
    row4 = np.zeros(64, dtype=np.float32)
    row4[40] = 3.0                            # floor(log2 3) = 1 -> s = -1
    codes4, scales4 = mx.mx4_quantize(_bf16(row4))
    assert scales4.tolist() == [0, 126] and np.all(codes4[:32] == 0) and codes4[40] == 0x7


def test_mx4_quantization_error_bound():
    rng = np.random.default_rng(2)
    w_bits = _trunc_bf16(rng.normal(0, 0.02, (8, 512)))
    wv = (w_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    codes, scales = mx.mx4_quantize(w_bits)
    deq = mx.mx4_dequantize(codes, scales)
    s = np.repeat(scales.astype(np.float64) - 127.0, 32, axis=-1)
    u = np.abs(wv) / np.exp2(s)               # in [0, 8)
    # half a grid step: 0.25 below 2, 0.5 in [2, 4), 1 in [4, 6]; above 6 the clamp
    half = np.where(u < 2, 0.25, np.where(u < 4, 0.5, 1.0)) * np.exp2(s)
    ok = u <= 6
    assert np.all(np.abs(deq - wv)[ok] <= half[ok])
    assert np.array_equal(np.abs(deq)[~ok], (6 * np.exp2(s))[~ok])
    assert np.array_equal(mx.mx4_dequantize_bf16_bits(codes, scales),
                          (deq.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))


def test_mx4_lut_equals_the_definition():
    for w in _lut_cases():
        c0, s0 = mx.mx4_quantize(w)
        c1, s1 = mx.mx4_quantize_lut(w, rows_per_pass=5)
        assert np.array_equal(s0, s1) and np.array_equal(c0, c1)
        assert np.array_equal(mx.mx4_roundtrip_bf16_bits_lut(w), mx.mx4_dequantize_bf16_bits(c0, s0))
