"""CPU oracle for MXFP8 expert weights: E4M3 elements with one power-of-two (E8M0) scale
per block of 32 consecutive values along K.

TEST INFRASTRUCTURE ONLY, like moe_oracle: only the test-suite, the smoke check and the
benchmark's CPU leg may import it, and it shares no code with the HIP path.

Sources.  The AlphaMoE page (FlashInfer PR #6511 analysis) runs its routed-MoE kernels
on block-scaled 4-bit weights (NVFP4) to cut the bytes a decode step streams; the pages
give no recipe for it.  The recipe here is the published conversion of the OCP
Microscaling Formats (MX) v1.0 specification with FP8 E4M3 elements, written from its
definition:
  * E4M3 (the "fn" variant: no infinities): sign, 4 exponent bits with bias 7, 3 mantissa
    bits.  Exponent field 0 holds subnormals m/8 * 2^-6; fields 1..15 hold
    (1 + m/8) * 2^(field - 7), except S.1111.111, which is NaN.  Largest finite: 448.
  * A block V of 32 values gets the shared exponent
        s = floor(log2(max |V_i|)) - 8          (8 = exponent of E4M3's largest normal)
    stored as the E8M0 byte s + 127, clamped to [0, 254] (a block of zeros gets 0), and
    each element becomes E4M3(V_i / 2^s): round to nearest, ties to even, with
    magnitudes above 448 clamped to 448.
  * Dequantized value: E4M3 value * 2^s.  Every such value is exactly representable in
    bf16 (4 significant bits, exponents well inside bf16's range), so the layer can run
    its bf16 arithmetic on the dequantized weights unchanged.

Readings (listed in the design notes): only the expert weights W13 and W2 are quantized
(activations, router, residual and norm stay as in the bf16 layer); blocks run along the
contraction dimension K (H for W13 rows, I for W2 rows); a block of zeros gets scale byte
0 and zero elements.
"""
from __future__ import annotations

import numpy as np

__all__ = ["E4M3_MAX", "MX_BLOCK", "e4m3_decode", "e4m3_encode", "mx_quantize",
           "mx_dequantize", "mx_dequantize_bf16_bits"]

E4M3_MAX = 448.0
MX_BLOCK = 32


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 byte -> float64 by the field definition (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    field = (c >> 3) & 0xF
    mant = (c & 0x7).astype(np.float64)
    sub = mant / 8.0 * 2.0 ** -6
    nor = (1.0 + mant / 8.0) * np.exp2(field.astype(np.float64) - 7.0)
    val = sign * np.where(field == 0, sub, nor)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def e4m3_encode(v) -> np.ndarray:
    """Finite float64 -> E4M3 byte: round to nearest, ties to even, magnitudes above 448
    clamped to 448.  Zero (of either sign) encodes as +0."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    out = np.zeros(v.shape, dtype=np.uint8)
    nz = a > 0
    # grid spacing at |v|: 2^(E - 3) for binade E >= -6, 2^-9 below (subnormals)
    e = np.floor(np.log2(np.where(nz, a, 1.0)))
    e = np.clip(e, -6.0, 8.0)
    spacing = np.exp2(e - 3.0)
    q = np.round(a / spacing) * spacing          # numpy rounds halves to even; q <= 448
    # bits of the rounded magnitude
    qe = np.floor(np.log2(np.where(q > 0, q, 1.0)))
    normal = q >= 2.0 ** -6
    field = np.where(normal, qe + 7.0, 0.0)
    mant = np.where(normal, (q / np.exp2(qe) - 1.0) * 8.0, q / 2.0 ** -9)
    code = (field.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    code = np.where(q > 0, code, 0)
    sign = np.where((v < 0) & (q > 0), 0x80, 0)
    out[...] = (code | sign).astype(np.uint8)
    return out


def _bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def mx_quantize(w_bits, block: int = MX_BLOCK):
    """bf16 weights [..., K] (uint16 bits, K a multiple of `block`) -> (E4M3 codes
    [..., K] uint8, E8M0 scale bytes [..., K / block] uint8)."""
    w = _bf16_bits_to_f64(w_bits)
    K = w.shape[-1]
    assert K % block == 0, "K must be a multiple of the block"
    blocks = w.reshape(w.shape[:-1] + (K // block, block))
    amax = np.abs(blocks).max(axis=-1)
    s = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8.0, -127.0)
    s = np.clip(s, -127.0, 127.0)
    scales = (s + 127.0).astype(np.uint8)
    codes = e4m3_encode(blocks / np.exp2(s)[..., None])
    return codes.reshape(w.shape), scales


def mx_dequantize(codes, scales, block: int = MX_BLOCK) -> np.ndarray:
    """(E4M3 codes [..., K], E8M0 bytes [..., K / block]) -> float64 [..., K]."""
    c = np.asarray(codes, dtype=np.uint8)
    K = c.shape[-1]
    vals = e4m3_decode(c).reshape(c.shape[:-1] + (K // block, block))
    s = np.asarray(scales, dtype=np.float64) - 127.0
    return (vals * np.exp2(s)[..., None]).reshape(c.shape)


def mx_dequantize_bf16_bits(codes, scales, block: int = MX_BLOCK) -> np.ndarray:
    """Dequantized weights as bf16 bit patterns; every value is exact in bf16."""
    v = mx_dequantize(codes, scales, block)
    f32 = v.astype(np.float32)
    assert np.array_equal(f32.astype(np.float64), v), "dequantized value not exact in fp32"
    bits = f32.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0), "dequantized value not exact in bf16"
    return (bits >> 16).astype(np.uint16)


# ----------------------------------------------------------------------------------------
# The same conversion as tables over every bf16 bit pattern (for whole expert stacks)
# ----------------------------------------------------------------------------------------
# The scale of a block depends only on its largest magnitude, and a value's code only on
# its own bf16 bit pattern and that scale.  So the conversion above can be tabulated once:
# for every scale byte b (s = b - 127) and every bf16 pattern p, the code e4m3_encode(p / 2^s)
# and the dequantized bf16 pattern.  The tables are filled by the functions above and
# nothing else; mx_quantize_lut equals mx_quantize bit for bit (pinned by tests), it is
# only fast enough to convert all 256 experts of the real-shape layer.
_LUT = {}


def _luts():
    if not _LUT:
        patterns = np.arange(1 << 16, dtype=np.uint32)
        enc = np.empty((255, 1 << 16), dtype=np.uint8)
        dq = np.empty((255, 256), dtype=np.uint16)
        exact = np.empty((255, 256), dtype=bool)    # code * 2^s exact in bf16 (and finite)
        codes = np.arange(256, dtype=np.uint8)
        with np.errstate(all="ignore"):
            vals = (patterns << np.uint32(16)).view(np.float32).astype(np.float64)
            finite = np.isfinite(vals)
            vals = np.where(finite, vals, 0.0)
            for b in range(255):
                s = float(b) - 127.0
                enc[b] = np.where(finite, e4m3_encode(vals / np.exp2(s)), 0x7F)
                v = e4m3_decode(codes) * np.exp2(s)
                f32 = np.where(np.isfinite(v), v, 0.0).astype(np.float32)
                u = f32.view(np.uint32)
                exact[b] = np.isfinite(v) & (f32.astype(np.float64) == v) & ((u & 0xFFFF) == 0)
                dq[b] = (u >> 16).astype(np.uint16)
        _LUT["enc"], _LUT["dq"], _LUT["exact"] = enc, dq, exact
    return _LUT["enc"], _LUT["dq"]


def _block_scale_bytes(blocks_bits) -> np.ndarray:
    """E8M0 byte of each 32-value block of bf16 patterns [..., 32]: s = floor(log2 amax) - 8,
    clamped to [-127, 127], byte s + 127 (blocks of zeros -> 0).  For a finite bf16 the
    magnitude bits order like the magnitudes, and floor(log2) of a normal value is its
    exponent field - 127 (subnormal and zero maxima clamp to s = -127)."""
    amax = (blocks_bits & np.uint16(0x7FFF)).max(axis=-1)
    e = (amax >> 7).astype(np.int64)
    s = np.where(e > 0, e - 127 - 8, -127)
    return (np.clip(s, -127, 127) + 127).astype(np.uint8)


def mx_quantize_lut(w_bits, block: int = MX_BLOCK, rows_per_pass: int = 1024):
    """mx_quantize through the tables: (codes [..., K], scale bytes [..., K / block])."""
    enc, _ = _luts()
    w = np.asarray(w_bits, dtype=np.uint16)
    K = w.shape[-1]
    assert K % block == 0, "K must be a multiple of the block"
    flat = w.reshape(-1, K)
    codes = np.empty(flat.shape, dtype=np.uint8)
    scales = np.empty((flat.shape[0], K // block), dtype=np.uint8)
    enc_flat = enc.reshape(-1)
    for r0 in range(0, flat.shape[0], rows_per_pass):
        blk = flat[r0:r0 + rows_per_pass].reshape(-1, K // block, block)
        sb = _block_scale_bytes(blk)
        idx = (sb[..., None].astype(np.int64) << 16) | blk.astype(np.int64)
        codes[r0:r0 + rows_per_pass] = enc_flat[idx].reshape(-1, K)
        scales[r0:r0 + rows_per_pass] = sb
    return codes.reshape(w.shape), scales.reshape(w.shape[:-1] + (K // block,))


def _rt_table():
    """rt[b, p]: bf16 pattern of the dequantized value of pattern p under scale byte b."""
    if "rt" not in _LUT:
        enc, dq = _luts()
        rt = np.take_along_axis(dq, enc.astype(np.int64), axis=1)
        ok = np.take_along_axis(_LUT["exact"], enc.astype(np.int64), axis=1)
        # as mx_dequantize_bf16_bits asserts: the dequantized value of every pattern a block
        # can hold under scale byte b is a bf16 number (checked here once for the table).
        # Byte b comes from a finite block maximum with exponent field b + 8 <= 254 (or
        # less, for b = 0), so the block's patterns have exponent fields <= b + 8.
        p = np.arange(1 << 16, dtype=np.int64)
        b = np.arange(255)[:, None]
        reachable = (((p >> 7) & 0xFF)[None, :] <= b + 8) & (b + 8 <= 254)
        assert ok[reachable].all(), "dequantized value not exact in bf16"
        _LUT["rt"] = rt
    return _LUT["rt"]


def mx_roundtrip_bf16_bits_lut(w_bits, block: int = MX_BLOCK, rows_per_pass: int = 1024):
    """bf16 patterns of the dequantized MXFP8 weights, mx_dequantize_bf16_bits(mx_quantize(w)),
    through the tables."""
    rt = _rt_table().reshape(-1)
    w = np.asarray(w_bits, dtype=np.uint16)
    K = w.shape[-1]
    assert K % block == 0, "K must be a multiple of the block"
    flat = w.reshape(-1, K)
    out = np.empty(flat.shape, dtype=np.uint16)
    for r0 in range(0, flat.shape[0], rows_per_pass):
        blk = flat[r0:r0 + rows_per_pass].reshape(-1, K // block, block)
        sb = _block_scale_bytes(blk).astype(np.uint32)
        idx = (sb[..., None] << np.uint32(16)) | blk
        out[r0:r0 + rows_per_pass] = rt[idx].reshape(-1, K)
    return out.reshape(w.shape)


__all__ += ["mx_quantize_lut", "mx_roundtrip_bf16_bits_lut"]


# ----------------------------------------------------------------------------------------
# MXFP4: E2M1 elements, the same E8M0 block scale
# ----------------------------------------------------------------------------------------
# OCP MX v1.0 FP4 (E2M1): sign, 2 exponent bits with bias 1, 1 mantissa bit, no infinity or
# NaN.  Exponent field 0 holds the subnormals m * 0.5; fields 1..3 hold (1 + m/2) * 2^(f-1):
# magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.  The block's shared exponent is
#     s = floor(log2(max |V_i|)) - 2          (2 = exponent of E2M1's largest normal, 6)
# (E8M0 byte s + 127, a block of zeros gets 0), each element becomes E2M1(V_i / 2^s), round
# to nearest, ties to even (the even neighbour has mantissa bit 0), magnitudes above 6
# clamped to 6.  The AlphaMoE page's routed-MoE kernels stream 4-bit weights (NVFP4); this is
# the OCP 4-bit format with the same block of 32 and power-of-two scale as MXFP8 above.
E2M1_MAX = 6.0


def e2m1_decode(codes) -> np.ndarray:
    """E2M1 code (low 4 bits) -> float64 by the field definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    field = (c >> 1) & 0x3
    mant = (c & 0x1).astype(np.float64)
    sub = mant * 0.5
    nor = (1.0 + mant / 2.0) * np.exp2(field.astype(np.float64) - 1.0)
    return sign * np.where(field == 0, sub, nor)


def e2m1_encode(v) -> np.ndarray:
    """Finite float64 -> E2M1 code (uint8, low 4 bits): round to nearest, ties to even,
    magnitudes above 6 clamped to 6.  Zero (of either sign) encodes as +0."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E2M1_MAX)
    # grid spacing at |v|: 2^(E - 1) for binade E = floor(log2 |v|) in 0..2, 0.5 below 1
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, 0.0, 2.0)
    spacing = np.exp2(e - 1.0)
    q = np.round(a / spacing) * spacing              # halves to even; q <= 6
    qe = np.floor(np.log2(np.where(q > 0, q, 1.0)))
    normal = q >= 1.0
    field = np.where(normal, qe + 1.0, 0.0)
    mant = np.where(normal, (q / np.exp2(qe) - 1.0) * 2.0, q * 2.0)
    code = (field.astype(np.int64) << 1) | np.rint(mant).astype(np.int64)
    code = np.where(q > 0, code, 0)
    sign = np.where((v < 0) & (q > 0), 0x8, 0)
    return (code | sign).astype(np.uint8)


def mx4_quantize(w_bits, block: int = MX_BLOCK):
    """bf16 weights [..., K] (uint16 bits) -> (E2M1 codes [..., K] uint8, one code per byte,
    E8M0 scale bytes [..., K / block] uint8)."""
    w = _bf16_bits_to_f64(w_bits)
    K = w.shape[-1]
    assert K % block == 0, "K must be a multiple of the block"
    blocks = w.reshape(w.shape[:-1] + (K // block, block))
    amax = np.abs(blocks).max(axis=-1)
    s = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2.0, -127.0)
    s = np.clip(s, -127.0, 127.0)
    scales = (s + 127.0).astype(np.uint8)
    codes = e2m1_encode(blocks / np.exp2(s)[..., None])
    return codes.reshape(w.shape), scales


def mx4_dequantize(codes, scales, block: int = MX_BLOCK) -> np.ndarray:
    """(E2M1 codes [..., K], E8M0 bytes [..., K / block]) -> float64 [..., K]."""
    c = np.asarray(codes, dtype=np.uint8)
    K = c.shape[-1]
    vals = e2m1_decode(c).reshape(c.shape[:-1] + (K // block, block))
    s = np.asarray(scales, dtype=np.float64) - 127.0
    return (vals * np.exp2(s)[..., None]).reshape(c.shape)


def mx4_dequantize_bf16_bits(codes, scales, block: int = MX_BLOCK) -> np.ndarray:
    """Dequantized MXFP4 weights as bf16 bit patterns; every value is exact in bf16."""
    v = mx4_dequantize(codes, scales, block)
    f32 = v.astype(np.float32)
    assert np.array_equal(f32.astype(np.float64), v), "dequantized value not exact in fp32"
    bits = f32.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0), "dequantized value not exact in bf16"
    return (bits >> 16).astype(np.uint16)


def _luts4():
    """enc4[b, p]: E2M1 code of bf16 pattern p under scale byte b; rt4[b, p]: the bf16 pattern
    of its dequantized value -- both filled by the functions above."""
    if "rt4" not in _LUT:
        patterns = np.arange(1 << 16, dtype=np.uint32)
        enc = np.empty((255, 1 << 16), dtype=np.uint8)
        rt = np.empty((255, 1 << 16), dtype=np.uint16)
        codes = np.arange(16, dtype=np.uint8)
        with np.errstate(all="ignore"):
            vals = (patterns << np.uint32(16)).view(np.float32).astype(np.float64)
            finite = np.isfinite(vals)
            vals = np.where(finite, vals, 0.0)
            for b in range(255):
                s = float(b) - 127.0
                enc[b] = np.where(finite, e2m1_encode(vals / np.exp2(s)), 0)
                dq = e2m1_decode(codes) * np.exp2(s)
                f32 = np.where(np.isfinite(dq), dq, 0.0).astype(np.float32)
                u = f32.view(np.uint32)
                exact = np.isfinite(dq) & (f32.astype(np.float64) == dq) & ((u & 0xFFFF) == 0)
                # a scale byte b comes from a block maximum with exponent field b + 2 <= 254:
                # every dequantized value such a block can produce must be a bf16 number
                if b + 2 <= 254:
                    reach = ((patterns >> 7) & 0xFF) <= b + 2
                    assert exact[enc[b][reach]].all(), "dequantized value not exact in bf16"
                rt[b] = (u >> 16).astype(np.uint16)[enc[b]]
        _LUT["enc4"], _LUT["rt4"] = enc, rt
    return _LUT["enc4"], _LUT["rt4"]


def _block_scale_bytes4(blocks_bits) -> np.ndarray:
    """E8M0 byte of each 32-value block for E2M1: s = floor(log2 amax) - 2, clamped to
    [-127, 127] (exponent field - 127 - 2 for a normal maximum; subnormal and zero maxima
    clamp to s = -127)."""
    amax = (blocks_bits & np.uint16(0x7FFF)).max(axis=-1)
    e = (amax >> 7).astype(np.int64)
    s = np.where(e > 0, e - 127 - 2, -127)
    return (np.clip(s, -127, 127) + 127).astype(np.uint8)


def mx4_quantize_lut(w_bits, block: int = MX_BLOCK, rows_per_pass: int = 1024):
    """mx4_quantize through the tables: (codes [..., K], scale bytes [..., K / block])."""
    enc, _ = _luts4()
    w = np.asarray(w_bits, dtype=np.uint16)
    K = w.shape[-1]
    assert K % block == 0, "K must be a multiple of the block"
    flat = w.reshape(-1, K)
    codes = np.empty(flat.shape, dtype=np.uint8)
    scales = np.empty((flat.shape[0], K // block), dtype=np.uint8)
    enc_flat = enc.reshape(-1)
    for r0 in range(0, flat.shape[0], rows_per_pass):
        blk = flat[r0:r0 + rows_per_pass].reshape(-1, K // block, block)
        sb = _block_scale_bytes4(blk)
        idx = (sb[..., None].astype(np.uint32) << np.uint32(16)) | blk
        codes[r0:r0 + rows_per_pass] = enc_flat[idx].reshape(-1, K)
        scales[r0:r0 + rows_per_pass] = sb
    return codes.reshape(w.shape), scales.reshape(w.shape[:-1] + (K // block,))


def mx4_roundtrip_bf16_bits_lut(w_bits, block: int = MX_BLOCK, rows_per_pass: int = 1024):
    """bf16 patterns of mx4_dequantize_bf16_bits(mx4_quantize(w)), through the tables."""
    _, rt = _luts4()
    rt_flat = rt.reshape(-1)
    w = np.asarray(w_bits, dtype=np.uint16)
    K = w.shape[-1]
    flat = w.reshape(-1, K)
    out = np.empty(flat.shape, dtype=np.uint16)
    for r0 in range(0, flat.shape[0], rows_per_pass):
        blk = flat[r0:r0 + rows_per_pass].reshape(-1, K // block, block)
        sb = _block_scale_bytes4(blk).astype(np.uint32)
        out[r0:r0 + rows_per_pass] = rt_flat[(sb[..., None] << np.uint32(16)) | blk].reshape(-1, K)
    return out.reshape(w.shape)


__all__ += ["E2M1_MAX", "e2m1_decode", "e2m1_encode", "mx4_quantize", "mx4_dequantize",
            "mx4_dequantize_bf16_bits", "mx4_quantize_lut", "mx4_roundtrip_bf16_bits_lut"]
