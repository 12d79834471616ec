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
