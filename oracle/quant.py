"""Symmetric INTb quantizer, bit-packing and dequantizer, float64.

FADE post, sections "第二层：INT4量化存储" (middle tokens stored as 4-bit
codes with bit-packing), "第三层：INT2深度压缩" (optional 2-bit tier) and
"量化与Bit-Packing" (the scheme is symmetric; K stays INT4, V may drop to
INT2). The post gives no group size, scale type, rounding or pack order;
the readings taken are:

* Group: G consecutive channels of one (token, KV head); G = 32.
* Scale: s = fp16_RNE(amax / qmax), qmax = 2^(b-1) - 1 (7 for INT4, 1 for
  INT2) - the textbook symmetric quantizer with fp16 scales.
* Code: q = clamp(RNE(x / s), -qmax, qmax), rounding the exact real quotient
  half-to-even; a zero group (s == 0) gets q = 0 everywhere.
* Storage: offset binary u = q + 2^(b-1) (INT4 1..15, INT2 1..3).
* Pack: channel c of a row lives in byte floor(c*b/8) at bit (c*b) mod 8,
  so the lower channel sits in the low bits (little-endian).
* Dequant: x_hat = (u - 2^(b-1)) * s, exact in float32 and float64.
"""
import numpy as np


def qmax(bits):
    if bits not in (2, 4):
        raise ValueError("bits must be 2 or 4")
    return (1 << (bits - 1)) - 1


def offset(bits):
    return 1 << (bits - 1)


def scales_fp16(x16, bits, group):
    """Per-group fp16 scales of x16 [..., d]."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    d = x.shape[-1]
    xg = x.reshape(x.shape[:-1] + (d // group, group))
    amax = np.abs(xg).max(axis=-1)
    # float64 division is correctly rounded; float64 -> float16 is RNE.
    return (amax / qmax(bits)).astype(np.float16)


def codes_with_scale(x16, s16, bits, group):
    """Offset-binary codes of x16 [..., d] given per-group scales s16."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    d = x.shape[-1]
    xg = x.reshape(x.shape[:-1] + (d // group, group))
    s = np.asarray(s16, dtype=np.float16).astype(np.float64)[..., None]
    qm = qmax(bits)
    safe = np.where(s == 0.0, 1.0, s)
    q = np.rint(xg / safe)                      # RNE on the quotient
    q = np.clip(q, -qm, qm)
    q = np.where(s == 0.0, 0.0, q)
    u = (q + offset(bits)).astype(np.uint8)
    return u.reshape(x.shape)


def quantize(x16, bits, group=32):
    """Quantize rows x16 [..., d] -> (codes uint8 [..., d], scales fp16 [..., d/G])."""
    s16 = scales_fp16(x16, bits, group)
    return codes_with_scale(x16, s16, bits, group), s16


def dequantize(u, s16, bits, group=32):
    """x_hat [..., d] float64 from codes and scales."""
    u = np.asarray(u).astype(np.float64)
    d = u.shape[-1]
    ug = u.reshape(u.shape[:-1] + (d // group, group))
    s = np.asarray(s16, dtype=np.float16).astype(np.float64)[..., None]
    return ((ug - offset(bits)) * s).reshape(u.shape)


def pack(u, bits):
    """Pack codes u [..., d] (values < 2^bits) into bytes [..., d*bits/8]."""
    u = np.asarray(u, dtype=np.uint8)
    d = u.shape[-1]
    if (d * bits) % 8:
        raise ValueError("row does not fill whole bytes")
    out = np.zeros(u.shape[:-1] + (d * bits // 8,), dtype=np.uint8)
    for c in range(d):
        byte, shift = divmod(c * bits, 8)
        out[..., byte] |= (u[..., c] & ((1 << bits) - 1)) << shift
    return out


def unpack(packed, bits, d):
    """Inverse of `pack`."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.zeros(packed.shape[:-1] + (d,), dtype=np.uint8)
    for c in range(d):
        byte, shift = divmod(c * bits, 8)
        out[..., c] = (packed[..., byte] >> shift) & ((1 << bits) - 1)
    return out


def roundtrip(x16, bits, group=32):
    """quantize then dequantize (float64)."""
    u, s = quantize(x16, bits, group)
    return dequantize(u, s, bits, group)
