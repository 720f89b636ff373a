"""Test-side helpers, independent of the oracle's vectorised unpacker.

``pack_codes`` builds each packed row as one Python integer bit stream (code c
at bits [c*b, c*b+b)) and splits it into little-endian 32-bit words.
"""
import math
from fractions import Fraction

import numpy as np

from synth import FormatSpec, QTensor


def pack_codes(codes, bits):
    codes = np.asarray(codes)
    rows, cols = codes.shape
    assert (cols * bits) % 32 == 0
    nw = cols * bits // 32
    out = np.zeros((rows, nw), dtype=np.uint32)
    for r in range(rows):
        stream = 0
        for c in range(cols):
            q = int(codes[r, c])
            assert 0 <= q < (1 << bits)
            stream |= q << (c * bits)
        for i in range(nw):
            out[r, i] = (stream >> (32 * i)) & 0xFFFFFFFF
    return out


def make_affine(codes_list, scales_list, biases_list, bits, group):
    """QTensor (n experts) from explicit integer codes and fp16 scale/bias arrays."""
    spec = FormatSpec("affine", bits, group)
    codes = np.stack([pack_codes(c, bits) for c in codes_list])
    rows, cols = np.asarray(codes_list[0]).shape
    return QTensor(spec, rows, cols, codes,
                   np.stack([np.asarray(s, dtype=np.float16) for s in scales_list]),
                   np.stack([np.asarray(b, dtype=np.float16) for b in biases_list]))


def make_mxfp4(codes_list, scale_bytes_list):
    spec = FormatSpec("mxfp4", 4, 32)
    codes = np.stack([pack_codes(c, 4) for c in codes_list])
    rows, cols = np.asarray(codes_list[0]).shape
    return QTensor(spec, rows, cols, codes,
                   np.stack([np.asarray(s, dtype=np.uint8) for s in scale_bytes_list]), None)


def make_mxfp8(codes_list, scale_bytes_list):
    spec = FormatSpec("mxfp8", 8, 32)
    codes = np.stack([pack_codes(c, 8) for c in codes_list])
    rows, cols = np.asarray(codes_list[0]).shape
    return QTensor(spec, rows, cols, codes,
                   np.stack([np.asarray(s, dtype=np.uint8) for s in scale_bytes_list]), None)


def e4m3_table_torch():
    """The 256 e4m3 code values through torch's float8_e4m3fn conversion (an
    implementation independent of the oracle's decoder)."""
    import torch
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def finite_e4m3_codes(rng, shape):
    """Uniform over the 254 non-NaN e4m3 codes (0x7F and 0xFF are NaN)."""
    b = rng.integers(0, 254, size=shape)
    return b + (b >= 0x7F)


def bf16_round_exact(v: float) -> float:
    """Nearest bf16 (ties to even) of a finite normal-range double, via exact rationals."""
    if v == 0.0 or not math.isfinite(v):
        return v
    _, e = math.frexp(v)
    scaled = Fraction(v) * Fraction(2) ** (8 - e)
    return float(round(scaled) * Fraction(2) ** (e - 8))
