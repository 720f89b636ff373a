"""Pins of the oracle's number formats against the pages and closed forms (CPU)."""
import json
import os
import struct

import numpy as np
import pytest
import torch

import oracle
from tests._packing import (bf16_round_exact, e4m3_table_torch, finite_e4m3_codes, make_affine, make_mxfp4,
                            make_mxfp8, pack_codes)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32_from_bits(u):
    return struct.unpack("<f", struct.pack("<I", u))[0]


# --------------------------------------------------------------------------- e2m1 / e8m0

def check_e2m1_table():
    with open(os.path.join(GOLDEN, "e2m1_values.json")) as f:
        want = json.load(f)["code_to_value"]
    got = oracle.e2m1_decode(np.arange(16))
    assert np.array_equal(got, np.array(want))
    # sign of zero: code 8 is -0
    assert np.signbit(got[8]) and not np.signbit(got[0])


def test_e2m1_table_matches_golden():
    check_e2m1_table()


def test_e2m1_times_e8m0_is_exact_in_bf16():
    """Every e2m1 value times 2^(118..124 - 127) is a bf16 value: the fp4 source
    format fits losslessly in bf16 (card 'DeepSeek-V4-Flash-0731-MLX-Serve-mixed-2-3-8bit',
    conversion paragraph)."""
    vals = oracle.e2m1_decode(np.arange(16))[:, None] * oracle.e8m0_decode(np.arange(118, 125))[None, :]
    t = torch.tensor(vals, dtype=torch.float64)
    assert torch.equal(t.to(torch.bfloat16).to(torch.float64), t)


def check_e8m0_exhaustive():
    got = oracle.e8m0_decode(np.arange(256))
    for b in range(1, 255):
        assert got[b] == _f32_from_bits(b << 23), b   # fp32 with exponent field b, zero mantissa
    assert got[0] == _f32_from_bits(1 << 22)            # 2^-127 is the fp32 subnormal 0x00400000
    assert np.isnan(got[255])


def test_e8m0_exhaustive():
    check_e8m0_exhaustive()


# --------------------------------------------------------------------------- e4m3

def check_e4m3_table():
    """All 256 codes against torch's float8_e4m3fn (the OCP E4M3 format), NaN
    codes included, and the format's closed-form landmarks."""
    got = oracle.e4m3_decode(np.arange(256))
    want = e4m3_table_torch()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))   # 0x80 is -0
    assert got[0x38] == 1.0 and got[0xB8] == -1.0
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0                 # largest magnitude
    assert got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6           # smallest subnormal / normal
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def test_e4m3_table():
    check_e4m3_table()


def test_e4m3_times_e8m0_is_exact_in_bf16():
    """Every finite e4m3 value times 2^(s - 127) over the synthetic scale bytes
    is a bf16 value (3 mantissa bits fit in bf16's 7), so the kernels may
    dequantise to bf16 without rounding."""
    v = oracle.e4m3_decode(np.arange(256))
    v = v[~np.isnan(v)][:, None] * oracle.e8m0_decode(np.arange(108, 122))[None, :]
    t = torch.tensor(v, dtype=torch.float64)
    assert torch.equal(t.to(torch.bfloat16).to(torch.float64), t)


def check_mxfp8_rule():
    rng = np.random.default_rng(45)
    rows, cols = 2, 64
    codes = finite_e4m3_codes(rng, (rows, cols))
    sb = rng.integers(108, 122, size=(rows, cols // 32))
    q = make_mxfp8([codes], [sb])
    table = e4m3_table_torch()
    got = oracle.dequant(q, 0)
    for r in range(rows):
        for c in range(cols):
            assert got[r, c] == table[codes[r, c]] * 2.0 ** (int(sb[r, c // 32]) - 127)


def test_mxfp8_rule():
    check_mxfp8_rule()


def test_mxfp8_byte_order():
    """Byte j of a row (little-endian words) holds element j; the scale byte of
    inputs 32..63 is the row's second one."""
    q = make_mxfp8([np.zeros((1, 64), np.int64)], [np.array([[127, 128]])])
    q.codes[0] = np.zeros((1, 16), np.uint32)
    q.codes[0, 0, 0] = 0x0000B838        # element 0 = 1.0, element 1 = -1.0
    q.codes[0, 0, 8] = 0x7E000000        # element 35 = 448
    w = oracle.dequant(q, 0)[0]
    assert w[0] == 1.0 and w[1] == -1.0 and w[35] == 896.0
    assert np.count_nonzero(w) == 3


# --------------------------------------------------------------------------- bit unpacking

@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("cols", [32, 64, 256])
def test_unpack_roundtrip_independent_packer(bits, cols):
    rng = np.random.default_rng(1000 * bits + cols)
    codes = rng.integers(0, 1 << bits, size=(5, cols))
    words = pack_codes(codes, bits)
    assert np.array_equal(oracle.unpack_codes(words, bits, cols), codes)


def check_unpack_known_words():
    # 4-bit: word 0x76543210 holds codes 0,1,...,7 (low nibble first)
    assert list(oracle.unpack_codes(np.array([[0x76543210]], np.uint32), 4, 8)[0]) == list(range(8))
    # 8-bit: bytes in little-endian order
    assert list(oracle.unpack_codes(np.array([[0x04030201]], np.uint32), 8, 4)[0]) == [1, 2, 3, 4]
    # 2-bit: 0b...11100100 -> 0,1,2,3 then zeros
    assert list(oracle.unpack_codes(np.array([[0xE4]], np.uint32), 2, 16)[0][:5]) == [0, 1, 2, 3, 0]
    # 3-bit: code 10 occupies stream bits 30..32 and straddles words 0 and 1
    codes = np.zeros((1, 32), np.int64)
    codes[0, 10] = 0b101
    w = np.zeros((1, 3), np.uint32)
    w[0, 0] = 0b01 << 30          # low two bits of code 10
    w[0, 1] = 0b1                 # high bit of code 10
    assert np.array_equal(oracle.unpack_codes(w, 3, 32), codes)


def test_unpack_known_words():
    check_unpack_known_words()


# --------------------------------------------------------------------------- dequant rules

def check_affine_rule(bits, group):
    rng = np.random.default_rng(bits * 7 + group)
    rows, cols = 3, 2 * group
    codes = rng.integers(0, 1 << bits, size=(rows, cols))
    s = rng.uniform(0.001, 0.01, size=(rows, cols // group)).astype(np.float16)
    b = (-rng.uniform(0.0, 0.1, size=(rows, cols // group))).astype(np.float16)
    q = make_affine([codes], [s], [b], bits, group)
    got = oracle.dequant(q, 0)
    for r in range(rows):
        for c in range(cols):
            want = float(s[r, c // group]) * int(codes[r, c]) + float(b[r, c // group])
            assert got[r, c] == want


@pytest.mark.parametrize("bits,group", [(2, 128), (3, 128), (4, 64), (8, 64), (4, 32)])
def test_affine_rule(bits, group):
    check_affine_rule(bits, group)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_affine_centred_codes(bits):
    """With bias = -2^(b-1) * scale, w = scale * (q - 2^(b-1)); the middle code is exactly 0."""
    rows, cols, g = 2, 128, 64
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 1 << bits, size=(rows, cols))
    codes[:, :5] = 1 << (bits - 1)
    s = rng.uniform(0.001, 0.01, size=(rows, cols // g)).astype(np.float16)
    b = (np.float32(-(1 << (bits - 1))) * s.astype(np.float32)).astype(np.float16)
    w = oracle.dequant(make_affine([codes], [s], [b], bits, g), 0)
    assert np.all(w[:, :5] == 0.0)
    assert np.array_equal(w, np.repeat(s.astype(np.float64), g, -1) * (codes - (1 << (bits - 1))))


def check_mxfp4_rule():
    rng = np.random.default_rng(44)
    rows, cols = 2, 64
    codes = rng.integers(0, 16, size=(rows, cols))
    sb = rng.integers(118, 125, size=(rows, cols // 32))
    q = make_mxfp4([codes], [sb])
    with open(os.path.join(GOLDEN, "e2m1_values.json")) as f:
        table = json.load(f)["code_to_value"]
    got = oracle.dequant(q, 0)
    for r in range(rows):
        for c in range(cols):
            assert got[r, c] == table[codes[r, c]] * 2.0 ** (int(sb[r, c // 32]) - 127)


def test_mxfp4_rule():
    check_mxfp4_rule()


def test_mxfp4_byte_order():
    """Byte j of a row holds element 2j in its low nibble and 2j+1 in its high nibble."""
    words = np.array([[0x000000F1, 0, 0, 0]], np.uint32)   # byte 0 = 0xF1
    q = make_mxfp4([np.zeros((1, 32), np.int64)], [np.array([[127]])])
    q.codes[0] = words
    w = oracle.dequant(q, 0)[0]
    assert w[0] == 0.5 and w[1] == -6.0 and np.all(w[2:] == 0)


# --------------------------------------------------------------------------- bf16 rounding

def check_bf16_rounding():
    rng = np.random.default_rng(7)
    v32 = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-38).astype(np.float32),   # subnormal range
        (rng.standard_normal(2000) * 1e37).astype(np.float32),
        np.array([3.3961775e38, -3.3961775e38, 1.0, 0.0, -0.0], np.float32),
    ])
    want = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(v32.astype(np.float64))
    assert np.array_equal(got, want)
    # ties to even, and a single rounding from float64 (no detour through fp32)
    assert oracle.round_bf16(1.0 + 2.0 ** -8) == 1.0
    assert oracle.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert oracle.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    vals = rng.standard_normal(500) * 10
    assert all(oracle.round_bf16(v) == bf16_round_exact(v) for v in vals)


def test_bf16_rounding():
    check_bf16_rounding()


def test_bf16_bits_roundtrip():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    v = oracle.bf16_bits_to_f64(bits)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    fin = np.isfinite(t)
    assert np.array_equal(v[fin], t[fin])
    assert np.array_equal(np.isnan(v), np.isnan(t))
