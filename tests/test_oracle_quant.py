"""Pins of the oracle's plain min/max affine quantiser (the conversion step
before the layer) and its bit packer, on the CPU."""
import numpy as np
import pytest

import oracle
from synth import f32_to_bf16_bits
from tests._packing import pack_codes as pack_ref


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_pack_codes_matches_independent_packer(bits):
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 1 << bits, size=(4, 96))
    assert np.array_equal(oracle.pack_codes(codes, bits), pack_ref(codes, bits))
    assert np.array_equal(oracle.unpack_codes(oracle.pack_codes(codes, bits), bits, 96), codes)


def _grid_group(rng, bits, group, s_exp, bmult):
    """Weights exactly on a grid s*q + b with s = 2^s_exp and b = bmult*s (both
    exact in fp16; |q + bmult| < 256 keeps every weight exact in bf16), codes
    spanning 0..2^b-1."""
    q = rng.integers(0, 1 << bits, size=group)
    q[0], q[-1] = 0, (1 << bits) - 1
    w = np.ldexp((q + bmult).astype(np.float64), s_exp)
    return q, w


def check_grid_roundtrip():
    """Weights on an fp16-representable grid come back as exactly that grid:
    the same codes, scale and bias."""
    rng = np.random.default_rng(5)
    for bits, group in [(2, 128), (3, 64), (4, 64), (4, 32), (8, 64)]:
        qs, ws, bs = [], [], []
        grids = [(-9, -128), (-12, 0), (-7, -3)] if bits == 8 else [(-9, -8), (-12, 37), (-7, -100)]
        for j, (s_exp, bmult) in enumerate(grids):
            q, w = _grid_group(rng, bits, group, s_exp, bmult)
            qs.append(q)
            ws.append(w)
            bs.append((s_exp, bmult * 2.0 ** s_exp))
        w = np.concatenate(ws)[None, :]
        wb = f32_to_bf16_bits(w.astype(np.float32))
        assert np.array_equal(oracle.bf16_bits_to_f64(wb), w)      # exact in bf16
        codes, scale, bias = oracle.quantize_affine(wb, bits, group)
        assert np.array_equal(oracle.unpack_codes(codes, bits, w.shape[1])[0], np.concatenate(qs))
        for j, (s_exp, b) in enumerate(bs):
            assert float(scale[0, j]) == 2.0 ** s_exp and float(bias[0, j]) == b


def test_grid_roundtrip():
    check_grid_roundtrip()


def check_quant_bounds():
    """On random weights: each group's min gets code 0 and its max code 2^b-1,
    codes are monotone in the weight, and every weight is within half a step
    (plus the fp16 rounding of scale and bias) of its dequantised value."""
    rng = np.random.default_rng(6)
    for bits, group in [(2, 128), (3, 128), (4, 64), (8, 32)]:
        w = f32_to_bf16_bits((rng.standard_normal((5, 4 * group)) * 0.02).astype(np.float32))
        codes, scale, bias = oracle.quantize_affine(w, bits, group)
        q = oracle.unpack_codes(codes, bits, 4 * group).reshape(5, 4, group)
        wf = oracle.bf16_bits_to_f64(w).reshape(5, 4, group)
        s, b = scale.astype(np.float64), bias.astype(np.float64)
        lo, hi = wf.min(-1), wf.max(-1)
        exact = (hi - lo) / ((1 << bits) - 1)
        assert np.all(s > 0)
        lo_i, hi_i = wf.argmin(-1), wf.argmax(-1)
        assert np.all(np.take_along_axis(q, lo_i[..., None], -1) == 0)
        assert np.all(np.take_along_axis(q, hi_i[..., None], -1) == (1 << bits) - 1)
        order = np.argsort(wf, axis=-1, kind="stable")
        assert np.all(np.diff(np.take_along_axis(q, order, -1), axis=-1) >= 0)
        deq = s[..., None] * q + b[..., None]
        bound = 0.5 * s * (1 + 2.0 ** -10) + np.abs(b - lo) + ((1 << bits) - 1) * np.abs(s - exact)
        assert np.all(np.abs(deq - wf) <= bound[..., None] + 1e-12)


def test_quant_bounds():
    check_quant_bounds()


def test_constant_group_has_zero_scale():
    w = np.full((2, 64), 0x3F80, dtype=np.uint16)          # bf16 1.0
    w[1, 32:] = 0xBE00                                      # bf16 -0.125
    codes, scale, bias = oracle.quantize_affine(w, 4, 32)
    assert np.all(scale == 0) and np.array_equal(bias.astype(np.float64), [[1.0, 1.0], [1.0, -0.125]])
    assert np.all(oracle.unpack_codes(codes, 4, 64) == 0)
