"""The GPU affine quantiser against the oracle's (moe_quantize_affine): codes,
fp16 scales and biases bit for bit, on seeded bf16 weights with ragged row
counts, every bit width and group size, special groups (constant, tiny range,
large magnitude, one sign), the device error word, and a full expert-sized
stack; and quantised weights run through the layer."""
import numpy as np
import pytest
import torch

import oracle
import quantized_sparse_moe_amd as qm
import quantized_sparse_moe_amd._lib as _lib
import synth
from synth import f32_to_bf16_bits
from tests._gpu import xdev

pytestmark = pytest.mark.gpu


def _gpu_quant(w_bits, bits, group):
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    codes, scales, biases = qm.quantize_affine(xdev(w_bits), bits, group, err=err)
    torch.cuda.synchronize()
    return (codes.cpu().numpy().view(np.uint32), scales.cpu().numpy().view(np.float16),
            biases.cpu().numpy().view(np.float16), int(err.item()))


def _special_rows(cols, group):
    """Rows of special groups: constant, a range below fp16's smallest step, large
    magnitudes, one sign only, a single outlier."""
    rng = np.random.default_rng(77)
    rows = []
    rows.append(np.full(cols, 0.75, np.float32))
    rows.append((1.0 + rng.integers(0, 2, cols) * 2.0 ** -7).astype(np.float32))
    rows.append((rng.standard_normal(cols) * 3000.0).astype(np.float32))
    rows.append(np.abs(rng.standard_normal(cols)).astype(np.float32) * 0.01 + 0.5)
    r = (rng.standard_normal(cols) * 0.02).astype(np.float32)
    r[group // 2] = 1.5
    rows.append(r)
    rows.append((rng.standard_normal(cols) * 1e-6).astype(np.float32))
    return f32_to_bf16_bits(np.stack(rows))


@pytest.mark.parametrize("bits,group", [(2, 128), (3, 128), (4, 64), (8, 64), (2, 32), (3, 32), (4, 32), (8, 128)])
def test_quantize_matches_oracle(bits, group):
    w = np.concatenate([synth.gen_bf16_weights(11, bits * group, 37, 4 * group), _special_rows(4 * group, group)])
    codes, scales, biases, err = _gpu_quant(w, bits, group)
    rc, rs, rb = oracle.quantize_affine(w, bits, group)
    assert err == 0
    assert np.array_equal(codes, rc)
    assert np.array_equal(scales.view(np.uint16), rs.view(np.uint16))
    assert np.array_equal(biases.view(np.uint16), rb.view(np.uint16))


def _tie_rows(bits, group, cols):
    """Groups whose quotients (w - bias) / scale land exactly on half-integers,
    and one bf16 step either side of them: min 0 and max (2^b - 1) / 16 make
    the scale exactly 1/16, so w = (2k + 1) / 32 gives the quotient k + 1/2."""
    levels = (1 << bits) - 1
    ks = np.arange(min(levels, 128))
    ties = (2 * ks + 1) / 32.0
    rows = []
    for nudge in (0, 1, -1):
        g = np.resize(ties, group).astype(np.float32)
        g[0], g[1] = 0.0, levels / 16.0
        b = f32_to_bf16_bits(g).astype(np.int32)
        b[2:] += nudge          # one bf16 step up or down (all values positive)
        rows.append(np.tile(b.astype(np.uint16), cols // group))
    return np.stack(rows)


@pytest.mark.parametrize("bits,group", [(2, 32), (3, 64), (4, 64), (8, 128)])
def test_quantize_exact_and_near_ties(bits, group):
    """Exact ties round to even, neighbours one step away to their side: the
    same integers as the oracle's correctly rounded division."""
    w = _tie_rows(bits, group, 2 * group)
    codes, scales, biases, err = _gpu_quant(w, bits, group)
    rc, rs, rb = oracle.quantize_affine(w, bits, group)
    assert err == 0
    assert np.all(rs.astype(np.float32)[:1] == 1.0 / 16)
    assert np.array_equal(codes, rc)
    assert np.array_equal(scales.view(np.uint16), rs.view(np.uint16))
    assert np.array_equal(biases.view(np.uint16), rb.view(np.uint16))


def _biased_tie_rows(bits, group, cols, B, s):
    """Ties away from zero: min b = B s and max b + (2^b - 1) s make the scale
    exactly s and the bias b, and w = s (B + k + 1/2) gives the quotient
    k + 1/2 exactly; then one bf16 step either side of each tie. |B| up to 120
    makes the fast path's |b / s| term the larger part of its threshold."""
    levels = (1 << bits) - 1
    ks = np.arange(min(levels, 128))
    rows = []
    for nudge in (0, 1, -1):
        g = np.resize(s * (B + ks + 0.5), group).astype(np.float32)
        g[0], g[1] = s * B, s * (B + levels)
        b = f32_to_bf16_bits(g)
        assert np.array_equal(oracle.bf16_bits_to_f64(b), g.astype(np.float64))   # exact in bf16
        b = b.astype(np.int32)
        b[2:] += nudge
        rows.append(np.tile(b.astype(np.uint16), cols // group))
    return np.stack(rows)


@pytest.mark.parametrize("bits,group,B,s", [(2, 32, 64, 2.0 ** -6), (3, 64, 100, 1.0), (4, 64, 64, 2.0 ** -5),
                                            (4, 128, -120, 2.0 ** -3), (8, 128, -64, 2.0 ** -4)])
def test_quantize_ties_with_a_nonzero_minimum(bits, group, B, s):
    """Exact ties and their one-step neighbours in groups whose minimum (the
    bias) is up to 120 scale steps from zero: codes, scales and biases equal the
    oracle's correctly rounded division bit for bit."""
    w = _biased_tie_rows(bits, group, 2 * group, B, s)
    codes, scales, biases, err = _gpu_quant(w, bits, group)
    rc, rs, rb = oracle.quantize_affine(w, bits, group)
    assert err == 0
    assert np.all(rs.astype(np.float64)[0] == s) and np.all(rb.astype(np.float64)[0] == B * s)
    assert np.array_equal(codes, rc)
    assert np.array_equal(scales.view(np.uint16), rs.view(np.uint16))
    assert np.array_equal(biases.view(np.uint16), rb.view(np.uint16))


def test_quantize_ragged_tail_and_one_row():
    """Chunk counts that leave the last workgroup partly empty, and a single row."""
    for rows, cols, bits, group in [(3, 4096 + 64, 4, 64), (1, 64, 2, 64), (257, 96, 3, 32)]:
        w = synth.gen_bf16_weights(12, rows, rows, cols)
        codes, scales, biases, err = _gpu_quant(w, bits, group)
        rc, rs, rb = oracle.quantize_affine(w, bits, group)
        assert err == 0 and np.array_equal(codes, rc)
        assert np.array_equal(scales.view(np.uint16), rs.view(np.uint16))
        assert np.array_equal(biases.view(np.uint16), rb.view(np.uint16))


def test_quantize_flags_inputs_beyond_fp16():
    w = synth.gen_bf16_weights(13, 0, 2, 128)
    w[1, 5] = f32_to_bf16_bits(np.array([1.0e6], np.float32))[0]      # bias and scale beyond fp16
    *_, err = _gpu_quant(w, 4, 64)
    assert err & _lib.MOE_DEVERR_QUANT_INPUT
    w = synth.gen_bf16_weights(13, 0, 2, 128)
    w[0, 7] = 0x7FC0                                                  # bf16 NaN
    *_, err = _gpu_quant(w, 4, 64)
    assert err & _lib.MOE_DEVERR_QUANT_INPUT


def test_quantize_full_expert_stack():
    """Eight experts' gate projections stacked as rows = 8 * 2048, d = 4096
    (4-bit g64 and 2-bit g128): bit-exact on sampled rows."""
    w = synth.gen_bf16_weights(14, 0, 8 * 2048, 4096)
    for bits, group in [(4, 64), (2, 128)]:
        codes, scales, biases, err = _gpu_quant(w, bits, group)
        assert err == 0
        sample = np.array([0, 1, 2047, 2048, 9000, 8 * 2048 - 1])
        rc, rs, rb = oracle.quantize_affine(w[sample], bits, group)
        assert np.array_equal(codes[sample], rc)
        assert np.array_equal(scales[sample].view(np.uint16), rs.view(np.uint16))
        assert np.array_equal(biases[sample].view(np.uint16), rb.view(np.uint16))


def test_quantised_weights_run_through_the_layer():
    """Quantise a small layer's bf16 expert weights on the GPU, run the layer on
    them, and compare with the oracle's layer on the oracle's quantisation."""
    cfg = synth.variant("tiny", "quant_layer", 140, T=5, d=256, I=128, E=4, top_k=2)
    layer = synth.gen_layer(cfg)
    spec = cfg.gate_up
    for e in range(cfg.E):
        for m, q in enumerate((layer.routed.gate, layer.routed.up, layer.routed.down)):
            w = synth.gen_bf16_weights(15, 3 * e + m, q.rows, q.cols)
            codes, scales, biases, err = _gpu_quant(w, spec.bits, spec.group)
            assert err == 0
            q.codes[e], q.scales[e], q.biases[e] = codes, scales, biases
            rc, rs, rb = oracle.quantize_affine(w, spec.bits, spec.group)
            assert np.array_equal(codes, rc)
    dl = qm.DeviceLayer.from_host(layer)
    x = synth.gen_x(cfg, 0)
    out = qm.forward(dl, xdev(x), None, out_dtype="f32", ws=dl.workspace(cfg.T)).cpu().numpy()
    ref = oracle.forward(layer, x)
    err = np.abs(out - ref.y).max(axis=1) / np.abs(ref.y).max(axis=1)
    assert err.max() <= 2e-3
