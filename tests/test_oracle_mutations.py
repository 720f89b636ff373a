"""Each plausible mistake planted in the oracle (on the CPU, via monkeypatch) must
make at least one pin fail: evidence that the pins constrain every step."""
import numpy as np
import pytest

import oracle
import oracle.moe as om
from tests import test_oracle_formats as F
from tests import test_oracle_layer as L
from tests import test_oracle_quant as Q
from tests import test_oracle_router as R
from tests import test_oracle_sinkhorn as S


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(om, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _tiny_bruteforce_with_shared():
    layer, plain = L.build_tiny_layer(104, fmt="affine", bits=4, group=32, shared=8)
    x = L._x(4, 2, layer.cfg.d)
    ref = oracle.forward(layer, x)
    for t, (ids, w, y) in enumerate(L.brute_layer(layer, plain, x)):
        assert ref.ids[t].tolist() == ids
        assert np.allclose(ref.y[t], y, rtol=1e-9, atol=1e-12 * max(abs(v) for v in y))


def _tiny_bruteforce_mxfp4():
    layer, plain = L.build_tiny_layer(105, fmt="mxfp4")
    x = L._x(5, 2, layer.cfg.d)
    ref = oracle.forward(layer, x)
    for t, (ids, w, y) in enumerate(L.brute_layer(layer, plain, x)):
        assert np.allclose(ref.y[t], y, rtol=1e-9, atol=1e-12 * max(abs(v) for v in y))


orig = {n: getattr(om, n) for n in om.__all__}


def m_e2m1_sign_bit(n):
    return orig["e2m1_decode"](np.asarray(n).astype(np.int64) ^ 0x8)


def m_e4m3_bias_8(n):
    """e4m3 decoded with exponent bias 8 (the FNUZ variant's bias)."""
    return orig["e4m3_decode"](n) * 0.5


def _tiny_bruteforce_mxfp8():
    layer, plain = L.build_tiny_layer(106, fmt="mxfp8")
    x = L._x(6, 2, layer.cfg.d)
    ref = oracle.forward(layer, x)
    for t, (ids, w, y) in enumerate(L.brute_layer(layer, plain, x)):
        assert np.allclose(ref.y[t], y, rtol=1e-9, atol=1e-12 * max(abs(v) for v in y))


def m_quant_levels_pow2(w_bits, bits, group):
    """Scale from 2^b steps instead of 2^b - 1."""
    codes, scale, bias = orig["quantize_affine"](w_bits, bits + 0, group)
    w = om.bf16_bits_to_f64(w_bits).astype(np.float32)
    g = w.reshape(w.shape[0], -1, group)
    scale = ((g.max(-1) - g.min(-1)) / np.float32(1 << bits)).astype(np.float16)
    q = np.clip(np.rint((g - bias.astype(np.float32)[..., None]) / scale.astype(np.float32)[..., None]), 0,
                (1 << bits) - 1).astype(np.int64).reshape(w.shape)
    return om.pack_codes(q, bits), scale, bias


def m_quant_truncate(w_bits, bits, group):
    """Codes truncated instead of rounded to nearest."""
    w = om.bf16_bits_to_f64(w_bits).astype(np.float32)
    g = w.reshape(w.shape[0], -1, group)
    scale = ((g.max(-1) - g.min(-1)) / np.float32((1 << bits) - 1)).astype(np.float16)
    bias = g.min(-1).astype(np.float16)
    q = np.clip(np.floor((g - bias.astype(np.float32)[..., None]) / scale.astype(np.float32)[..., None]), 0,
                (1 << bits) - 1).astype(np.int64).reshape(w.shape)
    return om.pack_codes(q, bits), scale, bias


def m_sinkhorn_rows_first(logits, iters=10, eps=0.0):
    """Rows normalised before columns in each round."""
    l = np.asarray(logits, dtype=np.float64)
    m = np.exp(l - l.max(axis=-1, keepdims=True))
    m = m / m.sum(axis=-1, keepdims=True)
    for _ in range(iters):
        m = m / (m.sum(axis=-1, keepdims=True) + eps)
        m = m / (m.sum(axis=-2, keepdims=True) + eps)
    return m


def m_sinkhorn_no_max_shift(logits, iters=10, eps=0.0):
    l = np.asarray(logits, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        m = np.exp(l)
        m = m / m.sum(axis=-1, keepdims=True)
        for _ in range(iters):
            m = m / (m.sum(axis=-2, keepdims=True) + eps)
            m = m / (m.sum(axis=-1, keepdims=True) + eps)
    return m


def m_e8m0_off_by_one(b):
    return orig["e8m0_decode"](np.asarray(b).astype(np.int64) - 1)


def m_unpack_msb_first(words, bits, cols):
    """Codes taken from the top of each word down (MSB-first order)."""
    c = orig["unpack_codes"](words, bits, cols)
    if 32 % bits:
        return np.roll(c, 1, axis=-1)
    per = 32 // bits
    return np.flip(c.reshape(*c.shape[:-1], -1, per), -1).reshape(c.shape)


def m_dequant_no_bias(q, e=0):
    if q.spec.fmt != "affine":
        return orig["dequant"](q, e)
    codes = om.unpack_codes(q.codes[e], q.spec.bits, q.cols)
    return np.repeat(q.scales[e].astype(np.float64), q.spec.group, -1) * codes


def m_mxfp4_scale_halved(q, e=0):
    w = orig["dequant"](q, e)
    return w * 0.5 if q.spec.fmt == "mxfp4" else w


def m_sqrtsoftplus_sign(l):
    l = np.asarray(l, dtype=np.float64)
    return np.sqrt(np.maximum(-l, 0.0) + np.log1p(np.exp(-np.abs(l))))


def m_topk_ties_high(logits, bias, k, routed_scale=1.0):
    s = om.sqrtsoftplus(logits)
    key = s + (0.0 if bias is None else np.asarray(bias, np.float64)[None, :])
    T, E = key.shape
    ids = np.empty((T, k), np.int32)
    for t in range(T):
        ids[t] = np.lexsort((-np.arange(E), -key[t]))[:k]
    return ids, om.combine_weights_for_ids(s, ids, routed_scale), key, s


def m_weights_with_bias(logits, bias, k, routed_scale=1.0):
    ids, _, key, s = orig["route_topk"](logits, bias, k, routed_scale)
    return ids, om.combine_weights_for_ids(key, ids, routed_scale), key, s


def m_permute_reverse_in_bucket(ids, E):
    off, perm, cnt = orig["permute"](ids, E)
    perm = perm.copy()
    for e in range(E):
        perm[off[e]:off[e + 1]] = perm[off[e]:off[e + 1]][::-1]
    return off, perm, cnt


def m_swiglu_swapped(w1, w3, w2, x64, round_h=True):
    return orig["swiglu_expert"](w3, w1, w2, x64, round_h)


def m_swiglu_transposed_down(w1, w3, w2, x64, round_h=True):
    """The down projection read as if stored [I][d] instead of [d][I]."""
    h = om.silu(x64 @ w1.T) * (x64 @ w3.T)
    h = om.round_bf16(h) if round_h else h
    return h @ w2.reshape(w2.shape[1], w2.shape[0])


def m_swiglu_h_silu_on_up(w1, w3, x64):
    """silu applied to the up projection instead of the gate."""
    return (x64 @ w1.T) * om.silu(x64 @ w3.T)


def m_round_via_fp32(v):
    return orig["round_bf16"](np.asarray(v, np.float64).astype(np.float32).astype(np.float64))


def m_hash_sorted_ids(x64, wr, tid2eid, token_ids, routed_scale=1.0):
    ids, w, s = orig["route_hash"](x64, wr, tid2eid, token_ids, routed_scale)
    return np.sort(ids, axis=1), w, s


MUTATIONS = [
    ("e2m1_decode", m_e2m1_sign_bit, [F.check_e2m1_table, F.check_mxfp4_rule]),
    ("e8m0_decode", m_e8m0_off_by_one, [F.check_e8m0_exhaustive, F.check_mxfp4_rule]),
    ("e4m3_decode", m_e4m3_bias_8, [F.check_e4m3_table, F.check_mxfp8_rule, _tiny_bruteforce_mxfp8]),
    ("unpack_codes", m_unpack_msb_first, [F.check_unpack_known_words]),
    ("dequant", m_dequant_no_bias, [lambda: F.check_affine_rule(4, 64), L.check_zero_weights_give_zero]),
    ("dequant", m_mxfp4_scale_halved, [F.check_mxfp4_rule, _tiny_bruteforce_mxfp4]),
    ("sqrtsoftplus", m_sqrtsoftplus_sign, [R.check_sqrtsoftplus_closed_forms]),
    ("route_topk", m_topk_ties_high, [R.check_topk_bruteforce]),
    ("route_topk", m_weights_with_bias, [R.check_topk_bruteforce, _tiny_bruteforce_with_shared]),
    ("permute", m_permute_reverse_in_bucket, [L.check_permute_stable_sort]),
    ("swiglu_expert", m_swiglu_swapped, [L.check_one_hot_extracts_column]),
    ("swiglu_expert", m_swiglu_transposed_down, [L.check_one_hot_extracts_column]),
    ("swiglu_h", m_swiglu_h_silu_on_up, [L.check_swiglu_h_one_hot, L.check_one_hot_extracts_column]),
    ("round_bf16", m_round_via_fp32, [F.check_bf16_rounding]),
    ("route_hash", m_hash_sorted_ids, [R.check_hash_route_lookup]),
    ("quantize_affine", m_quant_levels_pow2, [Q.check_grid_roundtrip, Q.check_quant_bounds]),
    ("quantize_affine", m_quant_truncate, [Q.check_quant_bounds]),
    ("mhc_sinkhorn", m_sinkhorn_rows_first, [S.check_sinkhorn_properties]),
    ("mhc_sinkhorn", m_sinkhorn_no_max_shift, [S.check_sinkhorn_properties]),
]


@pytest.mark.parametrize("i", range(len(MUTATIONS)), ids=[f"{m[0]}:{m[1].__name__}" for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, i):
    name, fn, pins = MUTATIONS[i]
    # the unmutated oracle passes these pins
    for pin in pins:
        pin()
    _patch(monkeypatch, name, fn)
    caught = 0
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught > 0, f"no pin caught the planted mistake in {name}"


def test_forward_without_shared_is_caught(monkeypatch):
    real = om.forward

    def no_shared(layer, x_bits, token_ids=None, ids=None, round_h=True):
        r = real(layer, x_bits, token_ids, ids, round_h)
        r.y = r.y - r.y_shared
        return r
    _tiny_bruteforce_with_shared()
    monkeypatch.setattr(oracle, "forward", no_shared)
    with pytest.raises(AssertionError):
        _tiny_bruteforce_with_shared()
