"""Pins of the oracle's bucketing, experts and combine: stable sort, zero weights,
one-hot inputs, linearity, token-order equivariance, per-token independence and
pure-Python brute force on tiny layers (CPU)."""
import math
import struct
from types import SimpleNamespace

import numpy as np
import pytest

import oracle
from synth import ExpertWeights, FormatSpec, MoeConfig, f32_to_bf16_bits
from tests._packing import bf16_round_exact, e4m3_table_torch, finite_e4m3_codes, make_affine, make_mxfp4, make_mxfp8


# --------------------------------------------------------------------------- permutation

def check_permute_stable_sort():
    rng = np.random.default_rng(21)
    for T, k, E in [(1, 6, 256), (37, 2, 5), (200, 6, 16), (64, 3, 1)]:
        ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
        off, perm, cnt = oracle.permute(ids, E)
        flat = ids.reshape(-1).tolist()
        assert perm.tolist() == sorted(range(T * k), key=flat.__getitem__)
        assert off[0] == 0 and off[E] == T * k
        assert cnt.tolist() == [flat.count(e) for e in range(E)]
        for e in range(E):
            seg = perm[off[e]:off[e + 1]]
            assert all(flat[a] == e for a in seg) and list(seg) == sorted(seg)


def test_permute_is_stable_sort():
    check_permute_stable_sort()


def test_permute_rejects_out_of_range():
    with pytest.raises(AssertionError):
        oracle.permute(np.array([[0, 5]]), 5)


# --------------------------------------------------------------------------- tiny layers

def _bf16(v):
    return struct.unpack("<f", struct.pack("<I", int(v) << 16))[0]


def build_tiny_layer(seed, E=4, d=64, I=32, k=2, fmt="affine", bits=4, group=32, shared=None,
                     route="topk", vocab=0, zero_router=False):
    """A tiny layer with known integer codes; returns (layer, plain float weights)."""
    rng = np.random.default_rng(seed)
    plain = {}

    def proj(rows, cols, fmt_, bits_, group_):
        if fmt_ == "affine":
            codes = rng.integers(0, 1 << bits_, size=(rows, cols))
            s = rng.uniform(0.001, 0.01, size=(rows, cols // group_)).astype(np.float16) * np.float16(16 / 2 ** bits_)
            b = (np.float32(-(1 << (bits_ - 1))) * s.astype(np.float32)).astype(np.float16)
            q = make_affine([codes], [s], [b], bits_, group_)
            W = [[float(s[r, c // group_]) * int(codes[r, c]) + float(b[r, c // group_]) for c in range(cols)]
                 for r in range(rows)]
        elif fmt_ == "mxfp8":
            codes = finite_e4m3_codes(rng, (rows, cols))
            sb = rng.integers(110, 116, size=(rows, cols // 32))
            q = make_mxfp8([codes], [sb])
            tab8 = e4m3_table_torch()
            W = [[float(tab8[codes[r, c]]) * 2.0 ** (int(sb[r, c // 32]) - 127) for c in range(cols)]
                 for r in range(rows)]
        else:
            codes = rng.integers(0, 16, size=(rows, cols))
            sb = rng.integers(118, 125, size=(rows, cols // 32))
            q = make_mxfp4([codes], [sb])
            tab = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
            W = [[(-1.0 if codes[r, c] & 8 else 1.0) * tab[codes[r, c] & 7] * 2.0 ** (int(sb[r, c // 32]) - 127)
                  for c in range(cols)] for r in range(rows)]
        return q, W

    experts = []
    for e in range(E):
        g, Wg = proj(I, d, fmt, bits, group)
        u, Wu = proj(I, d, fmt, bits, group)
        dn, Wd = proj(d, I, fmt, bits, group)
        experts.append(ExpertWeights(g, u, dn))
        plain[e] = (Wg, Wu, Wd)
    sh = None
    if shared is not None:
        g, Wg = proj(I, d, "affine", shared, 32)
        u, Wu = proj(I, d, "affine", shared, 32)
        dn, Wd = proj(d, I, "affine", shared, 32)
        sh = ExpertWeights(g, u, dn)
        plain["shared"] = (Wg, Wu, Wd)
    wr = (rng.standard_normal((E, d)) * 0.2).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.1).astype(np.float32)
    if zero_router:
        wr[:] = 0
        bias[:] = 0
    fs = FormatSpec(fmt, bits if fmt == "affine" else (8 if fmt == "mxfp8" else 4), group if fmt == "affine" else 32)
    cfg = MoeConfig("t", seed, T=1, d=d, I=I, E=E, top_k=k, route=route, gate_up=fs, down=fs,
                    shared=None if shared is None else FormatSpec("affine", shared, 32),
                    I_shared=I if shared is not None else 0, vocab=vocab,
                    bias_kind="none" if route == "hash" else "normal")
    tid2eid = None
    if route == "hash":
        tid2eid = rng.integers(0, E, size=(vocab, k)).astype(np.int32)
    layer = SimpleNamespace(cfg=cfg, wr=wr, bias=None if route == "hash" else bias, tid2eid=tid2eid,
                            shared=sh, routed_expert=lambda e: experts[e])
    plain["wr"], plain["bias"], plain["tid2eid"] = wr, bias, tid2eid
    return layer, plain


def brute_layer(layer, plain, x_bits, token_ids=None):
    """The layer in plain Python loops over the test's own float weights."""
    cfg = layer.cfg
    T, d, E, k = x_bits.shape[0], cfg.d, cfg.E, cfg.top_k
    xs = [[_bf16(v) for v in row] for row in x_bits]
    wr = plain["wr"]
    out = []
    for t in range(T):
        logit = [sum(xs[t][i] * float(wr[e][i]) for i in range(d)) for e in range(E)]
        s = [math.sqrt(math.log1p(math.exp(l))) for l in logit]
        if cfg.route == "hash":
            ids = [int(v) for v in plain["tid2eid"][token_ids[t]]]
        else:
            key = [s[e] + float(plain["bias"][e]) for e in range(E)]
            ids = sorted(range(E), key=lambda e: (-key[e], e))[:k]
        tot = sum(s[e] for e in ids)
        w = [s[e] / tot for e in ids]

        def expert(W):
            Wg, Wu, Wd = W
            h = []
            for i in range(len(Wg)):
                g = sum(Wg[i][c] * xs[t][c] for c in range(d))
                u = sum(Wu[i][c] * xs[t][c] for c in range(d))
                h.append(bf16_round_exact(g / (1.0 + math.exp(-g)) * u))
            return [sum(Wd[r][i] * h[i] for i in range(len(h))) for r in range(d)]

        y = [0.0] * d
        for j, e in enumerate(ids):
            ye = expert(plain[e])
            y = [y[r] + w[j] * ye[r] for r in range(d)]
        if "shared" in plain:
            ys = expert(plain["shared"])
            y = [y[r] + ys[r] for r in range(d)]
        out.append((ids, w, y))
    return out


def _x(seed, T, d, scale=1.0):
    return f32_to_bf16_bits(np.random.default_rng(seed).standard_normal((T, d)).astype(np.float32) * scale)


@pytest.mark.parametrize("fmt,bits,shared", [("affine", 4, None), ("affine", 2, 8), ("affine", 3, None),
                                             ("affine", 8, 4), ("mxfp4", 4, None), ("mxfp8", 8, None)])
def test_tiny_layer_bruteforce(fmt, bits, shared):
    group = 32
    layer, plain = build_tiny_layer(100 + bits, fmt=fmt, bits=bits, group=group, shared=shared)
    x = _x(bits, 3, layer.cfg.d)
    ref = oracle.forward(layer, x)
    for t, (ids, w, y) in enumerate(brute_layer(layer, plain, x)):
        assert ref.ids[t].tolist() == ids
        assert np.allclose(ref.w[t], w, rtol=1e-12)
        assert np.allclose(ref.y[t], y, rtol=1e-9, atol=1e-12 * max(abs(v) for v in y))


def test_tiny_hash_layer_bruteforce():
    layer, plain = build_tiny_layer(7, E=5, k=3, route="hash", vocab=11)
    x = _x(8, 4, layer.cfg.d)
    tok = np.array([3, 10, 0, 3], np.int32)
    ref = oracle.forward(layer, x, token_ids=tok)
    for t, (ids, w, y) in enumerate(brute_layer(layer, plain, x, tok)):
        assert ref.ids[t].tolist() == ids
        assert np.allclose(ref.w[t], w, rtol=1e-12)
        assert np.allclose(ref.y[t], y, rtol=1e-9, atol=1e-12 * max(abs(v) for v in y))


def check_one_hot_extracts_column():
    layer, plain = build_tiny_layer(31, E=2, k=1, zero_router=True)
    d = layer.cfg.d
    for c in (0, 17, d - 1):
        x = np.zeros((1, d), np.uint16)
        x[0, c] = 0x3F80                                   # bf16 1.0
        ref = oracle.forward(layer, x)
        assert ref.ids[0].tolist() == [0] and ref.w[0, 0] == 1.0
        Wg, Wu, Wd = plain[0]
        h = [bf16_round_exact(Wg[i][c] / (1.0 + math.exp(-Wg[i][c])) * Wu[i][c]) for i in range(len(Wg))]
        want = [sum(Wd[r][i] * h[i] for i in range(len(h))) for r in range(d)]
        assert np.allclose(ref.y[0], want, rtol=1e-12, atol=1e-15)


def test_one_hot_extracts_column():
    check_one_hot_extracts_column()


def check_swiglu_h_one_hot():
    """swiglu_h of a one-hot input at column c is silu(W1[:, c]) * W3[:, c]
    (a gate/up swap, a missing silu or a transposed operand fails), and it is
    the unrounded product that swiglu_expert rounds to bf16 before W2."""
    rng = np.random.default_rng(5)
    w1, w3, w2 = rng.standard_normal((6, 8)), rng.standard_normal((6, 8)), rng.standard_normal((8, 6))
    for c in (0, 5, 7):
        x = np.zeros((1, 8))
        x[0, c] = 1.0
        h = oracle.swiglu_h(w1, w3, x)[0]
        want = [w1[i, c] / (1.0 + math.exp(-w1[i, c])) * w3[i, c] for i in range(6)]
        assert np.allclose(h, want, rtol=1e-14, atol=0)
        y = oracle.swiglu_expert(w1, w3, w2, x)[0]
        assert np.array_equal(y, oracle.round_bf16(h) @ w2.T)


def test_swiglu_h_one_hot():
    check_swiglu_h_one_hot()


def check_zero_weights_give_zero():
    layer, _ = build_tiny_layer(41, shared=8)
    for ew in [layer.routed_expert(e) for e in range(layer.cfg.E)] + [layer.shared]:
        for q in (ew.gate, ew.up, ew.down):
            # every code at the middle value 2^(b-1), whose weight is exactly zero
            b = q.spec.bits
            mid = sum(1 << (b * i + b - 1) for i in range(32 // b)) if 32 % b == 0 else None
            if mid is not None:
                q.codes[:] = mid
            else:
                q.scales[:] = 0
                q.biases[:] = 0
    ref = oracle.forward(layer, _x(3, 3, layer.cfg.d))
    assert np.all(ref.y == 0.0) and np.all(ref.y_slot == 0.0)


def test_zero_weights_give_zero():
    check_zero_weights_give_zero()


def test_down_scale_linearity():
    layer, _ = build_tiny_layer(51)
    x = _x(4, 3, layer.cfg.d)
    y1 = oracle.forward(layer, x).y
    for e in range(layer.cfg.E):
        dn = layer.routed_expert(e).down
        dn.scales *= np.float16(2)
        dn.biases *= np.float16(2)
    y2 = oracle.forward(layer, x).y
    assert np.array_equal(y2, 2 * y1)


def test_token_order_equivariance_and_independence():
    layer, _ = build_tiny_layer(61, shared=8)
    x = _x(6, 5, layer.cfg.d)
    ref = oracle.forward(layer, x)
    p = np.array([3, 0, 4, 1, 2])
    refp = oracle.forward(layer, x[p])
    assert np.array_equal(refp.ids, ref.ids[p])
    assert np.allclose(refp.y, ref.y[p], rtol=1e-13, atol=0)
    for t in range(5):
        one = oracle.forward(layer, x[t:t + 1])
        assert np.array_equal(one.ids[0], ref.ids[t])
        assert np.allclose(one.y[0], ref.y[t], rtol=1e-13, atol=0)


def test_weights_sum_to_one_and_shared_is_additive():
    layer, _ = build_tiny_layer(71, shared=8)
    x = _x(7, 4, layer.cfg.d)
    ref = oracle.forward(layer, x)
    assert np.allclose(ref.w.sum(1), 1.0, rtol=1e-14)
    routed = sum(ref.w[:, j:j + 1] * ref.y_slot[j::layer.cfg.top_k] for j in range(layer.cfg.top_k))
    assert np.allclose(ref.y - routed, ref.y_shared, rtol=1e-12, atol=1e-15)


def test_forward_tokens_and_given_ids_agree_with_forward():
    layer, _ = build_tiny_layer(81, shared=8)
    x = _x(9, 4, layer.cfg.d)
    ref = oracle.forward(layer, x)
    again = oracle.forward(layer, x, ids=ref.ids)
    assert np.array_equal(again.y, ref.y)
    w, ys, ysh, y = oracle.forward_tokens(layer, x, [2, 0], ref.ids[[2, 0]])
    assert np.allclose(y, ref.y[[2, 0]], rtol=1e-13)
    assert np.allclose(ysh, ref.y_shared[[2, 0]], rtol=1e-13)


def test_unrounded_h_differs_only_slightly():
    layer, _ = build_tiny_layer(91)
    x = _x(10, 3, layer.cfg.d)
    a = oracle.forward(layer, x).y
    b = oracle.forward(layer, x, round_h=False).y
    rel = np.abs(a - b).max(1) / np.abs(b).max(1)
    assert np.all(rel < 2.0 ** -7)
