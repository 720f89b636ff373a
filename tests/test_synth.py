"""The seeded input generator: determinism, per-expert independence, value
ranges, and the layer byte model pinned by the pages' published sizes (CPU)."""
import json
import os

import numpy as np
import torch

import synth
from synth import CONFIGS, variant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_x_is_bf16_rne_of_normal_draw():
    cfg = variant("tiny", "t", 1234, T=8)
    bits = synth.gen_x(cfg, 0)
    a = np.random.Generator(np.random.PCG64(np.random.SeedSequence(1234, spawn_key=(2, 0)))) \
        .standard_normal((8, cfg.d), dtype=np.float32)
    want = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, want)
    assert np.array_equal(synth.gen_x(cfg, 0), bits)
    assert not np.array_equal(synth.gen_x(cfg, 1), bits)


def test_expert_alone_equals_stack_slice():
    cfg = variant("tiny", "t", 99, E=5, top_k=2)
    stack = synth.gen_routed_stacked(cfg)
    for e in (0, 3, 4):
        one = synth.gen_expert(cfg, e)
        for a, b in zip((one.gate, one.up, one.down), (stack.gate, stack.up, stack.down)):
            assert np.array_equal(a.codes[0], b.codes[e])
            assert np.array_equal(a.scales[0], b.scales[e])
            assert np.array_equal(a.biases[0], b.biases[e])


def test_value_ranges():
    cfg = variant("mixed", "m", 5, E=3, top_k=2, d=256, I=128)
    ex = synth.gen_expert(cfg, 1)
    for q, b in ((ex.gate, 2), (ex.down, 3)):
        s = q.scales.astype(np.float64)
        scale = 16.0 / 2 ** b
        assert s.min() >= 0.001 * scale * 0.999 and s.max() <= 0.01 * scale * 1.001
        assert np.array_equal(q.biases.astype(np.float64), -(2 ** (b - 1)) * s)
        assert q.codes.dtype == np.uint32 and q.codes.shape[-1] == q.cols * b // 32
    sh = synth.gen_shared(cfg)
    assert sh.gate.spec.bits == 8 and np.array_equal(sh.gate.biases.astype(np.float64),
                                                     -128 * sh.gate.scales.astype(np.float64))
    pf = variant("prefill", "p", 4, E=2, top_k=2, d=256, I=128)
    q = synth.gen_expert(pf, 0).gate
    assert q.biases is None and q.scales.dtype == np.uint8
    assert q.scales.min() >= 118 and q.scales.max() <= 124
    # uniform codes: every nibble value appears with about equal frequency
    nib = np.concatenate([(q.codes >> (4 * i)) & 0xF for i in range(8)]).ravel()
    cnt = np.bincount(nib, minlength=16)
    assert cnt.min() > 0.9 * cnt.mean()


def test_router_and_bias_kinds():
    wr, bias = synth.gen_router(variant("tiny", "t", 3))
    assert wr.dtype == np.float32 and abs(wr.std() - 0.02) < 0.002
    assert bias.dtype == np.float32 and abs(bias.std() - 0.1) < 0.04
    _, zb = synth.gen_router(variant("prefill", "p", 4, d=64))
    r = np.sort(np.exp(-zb.astype(np.float64) / 0.11))
    assert np.allclose(r, np.arange(1, 257), rtol=1e-5)
    _, hb = synth.gen_router(variant("hash", "h", 3, d=64, vocab=100))
    assert hb is None


def test_tid2eid_rows_are_distinct_subsets():
    cfg = variant("hash", "h", 3, vocab=5000)
    t = synth.gen_tid2eid(cfg)
    assert t.shape == (5000, 6) and t.dtype == np.int32
    assert t.min() >= 0 and t.max() < 256
    s = np.sort(t, 1)
    assert not np.any(s[:, 1:] == s[:, :-1])
    tok = synth.gen_token_ids(cfg, 0)
    assert tok.min() >= 0 and tok.max() < 5000 and len(tok) == cfg.T


def test_config_shapes():
    c = CONFIGS
    assert (c["tiny"].T, c["tiny"].d, c["tiny"].I, c["tiny"].E, c["tiny"].top_k) == (4, 256, 128, 16, 2)
    for n in ("decode", "hash", "prefill", "mixed"):
        assert (c[n].d, c[n].I, c[n].E, c[n].top_k) == (4096, 2048, 256, 6)
    assert c["decode"].T == 1 and c["decode"].steps == 64 and c["decode"].shared.bits == 8
    assert c["hash"].T == 512 and c["hash"].vocab == 129280
    assert c["prefill"].T == 4096 and c["prefill"].gate_up.fmt == "mxfp4"
    assert c["mixed"].T == 64 and (c["mixed"].gate_up.bits, c["mixed"].down.bits) == (2, 3)


def _expert_bytes(cfg, shared=False):
    if shared:
        return synth.gen_shared(cfg).nbytes_per_expert()
    fs_gu, fs_dn, I = cfg.gate_up, cfg.down, cfg.I
    d = cfg.d

    def qbytes(fs, rows, cols):
        b = rows * cols * fs.bits // 8 + rows * (cols // fs.group) * (2 if fs.fmt == "affine" else 1)
        return b + (rows * (cols // fs.group) * 2 if fs.fmt == "affine" else 0)
    return 2 * qbytes(fs_gu, I, d) + qbytes(fs_dn, d, I)


def test_byte_model_against_page_figures():
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        g = json.load(f)
    # bits per weight of affine b-bit g64 with 16-bit scale and bias
    assert abs((4 + 32 / 64) - g["bits_per_weight"]["affine4_g64"]["value"]) < 0.01
    assert abs((2 + 32 / 64) - g["bits_per_weight"]["affine2_g64"]["value"]) < 0.07
    # routed-expert parameters: 3 projections x d x I x E x layers
    sh = g["shape"]
    n = 3 * sh["hidden"] * sh["intermediate"] * sh["experts"] * g["num_layers"]["value"]
    assert n == 277_025_390_592 and abs(n - g["routed_expert_params"]["value"]) < 0.5e9
    # per-layer routed bytes fit the layer shards with fp16 scale/bias, and would not with fp32
    small = CONFIGS["mixed"]
    big = CONFIGS["decode"]
    per_small = _expert_bytes(small)
    per_big = _expert_bytes(big)
    assert per_small == 8_126_464 and per_big == 14_155_776
    assert _expert_bytes(big, shared=True) == 26_738_688
    E = sh["experts"]
    assert E * per_small / 1e9 <= g["shard_bytes_decimal_GB"]["layers_0_38_min"]["value"]
    assert E * per_big / 1e9 <= g["shard_bytes_decimal_GB"]["layers_39_42"]["value"]
    wts = 3 * sh["hidden"] * sh["intermediate"]
    fp32_small = (2 * wts / 3 * (2 + 64 / 128) + wts / 3 * (3 + 64 / 128)) / 8
    fp32_big = wts * (4 + 64 / 64) / 8
    assert E * fp32_small / 1e9 > g["shard_bytes_decimal_GB"]["layers_0_38_min"]["value"]
    assert E * fp32_big / 1e9 > g["shard_bytes_decimal_GB"]["layers_39_42"]["value"]
