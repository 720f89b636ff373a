"""GPU parity against the float64 oracle on seeded inputs small enough for the
oracle to finish in seconds, yet spanning several tiles, several tokens per
expert bucket and ragged tails (hidden sizes that leave lanes idle, token
counts that leave the last pass of a bucket partial).

Bar: routing ids equal the oracle's except certified float64 near-ties, and
equal a host brute-force top-k on the GPU's own fp32 keys bit for bit (order
and weights included); permutations equal the stable sort of the GPU's ids
exactly; routed, shared and combined outputs within max relative error 2e-3
per token (fp32 output mode); the bf16 output is the round-to-nearest-even of
the fp32 output, bit for bit; the one-shot forward (which for up to 4 tokens
takes the fused path) agrees with the four entry points called in turn within
the same bound; its bf16 h equals the oracle's rounding of float64 h except for flips at
rounding midpoints, and its down projection, shared expert and combine agree
with float64 arithmetic on that h to 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_sparse_moe_amd as qm
import synth
from synth import FormatSpec, variant
from tests._gpu import (TOL, check_forward_intermediates, check_topk_exact, check_topk_ids, read_ws, rel_err,
                        run_staged, stable_sort_perm, xdev)

pytestmark = pytest.mark.gpu

SMALL = [
    synth.config("tiny"),
    variant("decode", "decode_s", 102, T=3, d=512, I=256, E=32, I_shared=256, steps=2),
    variant("hash", "hash_s", 103, T=40, d=512, I=256, E=32, vocab=1000),
    variant("prefill", "prefill_s", 104, T=200, d=512, I=256, E=32),
    variant("mixed", "mixed_s", 105, T=24, d=512, I=256, E=32, I_shared=256),
    variant("decode", "ragged_g32", 106, T=7, d=2400, I=224, E=24, top_k=3, gate_up=FormatSpec("affine", 4, 32),
            down=FormatSpec("affine", 4, 32), shared=FormatSpec("affine", 8, 32), I_shared=96),
    variant("mixed", "mixed_2x8", 107, T=9, d=4096, I=256, E=16, top_k=4, gate_up=FormatSpec("affine", 8, 64),
            down=FormatSpec("affine", 2, 64), shared=FormatSpec("affine", 3, 32), I_shared=128),
    variant("prefill", "mxfp4_wide", 108, T=33, d=6144, I=128, E=8, top_k=2, bias_kind="normal"),
    # matrix-core paths: MXFP4 buckets spanning two 128-token tiles; affine
    # 4-bit buckets spanning several 32-token tiles, groups of 32, 64 and 128
    variant("prefill", "mxfp4_big_bucket", 112, T=300, d=256, I=128, E=4, top_k=2, bias_kind="normal"),
    # MXFP4 output widths off the 32 x 32 kernel's 128-column tile: gate/up of
    # 320 rows, down of 384 rows take the 16 x 16 kernel
    variant("prefill", "mxfp4_gateup_16x16", 124, T=150, d=256, I=320, E=4, top_k=2, bias_kind="normal"),
    variant("prefill", "mxfp4_down_16x16", 125, T=150, d=384, I=256, E=4, top_k=2, bias_kind="normal"),
    variant("prefill", "aff4_g32_g128_mfma", 113, T=96, d=512, I=256, E=8, top_k=2, bias_kind="normal",
            gate_up=FormatSpec("affine", 4, 32), down=FormatSpec("affine", 4, 128)),
    variant("prefill", "aff4_g64_mfma_shared", 114, T=80, d=768, I=384, E=16, top_k=4, bias_kind="normal",
            gate_up=FormatSpec("affine", 4, 64), down=FormatSpec("affine", 4, 64),
            shared=FormatSpec("affine", 8, 64), I_shared=128),
    # 2- and 3-bit codes on the matrix cores (4+ tokens per expert)
    variant("mixed", "aff2_3_mfma", 115, T=64, d=512, I=256, E=16, top_k=4, bias_kind="normal",
            gate_up=FormatSpec("affine", 2, 128), down=FormatSpec("affine", 3, 64),
            shared=FormatSpec("affine", 8, 64), I_shared=256),
    # (K = 768 and 384: the last 4-step weight block of a row is partial)
    variant("mixed", "aff3g64_2g128_mfma", 116, T=37, d=768, I=384, E=8, top_k=3, bias_kind="normal",
            gate_up=FormatSpec("affine", 3, 64), down=FormatSpec("affine", 2, 128)),
    variant("mixed", "aff4g32_3g32_mixed_paths", 118, T=40, d=512, I=256, E=8, top_k=2, bias_kind="normal",
            gate_up=FormatSpec("affine", 4, 32), down=FormatSpec("affine", 3, 32)),
    # 8-bit routed experts on the matrix cores (32- and 16-token tiles)
    variant("mixed", "aff8_mfma", 119, T=64, d=512, I=256, E=8, top_k=4, bias_kind="normal",
            gate_up=FormatSpec("affine", 8, 128), down=FormatSpec("affine", 8, 32), I_shared=256),
    # shared expert with its K split over workgroups (4 slices gate/up, 2 down)
    variant("mixed", "shared_splitk", 120, T=16, d=2048, I=128, E=8, top_k=2, bias_kind="normal", I_shared=1024),
    # single token on the fused path: k of 6 (shared expert), 2 (hidden 4096, none), 8 (40 experts)
    variant("decode", "fused_k6_shared", 121, T=1, d=1024, I=256, E=64, top_k=6, I_shared=256),
    variant("decode", "fused_k2_d4096", 122, T=1, d=4096, I=128, E=16, top_k=2, shared=None),
    variant("decode", "fused_k8_e40", 123, T=1, d=512, I=384, E=40, top_k=8, I_shared=128),
    # 2- and 3-bit codes on the streaming GEMV (under one token per expert)
    variant("mixed", "mixed_gemv", 117, T=20, d=512, I=256, E=128, top_k=4, I_shared=256),
    # MXFP8 (e4m3 + e8m0 per 32): matrix cores (10 tokens per expert), the
    # streaming GEMV (under one per expert), the fused single-token path with
    # an 8-bit shared expert, and MXFP8 as the shared expert (matrix cores)
    variant("mxfp8", "mxfp8_mfma", 126, T=40, d=512, I=256, E=8, top_k=2, bias_kind="normal"),
    variant("mxfp8", "mxfp8_gemv", 127, T=6, d=768, I=256, E=32, top_k=4),
    variant("mxfp8", "mxfp8_fused", 128, T=1, d=1024, I=256, E=16, top_k=4, shared=synth.configs.AFF8_G64,
            I_shared=256),
    variant("mxfp8", "mxfp8_shared", 129, T=16, d=512, I=256, E=8, top_k=2, shared=synth.configs.MXFP8,
            I_shared=256),
    # layers of the 43-layer stack at small sizes: a REAP25-pruned layer (192
    # experts) on the fused single-token path with 2/3-bit experts, and a
    # hash-routed single-token layer with a shared expert
    variant("mixed", "stack_pruned_fused", 130, T=1, d=1024, I=256, E=192, top_k=6, I_shared=256),
    variant("hash", "hash_fused_t3", 132, T=3, d=512, I=256, E=32, vocab=300),
    # 2-bit rows whose lanes load two adjacent chunks at once (even chunk
    # counts, 2 or 4 chunks per lane): fused single token at d=4096; GEMV with
    # d=3072 and I=2560 (lanes past the row masked); odd chunk count (d=4064,
    # groups of 32) keeps one chunk per load
    variant("mixed", "aff2_paired_fused", 133, T=1, d=4096, I=256, E=16, top_k=4, I_shared=256),
    variant("mixed", "aff2_paired_gemv", 134, T=6, d=3072, I=2560, E=64, top_k=4, shared=None,
            down=synth.configs.AFF2_G128),
    variant("mixed", "aff2_odd_chunks", 135, T=6, d=4064, I=256, E=64, top_k=4, shared=None,
            gate_up=synth.configs.FormatSpec("affine", 2, 32), down=synth.configs.FormatSpec("affine", 2, 32)),
    variant("hash", "stack_hash_shared", 131, T=1, d=1024, I=256, E=64, vocab=500,
            gate_up=synth.configs.AFF2_G128, down=synth.configs.AFF3_G128, shared=synth.configs.AFF8_G64,
            I_shared=256),
]


def check_layer(cfg, layer, dl, step):
    x = synth.gen_x(cfg, step)
    tok = synth.gen_token_ids(cfg, step)
    st, out_f32, out_bf16, ws = run_staged(dl, x, tok)
    ref = oracle.forward(layer, x, token_ids=tok)
    gids = st.ids.cpu().numpy()
    k, E = cfg.top_k, cfg.E
    if cfg.route == "topk":
        check_topk_ids(gids, ref.ids, ref.key, k)
    else:
        assert np.array_equal(gids, ref.ids)
    off, perm = stable_sort_perm(gids, E)
    assert np.array_equal(st.offsets.cpu().numpy(), off)
    assert np.array_equal(st.perm.cpu().numpy(), perm)
    if not np.array_equal(gids, ref.ids):
        ref = oracle.forward(layer, x, token_ids=tok, ids=gids)
    assert np.allclose(st.w.cpu().numpy(), ref.w, rtol=2e-6, atol=1e-7)
    e_slot = rel_err(st.y_slot.cpu().numpy(), ref.y_slot)
    assert e_slot.max() <= TOL, e_slot.max()
    if layer.shared is not None:
        e_sh = rel_err(st.y_shared.cpu().numpy(), ref.y_shared)
        assert e_sh.max() <= TOL, e_sh.max()
    e = rel_err(out_f32.cpu().numpy(), ref.y)
    assert e.max() <= TOL, e.max()
    # one-shot forward vs the four entry points: the one-shot call may run other
    # kernels (the fused small-batch path, gate/up on the matrix cores), whose
    # bf16 h can differ from the streaming GEMV's by rounding flips; each is
    # held to the oracle above and, on its own h, to 1e-5 below
    assert rel_err(out_f32.cpu().numpy(), st.out.cpu().numpy().astype(np.float64)).max() <= TOL
    assert torch.equal(out_f32.to(torch.bfloat16), out_bf16)
    flips = check_forward_intermediates(cfg, layer, dl, ws, x, tok, out_f32.cpu().numpy())
    print(f"{cfg.name} step {step}: {flips} h rounding flip(s) of {cfg.T * cfg.top_k * cfg.I}")
    return e.max()


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_small_layer_parity(cfg):
    layer = synth.gen_layer(cfg)
    dl = qm.DeviceLayer.from_host(layer)
    worst = max(check_layer(cfg, layer, dl, s) for s in range(min(cfg.steps, 2)))
    print(f"{cfg.name}: max rel err {worst:.2e}")


# The documented maxima: hidden (gate/up input width) 8192 on every path (the
# fused decode path at four 32-input chunks per lane, the streaming GEMV, the
# matrix-core GEMM), 1024 experts with top-8 (above the fused path's 256, so
# the general path at one token too), intermediate (down input width) 8192.
LIMITS = [
    variant("decode", "lim_d8192_fused_t1", 140, T=1, d=8192, I=128, E=16, top_k=4, I_shared=128),
    variant("decode", "lim_d8192_fused_t3", 141, T=3, d=8192, I=128, E=16, top_k=4, I_shared=128),
    variant("mixed", "lim_d8192_gemv", 142, T=6, d=8192, I=128, E=64, top_k=4, I_shared=128),
    variant("hash", "lim_d8192_mfma", 143, T=160, d=8192, I=128, E=8, vocab=1000),
    variant("tiny", "lim_E1024_t1", 144, T=1, d=256, I=128, E=1024, top_k=8),
    variant("tiny", "lim_E1024_t40", 145, T=40, d=256, I=128, E=1024, top_k=8),
    variant("decode", "lim_I8192_t2", 146, T=2, d=256, I=8192, E=4, top_k=2, I_shared=8192),
    variant("decode", "lim_I8192_t40", 147, T=40, d=256, I=8192, E=4, top_k=2, I_shared=8192),
]


@pytest.mark.parametrize("cfg", LIMITS, ids=[c.name for c in LIMITS])
def test_maximum_size_parity(cfg):
    layer = synth.gen_layer(cfg)
    dl = qm.DeviceLayer.from_host(layer)
    worst = check_layer(cfg, layer, dl, 0)
    print(f"{cfg.name}: max rel err {worst:.2e}")


# Every token routed to the same k experts (k buckets full, the rest empty):
# a bias far above the scores on experts 0..k-1 (the bias only ranks, so the
# weights are still the scores'), or a hash table whose rows all name them.
ONE_BUCKET = [
    variant("prefill", "same_mxfp4_mfma", 150, T=300, d=256, I=128, E=8, top_k=2, bias_kind="normal"),
    variant("hash", "same_hash_aff4_mfma", 151, T=96, d=512, I=256, E=16, vocab=500),
    variant("mixed", "same_gemv", 152, T=6, d=512, I=256, E=64, top_k=4, I_shared=128),
    variant("decode", "same_fused_t4", 153, T=4, d=512, I=256, E=32, I_shared=128),
]


@pytest.mark.parametrize("cfg", ONE_BUCKET, ids=[c.name for c in ONE_BUCKET])
def test_all_tokens_in_the_same_buckets(cfg):
    layer = synth.gen_layer(cfg)
    k = cfg.top_k
    if cfg.route == "hash":
        layer.tid2eid[:] = np.arange(k, dtype=layer.tid2eid.dtype)
    else:
        layer.bias[:k] += 10.0
    dl = qm.DeviceLayer.from_host(layer)
    check_layer(cfg, layer, dl, 0)
    ids = oracle.forward(layer, synth.gen_x(cfg, 0), token_ids=synth.gen_token_ids(cfg, 0)).ids
    assert np.array_equal(np.sort(ids, axis=1), np.tile(np.arange(k), (cfg.T, 1)))


# All router weights zero and no bias: every logit is exactly 0, every key
# ties, so each token takes experts 0..k-1 in that order with weights 1/k (the
# ties-to-the-lower-index rule, in closed form) on every router path: the
# fused decode path (its output checked against the staged entry points),
# the K-split and the 64 x 64 logits kernels.
ALL_TIED = [
    variant("decode", "tied_fused_t1", 160, T=1, d=512, I=256, E=32, I_shared=128, bias_kind="none"),
    variant("decode", "tied_fused_t3", 161, T=3, d=512, I=256, E=32, I_shared=128, bias_kind="none"),
    variant("tiny", "tied_ksplit_t40", 162, T=40, d=256, I=128, E=64, top_k=6, bias_kind="none"),
    variant("prefill", "tied_mfma_t600", 163, T=600, d=256, I=128, E=8, top_k=2, bias_kind="none"),
]


@pytest.mark.parametrize("cfg", ALL_TIED, ids=[c.name for c in ALL_TIED])
def test_all_keys_tied_pick_the_lowest_experts(cfg):
    layer = synth.gen_layer(cfg)
    layer.wr[:] = 0.0
    dl = qm.DeviceLayer.from_host(layer)
    check_layer(cfg, layer, dl, 0)
    st, _, _, _ = run_staged(dl, synth.gen_x(cfg, 0))
    k = cfg.top_k
    assert np.array_equal(st.ids.cpu().numpy(), np.tile(np.arange(k, dtype=np.int32), (cfg.T, 1)))
    assert np.allclose(st.w.cpu().numpy(), 1.0 / k, rtol=1e-6, atol=0)


@pytest.mark.parametrize("T,d,E", [(600, 1024, 64), (300, 1024, 64), (100, 1056, 40), (17, 4096, 256)])
def test_router_logits_and_topk_on_gpu_keys(T, d, E):
    """Logits within fp32 accumulation error of float64; moe_route's top-k
    equals a host brute-force top-k on the GPU's own fp32 keys, order and
    weights bit for bit. Shapes: the 64-token tile kernel (over 512 tokens);
    the K-split kernel with ragged tokens, experts and K steps; its full width."""
    cfg = variant("prefill", "logits", 111, T=T, d=d, I=128, E=E)
    wr, bias = synth.gen_router(cfg)
    layer = synth.Layer(cfg, wr, bias, None, synth.gen_routed_stacked(cfg), None)
    dl = qm.DeviceLayer.from_host(layer)
    x = synth.gen_x(cfg, 0)
    xd = xdev(x)
    logits = qm.router_logits(dl, xd).cpu().numpy()
    ref = oracle.router_logits(oracle.bf16_bits_to_f64(x), wr)
    scale = np.abs(oracle.bf16_bits_to_f64(x)) @ np.abs(wr.astype(np.float64)).T
    assert np.all(np.abs(logits - ref) <= 1e-5 * scale + 1e-30)
    ws = dl.workspace(T)
    ids, w = qm.route(dl, xd, ws=ws)
    # moe_route leaves logits, packed keys and scores in its workspace
    a = lambda n: (n + 255) // 256 * 256
    te = T * E
    r_logits = qm.ws_region(ws, 256, torch.float32, (T, E)).cpu().numpy()
    keys = qm.ws_region(ws, 256 + a(4 * te), torch.int64, (T, E)).cpu().numpy().view(np.uint64)
    scores = qm.ws_region(ws, 256 + a(4 * te) + a(8 * te), torch.float32, (T, E)).cpu().numpy()
    assert np.array_equal(r_logits, logits)
    check_topk_exact(keys, scores, bias, ids.cpu().numpy(), w.cpu().numpy(), cfg.top_k)
    # scores are sqrtsoftplus of the GPU's logits to a few fp32 ulps
    s64 = oracle.sqrtsoftplus(logits.astype(np.float64))
    assert np.all(np.abs(scores - s64) <= 4 * np.spacing(np.abs(s64).astype(np.float32)))
