"""Parity at the workloads' full sizes, through moe_forward as the benchmark
launches it. Routing ids and permutations are checked for every token; the
outputs are checked on sampled tokens, which the oracle evaluates one by one
(the layer is per-token, so a sampled token's output depends only on its own
activations and experts)."""
import gc

import numpy as np
import pytest
import torch

import oracle
import quantized_sparse_moe_amd as qm
import synth
from tests._gpu import TOL, check_topk_ids, rel_err, run_staged, stable_sort_perm

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def full():
    cache = {}

    def get(name):
        if name not in cache:
            cache.clear()
            gc.collect()
            torch.cuda.empty_cache()
            if name.startswith("stack43_l"):
                cfg = synth.stack_configs()[int(name[len("stack43_l"):])]
            else:
                cfg = synth.config(name)
            layer = synth.gen_layer(cfg)                 # stacked experts, uploaded once
            dl = qm.DeviceLayer.from_host(layer)
            layer.routed = None                          # oracle draws experts on demand
            cache[name] = (cfg, layer, dl, {})
        return cache[name]
    yield get
    cache.clear()
    gc.collect()
    torch.cuda.empty_cache()


def _check(cfg, layer, dl, ecache, x, tok, sample):
    st, out, out_bf16, _ = run_staged(dl, x, tok)
    gids = st.ids.cpu().numpy()
    x64 = oracle.bf16_bits_to_f64(x)
    if cfg.route == "hash":
        assert np.array_equal(gids, layer.tid2eid[tok])
    else:
        ref_ids, _, key, _ = oracle.route_topk(oracle.router_logits(x64, layer.wr), layer.bias, cfg.top_k)
        ties = check_topk_ids(gids, ref_ids, key, cfg.top_k, max_ties=max(2, cfg.T // 500))
        if ties:
            print(f"{cfg.name}: {ties} certified near-tie tokens")
    off, perm = stable_sort_perm(gids, cfg.E)
    assert np.array_equal(st.offsets.cpu().numpy(), off)
    assert np.array_equal(st.perm.cpu().numpy(), perm)
    w, y_slot, y_sh, y = oracle.forward_tokens(layer, x, sample, gids[sample], expert_cache=ecache)
    assert np.allclose(st.w.cpu().numpy()[sample], w, rtol=2e-6, atol=1e-7)
    ys = st.y_slot.cpu().numpy().reshape(cfg.T, cfg.top_k, cfg.d)[sample]
    assert rel_err(ys, y_slot).max() <= TOL
    if layer.shared is not None:
        assert rel_err(st.y_shared.cpu().numpy()[sample], y_sh).max() <= TOL
    e = rel_err(out.cpu().numpy()[sample], y)
    assert e.max() <= TOL, e.max()
    assert torch.equal(out.to(torch.bfloat16), out_bf16)
    return e.max()


def test_decode_batch1_full(full):
    cfg, layer, dl, ec = full("decode")
    worst = max(_check(cfg, layer, dl, ec, synth.gen_x(cfg, s), None, [0]) for s in (0, 1, 63))
    print(f"decode: max rel err {worst:.2e}")


def test_mixed_lowbit_full(full):
    cfg, layer, dl, ec = full("mixed")
    worst = _check(cfg, layer, dl, ec, synth.gen_x(cfg, 0), None, [0, 37, 63])
    print(f"mixed: max rel err {worst:.2e}")


def test_hash_routed_full(full):
    cfg, layer, dl, ec = full("hash")
    worst = _check(cfg, layer, dl, ec, synth.gen_x(cfg, 0), synth.gen_token_ids(cfg, 0), [0, 511])
    print(f"hash: max rel err {worst:.2e}")


def test_prefill_mxfp4_full(full):
    cfg, layer, dl, ec = full("prefill")
    worst = _check(cfg, layer, dl, ec, synth.gen_x(cfg, 0), None, [0, 4095])
    print(f"prefill: max rel err {worst:.2e}")


def test_mxfp8_full(full):
    cfg, layer, dl, ec = full("mxfp8")
    worst = _check(cfg, layer, dl, ec, synth.gen_x(cfg, 0), None, [0, 511])
    print(f"mxfp8: max rel err {worst:.2e}")


@pytest.mark.parametrize("layer", [0, 3, 42])
def test_stack43_layer_full(full, layer):
    """Layers of the 43-layer stack at full size, one token: a hash layer over
    256 experts, a REAP25-pruned 2/3-bit layer and a pruned 4-bit layer (each
    with its 8-bit shared expert)."""
    cfg, lyr, dl, ec = full(f"stack43_l{layer}")
    hashed = cfg.route == "hash"
    worst = max(_check(cfg, lyr, dl, ec, synth.gen_x(cfg, s), synth.gen_token_ids(cfg, s) if hashed else None, [0])
                for s in (0, 1))
    print(f"stack43 layer {layer}: max rel err {worst:.2e}")
