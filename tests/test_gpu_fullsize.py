"""Parity at the workloads' full sizes, through moe_forward as the benchmark
launches it.

For every workload: routing ids equal the oracle's (certified float64
near-ties aside) and equal a host brute-force top-k on the GPU's own fp32 keys
bit for bit; permutations equal the stable sort of the GPU's ids. Outputs, per
workload:
  * the heaviest and the lightest non-empty expert bucket: every slot's y_slot
    against the oracle, every element of their bf16 h against the oracle's
    rounding of float64 h (flips only at rounding midpoints), and y_slot
    against float64 arithmetic on the GPU's own h to 1e-5;
  * sampled tokens' combined outputs (all 64 tokens of the mixed workload).
The oracle evaluates only the experts it needs (the layer is per-token and
per-expert), dequantising them in a thread pool.
"""
import gc
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import quantized_sparse_moe_amd as qm
import synth
from tests._gpu import (TIGHT, TOL, check_forward_intermediates, check_h, check_topk_ids, check_topk_exact,
                        check_weights_exact, expert_reference, read_ws, rel_err, run_staged, stable_sort_perm)

pytestmark = pytest.mark.gpu

THREADS = min(16, len(os.sched_getaffinity(0)))


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
            cache[name] = (cfg, layer, dl)
        return cache[name]
    yield get
    cache.clear()
    gc.collect()
    torch.cuda.empty_cache()


def _routing(cfg, layer, x, tok, st, r):
    gids = st.ids.cpu().numpy()
    assert np.array_equal(r["ids"], gids)
    if cfg.route == "hash":
        assert np.array_equal(gids, layer.tid2eid[tok])
        if r["scores"] is not None:
            check_weights_exact(r["scores"], gids, r["w"])
    else:
        x64 = oracle.bf16_bits_to_f64(x)
        ref_ids, _, key, _ = oracle.route_topk(oracle.router_logits(x64, layer.wr), layer.bias, cfg.top_k)
        ties = check_topk_ids(gids, ref_ids, key, cfg.top_k, max_ties=max(2, cfg.T // 500))
        if ties:
            print(f"{cfg.name}: {ties} certified near-tie tokens")
        check_topk_exact(r["keys"], r["scores"], layer.bias, gids, r["w"], cfg.top_k)
    off, perm = stable_sort_perm(gids, cfg.E)
    assert np.array_equal(st.offsets.cpu().numpy(), off)
    assert np.array_equal(st.perm.cpu().numpy(), perm)
    if not r["fused"]:
        assert np.array_equal(r["offsets"], off) and np.array_equal(r["perm"], perm)
    return gids, off, perm


def _bucket(cfg, layer, x, r, off, perm, e):
    """Every slot of expert e's bucket: h and y_slot."""
    k = cfg.top_k
    slots = perm[off[e]:off[e + 1]]
    ref = expert_reference(layer.routed_expert(int(e)), 0, x[slots // k])
    h_gpu = r["h"][off[e]:off[e + 1]]
    flips = check_h(h_gpu, ref)
    y_gpu = r["y_slot"][slots]
    e_or = rel_err(y_gpu, ref["y"]).max()
    assert e_or <= TOL, e_or
    assert rel_err(y_gpu, oracle.bf16_bits_to_f64(h_gpu) @ ref["w2"].T).max() <= TIGHT
    return flips, e_or, len(slots)


def _tokens_out(cfg, layer, x, gids, out, tokens):
    """Combined outputs of `tokens` against the oracle, each touched expert
    dequantised once (in a thread pool)."""
    k = cfg.top_k
    tokens = np.asarray(tokens)
    need = {}
    for i, t in enumerate(tokens):
        for j in range(k):
            need.setdefault(int(gids[t, j]), []).append((i, j))

    def run(e):
        sel = need[e]
        ref = expert_reference(layer.routed_expert(e), 0, x[tokens[[i for i, _ in sel]]], bound=False)
        return e, sel, ref["y"]

    y_slot = np.zeros((len(tokens), k, cfg.d))
    with ThreadPoolExecutor(THREADS) as ex:
        for e, sel, y in ex.map(run, list(need)):
            for row, (i, j) in enumerate(sel):
                y_slot[i, j] = y[row]
    x64 = oracle.bf16_bits_to_f64(x[tokens])
    s = oracle.sqrtsoftplus(oracle.router_logits(x64, layer.wr))
    w = oracle.combine_weights_for_ids(s, gids[tokens])
    y = np.einsum("nk,nkd->nd", w, y_slot)
    if layer.shared is not None:
        y += oracle.swiglu_expert(*oracle.expert_mats(layer.shared), x64)
    e = rel_err(out[tokens], y)
    assert e.max() <= TOL, e.max()
    return e.max()


def _check(cfg, layer, dl, x, tok, sample, buckets=True):
    st, out, out_bf16, ws = run_staged(dl, x, tok)
    assert torch.equal(out.to(torch.bfloat16), out_bf16)
    r = read_ws(dl, ws, cfg.T)
    gids, off, perm = _routing(cfg, layer, x, tok, st, r)
    out = out.cpu().numpy()
    worst = _tokens_out(cfg, layer, x, gids, out, sample)
    if buckets and not r["fused"]:
        cnt = np.diff(off)
        nz = np.nonzero(cnt)[0]
        heavy, light = int(nz[np.argmax(cnt[nz])]), int(nz[np.argmin(cnt[nz])])
        for e in (heavy, light):
            flips, err, n = _bucket(cfg, layer, x, r, off, perm, e)
            print(f"{cfg.name}: expert {e} bucket of {n} slots: max rel err {err:.2e}, "
                  f"{flips} h rounding flip(s) of {n * cfg.I}")
            worst = max(worst, err)
    return worst, r


def test_decode_batch1_full(full):
    """The fused single-token path: outputs; routing on the GPU's keys; every
    slot's h (slot order) and the shared expert's h against the oracle; the
    fused down + shared + combine on the GPU's own h to 1e-5."""
    cfg, layer, dl = full("decode")
    worst = 0.0
    for s in (0, 1, 63):
        x = synth.gen_x(cfg, s)
        st, out, out_bf16, ws = run_staged(dl, x, None)
        w, r = _check(cfg, layer, dl, x, None, [0])
        assert r["fused"]
        flips = check_forward_intermediates(cfg, layer, dl, ws, x, None, out.cpu().numpy())
        print(f"decode step {s}: {flips} h rounding flip(s) of {cfg.top_k * cfg.I + cfg.I_shared}")
        worst = max(worst, w)
    print(f"decode: max rel err {worst:.2e}")


def test_mixed_lowbit_full(full):
    cfg, layer, dl = full("mixed")
    worst, _ = _check(cfg, layer, dl, synth.gen_x(cfg, 0), None, range(cfg.T))
    print(f"mixed: all {cfg.T} tokens, max rel err {worst:.2e}")


def test_hash_routed_full(full):
    cfg, layer, dl = full("hash")
    worst, _ = _check(cfg, layer, dl, synth.gen_x(cfg, 0), synth.gen_token_ids(cfg, 0), [0, 255, 511])
    print(f"hash: max rel err {worst:.2e}")


def test_prefill_mxfp4_full(full):
    cfg, layer, dl = full("prefill")
    worst, _ = _check(cfg, layer, dl, synth.gen_x(cfg, 0), None, [0, 2047, 4095])
    print(f"prefill: max rel err {worst:.2e}")


def test_mxfp8_full(full):
    cfg, layer, dl = full("mxfp8")
    worst, _ = _check(cfg, layer, dl, synth.gen_x(cfg, 0), None, [0, 511])
    print(f"mxfp8: max rel err {worst:.2e}")


@pytest.mark.parametrize("layer", [0, 3, 42])
def test_stack43_layer_full(full, layer):
    """Layers of the 43-layer stack at full size, one token: a hash layer over
    256 experts, a REAP25-pruned 2/3-bit layer and a pruned 4-bit layer (each
    with its 8-bit shared expert)."""
    cfg, lyr, dl = full(f"stack43_l{layer}")
    hashed = cfg.route == "hash"
    worst = 0.0
    for s in (0, 1):
        x, tok = synth.gen_x(cfg, s), synth.gen_token_ids(cfg, s) if hashed else None
        _, out, _, ws = run_staged(dl, x, tok)
        worst = max(worst, _check(cfg, lyr, dl, x, tok, [0])[0])
        flips = check_forward_intermediates(cfg, lyr, dl, ws, x, tok, out.cpu().numpy())
        print(f"stack43 layer {layer} step {s}: {flips} h rounding flip(s)")
    print(f"stack43 layer {layer}: max rel err {worst:.2e}")
