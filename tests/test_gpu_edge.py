"""Edge cases on the GPU: k = E, a single expert, duplicate hash-table ids,
zero weights, zero tokens, device error words for out-of-range ids (forced
from the host with in-bounds fallbacks), and determinism with a poisoned
workspace."""
import numpy as np
import pytest
import torch

import oracle
import quantized_sparse_moe_amd as qm
import synth
from quantized_sparse_moe_amd import _lib
from synth import variant
from tests._gpu import TOL, rel_err, run_staged, stable_sort_perm, xdev

pytestmark = pytest.mark.gpu


def _parity(cfg, layer, x, tok=None):
    dl = qm.DeviceLayer.from_host(layer)
    st, out, _, _ = run_staged(dl, x, tok)
    ref = oracle.forward(layer, x, token_ids=tok)
    assert np.array_equal(st.ids.cpu().numpy(), ref.ids)
    assert rel_err(out.cpu().numpy(), ref.y).max() <= TOL
    return st, ref


def test_k_equals_E():
    cfg = variant("tiny", "kE", 201, E=8, top_k=8, T=5)
    layer = synth.gen_layer(cfg)
    st, _ = _parity(cfg, layer, synth.gen_x(cfg, 0))
    assert np.all(np.sort(st.ids.cpu().numpy(), 1) == np.arange(8))


def test_single_expert():
    cfg = variant("tiny", "E1", 202, E=1, top_k=1, T=6)
    layer = synth.gen_layer(cfg)
    st, _ = _parity(cfg, layer, synth.gen_x(cfg, 0))
    assert np.all(st.w.cpu().numpy() == 1.0)


def test_hash_duplicate_ids_are_separate_slots():
    cfg = variant("hash", "dup", 203, T=12, d=256, I=128, E=8, top_k=3, vocab=10)
    layer = synth.gen_layer(cfg)
    layer.tid2eid[:] = np.array([[1, 1, 5]] * 10, np.int32)
    layer.tid2eid[3] = [7, 7, 7]
    x = synth.gen_x(cfg, 0)
    tok = synth.gen_token_ids(cfg, 0)
    tok[0] = 3
    _parity(cfg, layer, x, tok)


def test_zero_weights_give_zero_output():
    cfg = variant("mixed", "zero", 204, T=4, d=256, I=128, E=8, top_k=2, I_shared=128)
    layer = synth.gen_layer(cfg)
    for ew in (layer.routed, layer.shared):
        for q in (ew.gate, ew.up, ew.down):
            q.scales[:] = 0
            q.biases[:] = 0
    dl = qm.DeviceLayer.from_host(layer)
    out = qm.forward(dl, xdev(synth.gen_x(cfg, 0)), out_dtype="f32")
    assert torch.count_nonzero(out).item() == 0


def test_zero_tokens_launches_nothing():
    cfg = synth.config("tiny")
    dl = qm.DeviceLayer.from_host(synth.gen_layer(cfg))
    x = torch.empty((0, cfg.d), dtype=torch.int16, device="cuda")
    ws = dl.workspace(1)
    out = qm.forward(dl, x, out_dtype="f32", ws=ws)
    assert out.shape == (0, cfg.d)
    st = qm.forward_staged(dl, x, ws=ws)
    assert st.out.shape == (0, cfg.d) and st.ids.shape == (0, cfg.top_k)


# T=8: the staged path (k_hash); T=3: the fused small-batch path
@pytest.mark.parametrize("T,bad", [(8, 3), (3, 1)])
def test_out_of_range_token_id_sets_error_word(T, bad):
    cfg = variant("hash", "badtok", 205, T=T, d=256, I=128, E=16, top_k=2, vocab=50)
    layer = synth.gen_layer(cfg)
    dl = qm.DeviceLayer.from_host(layer)
    x = synth.gen_x(cfg, 0)
    tok = synth.gen_token_ids(cfg, 0)
    good = tok.copy()
    tok[bad] = 50
    ws = dl.workspace(cfg.T)
    out = qm.forward(dl, xdev(x), torch.from_numpy(tok).cuda(), out_dtype="f32", ws=ws)
    assert qm.device_error(ws) & _lib.MOE_DEVERR_TOKEN_ID
    ref = oracle.forward(layer, x, token_ids=good)
    keep = [t for t in range(cfg.T) if t != bad]
    assert rel_err(out.cpu().numpy()[keep], ref.y[keep]).max() <= TOL
    assert torch.count_nonzero(out[bad]).item() == 0
    qm.workspace_init(ws)
    assert qm.device_error(ws) == 0


def test_out_of_range_table_entry_sets_error_word():
    cfg = variant("hash", "badtab", 206, T=4, d=256, I=128, E=16, top_k=2, vocab=20)
    layer = synth.gen_layer(cfg)
    layer.tid2eid[:, 1] = 16
    dl = qm.DeviceLayer.from_host(layer)
    ws = dl.workspace(cfg.T)
    tok = torch.from_numpy(synth.gen_token_ids(cfg, 0)).cuda()
    qm.forward(dl, xdev(synth.gen_x(cfg, 0)), tok, ws=ws)
    assert qm.device_error(ws) & _lib.MOE_DEVERR_HASH_ID


def test_permute_flags_bad_expert_ids():
    ids = torch.tensor([[0, 3], [9, 1], [2, -1]], dtype=torch.int32, device="cuda")
    ws = torch.empty(4096, dtype=torch.uint8, device="cuda")
    qm.workspace_init(ws)
    off, perm = qm.permute(ids, 4, ws)
    assert qm.device_error(ws) & _lib.MOE_DEVERR_EXPERT_ID
    p = perm.cpu().numpy()
    assert sorted(p.tolist()) == list(range(6))   # still a permutation
    assert off.cpu().numpy()[-1] == 6


# (4096, 256): perm staged in LDS, ids kept in registers; (6000, 256): too
# large for either (global scatter, ids reloaded for the fifth batch)
@pytest.mark.parametrize("T,E", [(1, 256), (700, 64), (4096, 256), (1500, 1000), (2000, 1024), (6000, 256)])
def test_permute_large_and_wide(T, E):
    rng = np.random.default_rng(T + E)
    k = 6
    ids_np = rng.integers(0, E, size=(T, k)).astype(np.int32)
    ws = torch.empty(4096, dtype=torch.uint8, device="cuda")
    qm.workspace_init(ws)
    off, perm = qm.permute(torch.from_numpy(ids_np).cuda(), E, ws)
    o, p = stable_sort_perm(ids_np, E)
    assert np.array_equal(off.cpu().numpy(), o) and np.array_equal(perm.cpu().numpy(), p)
    assert qm.device_error(ws) == 0


def test_single_token_repeatable():
    """One token per step: the gate/up launch hands rows to its waves
    dynamically, so which wave computes a row varies from call to call; the
    outputs must still be identical bit for bit (repeated calls, other inputs
    in between, a fresh workspace)."""
    cfg = variant("decode", "rep1", 221, T=1, d=4096, I=256, E=64, I_shared=256)
    dl = qm.DeviceLayer.from_host(synth.gen_layer(cfg))
    xs = [xdev(synth.gen_x(cfg, s)) for s in range(3)]
    ws = dl.workspace(1)
    first = [qm.forward(dl, x, out_dtype="f32", ws=ws).clone() for x in xs]
    for _ in range(8):
        for x, ref in zip(xs, first):
            assert torch.equal(qm.forward(dl, x, out_dtype="f32", ws=ws), ref)
    fresh = dl.workspace(1)
    assert torch.equal(qm.forward(dl, xs[0], out_dtype="f32", ws=fresh), first[0])
    torch.cuda.synchronize()
    assert qm.device_error(ws) == 0


def test_deterministic_with_poisoned_workspace():
    cfg = variant("mixed", "det", 207, T=16, d=512, I=256, E=32, I_shared=256)
    layer = synth.gen_layer(cfg)
    dl = qm.DeviceLayer.from_host(layer)
    x = xdev(synth.gen_x(cfg, 0))
    clean = dl.workspace(cfg.T)
    a = qm.forward(dl, x, out_dtype="f32", ws=clean)
    ws = torch.full((dl.workspace_size(cfg.T),), 0xFF, dtype=torch.uint8, device="cuda")
    qm.workspace_init(ws)
    b = qm.forward(dl, x, out_dtype="f32", ws=ws)
    c = qm.forward(dl, x, out_dtype="f32", ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(b, c)
    assert qm.device_error(ws) == 0


@pytest.mark.parametrize("cfg,expect", [
    (variant("decode", "disp_dec", 213, T=2, d=512, I=256, E=32, I_shared=256),
     ["dec_router", "dec_gateup", "dec_down_combine"]),
    (variant("decode", "disp_dec1", 220, T=1, d=512, I=256, E=32, I_shared=256),
     ["dec_router", "dec_gateup", "dec_down_combine"]),
    (variant("decode", "disp_dec1_k8", 225, T=1, d=512, I=256, E=32, top_k=8, I_shared=256),
     ["dec_router", "dec_gateup", "dec_down_combine"]),
    (variant("hash", "disp_hash_dec1", 226, T=1, d=512, I=256, E=64, vocab=1000),
     ["dec_router", "dec_gateup", "dec_down_combine"]),
    (variant("mixed", "disp_mixed_gemv", 214, T=20, d=512, I=256, E=128, top_k=4, I_shared=256),
     ["router_logits", "router_topk", "permute", "shared_gateup_mfma", "routed_gateup", "shared_down_mfma",
      "routed_down", "combine"]),
    (variant("mixed", "disp_mixed_mfma", 215, T=64, d=512, I=256, E=16, top_k=4, I_shared=256),
     ["router_logits", "router_topk", "permute", "shared_gateup_mfma", "routed_gateup_mfma", "shared_down_mfma",
      "routed_down_mfma", "combine"]),
    (variant("mixed", "disp_shared_split", 219, T=16, d=2048, I=128, E=8, top_k=2, I_shared=1024),
     ["router_logits", "router_topk", "permute", "shared_gateup_mfma", "shared_swiglu", "routed_gateup_mfma",
      "shared_down_mfma", "shared_sum", "routed_down_mfma", "combine"]),
    (variant("mixed", "disp_shared_gemv", 218, T=7, d=512, I=256, E=128, top_k=4, I_shared=256),
     ["router_logits", "router_topk", "permute", "shared_gateup", "routed_gateup", "shared_down", "routed_down",
      "combine"]),
    (variant("hash", "disp_hash_gemv", 216, T=40, d=512, I=256, E=64, vocab=1000),
     ["router_hash", "permute", "routed_gateup", "routed_down", "combine"]),
    (variant("hash", "disp_hash_fused", 224, T=2, d=512, I=256, E=64, vocab=1000),
     ["dec_router", "dec_gateup", "dec_down_combine"]),
    (variant("prefill", "disp_mxfp4", 217, T=64, d=512, I=256, E=8, top_k=2, bias_kind="normal"),
     ["router_logits", "router_topk", "permute", "routed_gateup_mfma", "routed_down_mfma", "combine"]),
    (variant("mxfp8", "disp_mxfp8_mfma", 222, T=40, d=512, I=256, E=8, top_k=2),
     ["router_logits", "router_topk", "permute", "routed_gateup_mfma", "routed_down_mfma", "combine"]),
    (variant("mxfp8", "disp_mxfp8_gemv", 223, T=6, d=512, I=256, E=32, top_k=4),
     ["router_logits", "router_topk", "permute", "routed_gateup", "routed_down", "combine"]),
], ids=lambda v: v.name if hasattr(v, "name") else "")
def test_dispatch_picks_expected_kernels(cfg, expect):
    """Which kernels a step runs: the fused path for up to 4 tokens (top-k or
    hash routing); the streaming GEMV under one token per expert (2/3-bit) or four (4-bit); the
    matrix-core grouped GEMM above that; the shared expert on the matrix cores
    from 8 tokens, its K split over workgroups (with finishers) while its
    tiles are few."""
    layer = synth.gen_layer(cfg)
    dl = qm.DeviceLayer.from_host(layer)
    x = xdev(synth.gen_x(cfg, 0))
    tok = synth.gen_token_ids(cfg, 0)
    tok = None if tok is None else torch.from_numpy(tok).to("cuda")
    ws = dl.workspace(cfg.T)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(32)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    out = torch.empty((cfg.T, cfg.d), dtype=torch.float32, device="cuda")
    names = qm.forward_probed(dl, x, tok, out, ws, evs)
    torch.cuda.synchronize()
    assert names == expect


def test_forward_probed_matches_forward_and_times_each_kernel():
    """The probed step gives the same output; every kernel gets its own event
    pair with a positive duration, and a too-short event list is rejected."""
    for cfg in (variant("decode", "probe_dec", 211, T=2, d=512, I=256, E=32, I_shared=256),
                variant("prefill", "probe_pf", 212, T=64, d=512, I=256, E=8, top_k=2, bias_kind="normal")):
        layer = synth.gen_layer(cfg)
        dl = qm.DeviceLayer.from_host(layer)
        x = xdev(synth.gen_x(cfg, 0))
        ws = dl.workspace(cfg.T)
        ref = qm.forward(dl, x, ws=ws, out_dtype="f32").clone()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(32)]
        for e in evs:
            e.record()
        torch.cuda.synchronize()
        out = torch.empty((cfg.T, cfg.d), dtype=torch.float32, device="cuda")
        names = qm.forward_probed(dl, x, None, out, ws, evs)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert names and all(isinstance(n, str) and n for n in names)
        assert all(evs[2 * i].elapsed_time(evs[2 * i + 1]) > 0 for i in range(len(names)))
        if len(names) > 1:
            with pytest.raises(RuntimeError):
                qm.forward_probed(dl, x, None, out, ws, evs[:2])
            torch.cuda.synchronize()
