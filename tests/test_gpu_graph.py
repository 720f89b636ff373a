"""HIP-graph capture of whole steps (the way bench.py times them): a graph of
several steps, replayed several times with the program's own eager work and
synchronisations in between, gives on every replay exactly the eager outputs.
Covers the fused decode path (top-k and hash routed), the GEMV path and the
matrix-core paths (MXFP4, affine, MXFP8)."""
import numpy as np
import pytest
import torch

import quantized_sparse_moe_amd as qm
import synth
from synth import variant
from tests._gpu import xdev

pytestmark = pytest.mark.gpu

CASES = [
    variant("decode", "graph_dec", 301, T=1, d=512, I=256, E=32, I_shared=256, steps=3),
    variant("mixed", "graph_gemv", 302, T=16, d=512, I=256, E=32, I_shared=256, steps=3),
    variant("prefill", "graph_mx", 303, T=128, d=512, I=256, E=8, top_k=2, bias_kind="normal", steps=3),
    variant("hash", "graph_aff", 304, T=48, d=512, I=256, E=16, vocab=1000, steps=3),
    variant("hash", "graph_hash_dec", 305, T=1, d=512, I=256, E=16, vocab=1000, steps=3),
    variant("mxfp8", "graph_mxfp8", 306, T=64, d=512, I=256, E=16, steps=3),
]


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_graph_replays_equal_eager(cfg):
    layer = synth.gen_layer(cfg)
    dl = qm.DeviceLayer.from_host(layer)
    xs = [xdev(synth.gen_x(cfg, s)) for s in range(cfg.steps)]
    toks = ([torch.from_numpy(synth.gen_token_ids(cfg, s)).cuda() for s in range(cfg.steps)]
            if cfg.route == "hash" else [None] * cfg.steps)
    ws = dl.workspace(cfg.T)
    eager = [qm.forward(dl, xs[s], toks[s], ws=ws, out_dtype="f32").clone() for s in range(cfg.steps)]
    outs = [torch.empty((cfg.T, cfg.d), dtype=torch.float32, device="cuda") for _ in range(cfg.steps)]
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            for s in range(cfg.steps):
                qm.forward(dl, xs[s], toks[s], ws=ws, out=outs[s])
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()

    scratch = torch.empty(1 << 20, device="cuda")
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for s in range(cfg.steps):
            assert torch.equal(outs[s], eager[s]), (rep, s)
        # the program's own eager work between replays, including an eager step
        scratch.normal_()
        again = qm.forward(dl, xs[rep % cfg.steps], toks[rep % cfg.steps], ws=ws, out_dtype="f32")
        torch.cuda.synchronize()
        assert torch.equal(again, eager[rep % cfg.steps])
    assert qm.device_error(ws) == 0
