"""The fused mHC Sinkhorn kernel (moe_mhc_sinkhorn) against the float64
oracle: every matrix size, round counts, eps, ragged token counts, in place,
shifted logits; fp32 against float64 within 1e-5 (relative to each entry,
entries are in (0, 1])."""
import numpy as np
import pytest
import torch

import oracle
import quantized_sparse_moe_amd as qm

pytestmark = pytest.mark.gpu


def _logits(seed, T, n, std=1.0, shift=0.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, n, n)) * std + shift).astype(np.float32)


@pytest.mark.parametrize("n", [2, 4, 8])
@pytest.mark.parametrize("iters,eps", [(0, 0.0), (1, 0.0), (10, 0.0), (50, 1e-6)])
def test_sinkhorn_matches_oracle(n, iters, eps):
    l = _logits(n * 100 + iters, 1000, n, std=1.5)
    got = qm.mhc_sinkhorn(torch.from_numpy(l).cuda(), iters, eps).cpu().numpy()
    ref = oracle.mhc_sinkhorn(l, iters, eps)
    assert np.all(np.abs(got - ref) <= 1e-5 * ref + 1e-7)


@pytest.mark.parametrize("T", [1, 255, 257, 4097])
def test_sinkhorn_ragged_counts_and_in_place(T):
    l = _logits(T, T, 4)
    d = torch.from_numpy(l).cuda()
    ref = oracle.mhc_sinkhorn(l, 10)
    out = qm.mhc_sinkhorn(d, 10, out=d)            # in place
    assert out.data_ptr() == d.data_ptr()
    got = d.cpu().numpy()
    assert np.all(np.abs(got - ref) <= 1e-5 * ref + 1e-7)
    assert np.allclose(got.sum(-1), 1.0, atol=2e-6)


def test_sinkhorn_large_logits_and_empty():
    l = _logits(7, 64, 4, std=3.0, shift=700.0)
    got = qm.mhc_sinkhorn(torch.from_numpy(l).cuda(), 10).cpu().numpy()
    ref = oracle.mhc_sinkhorn(l, 10)
    assert np.all(np.isfinite(got)) and np.all(np.abs(got - ref) <= 1e-5 * ref + 1e-7)
    assert qm.mhc_sinkhorn(torch.empty((0, 4, 4), device="cuda")).shape == (0, 4, 4)


def test_sinkhorn_graph_replays_equal_eager():
    """Several calls captured as one HIP graph (the way the op is timed),
    replayed three times with eager work in between: every replay gives the
    eager results bit for bit."""
    rng = np.random.default_rng(93)
    ls = [torch.from_numpy(rng.standard_normal((300, 4, 4)).astype(np.float32)).cuda() for _ in range(3)]
    eager = [qm.mhc_sinkhorn(l, 10, 0.0).clone() for l in ls]
    outs = [torch.empty_like(l) for l in ls]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            for l, o in zip(ls, outs):
                qm.mhc_sinkhorn(l, 10, 0.0, out=o)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    scratch = torch.empty(1 << 20, device="cuda")
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for i in range(len(ls)):
            assert torch.equal(outs[i], eager[i]), (rep, i)
        scratch.normal_()
        again = qm.mhc_sinkhorn(ls[rep], 10, 0.0)
        torch.cuda.synchronize()
        assert torch.equal(again, eager[rep])
