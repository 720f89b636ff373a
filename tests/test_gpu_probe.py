"""The measurement kernels behind the benchmark's calibration: the stream reads
touch exactly the bytes they claim (the XOR of every word read equals the
host's), the stream write writes every 16-byte piece once, and the MFMA loop
runs every wave and records a rising shader clock and wall clock."""
import numpy as np
import pytest
import torch

import quantized_sparse_moe_amd as qm

pytestmark = pytest.mark.gpu


def test_stream_reads_cover_exactly_their_bytes():
    rng = np.random.default_rng(3)
    host = rng.integers(0, 2 ** 32, size=(1 << 22), dtype=np.uint32)          # 16 MiB
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    for mode, want in [(0, np.bitwise_xor.reduce(host)),
                       (1, np.bitwise_xor.reduce(host.reshape(-1, 32)[:, :8].ravel()))]:
        sink = torch.full((2048,), -1, dtype=torch.int32, device="cuda")
        qm.probe_stream(buf, mode, sink)
        torch.cuda.synchronize()
        assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == want, mode


def test_stream_write_covers_every_piece():
    buf = torch.full((1 << 20,), -1, dtype=torch.int32, device="cuda")        # 4 MiB
    qm.probe_stream(buf, 2)
    got = buf.cpu().numpy().view(np.uint32).reshape(-1, 4)
    assert np.array_equal(got, np.repeat(np.arange(got.shape[0], dtype=np.uint32)[:, None], 4, axis=1))


def test_mfma_probe_runs_every_wave():
    out = torch.zeros(5, dtype=torch.int64, device="cuda")
    qm.probe_mfma(64, 200, out)
    torch.cuda.synchronize()
    c0, c1, w0, w1, waves = out.cpu().tolist()
    assert c1 > c0 and w1 > w0 and waves == 64 * 4
