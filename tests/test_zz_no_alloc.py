"""moe_forward_noalloc (the library's own per-GPU workspace) against
moe_forward (a caller workspace), through the C ABI: bit-identical outputs
on two calls in a row, the second with fewer tokens, on the general and the
fused small-batch paths, top-k and hash routing; sizes beyond the static
workspace are refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import quantized_sparse_moe_amd as qm
import synth
from quantized_sparse_moe_amd import _lib
from synth import variant
from tests._gpu import xdev

pytestmark = pytest.mark.gpu

CASES = [
    variant("mixed", "na_mixed", 190, T=48, d=512, I=256, E=32, top_k=4, I_shared=256),
    variant("decode", "na_decode", 191, T=40, d=1024, I=256, E=64, top_k=6, I_shared=256),
    variant("hash", "na_hash", 192, T=64, d=512, I=256, E=16, vocab=700),
    variant("prefill", "na_mxfp4", 193, T=160, d=256, I=128, E=8, top_k=2, bias_kind="normal"),
]


def _both(dl, cfg, T, out_dtype):
    x = xdev(synth.gen_x(cfg, T, T=T))
    tok = synth.gen_token_ids(cfg, T, T=T)
    tok = None if tok is None else torch.from_numpy(tok).cuda()
    dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    ref = qm.forward(dl, x, tok, out=torch.empty((T, cfg.d), dtype=dt, device="cuda"), ws=dl.workspace(T))
    got = torch.full((T, cfg.d), float("nan"), dtype=dt, device="cuda")
    qm.forward_noalloc(dl, x, tok, got)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_noalloc_equals_forward(cfg):
    dl = qm.DeviceLayer.from_host(synth.gen_layer(cfg))
    for T, out_dtype in [(cfg.T, "f32"), (max(1, cfg.T // 3), "f32"), (3, "bf16"), (1, "f32")]:
        ref, got = _both(dl, cfg, T, out_dtype)
        assert torch.equal(ref, got), (cfg.name, T, out_dtype)
        assert torch.isfinite(got.float()).all()


def test_noalloc_refuses_sizes_beyond_its_workspace():
    cfg = variant("tiny", "na_big", 194, T=4)
    dl = qm.DeviceLayer.from_host(synth.gen_layer(cfg))
    T = 40000                                  # y_slot alone is 40000 * 2 * 256 * 4 bytes > 64 MiB
    assert dl.workspace_layout(T)["total"] > 64 << 20
    x = torch.zeros((1, cfg.d), dtype=torch.int16, device="cuda")
    out = torch.zeros((1, cfg.d), dtype=torch.float32, device="cuda")
    st = _lib.load().moe_forward_noalloc(ctypes.byref(dl.c), ctypes.c_void_p(x.data_ptr()), None, T,
                                         _lib.MOE_OUT_F32, ctypes.c_void_p(out.data_ptr()),
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == _lib.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
