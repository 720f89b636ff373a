"""Every expert kernel path on weights made by the plain min/max quantiser
(bias = the group's minimum, independent of the scale), not the generator's
centred bias = -2^(b-1) scale: the affine epilogues' bias term then carries a
value of its own on the streaming GEMV, the fused small-batch kernels, the
matrix-core GEMMs and the K-split shared expert, for 2-, 3-, 4- and 8-bit
codes. Each case asserts which kernels moe_forward launched, then runs the
full parity check (routing, outputs, h, down projection and combine)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_sparse_moe_amd as qm
import synth
from synth import FormatSpec, variant
from synth.configs import AFF2_G128, AFF3_G128, AFF8_G64
from tests._gpu import xdev
from tests.test_gpu_parity import check_layer

pytestmark = pytest.mark.gpu


def quantised_layer(cfg):
    """The seeded layer with every affine projection replaced by the oracle's
    min/max quantisation of seeded bf16 N(0, 0.02) weights."""
    layer = synth.gen_layer(cfg)
    idx = 0
    sets = [(layer.routed, cfg.E)] + ([(layer.shared, 1)] if layer.shared is not None else [])
    for ew, n in sets:
        for q in (ew.gate, ew.up, ew.down):
            if q.spec.fmt != "affine":
                continue
            for e in range(n):
                w = synth.gen_bf16_weights(cfg.seed, idx, q.rows, q.cols)
                idx += 1
                q.codes[e], q.scales[e], q.biases[e] = oracle.quantize_affine(w, q.spec.bits, q.spec.group)
    return layer


def launched(dl, cfg):
    x = xdev(synth.gen_x(cfg, 0))
    tok = synth.gen_token_ids(cfg, 0)
    tok = None if tok is None else torch.from_numpy(tok).cuda()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(32)]
    for e in evs:
        e.record()
    out = torch.empty((cfg.T, cfg.d), dtype=torch.float32, device="cuda")
    names = qm.forward_probed(dl, x, tok, out, dl.workspace(cfg.T), evs)
    torch.cuda.synchronize()
    return set(names)


AFF4_G32, AFF4_G64, AFF4_G128 = FormatSpec("affine", 4, 32), FormatSpec("affine", 4, 64), FormatSpec("affine", 4, 128)
AFF3_G64, AFF8_G32, AFF8_G128 = FormatSpec("affine", 3, 64), FormatSpec("affine", 8, 32), FormatSpec("affine", 8, 128)
GEMV = {"routed_gateup", "routed_down"}
MFMA = {"routed_gateup_mfma", "routed_down_mfma"}
FUSED = {"dec_router", "dec_gateup", "dec_down_combine"}

CASES = [
    (variant("decode", "q_gemv4", 170, T=5, d=512, I=256, E=32, top_k=2, I_shared=256),
     GEMV | {"shared_gateup", "shared_down"}),
    (variant("mixed", "q_gemv23", 171, T=6, d=512, I=256, E=64, top_k=4, I_shared=256),
     GEMV | {"shared_gateup", "shared_down"}),
    (variant("mixed", "q_gemv8", 172, T=6, d=512, I=256, E=32, top_k=2, gate_up=AFF8_G64, down=AFF8_G128,
             shared=None), GEMV),
    (variant("decode", "q_fused4_t1", 173, T=1, d=512, I=256, E=32, top_k=4, I_shared=256), FUSED),
    (variant("decode", "q_fused4_t2", 174, T=2, d=512, I=256, E=32, top_k=4, I_shared=256), FUSED),
    (variant("decode", "q_fused4_t3", 175, T=3, d=512, I=256, E=32, top_k=4, I_shared=256), FUSED),
    (variant("decode", "q_fused4_t4", 176, T=4, d=512, I=256, E=32, top_k=4, I_shared=256), FUSED),
    (variant("mixed", "q_fused23_t1", 177, T=1, d=1024, I=256, E=64, top_k=6, I_shared=256), FUSED),
    (variant("mixed", "q_fused23_t1_k8", 185, T=1, d=1024, I=256, E=64, top_k=8, I_shared=256), FUSED),
    (variant("mixed", "q_fused8_t2", 178, T=2, d=512, I=256, E=16, top_k=2, gate_up=AFF8_G64, down=AFF8_G32,
             I_shared=256), FUSED),
    (variant("prefill", "q_mfma4", 179, T=96, d=512, I=256, E=8, top_k=2, bias_kind="normal", gate_up=AFF4_G64,
             down=AFF4_G128, shared=AFF8_G64, I_shared=256), MFMA | {"shared_gateup_mfma", "shared_down_mfma"}),
    (variant("prefill", "q_mfma4_g32", 180, T=64, d=512, I=256, E=8, top_k=2, bias_kind="normal", gate_up=AFF4_G32,
             down=AFF4_G32), MFMA),
    (variant("mixed", "q_mfma23", 181, T=64, d=512, I=256, E=16, top_k=4, gate_up=AFF2_G128, down=AFF3_G64,
             I_shared=256), MFMA | {"shared_gateup_mfma", "shared_down_mfma"}),
    (variant("mixed", "q_mfma8", 182, T=64, d=512, I=256, E=8, top_k=4, gate_up=AFF8_G128, down=AFF8_G32,
             I_shared=256), MFMA),
    (variant("mixed", "q_mfma3_g128", 183, T=40, d=768, I=384, E=8, top_k=3, gate_up=AFF3_G128, down=AFF2_G128,
             shared=None), MFMA),
    (variant("mixed", "q_shared_splitk", 184, T=16, d=2048, I=128, E=8, top_k=2, I_shared=1024),
     {"shared_gateup_mfma", "shared_swiglu", "shared_down_mfma", "shared_sum"}),
]


@pytest.mark.parametrize("cfg,paths", CASES, ids=[c.name for c, _ in CASES])
def test_min_bias_weights_on_every_path(cfg, paths):
    layer = quantised_layer(cfg)
    # the quantiser's biases are the group minima, not tied to the scales
    q = layer.routed.gate
    if q.spec.fmt == "affine":
        ratio = q.biases.astype(np.float64) / q.scales.astype(np.float64)
        assert np.ptp(ratio) > 1.0
    dl = qm.DeviceLayer.from_host(layer)
    names = launched(dl, cfg)
    assert paths <= names, f"{cfg.name}: expected {sorted(paths)} among {sorted(names)}"
    worst = max(check_layer(cfg, layer, dl, s) for s in range(min(cfg.steps, 2)))
    print(f"{cfg.name}: kernels {sorted(names)}, max rel err {worst:.2e}")
