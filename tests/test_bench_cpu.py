"""bench.py's host-side parts, on the CPU: the multi-GPU refusal, the
algorithmic byte and flop model the roofline uses, and the rule that stored
counter readings are reported only for the kernel sources they were taken on."""
import json
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


class _Proj:
    def __init__(self, rows, cols, bits, group, fmt="affine"):
        self.rows, self.cols, self.bits, self.group, self.fmt = rows, cols, bits, group, fmt

    def nbytes_per_expert(self):
        codes = self.rows * self.cols * self.bits // 8
        per_group = 1 if self.fmt == "mxfp4" else 4  # e8m0 byte, or fp16 scale + fp16 bias
        return codes + self.rows * (self.cols // self.group) * per_group


class _Experts:
    def __init__(self, gate, up, down):
        self.gate, self.up, self.down = gate, up, down

    def nbytes_per_expert(self):
        return sum(p.nbytes_per_expert() for p in (self.gate, self.up, self.down))


class _Layer:
    def __init__(self, cfg):
        f = cfg.gate_up
        g = _Proj(cfg.I, cfg.d, f.bits, f.group, f.fmt)
        dn = _Proj(cfg.d, cfg.I, cfg.down.bits, cfg.down.group, cfg.down.fmt)
        self.routed = _Experts(g, g, dn)
        if cfg.shared is not None:
            s = cfg.shared
            sg = _Proj(cfg.I_shared, cfg.d, s.bits, s.group, s.fmt)
            self.shared = _Experts(sg, sg, _Proj(cfg.d, cfg.I_shared, s.bits, s.group, s.fmt))
        else:
            self.shared = None


def test_byte_model_matches_the_layer_sizes():
    cfg = synth.config("decode")
    dl = _Layer(cfg)
    # 4-bit g64 routed expert: gate+up 9,437,184 B, down 4,718,592 B; shared 8-bit g64: 26,738,688 B
    assert bench.kernel_bytes("dec_gateup", cfg, dl, 1, 6) - 6 * 9437184 < 64 * 1024
    assert dl.routed.down.nbytes_per_expert() == 4718592
    assert dl.shared.nbytes_per_expert() == 17825792 + 8912896
    step = bench.step_bytes(cfg, dl, 1, 6)
    assert abs(step - 115.9e6) < 0.1e6  # touched experts + shared + router + x/out


def test_mfma_flops_and_bound_choice():
    pf, hs = synth.config("prefill"), synth.config("hash")
    assert bench.kernel_flops("routed_gateup_mfma", pf, pf.T) == 2.0 * pf.T * pf.top_k * pf.d * 2 * pf.I
    assert bench.kernel_flops("routed_down_mfma", pf, pf.T) == 2.0 * pf.T * pf.top_k * pf.I * pf.d
    assert bench.kernel_flops("dec_gateup", pf, 1) is None
    # prefill gate/up is matrix-core bound, the hash-routed one is HBM bound
    for cfg, mfma in ((pf, True), (hs, False)):
        fl = bench.kernel_flops("routed_gateup_mfma", cfg, cfg.T)
        by = bench.kernel_bytes("routed_gateup_mfma", cfg, _Layer(cfg), cfg.T, cfg.E)
        assert (fl / (bench.MFMA_BF16_PEAK_TFLOPS * 1e12) >= by / (bench.HBM_PEAK_GBS * 1e9)) == mfma


def test_stored_traffic_needs_the_same_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"decode": {"kernel": "dec_gateup", "fetch_kib": 1000.0, "write_kib": 10.0, "fetch_scale": 2.0,
                      "write_scale": 1.0, "source_hash": bench.source_hash()}}
    (prof / "hbm_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda: rec["decode"]["source_hash"])
    assert bench.measured_traffic("decode", "dec_gateup") == 1000 * 1024 * 2 + 10 * 1024
    assert bench.measured_traffic("decode", "dec_down_combine") is None
    assert bench.measured_traffic("prefill", "routed_gateup_mfma") is None
    monkeypatch.setattr(bench, "source_hash", lambda: "changed")
    assert bench.measured_traffic("decode", "dec_gateup") is None
