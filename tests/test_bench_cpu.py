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
    # a single token's gate/up launch also streams the shared expert's down rows
    # (8-bit g64, 8,912,896 B), which its down launch then only adds
    gu1 = bench.kernel_bytes("dec_gateup", cfg, dl, 1, 6)
    assert 0 <= gu1 - (6 * 9437184 + 8912896) < 64 * 1024
    assert 0 <= bench.kernel_bytes("dec_down_combine", cfg, dl, 1, 6) - 6 * 4718592 < 64 * 1024
    # over four tokens the gate/up launch streams only the routed gate/up rows
    assert 0 <= bench.kernel_bytes("dec_gateup", cfg, dl, 4, 6) - 6 * 9437184 < 256 * 1024
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


def _write_counter_csv(path, rows):
    """A rocprofv3 counter-collection CSV: one row per (dispatch, counter)."""
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w") as f:
        f.write("Correlation_Id,Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for disp, kernel, counters in rows:
            for name, v in counters.items():
                f.write(f'{disp},{disp},"{kernel}",{name},{v}\n')


def _counters_for(read_bytes, write_bytes, req=128):
    """Counter values of a dispatch that reads/writes the given bytes in
    requests of `req` bytes (128, 64 or 32), as the formulas read them."""
    n = read_bytes // req
    return ({"TCC_EA0_RDREQ_sum": n, "TCC_EA0_RDREQ_32B_sum": n if req == 32 else 0,
             "TCC_BUBBLE_sum": n if req == 128 else 0, "TCC_EA0_RDREQ_DRAM_32B_sum": read_bytes // 32},
            {"TCC_EA0_WRREQ_sum": write_bytes // 64, "TCC_EA0_WRREQ_64B_sum": write_bytes // 64,
             "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum": write_bytes // 32, "TCC_EA0_RDREQ_DRAM_sum": n})


def test_counter_ingestion_calibrates_and_records(tmp_path, monkeypatch):
    """Ingestion checks the byte formulas on the three streams of known
    traffic, then records every kernel's bytes per launch keyed by the label
    moe_forward_probed gives it; the readings serve only the same sources."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_PATH", str(prof / "hbm_traffic.json"))
    monkeypatch.setattr(bench, "source_hash", lambda: "sources-of-this-run")
    C = bench.CAL_BYTES
    # the 32-of-128-byte stream moves whole lines at DRAM (its 32-byte requests become 128-byte fetches)
    streams = [("void qsmoe::k_probe_read<0>(unsigned int const*, unsigned long, unsigned int*)", C, 0, 128),
               ("void qsmoe::k_probe_read<1>(unsigned int const*, unsigned long, unsigned int*)", C, 0, 128),
               ("void qsmoe::k_probe_write(unsigned int*, unsigned long)", 0, C, 128)]
    kernels = [("void qsmoe::k_dec_gateup1<0, 4, 2>(qsmoe::DecodeArgs)", 60_000_000, 30_000, 128),
               ("void qsmoe::k_dec_down_combine<0, 4, 6, true>(qsmoe::DecodeArgs)", 38_000_000, 16_384, 64)]
    for run, rows in (("calibrate", streams), ("decode", kernels)):
        for p_, idx in (("_p1", 0), ("_p2", 1)):
            _write_counter_csv(tmp_path / "out" / (run + p_) / "host" / "run_counter_collection.csv",
                               [(d, k, _counters_for(r, w, q)[idx]) for d, (k, r, w, q) in enumerate(rows)])
    bench.ingest_counters(str(tmp_path / "out"))
    rec = json.loads((prof / "hbm_traffic.json").read_text())
    assert rec["validated"] and rec["read_formula_max_error"] <= 0.05
    dec = rec["workloads"]["decode"]
    assert set(dec) == {"k_dec_gateup1<0, 4, 2>", "k_dec_down_combine<0, 4, 6, true>"}
    g = dec["k_dec_gateup1<0, 4, 2>"]
    assert abs(g["read_bytes"] - 60_000_000) < 128
    assert (prof / "hbm_traffic.md").exists()
    cfg = synth.config("decode")
    assert bench.measured_traffic("decode", "dec_gateup", cfg) == g["read_bytes"] + g["write_bytes"]
    assert bench.measured_traffic("decode", "dec_router", cfg) is None
    monkeypatch.setattr(bench, "source_hash", lambda: "changed")
    assert bench.measured_traffic("decode", "dec_gateup", cfg) is None


def test_rocprof_names_match_probe_labels_by_format():
    """The routed experts' kernel, not the shared expert's, answers for a label."""
    key = bench.kernel_key
    assert key("void qsmoe::k_mfma_affine<true, 2, 128, 16, 0>(qsmoe::MfmaArgs)") == "k_mfma_affine<true, 2, 128, 16, 0>"
    assert key("void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<int>>(int, ...)") is None
    mixed, prefill, mx8 = synth.config("mixed"), synth.config("prefill"), synth.config("mxfp8")
    m = bench.kernel_matches
    assert m("routed_gateup_mfma", mixed, "k_mfma_affine<true, 2, 128, 16, 0>")
    assert not m("routed_gateup_mfma", mixed, "k_mfma_affine<true, 8, 64, 16, 0>")     # the shared expert
    assert m("routed_down_mfma", mixed, "k_mfma_affine<false, 3, 128, 16, 0>")
    assert m("routed_gateup_mfma", prefill, "k_mfma_mxfp4_w<true, 4>")
    assert not m("routed_gateup_mfma", prefill, "k_mfma_mxfp4_w<false, 4>")
    assert m("routed_down_mfma", mx8, "k_mfma_affine<false, 8, 32, 16, 2>")
    assert m("routed_gateup_mfma", mx8, "k_mfma_affine<true, 8, 32, 32, 2>")
    assert not m("routed_gateup_mfma", mx8, "k_mfma_affine<true, 8, 32, 32, 0>")
    assert m("routed_gateup", mixed, "k_ffn_stream<0, 2, 2, 1, true>")
    assert not m("routed_gateup", mixed, "k_ffn_stream<0, 8, 2, 1, true>")
    assert m("dec_gateup", mixed, "k_dec_gateup1<0, 2, 2>") and m("dec_router", mixed, "k_dec_router<1, 2, 1>")
