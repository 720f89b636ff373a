#!/usr/bin/env python3
"""Throughput of the routed-expert MoE layer on one MI355X.

Default run: batch-1 decode (T=1 token per step; d=4096, I=2048, E=256 routed
experts with affine 4-bit g64 weights, top-6, plus the always-on shared expert
in affine 8-bit g64; 64 seeded activation steps) as the headline record, with
the 4096-token MXFP4 prefill (Zipf-skewed routing, the matrix-core half of the
metric) as a sub-record in the same JSON line. A step is one moe_forward
(route, bucket, experts, combine) of one batch.

Timed region: K steps captured once in a HIP graph; the graph is replayed R
times (default 5), each replay between a torch.cuda.synchronize() on each
side and timed with events; ms_per_step is the median replay / K. Inputs and
weights are resident in HBM. Decode steps rotate over several device copies of
the layer so that no step finds its weights in the 256 MB Infinity Cache left
there by a recent step; separately, single cold steps each follow a 1 GiB
write that evicts the L2s and the Infinity Cache (median and p90 reported).

Also reported: the dominant kernel's roofline from HIP events that the
dispatches on the library's stream timestamp at kernel start and end
(moe_forward_probed); its HBM traffic from committed rocprofv3 counter
readings (validated against kernels of known traffic); the CPU oracle timed on
a bounded sample of the same workload on the host cores; and the measured
context of the peaks: streaming-read bandwidth, sustained shader clock and
dense bf16 MFMA rate on this GPU, and the host CPU model.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, MI355X
METRIC = "MoE-layer tokens/s + achieved HBM GB/s (decode) / MFMA % (prefill)"
TRAFFIC_PATH = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CAL_BYTES = 1 << 30          # bytes each calibration stream covers
FLUSH_BYTES = 1 << 30        # write before each cold step (L2s + 256 MB Infinity Cache)
WORKLOADS = ["decode", "tiny", "hash", "prefill", "mixed", "mxfp8", "stack43", "quantize", "sinkhorn"]


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=256)
    p.add_argument("--warmup", type=int, default=16)
    p.add_argument("--workload", default="decode", choices=WORKLOADS)
    p.add_argument("--copies", type=int, default=0, help="device copies of the layer to rotate over (0: auto)")
    p.add_argument("--replays", type=int, default=5, help="timed replays of the K-step graph (median reported)")
    p.add_argument("--cold-steps", type=int, default=64, help="decode: single steps each after a 1 GiB flush")
    p.add_argument("--no-prefill", action="store_true", help="default run: skip the prefill sub-record")
    p.add_argument("--no-context", action="store_true", help="skip the measured peaks and host description")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target length of the CPU oracle sample")
    p.add_argument("--eager", action="store_true", help="time eager launches instead of a graph replay")
    p.add_argument("--calibrate", action="store_true",
                   help="only run the three streams of known traffic (for the HBM byte counters)")
    p.add_argument("--ingest-counters", metavar="DIR",
                   help="turn rocprofv3 --pmc runs under DIR into profiles/hbm_traffic.json (no GPU needed)")
    return p.parse_args()


def workload_text(cfg) -> str:
    def fmt(f):
        if f.fmt in ("mxfp4", "mxfp8"):
            return f"{f.fmt} {'e2m1' if f.fmt == 'mxfp4' else 'e4m3'}+e8m0/32"
        return f"affine {f.bits}-bit g{f.group}"
    s = (f"{cfg.name}: T={cfg.T} tokens/step, d={cfg.d}, I={cfg.I}, E={cfg.E}, top-{cfg.top_k} "
         f"{'tid2eid hash' if cfg.route == 'hash' else 'sqrtsoftplus+bias'} routing, gate/up {fmt(cfg.gate_up)}, "
         f"down {fmt(cfg.down)}")
    if cfg.shared is not None:
        s += f", shared expert I={cfg.I_shared} {fmt(cfg.shared)}"
    return s + f", {cfg.steps} seeded activation batch(es)"


def kernel_bytes(name, cfg, dl, T, touched):
    """Algorithmic HBM bytes of one launch: the weights the kernel must read
    (touched experts only) plus its activation inputs and outputs."""
    k, d, E, I = cfg.top_k, cfg.d, cfg.E, cfg.I
    r = dl.routed
    sh = dl.shared
    tk = T * k
    if name == "router_logits":
        return E * d * 4 + T * d * 2 + T * E * 4
    if name == "router_topk":
        return T * E * 4 + E * 4 + tk * 8
    if name == "router_hash":
        return min(E, tk) * d * 4 + T * d * 2 + T * 4 + tk * 4 + tk * 8
    if name == "permute":
        return tk * 4 + (E + 1) * 4 + tk * 4
    if name in ("routed_gateup", "routed_gateup_mfma"):
        return touched * (r.gate.nbytes_per_expert() + r.up.nbytes_per_expert()) + T * d * 2 + tk * I * 2
    if name in ("routed_down", "routed_down_mfma"):
        return touched * r.down.nbytes_per_expert() + tk * I * 2 + tk * d * 4
    if name in ("shared_gateup", "shared_gateup_mfma"):
        return sh.gate.nbytes_per_expert() + sh.up.nbytes_per_expert() + T * d * 2 + T * cfg.I_shared * 2
    if name in ("shared_down", "shared_down_mfma"):
        return sh.down.nbytes_per_expert() + T * cfg.I_shared * 2 + T * d * 4
    # finishers of a K-split shared expert: one slice of fp32 partials in, the result out
    if name == "shared_swiglu":
        return T * cfg.I_shared * (2 * 4 + 2)
    if name == "shared_sum":
        return T * d * (4 + 4)
    if name == "combine":
        return tk * d * 4 + tk * 4 + (T * d * 4 if sh is not None else 0) + T * d * 2
    # fused small-batch path (a single token streams the shared expert's down
    # rows in its gate/up launch)
    sh_gu = sh.gate.nbytes_per_expert() + sh.up.nbytes_per_expert() + T * cfg.I_shared * 2 if sh is not None else 0
    sh_dn = sh.down.nbytes_per_expert() + T * cfg.I_shared * 2 if sh is not None else 0
    sh_dn_in_gu = T == 1 and d <= 4096
    gu = touched * (r.gate.nbytes_per_expert() + r.up.nbytes_per_expert()) + T * E * 12 + T * d * 2 + tk * I * 2
    if name == "dec_router":
        return E * d * 4 + T * d * 2 + T * E * 16 + sh_gu
    if name == "dec_gateup":
        return gu + tk * 8 + (sh_dn + T * d * 4 if sh_dn_in_gu else 0)
    if name == "dec_down_combine":
        sh_part = T * d * 4 if sh_dn_in_gu else sh_dn
        return touched * r.down.nbytes_per_expert() + sh_part + T * E * 4 + tk * I * 2 + T * d * 2
    raise KeyError(name)


def kernel_flops(name, cfg, T):
    """Algorithmic flops of one launch of an MFMA expert kernel (2 per
    multiply-add over every routed (token, expert) pair)."""
    tk = T * cfg.top_k
    if name == "routed_gateup_mfma":
        return 2.0 * tk * cfg.d * 2 * cfg.I
    if name == "routed_down_mfma":
        return 2.0 * tk * cfg.I * cfg.d
    if name == "shared_gateup_mfma":
        return 2.0 * T * cfg.d * 2 * cfg.I_shared
    if name == "shared_down_mfma":
        return 2.0 * T * cfg.I_shared * cfg.d
    return None


def step_bytes(cfg, dl, T, touched):
    """Algorithmic bytes of a whole step: touched routed experts, shared
    expert, router weights, activations in and out."""
    b = touched * dl.routed.nbytes_per_expert() + cfg.E * cfg.d * 4 + T * cfg.d * 2 * 2
    if dl.shared is not None:
        b += dl.shared.nbytes_per_expert()
    return b


def source_hash() -> str:
    """Hash of the kernel sources and the C ABI header: stored counter readings
    are used only for the exact sources they were taken on."""
    import hashlib
    h = hashlib.sha256()
    for sub in ("quantized_sparse_moe_amd/csrc", "include"):
        d = os.path.join(ROOT, sub)
        for name in sorted(os.listdir(d)):
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# HBM traffic from rocprofv3 counters
#
# Two --pmc passes per workload (4 L2-channel counters each):
READ_COUNTERS = ["TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_BUBBLE_sum", "TCC_EA0_RDREQ_DRAM_32B_sum"]
WRITE_COUNTERS = ["TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum", "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum",
                  "TCC_EA0_RDREQ_DRAM_sum"]
# Byte formulas from those counters (per dispatch):
READ_FORMULAS = {
    # requests by size: 128-byte (TCC_BUBBLE), 32-byte, the rest 64-byte
    "request_sizes": lambda c: (128 * c["TCC_BUBBLE_sum"] + 32 * c["TCC_EA0_RDREQ_32B_sum"]
                                + 64 * (c["TCC_EA0_RDREQ_sum"] - c["TCC_BUBBLE_sum"] - c["TCC_EA0_RDREQ_32B_sum"])),
    # DRAM read traffic counted in 32-byte units (a 64-byte request counts 2, a 128-byte one 4)
    "dram_32b_units": lambda c: 32 * c["TCC_EA0_RDREQ_DRAM_32B_sum"],
}
WRITE_FORMULAS = {
    "request_sizes": lambda c: (64 * c["TCC_EA0_WRREQ_64B_sum"]
                                + 32 * (c["TCC_EA0_WRREQ_sum"] - c["TCC_EA0_WRREQ_64B_sum"])),
    "dram_32b_units": lambda c: 32 * c["TCC_EA0_WRREQ_WRITE_DRAM_32B_sum"],
}


def kernel_key(kernel_name: str):
    """A library kernel's rocprofv3 name without namespace and argument list
    (e.g. "k_mfma_affine<true, 2, 128, 16, 0>"); None for other kernels."""
    n = kernel_name.replace("void ", "").replace("qsmoe::", "").strip()
    if not n.startswith("k_"):
        return None
    depth = 0
    for i, ch in enumerate(n):
        depth += ch == "<"
        depth -= ch == ">"
        if ch == "(" and depth == 0:
            return n[:i]
    return n


def _fmt_tag(f, gateup):
    """The kernel-name prefix of the routed experts' matrix-core kernel for format f."""
    gu = "true" if gateup else "false"
    if f.fmt == "mxfp4":
        return f"k_mfma_mxfp4"
    if f.fmt == "mxfp8":
        return f"k_mfma_affine<{gu}, 8, 32, "  # 16- or 32-token tiles, format 2 (checked below)
    return f"k_mfma_affine<{gu}, {f.bits}, "


def kernel_matches(label, cfg, key):
    """Does the kernel `key` (kernel_key) implement the probe label `label`
    for the routed experts of workload cfg?"""
    fixed = {"dec_router": "k_dec_router<", "dec_gateup": "k_dec_gateup", "dec_down_combine": "k_dec_down_combine<",
             "router_logits": "k_logits", "router_topk": "k_topk", "router_hash": "k_hash", "permute": "k_permute",
             "combine": "k_combine", "shared_swiglu": "k_swiglu_parts", "shared_sum": "k_sum_parts",
             "k_quantize_affine": "k_quantize_affine", "k_mhc_sinkhorn": "k_mhc_sinkhorn"}
    if label in fixed:
        return key.startswith(fixed[label])
    if label in ("routed_gateup_mfma", "routed_down_mfma"):
        gateup = label == "routed_gateup_mfma"
        f = cfg.gate_up if gateup else cfg.down
        tag = _fmt_tag(f, gateup)
        if f.fmt == "mxfp4":
            return key.startswith(tag) and ("<true" in key) == gateup
        if f.fmt == "mxfp8":
            return key.startswith(tag) and key.endswith(", 2>")
        return key.startswith(tag)
    if label in ("routed_gateup", "routed_down"):
        gateup = label == "routed_gateup"
        f = cfg.gate_up if gateup else cfg.down
        F = {"affine": 0, "mxfp4": 1, "mxfp8": 2}[f.fmt]
        return key.startswith(f"k_ffn_stream<{F}, {f.bits}, ") and key.endswith(", true>" if gateup else ", false>")
    return False


def _read_counter_csvs(d):
    """Mean counter value per (kernel, counter) over the dispatches in the
    rocprofv3 counter-collection CSVs under d; also the dispatch counts."""
    sums, counts = {}, {}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        per_dispatch = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                label = kernel_key(row["Kernel_Name"])
                if label is None:
                    continue
                key = (label, row["Dispatch_Id"])
                per_dispatch.setdefault(key, {})[row["Counter_Name"]] = float(row["Counter_Value"])
        for (label, _), ctr in per_dispatch.items():
            counts[label] = counts.get(label, 0) + 1
            for name, v in ctr.items():
                sums[(label, name)] = sums.get((label, name), 0.0) + v
    return {(l, n): v / counts[l] for (l, n), v in sums.items()}, counts


def ingest_counters(root):
    """Counter runs under root/<run>_p1 (read counters) and root/<run>_p2
    (write counters), run = calibrate or a workload: calibrate the byte
    formulas on the three streams of known traffic, then record the bytes per
    launch of every kernel of every workload (profiles/hbm_traffic.json) and a
    text summary (profiles/hbm_traffic.md)."""
    runs = sorted({os.path.basename(p)[:-3] for p in glob.glob(os.path.join(root, "*_p1"))})
    data = {}
    for r in runs:
        m1, c1 = _read_counter_csvs(os.path.join(root, r + "_p1"))
        m2, c2 = _read_counter_csvs(os.path.join(root, r + "_p2"))
        labels = sorted({l for l, _ in m1} & {l for l, _ in m2})
        data[r] = {l: ({n: m1[(l, n)] for n in READ_COUNTERS if (l, n) in m1},
                       {n: m2[(l, n)] for n in WRITE_COUNTERS if (l, n) in m2}, min(c1[l], c2[l])) for l in labels}
    cal = data.get("calibrate")
    if not cal:
        raise SystemExit(f"no calibrate_p1/_p2 runs under {root}")
    # known DRAM traffic: every byte of the dense streams; for the stream that
    # requests 32 bytes of each 128-byte line, whole lines (CAL_BYTES / 4
    # requested): HBM moves whole lines, as its run time beside the dense
    # read shows (context.stream_read_32b_of_128b_time_vs_dense)
    known = {"k_probe_read<0>": (CAL_BYTES, 0), "k_probe_read<1>": (CAL_BYTES, 0), "k_probe_write": (0, CAL_BYTES)}
    calib = {}
    for label, (want_r, want_w) in known.items():
        rd, wr, n = cal[label]
        calib[label] = {"known_read_bytes": want_r, "known_write_bytes": want_w, "dispatches": n,
                        "read": {f: fn(rd) for f, fn in READ_FORMULAS.items()},
                        "write": {f: fn(wr) for f, fn in WRITE_FORMULAS.items()}}

    def pick(kind, formulas, want_key, labels):
        best, err = None, None
        for f in formulas:
            e = max(abs(calib[l][kind][f] / calib[l][want_key] - 1.0) for l in labels)
            if err is None or e < err:
                best, err = f, e
        return best, err
    rf, rerr = pick("read", READ_FORMULAS, "known_read_bytes", ["k_probe_read<0>", "k_probe_read<1>"])
    wf, werr = pick("write", WRITE_FORMULAS, "known_write_bytes", ["k_probe_write"])
    valid = rerr <= 0.05 and werr <= 0.05
    out = {"calibration": calib, "read_formula": rf, "read_formula_max_error": rerr, "write_formula": wf,
           "write_formula_max_error": werr, "validated": valid, "source_hash": source_hash(),
           "read_counters": READ_COUNTERS, "write_counters": WRITE_COUNTERS, "workloads": {}}
    for r, kernels in data.items():
        if r == "calibrate":
            continue
        out["workloads"][r] = {l: {"read_bytes": READ_FORMULAS[rf](rd), "write_bytes": WRITE_FORMULAS[wf](wr),
                                   "dispatches": n, "counters": {**rd, **wr}} for l, (rd, wr, n) in kernels.items()}
    with open(TRAFFIC_PATH, "w") as f:
        json.dump(out, f, indent=1)
    lines = ["# HBM traffic per kernel launch from L2-to-fabric counters", "",
             "Two `rocprofv3 --pmc` passes per run, from the repository root on the MI355X box (`TMPDIR=/tmp`):", "",
             f"    rocprofv3 --pmc {' '.join(READ_COUNTERS)} --output-format csv -d OUT/RUN_p1 -o run -- python3 bench.py ARGS",
             f"    rocprofv3 --pmc {' '.join(WRITE_COUNTERS)} --output-format csv -d OUT/RUN_p2 -o run -- python3 bench.py ARGS",
             "    python3 bench.py --ingest-counters OUT", "",
             "ARGS: `--calibrate` for RUN = calibrate; `--workload RUN --steps 2 --warmup 1 --replays 1 "
             "--cold-steps 0 --no-prefill --no-context --no-cpu-baseline` for each workload.", "",
             "## Calibration on streams of known traffic (1 GiB each)", "",
             "Streams: `k_probe_read<0>` reads every byte of 1 GiB once (16 bytes per lane); `k_probe_read<1>` "
             "requests the first 32 bytes of every 128-byte line of 1 GiB (256 MiB requested, every line "
             "touched); `k_probe_write` writes every byte of 1 GiB once. Known DRAM traffic counts whole lines.", "",
             "| stream | known read | known write | " + " | ".join(f"read: {f}" for f in READ_FORMULAS) + " | "
             + " | ".join(f"write: {f}" for f in WRITE_FORMULAS) + " |",
             "|---|---|---|" + "---|" * (len(READ_FORMULAS) + len(WRITE_FORMULAS))]
    for l, c in calib.items():
        lines.append(f"| {l} | {c['known_read_bytes'] / 2**20:.0f} MiB | {c['known_write_bytes'] / 2**20:.0f} MiB | "
                     + " | ".join(f"{v / 2**20:.1f} MiB" for v in c["read"].values()) + " | "
                     + " | ".join(f"{v / 2**20:.1f} MiB" for v in c["write"].values()) + " |")
    lines += ["", f"Chosen: reads by `{rf}` (max error {100 * rerr:.1f} % on the two read streams), writes by "
              f"`{wf}` ({100 * werr:.1f} %); {'validated within 5 %' if valid else 'NOT validated (over 5 %)'}.", "",
              "## Bytes per launch (read + write) of each kernel", "",
              "| run | kernel | dispatches | read MB | write MB |", "|---|---|---|---|---|"]
    for r, ks in out["workloads"].items():
        for l, v in sorted(ks.items(), key=lambda kv: -kv[1]["read_bytes"]):
            lines.append(f"| {r} | `{l}` | {v['dispatches']} | {v['read_bytes'] / 1e6:.2f} | "
                         f"{v['write_bytes'] / 1e6:.2f} |")
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def measured_traffic(workload, label, cfg):
    """HBM bytes (read + write) per launch of the kernel `label` (for the
    routed experts of cfg) in `workload` from the committed counter readings,
    or None when there is none, the byte formulas did not validate, or the
    kernels changed since."""
    try:
        with open(TRAFFIC_PATH) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if not rec.get("validated") or rec.get("source_hash") != source_hash():
        return None
    hits = [v for k, v in rec.get("workloads", {}).get(workload, {}).items() if kernel_matches(label, cfg, k)]
    return hits[0]["read_bytes"] + hits[0]["write_bytes"] if len(hits) == 1 else None


def calibrate():
    """The three streams of known traffic: a dense 16-byte-per-lane read of
    1 GiB, a read of the first 32 bytes of every 128-byte line of 1 GiB, a
    dense write of 1 GiB (three launches each)."""
    import torch
    import quantized_sparse_moe_amd as qm
    qm.load()
    buf = torch.empty(CAL_BYTES // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(2048, dtype=torch.int32, device="cuda")
    for _ in range(3):
        qm.probe_stream(buf, 2)
        qm.probe_stream(buf, 0, sink)
        qm.probe_stream(buf, 1, sink)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_bytes": CAL_BYTES, "launches_per_stream": 3}))


# ---------------------------------------------------------------------------
# Context: the host, and the GPU's measured rates beside the nominal peaks

def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return 1


def context_info():
    """Streaming-read GB/s of a dense 4 GiB read (moe_probe_stream), the
    sustained shader clock and dense bf16 MFMA TFLOP/s of all CUs running
    V_MFMA_F32_32X32X16_BF16 chains (moe_probe_mfma), and the host."""
    import torch
    import quantized_sparse_moe_amd as qm
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    info = {"gpu": props.name, "compute_units": cus, "cpu_model": cpu_model(),
            "host_cpus": len(os.sched_getaffinity(0))}
    buf = torch.empty(1 << 30, dtype=torch.int32, device="cuda")          # 4 GiB
    sink = torch.zeros(2048, dtype=torch.int32, device="cuda")
    qm.probe_stream(buf, 0, sink)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
    for a, b in ev:
        a.record()
        qm.probe_stream(buf, 0, sink)
        b.record()
    torch.cuda.synchronize()
    ms = statistics.median(a.elapsed_time(b) for a, b in ev)
    info["stream_read_gbps"] = buf.numel() * 4 / (ms * 1e-3) / 1e9
    for a, b in ev:
        a.record()
        qm.probe_stream(buf, 1, sink)
        b.record()
    torch.cuda.synchronize()
    # requesting 32 bytes of every 128-byte line takes as long as reading
    # every byte when HBM moves whole lines
    info["stream_read_32b_of_128b_time_vs_dense"] = statistics.median(a.elapsed_time(b) for a, b in ev) / ms
    del buf
    out = torch.zeros(5, dtype=torch.int64, device="cuda")
    wg, iters = 2 * cus, 20000
    qm.probe_mfma(wg, 500, out)
    torch.cuda.synchronize()
    out.zero_()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    qm.probe_mfma(wg, iters, out)
    b.record()
    torch.cuda.synchronize()
    c0, c1, w0, w1, _ = out.cpu().tolist()
    ms = a.elapsed_time(b)
    info["mfma_bf16_dense_tflops"] = wg * 4 * iters * 8 * (2 * 32 * 32 * 16) / (ms * 1e-3) / 1e12
    info["sustained_sclk_mhz"] = (c1 - c0) / ((w1 - w0) / 1e8) / 1e6 if w1 > w0 else None
    info["note"] = ("measured on this GPU in this run; rooflines use the published peaks (HBM 8 TB/s, dense bf16 "
                    "MFMA 2.5 PFLOP/s)")
    return info


# ---------------------------------------------------------------------------
# The layer workloads

def cpu_baseline(cfg, layer, xs, toks, target_s, T_sample):
    """The float64 oracle, as it stands, on a bounded sample of the workload:
    whole oracle forward calls of the workload's first T_sample tokens."""
    import oracle
    n_tok = 0
    steps = 0
    t0 = time.perf_counter()
    while True:
        s = steps % len(xs)
        x = xs[s][:T_sample]
        tok = None if toks is None else toks[s][:T_sample]
        oracle.forward(layer, x, token_ids=tok)
        n_tok += x.shape[0]
        steps += 1
        el = time.perf_counter() - t0
        if el >= target_s or steps >= 64:
            break
    sample = (f"{steps} oracle forward call(s) of {T_sample} token(s) each on the same workload "
              f"(each call dequantises its touched experts to float64), {el:.1f} s")
    return {"value": n_tok / el, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle", "sample": sample,
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}


def time_graph(step, K, W, replays, eager=False):
    """W untimed steps, then K steps captured in one HIP graph (or launched
    eagerly) and timed `replays` times, each between synchronisations.
    Returns the per-replay milliseconds and the wall time of the timed replays."""
    import torch
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    graph = None
    if not eager:
        graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                for i in range(K):
                    step(i)
        torch.cuda.current_stream().wait_stream(s)
        graph.replay()  # untimed
        torch.cuda.synchronize()
    ms = []
    t0 = time.perf_counter()
    for _ in range(replays):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        if eager:
            for i in range(K):
                step(i)
        else:
            graph.replay()
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    return ms, time.perf_counter() - t0


def cold_steps(dl, xs, toks, ws, out, n):
    """n single steps (one token batch each, captured once as a graph), each
    preceded, outside its timed region, by a 1 GiB write that leaves none of
    the layer in the L2s or the Infinity Cache. Returns microseconds per step."""
    import torch
    import quantized_sparse_moe_amd as qm
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
    x_in = torch.empty_like(xs[0])
    tok_in = None if toks[0] is None else torch.empty_like(toks[0])
    qm.forward(dl, x_in.copy_(xs[0]), None if tok_in is None else tok_in.copy_(toks[0]), ws=ws, out=out)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            qm.forward(dl, x_in, tok_in, ws=ws, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    evs = []
    for i in range(n):
        x_in.copy_(xs[i % len(xs)])
        if tok_in is not None:
            tok_in.copy_(toks[i % len(toks)])
        qm.probe_stream(flush, 2)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in evs]


def roofline(label, cfg, dl, T, touched, kern_us, workload):
    """Roofline of the kernel `label`: MFMA (bf16 dense) when its algorithmic
    flops take longer at peak than its algorithmic bytes, else HBM."""
    b = kernel_bytes(label, cfg, dl, T, touched)
    fl = kernel_flops(label, cfg, T)
    if fl is not None and fl / (MFMA_BF16_PEAK_TFLOPS * 1e12) < b / (HBM_PEAK_GBS * 1e9):
        fl = None
    us = kern_us[label]
    if fl is None:
        a = b / (us * 1e-6) / 1e9
        return {"bound": "hbm", "kernel": label, "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": a / HBM_PEAK_GBS, "traffic": measured_traffic(workload, label, cfg),
                "algorithmic_bytes_per_launch": b, "avg_launch_us": us}
    a = fl / (us * 1e-6) / 1e12
    return {"bound": "mfma", "kernel": label, "achieved": a, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": a / MFMA_BF16_PEAK_TFLOPS, "traffic": measured_traffic(workload, label, cfg),
            "algorithmic_flops_per_launch": fl, "algorithmic_bytes_per_launch": b, "avg_launch_us": us}


def run_layer(args, name, K, W, replays, cold=0, cpu_T_sample=None, copies=0):
    """One layer workload: setup, timed graph replays, per-kernel times, the
    dominant kernel's roofline, optional cold steps and CPU-oracle sample."""
    import numpy as np
    import torch
    import quantized_sparse_moe_amd as qm
    import synth

    dev = torch.device("cuda:0")
    cfg = synth.config(name)
    T = cfg.T
    t_gen = time.perf_counter()
    layer = synth.gen_layer(cfg)
    base = qm.DeviceLayer.from_host(layer, dev)
    per_step_guess = step_bytes(cfg, base, T, min(cfg.E, T * cfg.top_k))
    copies = copies or max(1, min(8, math.ceil(1.0e9 / per_step_guess)))
    layers = [base] + [base.clone() for _ in range(copies - 1)]
    n_x = max(1, cfg.steps)
    xs_host = [synth.gen_x(cfg, s) for s in range(n_x)]
    toks_host = [synth.gen_token_ids(cfg, s) for s in range(n_x)] if cfg.route == "hash" else None
    xs = [torch.from_numpy(x.view(np.int16)).to(dev) for x in xs_host]
    toks = [torch.from_numpy(t).to(dev) for t in toks_host] if toks_host else [None] * n_x
    ws = base.workspace(T)
    out = torch.empty((T, cfg.d), dtype=torch.bfloat16, device=dev)
    gen_s = time.perf_counter() - t_gen

    touched = []
    for i in range(n_x):
        ids, _ = qm.route(base, xs[i], toks[i], ws)
        touched.append(int(torch.unique(ids).numel()))
    touched_mean = float(np.mean(touched))

    def step(i):
        qm.forward(layers[i % copies], xs[i % n_x], toks[i % n_x], ws=ws, out=out)

    replay_ms, wall = time_graph(step, K, W, replays, eager=args.eager)
    assert qm.device_error(ws) == 0
    ms = statistics.median(replay_ms) / K

    # per-kernel durations: each kernel's own start/stop timestamps (events
    # taken by the dispatch), on the library's stream
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(32)]
    for e in evs:
        e.record()  # torch creates the HIP event on first use
    torch.cuda.synchronize()
    sums = {}
    for i in range(min(K, 64)):
        names = qm.forward_probed(layers[i % copies], xs[i % n_x], toks[i % n_x], out, ws, evs)
        torch.cuda.synchronize()
        for j, n in enumerate(names):
            sums.setdefault(n, []).append(evs[2 * j].elapsed_time(evs[2 * j + 1]) * 1e3)
    kern = {n: float(np.mean(v)) for n, v in sums.items()}
    dom = max(kern, key=kern.get)
    roof = roofline(dom, cfg, base, T, touched_mean, kern, name)
    sbytes = step_bytes(cfg, base, T, touched_mean)
    rec = {
        "metric": METRIC, "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload_text(cfg), "tokens_per_step": T, "layer_copies": copies,
                   "timing": f"median of {replays} {'eager' if args.eager else 'hipgraph'} replays of {K} steps",
                   "touched_experts_per_step": touched_mean},
        "replay_ms": replay_ms,
        "hbm_gbps": sbytes / (ms * 1e-3) / 1e9,
        "step_algorithmic_bytes": sbytes,
        "roofline": roof,
        "kernels_us": kern,
        "wall_s": wall,
        "setup_s": gen_s,
    }
    fl_step = sum(kernel_flops(n, cfg, T) or 0.0 for n in kern)
    if fl_step:
        rec["mfma_frac_of_step"] = fl_step / (ms * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    if cold:
        us = cold_steps(base, xs, toks, ws, out, cold)
        q = statistics.quantiles(us, n=10)
        rec["cold_step_us"] = {"median": statistics.median(us), "p90": q[-1], "min": min(us), "steps": cold,
                               "flush_bytes_before_each": FLUSH_BYTES,
                               "tokens_per_s_at_median": T / (statistics.median(us) * 1e-6)}
    if not args.no_cpu_baseline:
        Ts = cpu_T_sample or (T if T <= 4 else 2)
        rec["cpu_baseline"] = cpu_baseline(cfg, layer, xs_host, toks_host, args.cpu_seconds, Ts)
    del layers, base, ws, xs, toks
    return rec


def main_quantize(args):
    """The conversion step before the layer: plain min/max affine quantisation
    (4-bit, groups of 64) of 128 experts' bf16 gate projections, [2048][4096]
    each, stacked as one [262144][4096] matrix: one launch per step."""
    import numpy as np
    import torch
    import quantized_sparse_moe_amd as qm
    import synth

    qm.load()
    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    experts, rows, cols, bits, group = 128, 2048, 4096, 4, 64
    t_gen = time.perf_counter()
    w = torch.empty((experts * rows, cols), dtype=torch.int16, device=dev)
    for e in range(experts):
        w[e * rows:(e + 1) * rows] = torch.from_numpy(synth.gen_bf16_weights(21, e, rows, cols).view(np.int16)).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    gen_s = time.perf_counter() - t_gen
    n = experts * rows * cols
    K, W = args.steps, args.warmup
    for _ in range(W):
        qm.quantize_affine(w, bits, group, err=err)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(K):
        qm.quantize_affine(w, bits, group, err=err)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(stop) / K
    assert int(err.item()) == 0
    nbytes = n * 2 + n * bits // 8 + (n // group) * 4   # bf16 in; codes, fp16 scale and bias out
    achieved = nbytes / (ms * 1e-3) / 1e9
    rec = {
        "metric": "affine quantiser weights/s (conversion step before the layer)", "value": n / (ms * 1e-3),
        "unit": "weights/s", "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"quantize: {experts} x [{rows}][{cols}] bf16 N(0, 0.02) weights -> affine "
                               f"{bits}-bit g{group} (one launch)", "timing": "eager, one launch per step"},
        "roofline": {"bound": "hbm", "kernel": "k_quantize_affine", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(args.workload,
                                                                                                  "k_quantize_affine",
                                                                                                  None),
                     "algorithmic_bytes_per_launch": nbytes, "avg_launch_us": ms * 1e3},
        "wall_s": wall, "setup_s": gen_s,
    }
    if not args.no_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        done = 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 10.0):
            oracle.quantize_affine(synth.gen_bf16_weights(21, done, 256, cols), bits, group)
            done += 1
        el = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": done * 256 * cols / el, "unit": "weights/s", "cores": 1, "kind": "oracle",
                               "sample": f"{done} oracle calls on [256][{cols}] blocks ({el:.1f} s)",
                               "host_cpus": len(os.sched_getaffinity(0))}
    print(json.dumps(rec), flush=True)


def main_sinkhorn(args):
    """mHC mix matrices of a 4096-token batch (4 x 4 per token, 10 rounds): the
    fused kernel, one launch per step; the unfused torch loop (a softmax and
    four launches per round) is timed beside it for context."""
    import numpy as np
    import torch
    import quantized_sparse_moe_amd as qm

    qm.load()
    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T, n, iters = 4096, 4, 10
    rng = np.random.default_rng(31)
    l = torch.from_numpy(rng.standard_normal((T, n, n)).astype(np.float32)).to(dev)
    out = torch.empty_like(l)
    K, W = args.steps, args.warmup

    def timed(fn):
        """K calls captured once as a HIP graph, replayed between events (host
        launch overhead outside the timed region, as for the layer)."""
        for _ in range(W):
            fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            with torch.cuda.graph(graph, stream=st):
                for _ in range(K):
                    fn()
        torch.cuda.current_stream().wait_stream(st)
        graph.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / K

    def unfused():
        m = torch.softmax(l, dim=-1)
        for _ in range(iters):
            m = m / m.sum(dim=-2, keepdim=True)
            m = m / m.sum(dim=-1, keepdim=True)
        return m

    ms = timed(lambda: qm.mhc_sinkhorn(l, iters, 0.0, out=out))
    ms_unfused = timed(unfused)
    nbytes = T * n * n * 4 * 2
    achieved = nbytes / (ms * 1e-3) / 1e9
    rec = {
        "metric": "mHC Sinkhorn mix matrices/s (op beside the MoE layer)", "value": T / (ms * 1e-3),
        "unit": "matrices/s", "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"sinkhorn: {T} tokens x {n}x{n} fp32 logits N(0,1), {iters} rounds, eps 0",
                   "timing": "hipgraph, one launch per step", "unfused_torch_ms": ms_unfused,
                   "speedup_vs_unfused": ms_unfused / ms},
        "roofline": {"bound": "hbm", "kernel": "k_mhc_sinkhorn", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(args.workload, "k_mhc_sinkhorn", None),
                     "algorithmic_bytes_per_launch": nbytes, "avg_launch_us": ms * 1e3,
                     "note": "0.5 MB per launch: bound by launch and memory latency, not HBM bandwidth"},
    }
    if not args.no_cpu_baseline:
        import oracle
        ln = l.cpu().numpy()
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 2.0:
            oracle.mhc_sinkhorn(ln, iters)
            reps += 1
        el = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": reps * T / el, "unit": "matrices/s", "cores": 1, "kind": "oracle",
                               "sample": f"{reps} oracle calls on the {T}-token batch ({el:.1f} s)",
                               "host_cpus": len(os.sched_getaffinity(0))}
    print(json.dumps(rec), flush=True)


def main_stack(args):
    """One decode token through the 43 MoE layers of the model (each layer with
    its own experts, formats and expert count, and its own seeded activations:
    attention and the residual stream between the layers are not part of the
    layer). A step is the 43 layers in order on one stream, captured once as a
    HIP graph."""
    import numpy as np
    import torch
    import quantized_sparse_moe_amd as qm
    import synth

    qm.load()
    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfgs = synth.stack_configs(T=1, steps=16)
    T, L = 1, len(cfgs)
    t_gen = time.perf_counter()
    dls, xs, toks, touched, host_layers = [], [], [], [], []
    for l, cfg in enumerate(cfgs):
        layer = synth.gen_layer(cfg)
        dls.append(qm.DeviceLayer.from_host(layer, dev))
        host_layers.append(layer if l in (0, 3, L - 1) else None)   # kept for the CPU baseline sample
        xs.append([torch.from_numpy(synth.gen_x(cfg, s).view(np.int16)).to(dev) for s in range(cfg.steps)])
        tk = [synth.gen_token_ids(cfg, s) for s in range(cfg.steps)] if cfg.route == "hash" else None
        toks.append([torch.from_numpy(t).to(dev) for t in tk] if tk else [None] * cfg.steps)
        del layer
        print(f"stack43: layer {l} built ({time.perf_counter() - t_gen:.0f} s)", file=sys.stderr, flush=True)
    ws = max((dl.workspace(T) for dl in dls), key=lambda w: w.numel())
    out = torch.empty((T, cfgs[0].d), dtype=torch.bfloat16, device=dev)
    for l, cfg in enumerate(cfgs):
        n = []
        for i in range(cfg.steps):
            ids, _ = qm.route(dls[l], xs[l][i], toks[l][i], ws)
            n.append(int(torch.unique(ids).numel()))
        touched.append(float(np.mean(n)))
    gen_s = time.perf_counter() - t_gen

    def step(i):
        for l in range(L):
            j = i % cfgs[l].steps
            qm.forward(dls[l], xs[l][j], toks[l][j], ws=ws, out=out)

    K, W = args.steps, args.warmup
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    assert qm.device_error(ws) == 0
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            for i in range(K):
                step(i)
    torch.cuda.current_stream().wait_stream(s)
    graph.replay()  # untimed
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    graph.replay()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(stop) / K
    assert qm.device_error(ws) == 0

    # per-kernel durations (HIP events taken by the dispatch), summed per step
    # over the layers; the dominant kernel's bytes and time are averaged over
    # its launches
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(32)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    per_launch, per_bytes = {}, {}
    probe_steps = min(K, 4)
    for i in range(probe_steps):
        for l, cfg in enumerate(cfgs):
            j = i % cfg.steps
            names = qm.forward_probed(dls[l], xs[l][j], toks[l][j], out, ws, evs)
            torch.cuda.synchronize()
            for q, n in enumerate(names):
                per_launch.setdefault(n, []).append(evs[2 * q].elapsed_time(evs[2 * q + 1]) * 1e3)
                per_bytes.setdefault(n, []).append(kernel_bytes(n, cfg, dls[l], T, touched[l]))
    step_us = {n: float(np.sum(v)) / probe_steps for n, v in per_launch.items()}
    dom = max(step_us, key=step_us.get)
    dom_us, dom_bytes = float(np.mean(per_launch[dom])), float(np.mean(per_bytes[dom]))
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    roof = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(args.workload, dom, cfgs[-1]),
            "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_us": dom_us,
            "launches_per_step": len(per_launch[dom]) // probe_steps}
    sbytes = sum(step_bytes(cfg, dls[l], T, touched[l]) for l, cfg in enumerate(cfgs))
    rec = {
        "metric": METRIC, "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (f"stack43: one decode token through 43 MoE layers, d=4096, I=2048, top-6; layers "
                                f"0-2 tid2eid hash over 256 experts, layers 3-42 top-6 over the 192 REAP25 "
                                f"survivors; routed gate/up affine 2-bit g128 and down 3-bit g128 in layers 0-38, "
                                f"affine 4-bit g64 in 39-42; shared expert I=2048 affine 8-bit g64 in every layer; "
                                f"each layer reads its own seeded activations (16 batches)"),
                   "tokens_per_step": T, "layers": L, "timing": "hipgraph",
                   "touched_experts_per_layer": float(np.mean(touched))},
        "hbm_gbps": sbytes / (ms * 1e-3) / 1e9,
        "step_algorithmic_bytes": sbytes,
        "roofline": roof,
        "kernels_us": step_us,
        "wall_s": wall,
        "setup_s": gen_s,
    }
    if not args.no_cpu_baseline:
        # the oracle on one token through a sample of the layers (a hash layer,
        # a pruned 2/3-bit layer, a 4-bit layer), scaled to the 43 layers
        import oracle
        smp = [l for l in range(L) if host_layers[l] is not None]
        t0 = time.perf_counter()
        for l in smp:
            oracle.forward(host_layers[l], synth.gen_x(cfgs[l], 0),
                           token_ids=synth.gen_token_ids(cfgs[l], 0) if cfgs[l].route == "hash" else None)
        el = time.perf_counter() - t0
        per_layer = el / len(smp)
        rec["cpu_baseline"] = {"value": 1.0 / (per_layer * L), "unit": "tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"one token through layers {smp} ({el:.1f} s), scaled to {L} layers",
                               "host_cpus": len(os.sched_getaffinity(0))}
        try:
            from threadpoolctl import threadpool_info
            rec["cpu_baseline"]["cores"] = int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
        except Exception:  # pragma: no cover
            pass
    print(json.dumps(rec), flush=True)


def main():
    args = parse()
    if args.ingest_counters:
        ingest_counters(args.ingest_counters)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import quantized_sparse_moe_amd as qm

    qm.load()  # fails loudly if the HIP library is not built
    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    torch.cuda.set_device(0)
    if args.calibrate:
        calibrate()
        return
    if args.workload in ("stack43", "quantize", "sinkhorn"):
        {"stack43": main_stack, "quantize": main_quantize, "sinkhorn": main_sinkhorn}[args.workload](args)
        return

    K, W, R = args.steps, args.warmup, max(1, args.replays)
    rec = run_layer(args, args.workload, K, W, R, cold=args.cold_steps if args.workload == "decode" else 0)
    if args.workload == "decode" and not args.no_prefill:
        # the matrix-core half of the metric: the 4096-token MXFP4 prefill,
        # its own steps (at most 16 per replay) and CPU-oracle sample (1 token)
        import gc
        gc.collect()
        torch.cuda.empty_cache()
        sub = run_layer(args, "prefill", min(K, 16), min(W, 4), R, cpu_T_sample=1, copies=1)
        rec["prefill"] = {k: sub[k] for k in ("value", "unit", "ms_per_step", "steps", "warmup", "replay_ms",
                                               "config", "roofline", "mfma_frac_of_step", "hbm_gbps",
                                               "kernels_us", "cpu_baseline") if k in sub}
    if not args.no_context:
        rec["context"] = context_info()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
