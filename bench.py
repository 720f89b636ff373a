#!/usr/bin/env python3
"""Throughput of the routed-expert MoE layer on one MI355X.

Default workload: batch-1 decode (T=1 token per step; d=4096, I=2048, E=256
routed experts with affine 4-bit g64 weights, top-6, plus the always-on shared
expert in affine 8-bit g64; 64 seeded activation steps). A step is one
moe_forward (route, bucket, experts, combine) of one batch.

Timed region: K steps captured in one HIP graph and replayed once, between a
torch.cuda.synchronize() on each side; inputs and weights are resident in HBM.
Steps rotate over several device copies of the layer so that no step finds its
weights in the 256 MB Infinity Cache left there by a recent step.

Also reported: the dominant kernel's roofline from HIP events that the
dispatches on the library's stream timestamp at kernel start and end
(moe_forward_probed), and the CPU oracle timed on a bounded sample of the same
workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, MI355X
METRIC = "MoE-layer tokens/s + achieved HBM GB/s (decode) / MFMA % (prefill)"


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=256)
    p.add_argument("--warmup", type=int, default=16)
    p.add_argument("--workload", default="decode",
                   choices=["decode", "tiny", "hash", "prefill", "mixed", "mxfp8", "stack43", "quantize",
                            "sinkhorn"])
    p.add_argument("--copies", type=int, default=0, help="device copies of the layer to rotate over (0: auto)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target length of the CPU oracle sample")
    p.add_argument("--eager", action="store_true", help="time eager launches instead of a graph replay")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run an elementwise copy of MIB MiB a few times (scale for HBM byte counters)")
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
    # fused small-batch path
    sh_gu = sh.gate.nbytes_per_expert() + sh.up.nbytes_per_expert() + T * cfg.I_shared * 2 if sh is not None else 0
    sh_dn = sh.down.nbytes_per_expert() + T * cfg.I_shared * 2 if sh is not None else 0
    if name == "dec_router":
        return E * d * 4 + T * d * 2 + T * E * 16 + sh_gu
    if name == "dec_gateup":
        return (touched * (r.gate.nbytes_per_expert() + r.up.nbytes_per_expert()) + T * E * 12 + T * d * 2
                + tk * I * 2 + tk * 8)
    if name == "dec_down_combine":
        return touched * r.down.nbytes_per_expert() + sh_dn + T * E * 4 + tk * I * 2 + T * d * 2
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


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter readings
    (profiles/hbm_traffic.json: FETCH_SIZE and WRITE_SIZE per dispatch from two
    rocprofv3 --pmc runs of this script, each scaled by what the same counter
    reads for an elementwise copy of known size), or None when there is no
    reading for this kernel or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel") != kernel or rec.get("source_hash") != source_hash():
        return None
    return rec["fetch_kib"] * 1024 * rec["fetch_scale"] + rec["write_kib"] * 1024 * rec["write_scale"]


def cpu_baseline(cfg, layer, xs, toks, target_s):
    """The float64 oracle, as it stands, on a bounded sample of the workload."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    n_tok = 0
    steps = 0
    t0 = time.perf_counter()
    T_sample = cfg.T if cfg.T <= 4 else 2
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
    return {"value": n_tok / el, "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": sample, "host_cpus": len(os.sched_getaffinity(0))}


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
                                                                                                  "k_quantize_affine"),
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
                     "traffic": measured_traffic(args.workload, "k_mhc_sinkhorn"),
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
            "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(args.workload, dom),
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
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)  # reads n bytes, writes n bytes
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n, "calibrate_copy_bytes_written": n, "launches": 3}))
        return

    if args.workload == "stack43":
        main_stack(args)
        return
    if args.workload == "quantize":
        main_quantize(args)
        return
    if args.workload == "sinkhorn":
        main_sinkhorn(args)
        return

    import quantized_sparse_moe_amd as qm
    import synth

    qm.load()  # fails loudly if the HIP library is not built
    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.config(args.workload)
    T = cfg.T

    t_gen = time.perf_counter()
    layer = synth.gen_layer(cfg)
    base = qm.DeviceLayer.from_host(layer, dev)
    per_step_guess = step_bytes(cfg, base, T, min(cfg.E, T * cfg.top_k))
    copies = args.copies or max(1, min(8, math.ceil(1.0e9 / per_step_guess)))
    layers = [base] + [base.clone() for _ in range(copies - 1)]
    n_x = max(1, cfg.steps)
    xs_host = [synth.gen_x(cfg, s) for s in range(n_x)]
    toks_host = [synth.gen_token_ids(cfg, s) for s in range(n_x)] if cfg.route == "hash" else None
    xs = [torch.from_numpy(x.view(np.int16)).to(dev) for x in xs_host]
    toks = [torch.from_numpy(t).to(dev) for t in toks_host] if toks_host else [None] * n_x
    ws = base.workspace(T)
    out = torch.empty((T, cfg.d), dtype=torch.bfloat16, device=dev)
    gen_s = time.perf_counter() - t_gen

    # distinct experts touched per activation batch (same for every layer copy)
    touched = []
    for i in range(n_x):
        ids, _ = qm.route(base, xs[i], toks[i], ws)
        touched.append(int(torch.unique(ids).numel()))
    touched_mean = float(np.mean(touched))

    def step(i):
        qm.forward(layers[i % copies], xs[i % n_x], toks[i % n_x], ws=ws, out=out)

    K, W = args.steps, args.warmup
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    assert qm.device_error(ws) == 0

    mode = "eager" if args.eager else "hipgraph"
    if not args.eager:
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
    t0 = time.perf_counter()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    if args.eager:
        for i in range(K):
            step(i)
    else:
        graph.replay()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(stop) / K
    assert qm.device_error(ws) == 0

    # per-kernel durations: each kernel's own start/stop timestamps (events
    # taken by the dispatch), on the library's stream
    n_ev = 32
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    for e in evs:
        e.record()  # torch creates the HIP event on first use
    torch.cuda.synchronize()
    probe_steps = min(K, 64)
    sums = {}
    for i in range(probe_steps):
        names = qm.forward_probed(layers[i % copies], xs[i % n_x], toks[i % n_x], out, ws, evs)
        torch.cuda.synchronize()
        for j, n in enumerate(names):
            sums.setdefault(n, []).append(evs[2 * j].elapsed_time(evs[2 * j + 1]) * 1e3)
    kern = {n: float(np.mean(v)) for n, v in sums.items()}
    dom = max(kern, key=kern.get)
    dom_bytes = kernel_bytes(dom, cfg, base, T, touched_mean)
    dom_flops = kernel_flops(dom, cfg, T)
    # the bound is whichever roof takes longer for the kernel's algorithmic work
    if dom_flops is not None and dom_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) < dom_bytes / (HBM_PEAK_GBS * 1e9):
        dom_flops = None
    if dom_flops is None:
        achieved = dom_bytes / (kern[dom] * 1e-6) / 1e9
        roof = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(args.workload, dom),
                "algorithmic_bytes_per_launch": dom_bytes,
                "avg_launch_us": kern[dom]}
    else:
        achieved = dom_flops / (kern[dom] * 1e-6) / 1e12
        roof = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                "traffic": measured_traffic(args.workload, dom),
                "algorithmic_flops_per_launch": dom_flops, "algorithmic_bytes_per_launch": dom_bytes,
                "avg_launch_us": kern[dom]}

    sbytes = step_bytes(cfg, base, T, touched_mean)
    rec = {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload_text(cfg), "tokens_per_step": T, "layer_copies": copies,
                   "timing": mode, "touched_experts_per_step": touched_mean},
        "hbm_gbps": sbytes / (ms * 1e-3) / 1e9,
        "step_algorithmic_bytes": sbytes,
        "roofline": roof,
        "kernels_us": kern,
        "wall_s": wall,
        "setup_s": gen_s,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, layer, xs_host, toks_host, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
