"""Helpers for the GPU parity tests: upload, error metric, routing comparison."""
import numpy as np
import torch

import oracle
import quantized_sparse_moe_amd as qm

# Max relative error of the fp32 output per token, max_j |y - y_ref| / max_j |y_ref|,
# against the float64 oracle (fp32 accumulation, bf16 activations).
TOL = 2e-3


def xdev(x_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda()


def rel_err(y, ref) -> np.ndarray:
    y = np.asarray(y, dtype=np.float64).reshape(ref.shape)
    den = np.abs(ref).max(axis=-1)
    den = np.where(den > 0, den, 1.0)
    return np.abs(y - ref).max(axis=-1) / den


def near_tie_ok(gpu_ids_t, key_t, k, tau_rel=1e-5):
    """A routing difference is accepted only where the float64 keys of the
    experts involved lie within tau of the k-th key (a certified near-tie):
    fp32 and float64 keys can order such experts differently."""
    order = sorted(range(len(key_t)), key=lambda e: (-key_t[e], e))
    kth = key_t[order[k - 1]]
    tau = tau_rel * (1.0 + abs(kth))
    ref_set, gpu_set = set(order[:k]), set(int(e) for e in gpu_ids_t)
    if len(gpu_set) != k:
        return False
    for e in ref_set ^ gpu_set:
        if abs(key_t[e] - kth) > tau:
            return False
    # order within the selection: adjacent keys must be non-increasing up to tau
    kg = [key_t[int(e)] for e in gpu_ids_t]
    return all(kg[i] >= kg[i + 1] - tau_rel * (1 + abs(kg[i])) for i in range(k - 1))


def check_topk_ids(gpu_ids: np.ndarray, ref_ids: np.ndarray, key: np.ndarray, k: int, max_ties: int = 2) -> int:
    """GPU ids equal the oracle's except at certified near-ties; returns their count."""
    ties = 0
    for t in range(gpu_ids.shape[0]):
        if not np.array_equal(gpu_ids[t], ref_ids[t]):
            assert near_tie_ok(gpu_ids[t], key[t], k), f"token {t}: gpu {gpu_ids[t]} oracle {ref_ids[t]}"
            ties += 1
    assert ties <= max_ties, f"{ties} near-tie tokens"
    return ties


def stable_sort_perm(ids: np.ndarray, E: int):
    flat = ids.reshape(-1)
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    off = np.zeros(E + 1, np.int64)
    off[1:] = np.cumsum(np.bincount(flat, minlength=E))
    return off, perm


def run_staged(dl, x_bits, token_ids=None):
    xd = xdev(x_bits)
    tok = None if token_ids is None else torch.from_numpy(np.ascontiguousarray(token_ids)).cuda()
    ws = dl.workspace(x_bits.shape[0])
    st = qm.forward_staged(dl, xd, tok, out_dtype="f32", ws=ws)
    out_f32 = qm.forward(dl, xd, tok, out_dtype="f32", ws=ws)
    out_bf16 = qm.forward(dl, xd, tok, out_dtype="bf16", ws=ws)
    torch.cuda.synchronize()
    assert qm.device_error(ws) == 0
    return st, out_f32, out_bf16, ws


# ---------------------------------------------------------------------------
# Intermediates of moe_forward, read from its workspace (moe_workspace_layout)

def read_ws(dl, ws, T):
    """moe_forward's intermediates for T tokens as numpy arrays (None where the
    call keeps no such region)."""
    lay = dl.workspace_layout(T)
    E, k, d, I = dl.E, dl.top_k, dl.d, dl.I
    Ish = dl.shared.gate.rows if dl.shared is not None else 0

    def get(name, dtype, shape, npdtype=None):
        off = lay[name]
        if off == 0:
            return None
        a = qm.ws_region(ws, off, dtype, shape).cpu().numpy()
        return a.view(npdtype) if npdtype is not None else a

    return {
        "fused": bool(lay["fused"]),
        "ids": get("ids", torch.int32, (T, k)),
        "w": get("weights", torch.float32, (T, k)),
        "logits": get("logits", torch.float32, (T, E)),
        "keys": get("keys", torch.int64, (T, E), np.uint64),
        "scores": get("scores", torch.float32, (T, E)),
        "offsets": get("offsets", torch.int32, (E + 1,)),
        "perm": get("perm", torch.int32, (T * k,)),
        "h": get("h", torch.int16, (T * k, I), np.uint16),
        "h_shared": get("h_shared", torch.int16, (T, Ish), np.uint16) if Ish else None,
        "y_slot": get("y_slot", torch.float32, (T * k, d)),
        "y_shared": get("y_shared", torch.float32, (T, d)) if Ish else None,
    }


def unpack_keys(keys):
    """Packed ranking keys (uint64: order-mapped fp32 key << 32 | 0xFFFFFFFF - e)
    -> (fp32 keys, expert indices)."""
    hi = (keys >> np.uint64(32)).astype(np.uint32)
    lo = (keys & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    bits = np.where(hi & np.uint32(0x80000000), hi & np.uint32(0x7FFFFFFF), ~hi).astype(np.uint32)
    return bits.view(np.float32), (np.uint32(0xFFFFFFFF) - lo).astype(np.int64)


def check_topk_exact(keys, scores, bias, ids, w, k, routed_scale=1.0):
    """The GPU's top-k on the GPU's own fp32 keys, bit for bit: every key is
    fp32(score + bias); the ids are the k largest keys in order (ties to the
    lower index) by host brute force on exactly those keys; the weights are the
    selected scores renormalised in fp32 in slot order."""
    key32, idx = unpack_keys(keys)
    T, E = key32.shape
    assert np.array_equal(idx, np.broadcast_to(np.arange(E), (T, E)))
    want = scores.astype(np.float32) + (np.float32(0) if bias is None else np.asarray(bias, np.float32)[None, :])
    assert np.array_equal(key32.view(np.uint32), want.astype(np.float32).view(np.uint32))
    ar = np.arange(E)
    for t in range(T):
        order = np.lexsort((ar, -key32[t].astype(np.float64)))[:k]
        assert ids[t].tolist() == order.tolist(), f"token {t}: gpu {ids[t].tolist()} brute force {order.tolist()}"
    check_weights_exact(scores, ids, w, routed_scale)


def check_weights_exact(scores, ids, w, routed_scale=1.0):
    """w[t, j] = fp32(s_j / (s_0 + ... + s_{k-1})) * routed_scale, summed in slot
    order in fp32, from the GPU's own scores (1/k when the sum is 0)."""
    T, k = ids.shape
    for t in range(T):
        s = scores[t, ids[t]].astype(np.float32)
        tot = np.float32(0.0)
        for j in range(k):
            tot = np.float32(tot + s[j])
        wt = (s / tot if tot > 0 else np.full(k, np.float32(1.0) / np.float32(k))).astype(np.float32)
        wt = (wt * np.float32(routed_scale)).astype(np.float32)
        assert np.array_equal(w[t].view(np.uint32), wt.view(np.uint32)), (t, w[t], wt)


# ---------------------------------------------------------------------------
# h = silu(gate) * up, rounded to bf16: the GPU's h against the oracle's

def _abs_terms(q, e):
    """|terms| the kernels sum per weight, as a [rows][cols] float64 bound:
    affine b <= 4 codes are summed as 2^b + q with the bias term b - 2^b s
    (8-bit: q with b), so |s| (off + q) + |b - off s|; MX formats |w|.
    2-bit codes are summed as q with b on the streaming and fused paths and
    in the grouped GEMM with groups of 64 or 128; the 2^b form kept here
    bounds those terms too, since |b| <= |b - 4 s| + 4 |s| gives
    |s| q + |b| <= |s| (4 + q) + |b - 4 s|."""
    spec = q.spec
    if spec.fmt == "affine":
        off = float(2 ** spec.bits) if spec.bits <= 4 else 0.0
        codes = oracle.unpack_codes(q.codes[e], spec.bits, q.cols).astype(np.float64)
        s = np.repeat(q.scales[e].astype(np.float64), spec.group, axis=-1)
        b = np.repeat(q.biases[e].astype(np.float64), spec.group, axis=-1)
        return np.abs(s) * (off + codes) + np.abs(b - off * s)
    return np.abs(oracle.dequant(q, e))


def expert_reference(ew, e, x_bits, bound=True):
    """For expert e of a weight set and the activation rows x_bits: the oracle's
    float64 h (unrounded) and the bf16-rounded path's output y; with `bound`,
    also what the rounding-flip bound needs (g, u and the absolute sums of the
    summed terms)."""
    x64 = oracle.bf16_bits_to_f64(x_bits)
    w1, w3, w2 = oracle.expert_mats(ew, e)
    h64 = oracle.swiglu_h(w1, w3, x64)
    ref = {"h64": h64, "y": oracle.round_bf16(h64) @ w2.T, "w2": w2, "d": x64.shape[1]}
    if bound:
        ax = np.abs(x64)
        ref.update(g=x64 @ w1.T, u=x64 @ w3.T, m1=ax @ _abs_terms(ew.gate, e).T, m3=ax @ _abs_terms(ew.up, e).T)
    return ref


def check_h(h_gpu_bits, ref):
    """The GPU's bf16 h is a round-to-nearest-even of a value within delta of
    the oracle's float64 h, RNE(h - delta) <= h_gpu <= RNE(h + delta), with
        delta = 4 sqrt(d / 32) 2^-24 (|silu'(g) u| M1 + |silu(g)| M3) + 2^-20 |h|:
    d / 32 fp32 additions of 32-input partial sums, each off by up to about
    one fp32 ulp of the magnitude M of the summed terms (M1, M3: absolute sums
    of the terms the kernels add for gate and up), independent errors growing
    as the square root of their count, four times over; carried through
    silu(g) u. (Measured on every path at d = 4096: the largest error needed
    is 0.53 of the single-ulp term, about 1/85 of delta.) Where h_gpu !=
    RNE(h), float64 h lies that close to a rounding boundary: a rounding flip.
    Returns the number of flips."""
    h64 = ref["h64"]
    hr = oracle.round_bf16(h64)
    hg = oracle.bf16_bits_to_f64(np.asarray(h_gpu_bits, np.uint16)).reshape(h64.shape)
    diff = hg != hr
    if not diff.any():
        return 0
    g, u = ref["g"][diff], ref["u"][diff]
    sig = 1.0 / (1.0 + np.exp(-g))
    dsilu = sig * (1.0 + g * (1.0 - sig))
    delta = 4.0 * np.sqrt(ref["d"] / 32) * 2.0 ** -24 * (np.abs(dsilu * u) * ref["m1"][diff]
                                                       + np.abs(g * sig) * ref["m3"][diff])
    delta += 2.0 ** -20 * np.abs(h64[diff])
    hv, gv = h64[diff], hg[diff]
    lo, hi = oracle.round_bf16(hv - delta), oracle.round_bf16(hv + delta)
    bad = (gv < lo) | (gv > hi)
    assert not bad.any(), (f"{int(bad.sum())} of {hv.size} differing h values outside RNE(h +- delta): e.g. "
                           f"h {hv[bad][:3]}, gpu {gv[bad][:3]}, delta {delta[bad][:3]}")
    return int(diff.sum())


# Down projection (and combine) given the GPU's own bf16 h: fp32 accumulation only.
TIGHT = 1e-5


def check_forward_intermediates(cfg, layer, dl, ws, x, tok, out_f32):
    """After moe_forward on workspace ws: routing bit-exact on the GPU's own
    keys; every assignment's bf16 h against the oracle (rounding flips only
    near midpoints); the down projection, shared expert and combine within
    TIGHT of float64 arithmetic on the GPU's own h. Returns the flip count."""
    T, k, E = x.shape[0], cfg.top_k, cfg.E
    r = read_ws(dl, ws, T)
    ids, w = r["ids"], r["w"]
    if cfg.route == "topk":
        check_topk_exact(r["keys"], r["scores"], layer.bias, ids, w, k)
    elif r["scores"] is not None:
        assert np.array_equal(ids, layer.tid2eid[tok])
        check_weights_exact(r["scores"], ids, w)
    # rows of the h region per expert: slot order (fused) or bucket order
    if r["fused"]:
        rows_of = {}
        for a in range(T * k):
            rows_of.setdefault(int(ids.reshape(-1)[a]), []).append((a, a))
    else:
        off, perm = r["offsets"], r["perm"]
        rows_of = {e: [(p, int(perm[p])) for p in range(off[e], off[e + 1])] for e in range(E) if off[e + 1] > off[e]}
    flips = 0
    y_tight = np.zeros((T * k, cfg.d))
    for e, rows in rows_of.items():
        hrow = np.array([p for p, _ in rows])
        slots = np.array([a for _, a in rows])
        ref = expert_reference(layer.routed_expert(e), 0, x[slots // k])
        flips += check_h(r["h"][hrow], ref)
        y_tight[slots] = oracle.bf16_bits_to_f64(r["h"][hrow]) @ ref["w2"].T
    y_sh = np.zeros((T, cfg.d))
    if layer.shared is not None:
        ref = expert_reference(layer.shared, 0, x)
        flips += check_h(r["h_shared"], ref)
        y_sh = oracle.bf16_bits_to_f64(r["h_shared"]) @ ref["w2"].T
    if not r["fused"]:
        assert rel_err(r["y_slot"], y_tight).max() <= TIGHT
    if r["y_shared"] is not None:
        assert rel_err(r["y_shared"], y_sh).max() <= TIGHT
    y = np.einsum("tk,tkd->td", w.astype(np.float64), y_tight.reshape(T, k, cfg.d)) + y_sh
    assert rel_err(out_f32, y).max() <= TIGHT
    return flips
