"""Plain float64 CPU oracle of the DeepSeek-V4 routed-expert MoE layer.

TEST INFRASTRUCTURE ONLY (imported by tests, the smoke check and the benchmark's
CPU-baseline leg; never by the GPU library). numpy only, float64 throughout,
no blocking, fusion or reordering beyond what each step's definition states.

Sources (web pages, cited by title and section):
  [PR1192]  mlx-lm pull request "Add DeepSeek-v4 (Flash/Pro)"
  [CARD4]   model card "mlx-community / DeepSeek-V4-Flash-4bit"
  [ALPHA]   model card "DeepSeek-V4-Flash-MLX-4bit" (alphaneural)
  [PR1190]  mlx-lm pull request "Add DeepSeek-V4 model and safetensors/tokenizer
            fallback handling"
  [SERVE]   model card "DeepSeek-V4-Flash-0731-MLX-Serve-mixed-2-3-8bit"

Readings taken where the pages are silent or ambiguous (each marked READING
below): e2m1 and e4m3 bit layouts and e8m0 0xFF = NaN from the public OCP MX format;
nibble/bit order LSB-first along the input dimension; the router bias only
ranks experts and does not enter the combine weights; hash-routed layers have
no bias; ties in the top-k go to the lower expert index and the k slots are
ordered by key descending; the shared expert is added with weight 1 after the
routed sum; SwiGLU is silu(w1 x) * (w3 x) without clamping; the SwiGLU
product h is rounded to bf16 (round to nearest even) before the down
projection, matching bf16 activations.

Parity pins: every function here is pinned by the CPU tests against values the
pages fix, closed forms, special cases or brute force, except the end-to-end
output values of a full layer, for which no worked example exists on the pages
(parity unpinned beyond the invariants the tests check: zero weights, one-hot
inputs, linearity in the down projection, token-order equivariance, per-token
independence and brute-force loops on tiny layers).
"""
from __future__ import annotations

from types import SimpleNamespace

import numpy as np

__all__ = [
    "bf16_bits_to_f64", "round_bf16", "e2m1_decode", "e4m3_decode", "e8m0_decode", "unpack_codes",
    "dequant", "sqrtsoftplus", "silu", "router_logits", "route_topk", "route_hash",
    "combine_weights_for_ids", "permute", "swiglu_h", "expert_mats", "swiglu_expert", "forward", "forward_tokens",
    "pack_codes", "quantize_affine", "mhc_sinkhorn",
]

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


# ----------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values (bf16 is the top half of fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def round_bf16(v) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even (single rounding).

    bf16 keeps 8 significant bits; below 2^-126 the spacing is fixed at 2^-133.
    Results above the largest finite bf16 become +-inf. Returned as float64.
    """
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        _, e = np.frexp(v)                     # v = m * 2^e with 0.5 <= |m| < 1
        quantum_exp = np.maximum(e - 8, -133)  # weight of the 8th significant bit
        r = np.ldexp(np.rint(np.ldexp(v, -quantum_exp)), quantum_exp)  # rint: ties to even
        r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, v), r)
    return np.where(np.isfinite(v), r, v)


def e2m1_decode(nibbles) -> np.ndarray:
    """FP4 e2m1 code -> value.

    [ALPHA] (section "What this port implements", closing paragraph) names the
    routed experts' format as FP4 e2m1 packed two per byte. READING: the OCP MX
    bit layout -- bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa;
    exponent 0 is subnormal (0 or 0.5).
    """
    n = np.asarray(nibbles).astype(np.int64) & 0xF
    sign = np.where(n & 8, -1.0, 1.0)
    exp = (n >> 1) & 3
    man = (n & 1).astype(np.float64)
    mag = np.where(exp == 0, 0.5 * man, np.ldexp(1.0 + 0.5 * man, exp - 1))
    return sign * mag


def e4m3_decode(codes) -> np.ndarray:
    """FP8 e4m3 code -> value.

    [PR1192] (FP8-to-bf16 requantization report) names the weight bytes FP8
    E4M3 and reads them with mx.dequantize in "mxfp8" mode; [PR1190] calls
    the layers MXFP8-quantized. READING: the OCP E4M3 layout ("e4m3fn") --
    bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa; exponent 0
    is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinities, so the
    largest magnitude is 1.75 * 2^8 = 448.
    """
    n = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(n & 0x80, -1.0, 1.0)
    exp = (n >> 3) & 0xF
    man = (n & 7).astype(np.float64)
    mag = np.where(exp == 0, np.ldexp(man / 8.0, -6), np.ldexp(1.0 + man / 8.0, exp - 7))
    mag = np.where((n & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e8m0_decode(b) -> np.ndarray:
    """e8m0 scale byte -> 2^(b - 127) ([PR1190] description: F8_E8M0 decoded as
    unsigned exponents). READING: 0xFF is NaN per OCP MX."""
    b = np.asarray(b).astype(np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))


def unpack_codes(words, bits: int, cols: int) -> np.ndarray:
    """Unsigned b-bit codes from a packed row.

    Codes are one contiguous LSB-first bit stream over little-endian uint32
    words along the input dimension (code c occupies stream bits
    [c*b, c*b + b)); a 3-bit code may straddle two words. [PR1192] stores the
    codes as ``weight.view(mx.uint32)`` (FP8/FP4 sanitize comment) and [SERVE]
    calls the packs byte-compatible with MLX's affine layout.
    words: uint32 [..., W] -> int64 [..., cols]
    """
    w = np.ascontiguousarray(words, dtype="<u4")
    lead = w.shape[:-1]
    stream = np.unpackbits(w.view(np.uint8), axis=-1, bitorder="little")  # [..., W*32]
    stream = stream[..., : cols * bits].reshape(*lead, cols, bits).astype(np.int64)
    codes = np.zeros((*lead, cols), dtype=np.int64)
    for i in range(bits):
        codes |= stream[..., i] << i
    return codes


def dequant(q, e: int = 0) -> np.ndarray:
    """Expert e of a stacked quantised projection -> float64 [rows][cols].

    affine: w = scale * q + bias with fp16 scale and bias per group of
            ``group`` consecutive inputs ({weight, scales, biases} triplets in
            [PR1192]'s pre-stacked expert patch; bit widths and group sizes from
            [CARD4] "Conversion" and the [SERVE] precision table).
    mxfp4:  w = e2m1(code) * 2^(scale_byte - 127), one scale byte per 32
            inputs ([PR1192] dequantize call with group_size=32, bits=4,
            mode="mxfp4"; e8m0 per [PR1190]).
    mxfp8:  w = e4m3(code) * 2^(scale_byte - 127), one byte per code and one
            scale byte per 32 inputs ([PR1192] requantization report:
            mx.dequantize with group_size=32, bits=8, mode="mxfp8").
    """
    spec = q.spec
    codes = unpack_codes(q.codes[e], spec.bits, q.cols)            # [rows][cols]
    if spec.fmt == "affine":
        s = np.repeat(q.scales[e].astype(np.float64), spec.group, axis=-1)
        b = np.repeat(q.biases[e].astype(np.float64), spec.group, axis=-1)
        return s * codes + b
    if spec.fmt == "mxfp4":
        scale = np.repeat(e8m0_decode(q.scales[e]), 32, axis=-1)
        return e2m1_decode(codes) * scale
    if spec.fmt == "mxfp8":
        scale = np.repeat(e8m0_decode(q.scales[e]), 32, axis=-1)
        return e4m3_decode(codes) * scale
    raise ValueError(spec.fmt)


def pack_codes(codes, bits: int) -> np.ndarray:
    """Inverse of unpack_codes: b-bit codes [..., cols] -> one LSB-first bit
    stream over little-endian uint32 words [..., cols*b/32]."""
    c = np.asarray(codes, dtype=np.int64)
    lead, cols = c.shape[:-1], c.shape[-1]
    assert (cols * bits) % 32 == 0 and c.min(initial=0) >= 0 and c.max(initial=0) < (1 << bits)
    stream = np.zeros((*lead, cols, bits), dtype=np.uint8)
    for i in range(bits):
        stream[..., i] = (c >> i) & 1
    stream = stream.reshape(*lead, cols * bits)
    return np.packbits(stream, axis=-1, bitorder="little").view("<u4")


def quantize_affine(w_bits, bits: int, group: int):
    """Plain min/max affine quantisation of bf16 weights [rows][cols], the
    conversion step before the layer ([CARD4] "Conversion": mlx_lm.convert
    -q --q-bits 4 --q-group-size 64; [SERVE] contrasts its calibrated search
    with plain min/max). READINGS (the pages give the recipe, not its
    arithmetic): per group of ``group`` consecutive inputs of a row,
        scale = fp16((max - min) / (2^b - 1)),  bias = fp16(min),
        q = clamp(rint((w - bias) / scale), 0, 2^b - 1)   (q = 0 if scale == 0),
    with fp16 round-to-nearest-even. The code is an integer that floating
    point decides, so it is computed in fp32 (the kernel's precision) with
    IEEE operations in this order: subtraction, division, rint (ties to even).
    Returns (codes uint32 [rows][cols*b/32], scales fp16, biases fp16 [rows][cols/group]).
    """
    w = bf16_bits_to_f64(w_bits).astype(np.float32)
    rows, cols = w.shape
    assert cols % group == 0
    g = w.reshape(rows, cols // group, group)
    lo, hi = g.min(axis=-1), g.max(axis=-1)
    levels = np.float32((1 << bits) - 1)
    scale = ((hi - lo) / levels).astype(np.float16)
    bias = lo.astype(np.float16)
    s32, b32 = scale.astype(np.float32)[..., None], bias.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.rint((g - b32) / s32)
    q = np.where(s32 == 0, 0.0, np.clip(t, 0, levels)).astype(np.int64).reshape(rows, cols)
    return pack_codes(q, bits), scale, bias


# ----------------------------------------------------------------------------
# Routing
# ----------------------------------------------------------------------------

def sqrtsoftplus(l) -> np.ndarray:
    """Expert score sqrt(softplus(l)) ([CARD4] "Architecture": sqrtsoftplus
    scoring instead of softmax), evaluated without overflow as
    sqrt(max(l, 0) + log(1 + exp(-|l|))) -- the log-sum-exp-stable
    logaddexp(l, 0) that [PR1192]'s review notes ask for."""
    l = np.asarray(l, dtype=np.float64)
    return np.sqrt(np.maximum(l, 0.0) + np.log1p(np.exp(-np.abs(l))))


def silu(z) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z))."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def router_logits(x64: np.ndarray, wr: np.ndarray) -> np.ndarray:
    """Gate logits l[t, e] = sum_i x[t, i] * Wr[e, i].

    [PR1192] cross-reference table, row "MoE gate dtype": the gate is computed
    in fp32 from the activations, in both the top-k and the hash router. Here
    in float64 from the exact bf16 activations and fp32 weights.
    """
    return x64 @ np.asarray(wr, dtype=np.float64).T


def route_topk(logits: np.ndarray, bias, k: int, routed_scale: float = 1.0):
    """Top-k routing on sqrtsoftplus scores plus per-expert bias.

    key[t, e] = s[t, e] + bias[e]. The k experts with the largest key are
    selected, in order of key descending, ties to the lower expert index
    (READING). The combine weights are the *unbiased* scores of the selected
    experts, renormalised to sum to one over the selected set ([ALPHA] "REAP-pruned
    builds": the router renormalises over the experts it keeps; READING: the
    bias, listed by [SERVE] among the verbatim router tensors, only ranks).
    A zero score sum (unreachable for finite logits above about -100) gives 1/k.
    Returns (ids int32 [T][k], w [T][k], key [T][E], s [T][E]).
    """
    s = sqrtsoftplus(logits)
    key = s + (0.0 if bias is None else np.asarray(bias, dtype=np.float64)[None, :])
    T, E = key.shape
    ids = np.empty((T, k), dtype=np.int32)
    idx = np.arange(E)
    for t in range(T):
        order = np.lexsort((idx, -key[t]))   # primary: key descending; then index ascending
        ids[t] = order[:k]
    w = combine_weights_for_ids(s, ids, routed_scale)
    return ids, w, key, s


def combine_weights_for_ids(s: np.ndarray, ids: np.ndarray, routed_scale: float = 1.0) -> np.ndarray:
    """w[t, j] = s[t, ids[t, j]] / sum_j' s[t, ids[t, j']] (times routed_scale)."""
    sel = np.take_along_axis(np.asarray(s, dtype=np.float64), ids.astype(np.int64), axis=1)
    tot = sel.sum(axis=1, keepdims=True)
    k = ids.shape[1]
    with np.errstate(invalid="ignore", divide="ignore"):
        w = np.where(tot > 0, sel / np.where(tot > 0, tot, 1.0), 1.0 / k)
    return w * routed_scale


def route_hash(x64: np.ndarray, wr: np.ndarray, tid2eid: np.ndarray, token_ids: np.ndarray,
               routed_scale: float = 1.0):
    """Hash routing for the first MoE layers ([CARD4] "Architecture": a
    deterministic tid2eid table, token id -> expert id; [ALPHA] table: keyed on
    token id, independent of context).

    ids[t, j] = tid2eid[token_ids[t], j] in table order (no bias, no top-k;
    duplicate ids stay as separate slots). Weights are the selected experts'
    sqrtsoftplus scores renormalised (READING, with [PR1192]'s note that the
    hash router also computes fp32 gate logits).
    Returns (ids int32 [T][k], w [T][k], s_sel [T][k]).
    """
    tid2eid = np.asarray(tid2eid)
    token_ids = np.asarray(token_ids).astype(np.int64)
    assert np.all((token_ids >= 0) & (token_ids < tid2eid.shape[0])), "token id out of range"
    ids = tid2eid[token_ids].astype(np.int32)
    E = wr.shape[0]
    assert np.all((ids >= 0) & (ids < E)), "tid2eid entry out of range"
    wr64 = np.asarray(wr, dtype=np.float64)
    T, k = ids.shape
    l = np.empty((T, k))
    for t in range(T):
        l[t] = wr64[ids[t]] @ x64[t]
    s = sqrtsoftplus(l)
    tot = s.sum(axis=1, keepdims=True)
    w = np.where(tot > 0, s / np.where(tot > 0, tot, 1.0), 1.0 / k) * routed_scale
    return ids, w, s


# ----------------------------------------------------------------------------
# Bucketing by expert
# ----------------------------------------------------------------------------

def permute(ids: np.ndarray, E: int):
    """Bucket the T*k (token, slot) assignments by expert.

    Assignment a = t*k + j has expert ids[t, j]. perm lists the assignments
    stably sorted by expert (within an expert, ascending a); counts is the
    per-expert histogram and offsets its exclusive prefix sum, offsets[E] = T*k.
    Needed to run the stacked experts ([PR1192]: experts pre-stacked as
    switch_mlp.{gate,up,down}_proj) over contiguous buckets.
    """
    flat = np.asarray(ids).reshape(-1).astype(np.int64)
    assert np.all((flat >= 0) & (flat < E)), "expert id out of range"
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    return offsets, perm, counts


# ----------------------------------------------------------------------------
# Experts and combine
# ----------------------------------------------------------------------------

def swiglu_h(w1: np.ndarray, w3: np.ndarray, x64: np.ndarray) -> np.ndarray:
    """h = silu(W1 x) * (W3 x) for each row x of x64, unrounded (float64).

    w1 = gate_proj, w3 = up_proj ([PR1192] pre-stacked expert rename:
    w1 -> gate_proj, w3 -> up_proj).
    """
    g = x64 @ w1.T
    u = x64 @ w3.T
    return silu(g) * u


def swiglu_expert(w1: np.ndarray, w3: np.ndarray, w2: np.ndarray, x64: np.ndarray,
                  round_h: bool = True) -> np.ndarray:
    """y = W2 (silu(W1 x) * (W3 x)) for each row x of x64.

    w2 = down_proj ([PR1192] pre-stacked expert rename: w2 -> down_proj). The
    product h (swiglu_h) is rounded to bf16 before the down projection when
    ``round_h`` (READING).
    """
    h = swiglu_h(w1, w3, x64)
    if round_h:
        h = round_bf16(h)
    return h @ w2.T


def expert_mats(ew, e: int = 0):
    """Expert e of a set of SwiGLU weights as float64 (w1, w3, w2)."""
    return dequant(ew.gate, e), dequant(ew.up, e), dequant(ew.down, e)


def forward(layer, x_bits, token_ids=None, ids=None, round_h: bool = True):
    """The whole layer for T tokens, float64.

    1. route (top-k or hash), or take ``ids`` as given and recompute their
       float64 weights (used to evaluate the layer on another router's ids);
    2. bucket the assignments by expert;
    3. for each touched expert, once: dequantise, run SwiGLU over its rows;
       y_slot[a] = expert(x[a // k]);
    4. shared expert over every token (weight 1, READING);
    5. combine y[t] = sum_j w[t, j] * y_slot[t*k + j] + y_shared[t].
    ``layer`` has: cfg, wr, bias, tid2eid, shared, routed_expert(e).
    """
    cfg = layer.cfg
    x = bf16_bits_to_f64(x_bits)
    T, d = x.shape
    k, E = cfg.top_k, cfg.E
    logits = router_logits(x, layer.wr)
    key = None
    if cfg.route == "hash":
        h_ids, h_w, _ = route_hash(x, layer.wr, layer.tid2eid, token_ids)
        if ids is None:
            ids, w = h_ids, h_w
        else:
            ids = np.asarray(ids, dtype=np.int32)
            assert np.array_equal(ids, h_ids)
            w = h_w
    else:
        r_ids, r_w, key, s = route_topk(logits, layer.bias, k)
        if ids is None:
            ids, w = r_ids, r_w
        else:
            ids = np.asarray(ids, dtype=np.int32).reshape(T, k)
            w = combine_weights_for_ids(s, ids)
    offsets, perm, counts = permute(ids, E)

    y_slot = np.zeros((T * k, d))
    for e in np.nonzero(counts)[0]:
        slots = perm[offsets[e]:offsets[e + 1]]
        w1, w3, w2 = expert_mats(layer.routed_expert(int(e)))
        y_slot[slots] = swiglu_expert(w1, w3, w2, x[slots // k], round_h)

    y_sh = np.zeros((T, d))
    if layer.shared is not None:
        w1, w3, w2 = expert_mats(layer.shared)
        y_sh = swiglu_expert(w1, w3, w2, x, round_h)

    y = np.zeros((T, d))
    for j in range(k):
        y += w[:, j:j + 1] * y_slot[j::k]
    y += y_sh
    return SimpleNamespace(logits=logits, key=key, ids=ids, w=w, offsets=offsets, perm=perm,
                           counts=counts, y_slot=y_slot, y_shared=y_sh, y=y)


def forward_tokens(layer, x_bits, tokens, ids, round_h: bool = True, expert_cache=None):
    """Outputs of selected tokens only, on the given ids (float64).

    For full-size checks: the layer is per-token, so y[t] depends only on x[t]
    and its own k experts (top-k or hash-table ids alike). Returns (w [n][k], y_slot [n][k][d], y_shared [n][d],
    y [n][d]) for tokens ``tokens``; ``ids`` are those tokens' expert ids.
    """
    cfg = layer.cfg
    x = bf16_bits_to_f64(np.asarray(x_bits)[list(tokens)])
    ids = np.asarray(ids, dtype=np.int32).reshape(len(tokens), cfg.top_k)
    # Hash layers weight the table's experts by the same renormalised scores,
    # and top-k weights never include the bias, so one formula serves both.
    logits = router_logits(x, layer.wr)
    s = sqrtsoftplus(logits)
    w = combine_weights_for_ids(s, ids)
    cache = {} if expert_cache is None else expert_cache
    n, k, d = len(tokens), cfg.top_k, cfg.d
    y_slot = np.zeros((n, k, d))
    for i in range(n):
        for j in range(k):
            e = int(ids[i, j])
            if e not in cache:
                cache[e] = expert_mats(layer.routed_expert(e))
            y_slot[i, j] = swiglu_expert(*cache[e], x[i:i + 1], round_h)[0]
    y_sh = np.zeros((n, d))
    if layer.shared is not None:
        y_sh = swiglu_expert(*expert_mats(layer.shared), x, round_h)
    y = np.einsum("nk,nkd->nd", w, y_slot) + y_sh
    return w, y_slot, y_sh, y


# ----------------------------------------------------------------------------
# mHC mix matrix (an op beside the MoE layer)
# ----------------------------------------------------------------------------

def mhc_sinkhorn(logits, iters: int = 10, eps: float = 0.0) -> np.ndarray:
    """Sinkhorn-normalised hyper-connection mix matrices, one n x n per token.

    [CARD4] "Architecture": the residual stream is hc_mult = 4 parallel copies
    recombined by a doubly-stochastic, Sinkhorn-normalised mix matrix; [PR1192]
    review notes: the unfused path is a softmax followed by iterations of a
    sum and a division (~40 launches per call). READINGS (iteration count and
    epsilon are not on the pages): softmax over each row, then ``iters``
    rounds of column normalisation followed by row normalisation, each a
    division by the sums (+ eps); 10 rounds make the pages' ~40 launches
    (1 + 10 x 2 x (sum + div)).
    logits: float [..., n, n] -> float64 [..., n, n]
    """
    l = np.asarray(logits, dtype=np.float64)
    m = np.exp(l - l.max(axis=-1, keepdims=True))
    m = m / m.sum(axis=-1, keepdims=True)
    for _ in range(iters):
        m = m / (m.sum(axis=-2, keepdims=True) + eps)
        m = m / (m.sum(axis=-1, keepdims=True) + eps)
    return m
