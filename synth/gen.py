"""Seeded generators for every input of the MoE layer.

Seeding: every array comes from its own PCG64 stream,
``SeedSequence(entropy=cfg.seed, spawn_key=key)``, so any one expert (or any
decode step's activations) can be drawn alone and is bit-identical to the
same slice of the fully stacked tensor:

  key (0,)        router weight Wr, fp32 N(0, wr_std)          [E][d]
  key (1,)        router bias, fp32 N(0, bias_std) or Zipf      [E]
  key (2, step)   activations, N(0,1) drawn in fp32 -> bf16 RNE  [T][d]
  key (3, step)   token ids, uniform over [0, vocab)             [T]
  key (4,)        tid2eid rows, each a uniform random k-subset  [vocab][k]
  key (5, m)      shared expert projection m (0 gate, 1 up, 2 down)
  key (6, e, m)   routed expert e, projection m
  key (7, i)      bf16 source weights for the quantiser, N(0, 0.02)

Packed codes are drawn directly as uniform uint32 words: for 2/4/8-bit codes,
for nibble pairs, and for 3-bit streams whose rows are a whole number of words
this is exactly "codes uniform over [0, 2^b)". Affine scales are
U(0.001, 0.01) * 16 / 2^b rounded to fp16 and biases are -2^(b-1) * scale, so
every affine format spans the same +-8*U(0.001, 0.01) weight range (for b=4
this is scale U(0.001, 0.01), bias -8*scale). e8m0 bytes are uniform over
118..124 (mxfp4) or 110..116 (mxfp8, whose codes reach 448). mxfp8 code bytes
are uniform over the 254 finite e4m3 codes (0x7F and 0xFF are NaN).

Layouts (row-major, rows = output features, cols = input features, codes
packed along cols as one LSB-first bit stream of little-endian uint32 words):
  codes  uint32  [n][rows][cols*bits/32]
  scales fp16    [n][rows][cols/group]   (affine)   | uint8 e8m0 [n][rows][cols/32] (mxfp4, mxfp8)
  biases fp16    [n][rows][cols/group]   (affine)   | None                          (mxfp4, mxfp8)
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import FormatSpec, MoeConfig


def _rng(cfg: MoeConfig, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=cfg.seed, spawn_key=key)))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


@dataclass
class QTensor:
    """A stack of n quantised [rows][cols] projections (see module doc)."""

    spec: FormatSpec
    rows: int
    cols: int
    codes: np.ndarray
    scales: np.ndarray
    biases: Optional[np.ndarray]

    @property
    def n(self) -> int:
        return self.codes.shape[0]

    @property
    def words_per_row(self) -> int:
        return self.cols * self.spec.bits // 32

    def expert(self, e: int) -> "QTensor":
        return QTensor(self.spec, self.rows, self.cols, self.codes[e:e + 1], self.scales[e:e + 1],
                       None if self.biases is None else self.biases[e:e + 1])

    def nbytes_per_expert(self) -> int:
        b = self.codes[0].nbytes + self.scales[0].nbytes
        if self.biases is not None:
            b += self.biases[0].nbytes
        return b


@dataclass
class ExpertWeights:
    gate: QTensor  # w1 [I][d]
    up: QTensor    # w3 [I][d]
    down: QTensor  # w2 [d][I]

    def expert(self, e: int) -> "ExpertWeights":
        return ExpertWeights(self.gate.expert(e), self.up.expert(e), self.down.expert(e))

    def nbytes_per_expert(self) -> int:
        return sum(q.nbytes_per_expert() for q in (self.gate, self.up, self.down))


@dataclass
class Layer:
    cfg: MoeConfig
    wr: np.ndarray                   # fp32 [E][d]
    bias: Optional[np.ndarray]       # fp32 [E]
    tid2eid: Optional[np.ndarray]    # int32 [vocab][k]
    routed: Optional[ExpertWeights]  # stacked [E], or None when drawn lazily
    shared: Optional[ExpertWeights]  # n = 1

    def routed_expert(self, e: int) -> ExpertWeights:
        if self.routed is not None:
            return self.routed.expert(e)
        return gen_expert(self.cfg, e)


def _empty_qtensor(spec: FormatSpec, rows: int, cols: int, n: int) -> QTensor:
    assert (cols * spec.bits) % 32 == 0 and cols % spec.group == 0
    w = cols * spec.bits // 32
    ng = cols // spec.group
    codes = np.empty((n, rows, w), dtype=np.uint32)
    if spec.fmt == "affine":
        return QTensor(spec, rows, cols, codes, np.empty((n, rows, ng), np.float16),
                       np.empty((n, rows, ng), np.float16))
    return QTensor(spec, rows, cols, codes, np.empty((n, rows, ng), np.uint8), None)


def _fill(q: QTensor, i: int, rng: np.random.Generator) -> None:
    rows, w = q.codes.shape[1], q.codes.shape[2]
    ng = q.scales.shape[2]
    if q.spec.fmt == "mxfp8":
        b = rng.integers(0, 254, size=(rows, 4 * w), dtype=np.uint16)
        b = (b + (b >= 0x7F)).astype(np.uint8)
        q.codes[i] = np.ascontiguousarray(b).view("<u4")
        q.scales[i] = rng.integers(110, 117, size=(rows, ng), dtype=np.uint8)
        return
    q.codes[i] = rng.integers(0, 2 ** 32, size=(rows, w), dtype=np.uint32)
    if q.spec.fmt == "affine":
        b = q.spec.bits
        s = (rng.uniform(0.001, 0.01, size=(rows, ng)) * (16.0 / 2 ** b)).astype(np.float16)
        q.scales[i] = s
        q.biases[i] = (np.float32(-(2 ** (b - 1))) * s.astype(np.float32)).astype(np.float16)
    else:
        q.scales[i] = rng.integers(118, 125, size=(rows, ng), dtype=np.uint8)


def _alloc_experts(cfg: MoeConfig, n: int, shared: bool) -> ExpertWeights:
    if shared:
        fmt_gu = fmt_dn = cfg.shared
        inter = cfg.I_shared
    else:
        fmt_gu, fmt_dn, inter = cfg.gate_up, cfg.down, cfg.I
    return ExpertWeights(_empty_qtensor(fmt_gu, inter, cfg.d, n),
                         _empty_qtensor(fmt_gu, inter, cfg.d, n),
                         _empty_qtensor(fmt_dn, cfg.d, inter, n))


def _fill_expert(ew: ExpertWeights, i: int, cfg: MoeConfig, key_prefix: tuple) -> None:
    for m, q in enumerate((ew.gate, ew.up, ew.down)):
        _fill(q, i, _rng(cfg, *key_prefix, m))


def gen_expert(cfg: MoeConfig, e: int) -> ExpertWeights:
    """Routed expert e alone (n = 1), identical to slice e of the stack."""
    assert 0 <= e < cfg.E
    ew = _alloc_experts(cfg, 1, shared=False)
    _fill_expert(ew, 0, cfg, (6, e))
    return ew


def gen_routed_stacked(cfg: MoeConfig) -> ExpertWeights:
    ew = _alloc_experts(cfg, cfg.E, shared=False)
    for e in range(cfg.E):
        _fill_expert(ew, e, cfg, (6, e))
    return ew


def gen_shared(cfg: MoeConfig) -> Optional[ExpertWeights]:
    if cfg.shared is None:
        return None
    ew = _alloc_experts(cfg, 1, shared=True)
    _fill_expert(ew, 0, cfg, (5,))
    return ew


def gen_bf16_weights(seed: int, i: int, rows: int, cols: int, std: float = 0.02) -> np.ndarray:
    """Unquantised bf16 weights (uint16 bits) [rows][cols], N(0, std), the
    quantiser's input (stream key (7, i) under ``seed``)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=(7, i))))
    return f32_to_bf16_bits(rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(std))


def gen_router(cfg: MoeConfig):
    wr = _rng(cfg, 0).standard_normal((cfg.E, cfg.d), dtype=np.float32) * np.float32(cfg.wr_std)
    rng = _rng(cfg, 1)
    if cfg.bias_kind == "normal":
        bias = (rng.standard_normal(cfg.E, dtype=np.float32) * np.float32(cfg.bias_std)).astype(np.float32)
    elif cfg.bias_kind == "zipf":
        r = rng.permutation(cfg.E).astype(np.float64) + 1.0
        bias = (-0.11 * np.log(r)).astype(np.float32)
    else:
        bias = None
    return np.ascontiguousarray(wr, dtype=np.float32), bias


def gen_tid2eid(cfg: MoeConfig) -> Optional[np.ndarray]:
    """Each row a uniform random k-subset of [0, E) (distinct entries)."""
    if cfg.route != "hash":
        return None
    rng = _rng(cfg, 4)
    t = rng.integers(0, cfg.E, size=(cfg.vocab, cfg.top_k), dtype=np.int32)
    while True:
        s = np.sort(t, axis=1)
        bad = np.any(s[:, 1:] == s[:, :-1], axis=1)
        nbad = int(bad.sum())
        if nbad == 0:
            return t
        t[bad] = rng.integers(0, cfg.E, size=(nbad, cfg.top_k), dtype=np.int32)


def gen_x(cfg: MoeConfig, step: int = 0, T: Optional[int] = None) -> np.ndarray:
    """Activations for one step: bf16 bits (uint16) [T][d]."""
    T = cfg.T if T is None else T
    a = _rng(cfg, 2, step).standard_normal((T, cfg.d), dtype=np.float32)
    return f32_to_bf16_bits(a)


def gen_token_ids(cfg: MoeConfig, step: int = 0, T: Optional[int] = None) -> Optional[np.ndarray]:
    if cfg.route != "hash":
        return None
    T = cfg.T if T is None else T
    return _rng(cfg, 3, step).integers(0, cfg.vocab, size=T, dtype=np.int32)


def gen_layer(cfg: MoeConfig, routed: bool = True) -> Layer:
    """The whole layer; with ``routed=False`` experts are drawn on demand."""
    wr, bias = gen_router(cfg)
    return Layer(cfg, wr, bias, gen_tid2eid(cfg), gen_routed_stacked(cfg) if routed else None,
                 gen_shared(cfg))
