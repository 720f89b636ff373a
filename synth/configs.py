"""The synthetic MoE-layer workloads and their small variants.

Shapes follow DeepSeek-V4-Flash as the pages pin them: hidden d=4096, expert
intermediate I=2048, E=256 routed experts, top-6 routing (the hash table is
``tid2eid[vocab, 6]`` on the alphaneural card "DeepSeek-V4-Flash-MLX-4bit",
table "What this port implements"; 3 projections x 4096 x 2048 x 256 experts
x 43 layers = 277.0e9 routed weights, the figure on the card
"DeepSeek-V4-Flash-0731-MLX-Serve-mixed-2-3-8bit", calibration paragraph).

Precision recipes:
  * affine 4-bit group 64 routed experts: the conversion command on the card
    "mlx-community / DeepSeek-V4-Flash-4bit", section "Conversion";
  * MXFP4 (e2m1 + e8m0 per 32) routed experts: the native expert format named
    in mlx-lm PR 1192 "Add DeepSeek-v4 (Flash/Pro)" (mxfp4-default comment) and
    on the alphaneural card (FP4 e2m1 packed two per byte);
  * gate/up 2-bit g128, down 3-bit g128, shared experts 8-bit g64: the precision
    table of the "MLX-Serve-mixed-2-3-8bit" card.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional


@dataclass(frozen=True)
class FormatSpec:
    """How one stacked projection is quantised.

    fmt   -- "affine" (w = scale*q + bias, unsigned b-bit codes), "mxfp4"
             (e2m1 nibbles with one e8m0 exponent byte per 32 values) or
             "mxfp8" (e4m3 bytes with one e8m0 exponent byte per 32 values)
    bits  -- code width: 2, 3, 4 or 8 for affine; 4 for mxfp4; 8 for mxfp8
    group -- values sharing one scale(/bias) along the input dimension
    """

    fmt: str
    bits: int
    group: int

    def __post_init__(self):
        if self.fmt == "affine":
            assert self.bits in (2, 3, 4, 8), self.bits
            assert self.group in (32, 64, 128), self.group
        elif self.fmt == "mxfp4":
            assert self.bits == 4 and self.group == 32
        elif self.fmt == "mxfp8":
            assert self.bits == 8 and self.group == 32
        else:
            raise ValueError(self.fmt)


AFF4_G64 = FormatSpec("affine", 4, 64)
AFF8_G64 = FormatSpec("affine", 8, 64)
AFF2_G128 = FormatSpec("affine", 2, 128)
AFF3_G128 = FormatSpec("affine", 3, 128)
MXFP4 = FormatSpec("mxfp4", 4, 32)
MXFP8 = FormatSpec("mxfp8", 8, 32)


@dataclass(frozen=True)
class MoeConfig:
    """One synthetic MoE-layer workload.

    T tokens per step, hidden d, expert intermediate I, E routed experts,
    top_k experts per token. ``route`` is "topk" (sqrtsoftplus scores + bias,
    top-k) or "hash" (tid2eid table lookup). ``bias_kind``: "normal" draws the
    router bias from N(0, 0.1); "zipf" gives expert e the bias -0.11*ln(r_e)
    with r a seeded permutation of 1..E; "none" means no bias. ``shared`` is
    the always-on shared expert's format (None: no shared expert).
    ``steps`` is the number of distinct seeded activation batches (decode
    steps) the workload cycles through.
    """

    name: str
    seed: int
    T: int
    d: int
    I: int
    E: int
    top_k: int
    route: str
    gate_up: FormatSpec
    down: FormatSpec
    shared: Optional[FormatSpec] = None
    I_shared: int = 0
    vocab: int = 0
    steps: int = 1
    bias_kind: str = "normal"
    wr_std: float = 0.02
    bias_std: float = 0.1

    def __post_init__(self):
        assert self.route in ("topk", "hash")
        assert self.bias_kind in ("normal", "zipf", "none")
        assert 1 <= self.top_k <= self.E
        if self.route == "hash":
            assert self.vocab > 0
        if self.shared is not None:
            assert self.I_shared > 0

    @property
    def slots(self) -> int:
        return self.T * self.top_k


CONFIGS = {
    # T=4, d=256, I=128, E=16, k=2; affine 4-bit g64, no shared expert.
    "tiny": MoeConfig("tiny", 1, T=4, d=256, I=128, E=16, top_k=2, route="topk",
                      gate_up=AFF4_G64, down=AFF4_G64),
    # Batch-1 decode over 64 seeded steps; 4-bit g64 routed + 8-bit g64 shared.
    "decode": MoeConfig("decode", 2, T=1, d=4096, I=2048, E=256, top_k=6, route="topk",
                        gate_up=AFF4_G64, down=AFF4_G64, shared=AFF8_G64, I_shared=2048,
                        steps=64),
    # Hash-routed layer: T=512 tokens, tid2eid[129280][6].
    "hash": MoeConfig("hash", 3, T=512, d=4096, I=2048, E=256, top_k=6, route="hash",
                      gate_up=AFF4_G64, down=AFF4_G64, vocab=129280, bias_kind="none"),
    # Prefill: T=4096 tokens, MXFP4 experts, Zipf-skewed router bias.
    "prefill": MoeConfig("prefill", 4, T=4096, d=4096, I=2048, E=256, top_k=6, route="topk",
                         gate_up=MXFP4, down=MXFP4, bias_kind="zipf"),
    # Mixed low-bit decode batch: gate/up 2-bit g128, down 3-bit g128, shared 8-bit g64.
    "mixed": MoeConfig("mixed", 5, T=64, d=4096, I=2048, E=256, top_k=6, route="topk",
                       gate_up=AFF2_G128, down=AFF3_G128, shared=AFF8_G64, I_shared=2048),
    # MXFP8 experts (e4m3 + e8m0 per 32), T=512 tokens, top-6 routing.
    "mxfp8": MoeConfig("mxfp8", 6, T=512, d=4096, I=2048, E=256, top_k=6, route="topk",
                       gate_up=MXFP8, down=MXFP8),
}


def config(name: str) -> MoeConfig:
    return CONFIGS[name]


# The 43 MoE layers of one decode token through the whole model.
#  * precision per layer from the "DeepSeek-V4-Flash-0731-MLX-Serve-mixed-2-3-8bit"
#    precision table: routed gate/up affine 2-bit g128 and down 3-bit g128 in
#    layers 0-38, affine 4-bit g64 in layers 39-42; shared experts 8-bit g64;
#  * expert counts from the "REAP-pruned builds" section of the alphaneural
#    card "DeepSeek-V4-Flash-MLX-4bit": layers 0-2 route through the tid2eid
#    table and keep all 256 experts; the other 40 keep the 192 survivors of
#    REAP25, with the router rows of the survivors only (top-6 renormalised
#    over them).
STACK_LAYERS = 43
STACK_HASH_LAYERS = 3
STACK_4BIT_FROM = 39
STACK_SURVIVORS = 192


def stack_configs(T: int = 1, steps: int = 16) -> list:
    """Per-layer configs of the 43-layer stack (seed 100 + layer)."""
    out = []
    for l in range(STACK_LAYERS):
        hash_layer = l < STACK_HASH_LAYERS
        fmt_gu, fmt_dn = (AFF4_G64, AFF4_G64) if l >= STACK_4BIT_FROM else (AFF2_G128, AFF3_G128)
        out.append(MoeConfig(f"stack43_l{l}", 100 + l, T=T, d=4096, I=2048,
                             E=256 if hash_layer else STACK_SURVIVORS, top_k=6,
                             route="hash" if hash_layer else "topk", gate_up=fmt_gu, down=fmt_dn,
                             shared=AFF8_G64, I_shared=2048, vocab=129280 if hash_layer else 0,
                             bias_kind="none" if hash_layer else "normal", steps=steps))
    return out


def variant(base: MoeConfig | str, name: str, seed: int, **changes) -> MoeConfig:
    """A smaller or reshaped copy of a workload under its own seed."""
    if isinstance(base, str):
        base = CONFIGS[base]
    return replace(base, name=name, seed=seed, **changes)
