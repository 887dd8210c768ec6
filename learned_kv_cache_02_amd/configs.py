"""The five synthetic workloads the Nectar hot path is measured and checked on.

Shapes follow Qwen3-4B, Qwen2.5-7B-1M and Llama-3.1-8B attention layers
(KV heads, query heads, head dim); the document lengths stand in for the
documents of Table 1 of the Nectar reading notes (section 3.1), which are not
available here.  Every tensor is drawn from a seeded N(0, 1) (modules:
N(0, 1/fan_in)); see ``synth.py`` for the recipe.

Local part (section 2.2 of the notes): a question's own tokens after the
document.  ``prompt`` tokens are already in the local cache; decode step ``s``
adds token ``prompt + s`` and its query sees local keys ``0 .. prompt + s``.
Prefill workloads (``decode_steps == 0``) run ``Tq == prompt`` causal query
tokens at once.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class MLPShape:
    Ht: int          # target hidden width (d -> Ht -> d)
    Hs: int          # score hidden width  (d -> Hs -> 1)

    def params(self, d: int) -> int:
        """Parameters per KV head including all biases."""
        return (d * self.Ht + self.Ht + self.Ht * d + d) + (d * self.Hs + self.Hs + self.Hs + 1)


@dataclass(frozen=True)
class DeepShape:
    """Deep module of Eq. (3.6): depths (D_b, D_s, D_t) of the shared backbone,
    score head and target head, and their widths (H_b, H_s, H_t)."""
    depth: Tuple[int, int, int]
    width: Tuple[int, int, int]

    def layers(self):
        """(width, input-state width) of every layer, backbone, score, target."""
        Db, Ds, Dt = self.depth
        out = []
        for part, D in enumerate(self.depth):
            H = self.width[part]
            for l in range(D):
                out.append((H, H if l > 0 else (self.width[0] if part > 0 and Db > 0 else 0)))
        return out

    def last_width(self, head: int) -> int:
        return self.width[head] if self.depth[head] > 0 else self.width[0]

    def params(self, d: int) -> int:
        """Parameters per KV head including all biases."""
        n = sum(H * d + H * H_in + H for H, H_in in self.layers())
        return n + (self.last_width(1) + 1) + (d * self.last_width(2) + d)


@dataclass(frozen=True)
class Config:
    name: str
    seed: int
    dtype: str               # "f32" or "bf16": storage type of q, caches and weights
    layers: int
    Hkv: int
    Hq: int
    d: int
    n: int                   # document tokens
    rope_base: float
    B: int                   # concurrent questions
    prompt: int              # local tokens per question before the first decode step
    decode_steps: int        # 0: one causal prefill chunk of `prompt` tokens per question
    mlps: Tuple[MLPShape, ...] = field(default_factory=tuple)
    kv_pairs: int = 0        # Quadrature pairs p (0: form not used)
    description: str = ""

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def prefill(self) -> bool:
        return self.decode_steps == 0

    @property
    def Tq(self) -> int:
        """Query tokens per question in one step."""
        return self.prompt if self.prefill else 1

    @property
    def R(self) -> int:
        """Query tokens per step."""
        return self.B * self.Tq

    @property
    def T_cap(self) -> int:
        """Local cache capacity per (question, KV head)."""
        return self.prompt if self.prefill else self.prompt + self.decode_steps

    def local_len(self, step: int = 0) -> int:
        """Valid local keys at a step."""
        return self.prompt if self.prefill else self.prompt + step + 1

    def q_offset(self, step: int = 0) -> int:
        """Local index seen by query token 0 of a step (it sees 0..q_offset+t)."""
        return 0 if self.prefill else self.prompt + step

    def query_pos(self, step: int = 0):
        """Absolute RoPE positions of the Tq query tokens of a step."""
        if self.prefill:
            return [self.n + t for t in range(self.prompt)]
        return [self.n + self.prompt + step]

    def rho(self, params_per_head: int) -> float:
        """Capacity ratio |theta| / (2 n d) per (layer, KV head)."""
        return params_per_head / (2.0 * self.n * self.d)


C1 = Config("c1_tiny_f32", 0, "f32", 1, 1, 2, 64, 512, 1e4, 1, 16, 0,
            (MLPShape(256, 256),), 0,
            "tiny single head, fp32: n=512, 16 local causal tokens")
C2 = Config("c2_qwen3_4b_decode", 1, "bf16", 1, 8, 32, 128, 61440, 1e6, 1, 512, 1,
            (MLPShape(4608, 2944),), 0,
            "Qwen3-4B-shaped layer, decode batch 1, n=61,440, 512 prompt + 1 decode token")
C3 = Config("c3_qwen25_7b_prefill", 2, "bf16", 28, 4, 28, 128, 131072, 1e7, 16, 1024, 0,
            (MLPShape(768, 512), MLPShape(7680, 5120)), 0,
            "Qwen2.5-7B-1M-shaped 28-layer stack, prefill 16 x 1,024 tokens, n=131,072")
C4 = Config("c4_llama31_8b_decode", 3, "bf16", 32, 8, 32, 128, 262144, 5e5, 64, 256, 128,
            (MLPShape(9984, 6144),), 0,
            "Llama-3.1-8B-shaped 32-layer stack, decode batch 64, n=262,144")
C5 = Config("c5_qwen25_7b_1m_decode", 4, "bf16", 28, 4, 28, 128, 1048576, 1e7, 8, 256, 128,
            (MLPShape(5120, 3072),), 10486,
            "Qwen2.5-7B-1M-shaped 28-layer stack, 1M-token document, decode batch 8")

CONFIGS = {c.name: c for c in (C1, C2, C3, C4, C5)}
BY_INDEX = [C1, C2, C3, C4, C5]

# Deep modules of Eq. (3.6) in the two depth shapes the notes plot, (0, 2, 3) and
# (2, 1, 2), sized to about the capacity of the Qwen3-4B-shaped layer's
# one-hidden-layer module (rho ~ 10 %).
DEEP_C2 = (DeepShape((0, 2, 3), (0, 576, 576)), DeepShape((2, 1, 2), (544, 544, 544)))


# Layer-wise capacity allocation (App. C.1, Table 10 of the notes): layer groups
# [0, 9), [9, 15), [15, 27), [27, 28) of a 28-layer stack with multipliers
# (1, 2, 5, 2), normalised so the total capacity stays that of the uniform
# allocation.  The score/target study of App. C.2 uses (1, 2, 8, 12) on the same
# groups.
TABLE10_BOUNDS = (0, 9, 15, 27, 28)
TABLE10_MULT = (1, 2, 5, 2)
TABLE11_MULT = (1, 2, 8, 12)


def layer_capacity_factors(bounds=TABLE10_BOUNDS, mult=TABLE10_MULT):
    """Per-layer capacity factor m_l / mean(m): the group multiplier divided by its
    layer-count-weighted mean (83/28 for Table 10), so the factors sum to the
    layer count."""
    sizes = [hi - lo for lo, hi in zip(bounds[:-1], bounds[1:])]
    L = bounds[-1] - bounds[0]
    mean = sum(n * m for n, m in zip(sizes, mult)) / L
    return [m / mean for n, m in zip(sizes, mult) for _ in range(n)]


def mlp_widths_for_budget(params: float, d: int, score_frac: float, multiple: int = 64):
    """Hidden widths (Ht, Hs) of a one-hidden-layer module with about `params`
    parameters per KV head, `score_frac` of them in the score net, each width
    rounded to a multiple of `multiple` (at least one multiple)."""
    def rnd(x):
        return max(multiple, int(round(x / multiple)) * multiple)
    pt, ps = params * (1.0 - score_frac), params * score_frac
    return rnd((pt - d) / (2 * d + 1)), rnd((ps - 1) / (d + 2))


def allocated_mlps(cfg: "Config", rho: float, score_frac: float, bounds=TABLE10_BOUNDS, mult=TABLE10_MULT):
    """Per-layer module shapes of a stack at total capacity ratio `rho`
    (|theta| / (2 n d) per layer and KV head on average), allocated by layer group."""
    base = rho * 2.0 * cfg.n * cfg.d
    return [MLPShape(*mlp_widths_for_budget(base * f, cfg.d, score_frac))
            for f in layer_capacity_factors(bounds, mult)]
