"""Seeded inputs for speculative decoding's accept / resample step.

Per sequence: target probabilities p over the vocabulary at the K drafted
positions and one more, draft probabilities q at the K drafted positions,
draft tokens drawn from q, one float32 uniform per draft and one 32-bit
integer per sequence. Distributions come from N(0, sigma^2) logits (a peaked
next-token distribution); the draft's logits are the target's plus
N(0, noise^2), so that the draft mostly agrees with the target, as the pages'
70-85% acceptance rates describe. Random numbers only: none of the accept /
resample arithmetic lives here.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

SEED = 218


@dataclass(frozen=True)
class SpecConfig:
    name: str
    cfg_id: int
    batch: int
    k: int              # drafted tokens per sequence
    vocab: int
    sigma: float = 6.0  # logit scale
    noise: float = 0.5  # draft logit noise


SPEC_CONFIGS = {
    c.name: c
    for c in [
        # 64 sequences, 5 drafts each (Blog #54's K = 5), Llama-3 vocabulary
        SpecConfig("spec_accept", 20, batch=64, k=5, vocab=128256),
        SpecConfig("spec_tiny", 21, batch=6, k=3, vocab=40),
    ]
}


def spec_config(name: str, **overrides) -> SpecConfig:
    return replace(SPEC_CONFIGS[name], **overrides)


def _softmax_f32(logits: np.ndarray) -> np.ndarray:
    z = logits - logits.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)


@dataclass
class SpecInputs:
    cfg: SpecConfig
    p: np.ndarray          # float32 [B][K+1][V]
    q: np.ndarray          # float32 [B][K][V]
    draft: np.ndarray      # int32 [B][K], drawn from q
    u_accept: np.ndarray   # float32 [B][K] in [0, 1)
    u_draw: np.ndarray     # uint32 [B]


def generate_spec(cfg: SpecConfig) -> SpecInputs:
    B, K, V = cfg.batch, cfg.k, cfg.vocab
    p = np.empty((B, K + 1, V), dtype=np.float32)
    q = np.empty((B, K, V), dtype=np.float32)
    draft = np.empty((B, K), dtype=np.int32)
    u_accept = np.empty((B, K), dtype=np.float32)
    u_draw = np.empty(B, dtype=np.uint32)
    for b in range(B):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, cfg.cfg_id, b])))
        logits = rng.standard_normal((K + 1, V)) * cfg.sigma
        p[b] = _softmax_f32(logits)
        q[b] = _softmax_f32(logits[:K] + rng.standard_normal((K, V)) * cfg.noise)
        # the draft model samples its tokens from q
        for k in range(K):
            c = np.cumsum(q[b, k].astype(np.float64))
            draft[b, k] = min(int(np.searchsorted(c, rng.random() * c[-1], side="right")), V - 1)
        u_accept[b] = rng.random(K, dtype=np.float32)
        u_draw[b] = rng.integers(0, 2 ** 32, dtype=np.uint64)
    return SpecInputs(cfg, p, q, draft, u_accept, u_draw)
