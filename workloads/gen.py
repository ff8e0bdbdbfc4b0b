"""Workload table and seeded generators.

Every workload is a batch of sequences that decode against a paged KV cache.
The shapes follow the pages' examples: a Llama-3-8B-shaped layer (32 query
heads, 8 KV heads, head dim 128), a Llama-3-70B-shaped layer (64/8/128) with
64 sequences of 8192 tokens, a shared system prompt with 5 drafted tokens for
speculative verification, and a 128K-token context split into 512-token
partitions.

Seeding: each sequence b of workload ``cfg_id`` owns the stream
``SeedSequence([218, cfg_id, b])`` (query rows, then keys, then values, then
the outlier positions), so any one sequence can be regenerated alone. Context
lengths, the pool's initial free order and a shared prefix each own a stream
of their own. Values are N(0, 1) float32; bf16 workloads round them to
bfloat16 with round-to-nearest-even and keep the raw uint16 bit patterns.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import List, Optional

import numpy as np

SEED = 218
_LEN_STREAM = 1_000_000
_PERM_STREAM = 1_000_001
_PREFIX_STREAM = 1_000_002
_TREE_STREAM = 1_000_003


@dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int
    batch: int
    q_len: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str                      # "f32" or "bf16": queries, outputs, K/V as written
    # K/V storage in the pool: "" = as dtype; "fp8" = OCP E4M3 codes with one
    # scale per (token, KV head), quantised from the bf16 rows when written
    kv_dtype: str = ""
    # context lengths: explicit list, constant, or integer-uniform [lo, hi]
    lens: Optional[tuple] = None
    len_const: int = 0
    len_lo: int = 0
    len_hi: int = 0
    # shared prefix (tokens) placed before every sequence's private tokens
    prefix_len: int = 0
    # physical pool: explicit size, or ceil(slack * blocks needed)
    num_blocks: int = 0
    pool_slack: float = 1.0
    # split-KV partition size in tokens requested by the workload (0 = auto)
    partition_tokens: int = 0
    # fraction of key vectors per (sequence, kv head) scaled by key_outlier_scale
    key_outlier_frac: float = 0.0
    key_outlier_scale: float = 1.0
    # shape of the q_len drafted tokens: "" = a chain (each continues the one
    # before), "random" = a random tree per sequence, "shared" = one random
    # tree for the whole batch. A tree is given by parent indices only.
    tree: str = ""

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


CONFIGS = {
    c.name: c
    for c in [
        Config("tiny_f32", 0, batch=4, q_len=1, num_q_heads=4, num_kv_heads=2,
               head_dim=64, block_size=16, dtype="f32", lens=(17, 33, 64, 100),
               num_blocks=32),
        Config("llama3_8b_decode", 1, batch=64, q_len=1, num_q_heads=32,
               num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16",
               len_lo=512, len_hi=4096, pool_slack=1.25),
        Config("llama3_70b_decode", 2, batch=64, q_len=1, num_q_heads=64,
               num_kv_heads=8, head_dim=128, block_size=32, dtype="bf16",
               len_const=8192),
        Config("prefix_verify", 3, batch=128, q_len=5, num_q_heads=32,
               num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16",
               prefix_len=512, len_lo=512, len_hi=3584, pool_slack=1.25),
        Config("long_ctx_split", 4, batch=4, q_len=1, num_q_heads=64,
               num_kv_heads=8, head_dim=128, block_size=32, dtype="bf16",
               len_const=131072, partition_tokens=512,
               key_outlier_frac=0.01, key_outlier_scale=8.0),
        # speculative verification of a tree of 8 drafted tokens per sequence
        # (4 query heads per KV head x 8 nodes = 32 rows per KV head)
        Config("tree_verify", 5, batch=128, q_len=8, num_q_heads=32,
               num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16",
               prefix_len=512, len_lo=512, len_hi=3584, pool_slack=1.25,
               tree="random"),
        # the 70B-shaped layer with an FP8 KV cache (same seeds and values as
        # llama3_70b_decode; the pool holds their E4M3 quantisation)
        Config("llama3_70b_decode_fp8", 2, batch=64, q_len=1, num_q_heads=64,
               num_kv_heads=8, head_dim=128, block_size=32, dtype="bf16",
               len_const=8192, kv_dtype="fp8"),
        # prefix-shared verification over an FP8 KV cache (same seeds and
        # values as prefix_verify)
        Config("prefix_verify_fp8", 3, batch=128, q_len=5, num_q_heads=32,
               num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16",
               prefix_len=512, len_lo=512, len_hi=3584, pool_slack=1.25,
               kv_dtype="fp8"),
    ]
}


def config(name: str, **overrides) -> Config:
    """A workload from the table, optionally resized (smaller batch, lengths...)."""
    return replace(CONFIGS[name], **overrides)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, *key])))


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = ((u + (((u >> 16) & 1) + np.uint32(0x7FFF))) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def context_lengths(cfg: Config) -> np.ndarray:
    """Total context length of each sequence, shared prefix included."""
    if cfg.lens is not None:
        lens = np.asarray(cfg.lens, dtype=np.int64)
        assert lens.size == cfg.batch
    elif cfg.len_const:
        lens = np.full(cfg.batch, cfg.len_const, dtype=np.int64)
    else:
        lens = _rng(cfg.cfg_id, _LEN_STREAM).integers(cfg.len_lo, cfg.len_hi + 1, size=cfg.batch)
    return (lens + cfg.prefix_len).astype(np.int32)


def pool_blocks(cfg: Config, lens: np.ndarray) -> int:
    """Physical pool size: explicit, or slack x (blocks the batch needs).

    With a shared prefix, the prefix's blocks are counted once and each
    sequence adds the blocks from the prefix's last full block onwards.
    """
    if cfg.num_blocks:
        return cfg.num_blocks
    bs = cfg.block_size
    per_seq = -(-lens.astype(np.int64) // bs)
    if cfg.prefix_len:
        need = -(-cfg.prefix_len // bs) + int((per_seq - cfg.prefix_len // bs).sum())
    else:
        need = int(per_seq.sum())
    return int(math.ceil(cfg.pool_slack * need))


def free_order(cfg: Config, num_blocks: int) -> np.ndarray:
    """Seeded permutation of the physical block ids: the pool's initial free order."""
    return _rng(cfg.cfg_id, _PERM_STREAM).permutation(num_blocks).astype(np.int32)


def _values(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    return x if dtype == "f32" else bf16_bits_from_f32(x)


def tree_parents(cfg: Config) -> Optional[np.ndarray]:
    """int32 [B][q_len] parent index of each drafted token (-1: continues the
    context), parents before children; None for a plain chain. Node j's parent
    is uniform over {-1, 0, ..., j-1}."""
    if not cfg.tree:
        return None
    if cfg.tree not in ("random", "shared"):
        raise ValueError(f"unknown tree shape {cfg.tree!r}")
    n_trees = 1 if cfg.tree == "shared" else cfg.batch
    out = np.empty((n_trees, cfg.q_len), dtype=np.int32)
    for t in range(n_trees):
        rng = _rng(cfg.cfg_id, _TREE_STREAM, t)
        out[t] = [rng.integers(-1, j) for j in range(cfg.q_len)]
    return np.repeat(out, cfg.batch, axis=0) if n_trees == 1 else out


@dataclass
class SeqData:
    """One sequence's query rows and its private (non-prefix) keys and values.

    q: [q_len][H_q][d]; k, v: [n_private][H_kv][d]; float32 or bf16 bits.
    """
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray


def sequence(cfg: Config, b: int, ctx_len: int) -> SeqData:
    rng = _rng(cfg.cfg_id, b)
    n_priv = int(ctx_len) - cfg.prefix_len
    shape = (n_priv, cfg.num_kv_heads, cfg.head_dim)
    q = rng.standard_normal((cfg.q_len, cfg.num_q_heads, cfg.head_dim), dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if cfg.key_outlier_frac:
        n_out = int(round(cfg.key_outlier_frac * n_priv))
        for g in range(cfg.num_kv_heads):
            pos = rng.choice(n_priv, size=n_out, replace=False)
            k[pos, g, :] *= np.float32(cfg.key_outlier_scale)
    if cfg.dtype == "bf16":
        q, k, v = bf16_bits_from_f32(q), bf16_bits_from_f32(k), bf16_bits_from_f32(v)
    return SeqData(q, k, v)


@dataclass
class Workload:
    cfg: Config
    lens: np.ndarray                 # int32 [B], total context incl. prefix
    num_blocks: int                  # physical pool size
    free_order: np.ndarray           # int32 [NB], initial free order
    seqs: List[SeqData] = field(default_factory=list)
    prefix_k: Optional[np.ndarray] = None   # [prefix_len][H_kv][d]
    prefix_v: Optional[np.ndarray] = None
    tree_parents: Optional[np.ndarray] = None   # int32 [B][q_len], or None (chain)

    @property
    def max_blocks(self) -> int:
        return int(-(-int(self.lens.max()) // self.cfg.block_size))

    def q_all(self) -> np.ndarray:
        """[B][q_len][H_q][d] query tensor."""
        return np.stack([s.q for s in self.seqs])

    def logical_kv(self, b: int):
        """Sequence b's contiguous K, V ([L_b][H_kv][d]), prefix first."""
        s = self.seqs[b]
        if self.prefix_k is None:
            return s.k, s.v
        return (np.concatenate([self.prefix_k, s.k]), np.concatenate([self.prefix_v, s.v]))


def generate(cfg: Config, threads: int = 8) -> Workload:
    lens = context_lengths(cfg)
    nb = pool_blocks(cfg, lens)
    w = Workload(cfg, lens, nb, free_order(cfg, nb), tree_parents=tree_parents(cfg))
    if cfg.prefix_len:
        rng = _rng(cfg.cfg_id, _PREFIX_STREAM)
        shape = (cfg.prefix_len, cfg.num_kv_heads, cfg.head_dim)
        w.prefix_k = _values(rng, shape, cfg.dtype)
        w.prefix_v = _values(rng, shape, cfg.dtype)
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        w.seqs = list(ex.map(lambda b: sequence(cfg, b, int(lens[b])), range(cfg.batch)))
    return w
