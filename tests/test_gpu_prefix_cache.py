"""Requests that reuse a cached prompt through the radix prefix cache give
the oracle's attention and the same bits as requests that wrote the prompt
themselves (MI355X)."""
import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from tests.gpu_util import assert_close, oracle_rows, out_bits, out_to_f64  # noqa: E402


@pytest.mark.parametrize("prefix_len", [64, 72])   # whole blocks / a partial last prompt block
def test_prefix_cache_reuse_matches_private_writes(prefix_len):
    from paged_kv_cache_218_amd.cache import (PagedKVCache, _to_device, lens_to_device,
                                              queries_to_device)
    cfg = workloads.config("prefix_verify", batch=5, prefix_len=prefix_len, len_lo=20, len_hi=90)
    w = workloads.generate(cfg)
    bs = cfg.block_size
    rng = np.random.default_rng(3)
    prompt = rng.integers(0, 32000, size=prefix_len).tolist()          # the shared prompt's token ids
    own = [rng.integers(0, 32000, size=int(w.lens[b]) - prefix_len).tolist() for b in range(cfg.batch)]
    tdt = torch.bfloat16
    print(f"prefix cache reuse, prompt {prefix_len}", flush=True)

    def build(use_cache):
        c = PagedKVCache(w.num_blocks * 2, bs, cfg.num_kv_heads, cfg.head_dim, tdt, cfg.batch, w.max_blocks,
                         w.free_order.tolist() + list(range(w.num_blocks, 2 * w.num_blocks)))
        pk, pv = _to_device(w.prefix_k, tdt, "cuda"), _to_device(w.prefix_v, tdt, "cuda")
        if use_cache:
            c.enable_prefix_cache()
        for b in range(cfg.batch):
            start = c.match_prefix(b, prompt + own[b]) if use_cache else 0
            if b > 0 and use_cache:
                assert start == prefix_len // bs * bs                  # the prompt's whole blocks
            if start < prefix_len:
                c.write(b, start, pk[start:], pv[start:])
            s = w.seqs[b]
            c.write(b, prefix_len, _to_device(s.k, tdt, "cuda"), _to_device(s.v, tdt, "cuda"))
            if use_cache and b == 0:
                assert c.insert_prefix(b, prompt) == prefix_len // bs
        return c

    outs = []
    for use_cache in (False, True):
        c = build(use_cache)
        q, lens = queries_to_device(w), lens_to_device(w)
        o = c.attention(q, c.tables_device(), lens, cfg.q_len, cfg.scale, int(w.lens.max()))
        torch.cuda.synchronize()
        outs.append((o, c))
    ref = oracle_rows(w, range(cfg.batch))
    got = out_to_f64(outs[1][0], cfg.dtype)
    for b in range(cfg.batch):
        assert_close(got[b], ref[b], cfg.dtype, f"seq {b}")
    assert np.array_equal(out_bits(outs[0][0]), out_bits(outs[1][0]))
    c = outs[1][1]
    import paged_kv_cache_218_amd as pa
    nblk = prefix_len // bs
    for j in range(nblk):                       # every request holds the cached prompt blocks
        assert pa.pa_block_refcount(c.pool, int(c.tables[0, j])) == cfg.batch
    assert (c.tables[:, :nblk] == c.tables[0, :nblk]).all()


def test_rewrite_of_cached_block_copies_it_on_device():
    """A request that rewrites a position inside a cached block gets a copy;
    the cached block (and every other request's output) is unchanged."""
    from paged_kv_cache_218_amd.cache import PagedKVCache, _to_device, lens_to_device, queries_to_device
    cfg = workloads.config("prefix_verify", batch=3, prefix_len=64, len_lo=20, len_hi=40)
    w = workloads.generate(cfg)
    tdt = torch.bfloat16
    prompt = list(range(64))
    c = PagedKVCache(w.num_blocks * 2, cfg.block_size, cfg.num_kv_heads, cfg.head_dim, tdt, cfg.batch,
                     w.max_blocks)
    c.enable_prefix_cache()
    pk, pv = _to_device(w.prefix_k, tdt, "cuda"), _to_device(w.prefix_v, tdt, "cuda")
    for b in range(cfg.batch):
        start = c.match_prefix(b, prompt)
        if start < 64:
            c.write(b, start, pk[start:], pv[start:])
        s = w.seqs[b]
        c.write(b, 64, _to_device(s.k, tdt, "cuda"), _to_device(s.v, tdt, "cuda"))
        if b == 0:
            c.insert_prefix(b, prompt)
    q, lens = queries_to_device(w), lens_to_device(w)
    before = c.attention(q, c.tables_device(), lens, cfg.q_len, cfg.scale, int(w.lens.max())).clone()
    cached_block = int(c.tables[2, 1])
    # request 2 overwrites position 20 (cached block 1) with its own K/V row
    row = _to_device(w.seqs[2].k[:1], tdt, "cuda")
    c.write(2, 20, row, row)
    print("prefix cache rewrite", flush=True)
    assert int(c.tables[2, 1]) != cached_block and int(c.tables[0, 1]) == cached_block
    after = c.attention(q, c.tables_device(), lens, cfg.q_len, cfg.scale, int(w.lens.max()))
    torch.cuda.synchronize()
    a, b_ = out_bits(before), out_bits(after)
    assert np.array_equal(a[:2], b_[:2]) and not np.array_equal(a[2], b_[2])
