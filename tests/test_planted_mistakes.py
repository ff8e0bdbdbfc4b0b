"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch each one: a wrong GQA head map, a wrong scale, an off-by-one causal
bound, K and V swapped, a transposed V slot, a wrong in-block offset, a
missing softmax normalisation, a merge without the max rescale, a doubled
byte count, a FIFO free list, two FP8 codec mistakes, two tree-mask
mistakes (ancestor sets cut to the parent, draft positions shifted by one)
three in the accept / resample step (resampling from p instead of the
residual, the acceptance ratio inverted, a non-strict inverse-CDF bound) and
two in the prefix cache (evicting blocks that still have cached children,
writing into a cached block in place)."""
import numpy as np
import pytest

import oracle.allocator as oalloc
import oracle.attention as oatt
import oracle.kvbytes as okv
import oracle.split as osplit
import oracle.store as ostore
from oracle.numerics import to_f64
from tests import test_oracle_pins as pins
from tests import test_allocator_model as apins
from tests import test_oracle_fp8 as fpins
import oracle.fp8 as ofp8
import oracle.tree as otree
import oracle.spec as ospec
import oracle.prefix_cache as opc
from tests import test_prefix_cache_model as pcpins
from tests import test_oracle_tree as tpins
from tests import test_oracle_spec as spins


def run_pins():
    """Run a representative set of pins; return the names of those that fail."""
    checks = {
        "brute": lambda: pins.test_oracle_vs_brute_force("bf16", 4, 4, 1, 64, 8, (4, 11, 20)),
        "brute_gqa": lambda: pins.test_oracle_vs_brute_force("bf16", 1, 8, 2, 32, 4, (3, 8, 13)),
        "brute_logical": lambda: pins.test_oracle_vs_brute_force_on_never_paged_kv(
            "bf16", 3, 8, 2, 32, 4, (3, 8, 13), 0),
        "sdpa_verify": lambda: pins.test_oracle_vs_torch_sdpa("prefix_verify"),
        "sdpa_decode": lambda: pins.test_oracle_vs_torch_sdpa("llama3_8b_decode"),
        "tables": lambda: [pins.test_printed_block_tables(c) for c in
                           pins.json.load(open(pins.os.path.join(pins.GOLDEN, "block_tables.json")))["cases"]],
        "one_token": pins.test_one_token_context_returns_v_exactly,
        "split": lambda: pins.test_split_merge_equals_direct(512),
        "kvbytes": lambda: [pins.test_kv_bytes_closed_form(c) for c in
                            pins.json.load(open(pins.os.path.join(pins.GOLDEN, "kv_bytes.json")))["cases"]],
        "lifo": apins.test_initial_free_order_and_lifo_reuse,
        "fp8_codec": fpins.test_decode_table_matches_torch_float8_e4m3fn,
        "fp8_attention": lambda: fpins.test_fp8_pool_attention_vs_torch_sdpa(
            "llama3_70b_decode_fp8", dict(batch=2, len_const=100)),
        "cow": apins.test_four_samples_share_prompt_then_copy_only_the_diverging_block,
        "tree_literal": tpins.test_ancestor_masks_literal,
        "spec_identity": spins.test_emitted_token_has_the_target_distribution,
        "spec_draw": spins.test_draw_boundaries_are_exact,
        "spec_accept": spins.test_acceptance_is_the_float32_comparison,
        "pc_lru": pcpins.test_lru_evicts_oldest_unreferenced_leaf_first,
        "pc_cow": pcpins.test_write_into_cached_block_copies_it,
        "pc_stream": lambda: pcpins.test_random_request_stream_invariants_and_longest_match(1),
        "tree_sdpa": lambda: tpins.test_tree_vs_torch_sdpa_with_parent_walk_mask(dict()),
    }
    failed = []
    for name, fn in checks.items():
        try:
            fn()
        except Exception:
            failed.append(name)
    return failed


def test_pins_pass_on_the_real_oracle():
    assert run_pins() == []


def _seq_mutant(head_map=None, scale_mul=1.0, causal_shift=0, swap_kv=False, normalise=True):
    def attention_paged_seq(q, pool, table, ctx_len, q_len, num_q_heads, scale):
        G = num_q_heads // pool.hkv
        qf = to_f64(q, pool.dtype)
        out = np.empty(qf.shape)
        for h in range(num_q_heads):
            g = head_map(h, G, pool.hkv) if head_map else h // G
            kr, vr = pool.gather_head(table, ctx_len, g)
            if swap_kv:
                kr, vr = vr, kr
            kf, vf = to_f64(kr, pool.dtype), to_f64(vr, pool.dtype)
            for i in range(q_len):
                last = min(ctx_len - 1, ctx_len - q_len + i + causal_shift)
                s = scale * scale_mul * (kf[:last + 1] @ qf[i, h])
                e = np.exp(s - s.max())
                p = e / e.sum() if normalise else e
                out[i, h] = p @ vf[:last + 1]
        return out
    return attention_paged_seq


def _gather_mutant(kind):
    def gather_head(self, table, ctx_len, g):
        pos = np.arange(ctx_len)
        blk = np.asarray(table, dtype=np.int64)[pos // self.bs]
        off = pos % self.bs
        kr = lambda o: self.k[blk, g, :, o, :].reshape(ctx_len, self.d)
        if kind == "v_transposed":
            flat = self.v[:, g].transpose(0, 2, 1)          # pretend v were [bs][d] row-major
            return kr(off), flat.reshape(self.nb, self.d, self.bs)[blk, :, off]
        if kind == "offset":
            off = (pos // self.bs) % self.bs
        return kr(off), self.v[blk, g, :, off]
    return gather_head


def _merge_no_rescale(m, l, o):
    w = l
    return (w[:, :, None] * o).sum(axis=0) / w.sum(axis=0)[:, None]


def _ancestors_parent_only(parents):
    return [(1 << i) | ((1 << int(p)) if p >= 0 else 0) for i, p in enumerate(parents)]


_real_visible = otree.visible_positions


def _visible_shifted(L, q_len, mask, i):
    pos = _real_visible(L, q_len, mask, i)
    ctx = L - q_len
    return np.where(pos >= ctx, pos - 1, pos)


def _accept_inverted(p_x, q_x, u):
    p_x, q_x, u = np.float32(p_x), np.float32(q_x), np.float32(u)
    return bool(q_x >= p_x or np.float32(u * p_x) < q_x)


def _draw_non_strict(weights, U):
    ints = ospec.fixed_weights(weights)
    S = sum(ints)
    if S == 0:
        raise ValueError("all weights are zero")
    T = (int(U) * S) >> ospec.FIXED_SHIFT
    run = 0
    for x, v in enumerate(ints):
        run += v
        if run >= T:
            return x
    return len(ints) - 1


def _evict_any(self):
    victim = min(self.unref_time, key=lambda b: (self.unref_time[b], b))
    del self.children[self.parent[victim]][self.key[victim]]
    for child in list(self.children[victim].values()):
        self.parent[child] = None                       # orphans re-hung under the root
    del self.children[victim], self.parent[victim], self.key[victim], self.unref_time[victim]
    return victim


class FifoPool(oalloc.BlockPoolModel):
    def alloc(self):
        if not self._stack:
            raise oalloc.PoolError(oalloc.ERR_NO_FREE_BLOCK)
        blk = self._stack.pop()
        self.refcount[blk] = 1
        return blk

    def free(self, blk):
        self._check(blk)
        if self.refcount[blk] == 0:
            raise oalloc.PoolError(oalloc.ERR_BAD_BLOCK)
        self.refcount[blk] -= 1
        if self.refcount[blk] == 0:
            self._stack.insert(0, blk)                       # tail instead of head


MUTANTS = {
    "head_map_modulo": lambda mp: mp.setattr(oatt, "attention_paged_seq", _seq_mutant(head_map=lambda h, G, H: h % H)),
    "scale_wrong": lambda mp: mp.setattr(oatt, "attention_paged_seq", _seq_mutant(scale_mul=np.sqrt(2.0))),
    "causal_off_by_one": lambda mp: mp.setattr(oatt, "attention_paged_seq", _seq_mutant(causal_shift=1)),
    "k_v_swapped": lambda mp: mp.setattr(oatt, "attention_paged_seq", _seq_mutant(swap_kv=True)),
    "softmax_unnormalised": lambda mp: mp.setattr(oatt, "attention_paged_seq", _seq_mutant(normalise=False)),
    "v_layout_transposed": lambda mp: mp.setattr(ostore.HostPool, "gather_head", _gather_mutant("v_transposed")),
    "in_block_offset": lambda mp: mp.setattr(ostore.HostPool, "gather_head", _gather_mutant("offset")),
    "merge_without_rescale": lambda mp: mp.setattr(osplit, "lse_merge", _merge_no_rescale),
    "kv_bytes_doubled": lambda mp: mp.setattr(okv, "kv_bytes_per_token", lambda L, H, d, e: 4 * L * H * d * e),
    "free_list_fifo": lambda mp: mp.setattr(apins, "BlockPoolModel", FifoPool),
    "fp8_exponent_bias_8": lambda mp: mp.setattr(ofp8, "_TABLE", ofp8.e4m3_decode_table() / 2.0),
    "fp8_scale_not_applied": lambda mp: mp.setattr(ofp8, "dequantize",
                                                   lambda c, s: ofp8.e4m3_decode(c) * 1.0),
    "tree_ancestors_parent_only": lambda mp: mp.setattr(otree, "ancestor_masks", _ancestors_parent_only),
    "tree_nodes_shifted": lambda mp: mp.setattr(otree, "visible_positions", _visible_shifted),
    "spec_resample_from_target": lambda mp: mp.setattr(ospec, "residual",
                                                       lambda p, q: np.asarray(p, dtype=np.float32)),
    "spec_ratio_inverted": lambda mp: mp.setattr(ospec, "accept_draft", _accept_inverted),
    "spec_draw_non_strict": lambda mp: mp.setattr(ospec, "draw", _draw_non_strict),
    "pc_evict_non_leaf": lambda mp: mp.setattr(opc.PrefixCachedPool, "_evict_one", _evict_any),
    "pc_write_in_place": lambda mp: mp.setattr(opc.PrefixCachedPool, "_must_copy",
                                               lambda self, blk: self.refcount[blk] > 1),
}


@pytest.mark.parametrize("mutant", list(MUTANTS))
def test_planted_mistake_is_caught(mutant, monkeypatch):
    MUTANTS[mutant](monkeypatch)
    assert run_pins(), f"no pin caught the planted mistake {mutant}"
