"""Host-side pieces of bench.py (CPU only): the source stamp that decides
whether committed HBM-traffic counters still describe the built kernels."""
import bench


def test_code_only_drops_comments_and_layout_keeps_literals():
    a = 'int a = 1; // note\n/* block\n comment */ const char* s = "//x /*y*/"; char c = \'"\';'
    b = 'int a = 1;\n\n   const char* s = "//x /*y*/";   char c = \'"\'; // other note'
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) == 'int a = 1; const char* s = "//x /*y*/"; char c = \'"\';'
    assert bench._code_only("int a = 1;") != bench._code_only("int a = 2;")


def test_source_digest_is_stable():
    assert bench.source_digest() == bench.source_digest()
    assert len(bench.source_digest()) == 64


def test_attention_flops_counts_visible_pairs():
    import numpy as np
    import workloads
    cfg = workloads.config("prefix_verify", batch=2, q_len=3)
    lens = np.array([10, 20])
    per_pair = 4 * cfg.num_q_heads * cfg.head_dim
    # a chain: row i sees L - q_len + i + 1 tokens
    assert bench.attention_flops(cfg, lens) == per_pair * sum(L - 3 + i + 1 for L in (10, 20) for i in range(3))
    # every drafted token hangs off the context: each sees the context and itself
    flat = np.full((2, 3), -1)
    assert bench.attention_flops(cfg, lens, flat) == per_pair * 3 * ((10 - 2) + (20 - 2))
    # a chain written as parents equals the causal count
    chain = np.array([[-1, 0, 1], [-1, 0, 1]])
    assert bench.attention_flops(cfg, lens, chain) == bench.attention_flops(cfg, lens)
