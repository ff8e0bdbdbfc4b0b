"""Seeded random configurations through the C ABI against the fp64 oracle
(MI355X): the combinations the named cases leave out, such as FP8 pools with
tree masks, 8- and 12-wave workgroups on short mixed segments, batches far
larger than a workgroup's threads (the step prefix sums span many chunks per
thread) and one-token contexts beside long ones."""
import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from tests.gpu_util import assert_close, oracle_rows, out_to_f64, run_gpu  # noqa: E402

N_CASES = 24


def random_case(i):
    """Configuration, waves per workgroup and partition size of case i."""
    rng = np.random.default_rng([218, 7000 + i])
    d = int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 32]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 4, 8]))
    q_len = int(rng.choice([1, 1, 2, 3, 5, 8]))
    while group * q_len > 32:  # the MFMA kernels' row limit
        q_len = max(1, q_len // 2)
    kv = "fp8" if rng.random() < 0.35 else ""
    tree = "random" if q_len > 1 and rng.random() < 0.5 else ""
    many = rng.random() < 0.2
    batch = int(rng.integers(300, 1500)) if many else int(rng.integers(1, 12))
    hi = 48 if many else int(rng.choice([40, 300, 1500]))
    lens = tuple(int(x) for x in rng.integers(q_len, hi + 1, size=batch))
    part = int(rng.choice([0, 0, 0, 64, 128]))
    waves = int(rng.choice([0, 1, 2, 4, 8, 12]))
    if part:
        waves = min(waves, 4)      # partition kernels: up to 4 waves
    elif group * q_len > 16:
        waves = min(waves, 8)      # two row tiles: up to 8 waves
    cfg = workloads.Config(f"random{i}", 7000 + i, batch=batch, q_len=q_len, num_q_heads=group * hkv,
                           num_kv_heads=hkv, head_dim=d, block_size=bs, dtype="bf16", kv_dtype=kv,
                           lens=lens, pool_slack=1.3, tree=tree)
    return cfg, waves, part


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_config_parity(i):
    cfg, waves, part = random_case(i)
    print(f"case {i}: B {cfg.batch} q_len {cfg.q_len} heads {cfg.num_q_heads}/{cfg.num_kv_heads} d {cfg.head_dim} "
          f"bs {cfg.block_size} kv {cfg.kv_dtype or 'bf16'} tree {cfg.tree or '-'} waves {waves} part {part} "
          f"max L {max(cfg.lens)}", flush=True)
    w = workloads.generate(cfg)
    kw = {}
    if w.tree_parents is not None:
        from paged_kv_cache_218_amd.cache import tree_masks_to_device
        kw = dict(tree_mask=tree_masks_to_device(w.tree_parents), mask_stride=cfg.q_len)
    out, _ = run_gpu(w, partition_tokens=part, waves=waves, **kw)
    rows = oracle_rows(w, range(cfg.batch))
    ref = np.stack([rows[b] for b in range(cfg.batch)])
    assert_close(out_to_f64(out, cfg.dtype).reshape(ref.shape), ref, cfg.dtype, f"random case {i}")
