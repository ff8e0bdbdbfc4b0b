"""Pins of the speculative accept / resample oracle (CPU only).

The identity the pages prove -- the emitted token has the target's
distribution p -- pins acceptance and residual together; the fixed-point
draw is pinned at its exact boundaries; special cases follow the pages'
narrative (all accepted plus one more token; a draft the target gives zero
probability is always rejected)."""
import numpy as np
import pytest

import workloads
from oracle import spec


def _dist(rng, v, sigma=1.5):
    l = rng.standard_normal(v) * sigma
    e = np.exp(l - l.max())
    return (e / e.sum()).astype(np.float32)


def test_emitted_token_has_the_target_distribution():
    """P(x) = min(q, p) + max(0, p - q) = p(x) (Blog #54, question 3)."""
    rng = np.random.default_rng(5)
    V = 6
    p0, p1, q0 = _dist(rng, V), _dist(rng, V), _dist(rng, V)
    N = 60000
    cq = np.cumsum(q0.astype(np.float64))
    drafts = np.minimum(np.searchsorted(cq, rng.random(N) * cq[-1], side="right"), V - 1)
    us = rng.random(N, dtype=np.float32)
    Us = rng.integers(0, 2 ** 32, size=N, dtype=np.uint64)
    counts = np.zeros(V)
    accepted = 0
    for i in range(N):
        n, toks = spec.accept_sequence(np.stack([p0, p1]), q0[None], [drafts[i]], [us[i]], int(Us[i]))
        counts[toks[0]] += 1
        accepted += n
    freq = counts / N
    sd = np.sqrt(p0 * (1 - p0) / N)
    assert np.all(np.abs(freq - p0) <= 5 * sd + 1e-9), (freq, p0)
    # the acceptance rate is sum_x min(p(x), q(x))
    rate = np.minimum(p0, q0).sum()
    assert abs(accepted / N - rate) <= 5 * np.sqrt(rate * (1 - rate) / N)


def test_draw_boundaries_are_exact():
    w = np.float32([0.25, 0.0, 0.5, 0.125, 0.125])
    ints = spec.fixed_weights(w)
    assert ints == [2 ** 30, 0, 2 ** 31, 2 ** 29, 2 ** 29]
    S = sum(ints)
    prefix = np.cumsum(ints)
    for t in range(len(w)):
        if ints[t] == 0:
            continue
        lo = -(-int(prefix[t] - ints[t]) * 2 ** 32 // S)     # first U drawing token t
        hi = -(-int(prefix[t]) * 2 ** 32 // S) - 1           # last U drawing token t
        assert spec.draw(w, lo) == t and spec.draw(w, hi) == t
        if lo > 0:
            assert spec.draw(w, lo - 1) != t
    assert spec.draw(w, 0) == 0 and spec.draw(w, 2 ** 32 - 1) == 4
    with pytest.raises(ValueError):
        spec.draw(np.float32([0, 0]), 5)


def test_all_accepted_then_one_more_token():
    """Blog #54, section 2.4: four drafts accepted, the pass yields a fifth."""
    rng = np.random.default_rng(6)
    V, K = 10, 4
    p = np.stack([_dist(rng, V) for _ in range(K + 1)])
    draft = [3, 1, 4, 1]
    q = p[:K].copy()                  # the draft agrees with the target: p >= q
    n, toks = spec.accept_sequence(p, q, draft, np.float32([0.99] * K), 12345)
    assert n == K and toks[:K] == draft
    assert toks[K] == spec.draw(p[K], 12345)


def test_zero_target_probability_always_rejected():
    rng = np.random.default_rng(7)
    V = 8
    p = np.stack([_dist(rng, V), _dist(rng, V)])
    p[0, 2] = 0.0
    q = _dist(rng, V)[None]
    for u in (np.float32(0.0), np.float32(0.5)):
        n, toks = spec.accept_sequence(p, q, [2], [u], 777)
        assert n == 0
        r = spec.residual(p[0], q[0])
        assert r[toks[0]] > 0 and toks[0] == spec.draw(r, 777)


def test_acceptance_is_the_float32_comparison():
    # u * q < p decides; p >= q always accepts
    assert spec.accept_draft(np.float32(0.3), np.float32(0.3), np.float32(0.999))
    assert spec.accept_draft(np.float32(0.2), np.float32(0.4), np.float32(0.49))
    assert not spec.accept_draft(np.float32(0.2), np.float32(0.4), np.float32(0.5))


def test_zero_residual_draws_from_target():
    p = np.float32([[0.5, 0.25, 0.25], [0.2, 0.3, 0.5]])
    q = p[:1].copy()
    q[0, 0] = np.float32(0.5) + np.float32(2.0 ** -22)   # u * q >= p for u just below 1: rejected
    n, toks = spec.accept_sequence(p, q, [0], [np.float32(1 - 2.0 ** -24)], 3 * 2 ** 30)
    assert n == 0 and sum(spec.fixed_weights(spec.residual(p[0], q[0]))) == 0
    assert toks[0] == spec.draw(p[0], 3 * 2 ** 30)


def test_workload_acceptance_rate_is_in_the_pages_range():
    w = workloads.generate_spec(workloads.spec_config("spec_accept", batch=8, vocab=4096))
    rates = [np.minimum(w.p[b, k], w.q[b, k]).sum() for b in range(8) for k in range(w.cfg.k)]
    assert 0.7 <= float(np.mean(rates)) <= 0.9
