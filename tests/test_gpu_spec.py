"""Speculative accept / resample on the HIP path vs the oracle (MI355X): the
number of kept drafts and every token must match bit for bit."""
import numpy as np
import pytest

import workloads
from oracle import spec

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def run_spec(w, q_none=False):
    import paged_kv_cache_218_amd as pa
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    B, K = w.draft.shape
    n = torch.empty(B, dtype=torch.int32, device="cuda")
    toks = torch.empty(B, K + 1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(pa.pa_spec_accept_workspace_size(B, w.p.shape[2]), dtype=torch.uint8, device="cuda")
    for rep in range(2):   # the second call checks that the first left its counters at zero
        pa.pa_spec_accept(d(w.p), None if q_none else d(w.q), d(w.draft), d(w.u_accept),
                          d(w.u_draw.view(np.int32)), n, toks, ws)
        torch.cuda.synchronize()
        if rep == 0:
            first = (n.cpu().numpy().copy(), toks.cpu().numpy().copy())
    assert int(ws[:4 * B].count_nonzero()) == 0
    assert np.array_equal(first[0], n.cpu().numpy()) and np.array_equal(first[1], toks.cpu().numpy())
    return first


def check(w, seqs=None):
    n, toks = run_spec(w)
    seqs = range(w.draft.shape[0]) if seqs is None else seqs
    for b in seqs:
        rn, rt = spec.accept_sequence(w.p[b], w.q[b], w.draft[b], w.u_accept[b], int(w.u_draw[b]))
        assert n[b] == rn and toks[b].tolist() == rt, (b, n[b], rn, toks[b], rt)
    return n, toks


@pytest.mark.parametrize("kw", [dict(), dict(vocab=37), dict(k=1, batch=9), dict(k=8, vocab=64, noise=2.0),
                                dict(vocab=4099, batch=3, noise=3.0)])
def test_spec_bit_exact_small(kw):
    w = workloads.generate_spec(workloads.spec_config("spec_tiny", **kw))
    print(f"spec small {kw}", flush=True)
    n, _ = check(w)
    assert 0 <= n.min() and n.max() <= w.cfg.k


def test_spec_bit_exact_llama3_vocab():
    w = workloads.generate_spec(workloads.spec_config("spec_accept", batch=6))
    print("spec llama3 vocab, 6 sequences", flush=True)
    check(w)


def test_spec_all_accepted_and_extra_token():
    w = workloads.generate_spec(workloads.spec_config("spec_tiny", vocab=48))
    w.q[:] = w.p[:, :w.cfg.k]                        # draft equals target: always kept
    print("spec all accepted", flush=True)
    n, toks = check(w)
    assert (n == w.cfg.k).all()


def test_spec_zero_target_probability_rejected():
    w = workloads.generate_spec(workloads.spec_config("spec_tiny", vocab=48))
    for b in range(w.cfg.batch):
        w.p[b, 0, w.draft[b, 0]] = 0.0                 # the first draft has no target mass
    print("spec forced rejection", flush=True)
    n, toks = check(w)
    assert (n == 0).all()
    for b in range(w.cfg.batch):
        if sum(spec.fixed_weights(spec.residual(w.p[b, 0], w.q[b, 0]))) > 0:   # else drawn from p
            assert w.p[b, 0, toks[b, 0]] > w.q[b, 0, toks[b, 0]]


def test_spec_no_drafts_draws_from_target():
    w = workloads.generate_spec(workloads.spec_config("spec_tiny", k=0, vocab=52))
    print("spec K = 0", flush=True)
    n, toks = run_spec(w, q_none=True)
    assert (n == 0).all()
    for b in range(w.cfg.batch):
        assert toks[b, 0] == spec.draw(w.p[b, 0], int(w.u_draw[b]))


def test_spec_bad_draft_token_marks_sequence():
    w = workloads.generate_spec(workloads.spec_config("spec_tiny", vocab=48))
    w.draft[1, 0] = 48
    w.draft[3, 1] = -2
    print("spec bad draft tokens", flush=True)
    n, toks = run_spec(w)
    assert n[1] == -1 and (toks[1] == -1).all()
    # a bad token after a rejection is never looked at; otherwise the sequence is marked
    rn, _ = spec.accept_sequence(w.p[3], w.q[3], [w.draft[3, 0]], w.u_accept[3][:1], int(w.u_draw[3]))
    assert n[3] == (-1 if rn == 1 else 0)
    for b in (0, 2, 4, 5):
        rn, rt = spec.accept_sequence(w.p[b], w.q[b], w.draft[b], w.u_accept[b], int(w.u_draw[b]))
        assert n[b] == rn and toks[b].tolist() == rt
