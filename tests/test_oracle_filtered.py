"""Oracle of truncated (top-k / top-p) and penalised speculative sampling,
pinned without reference to its own code:

* truncation: properties that define it (a leading set in probability order,
  top-k size, the smallest set reaching top_p of the top-k mass), on tiny
  distributions with ties, brute-forced over parameters;
* penalties: speculative rounds at top_k = 1 reproduce plain sequential
  greedy decoding of the penalised target (counts grow with every emitted
  token), and a planted mistake (row j not counting drafts 0..j-1) is caught;
* losslessness: the first committed token is distributed as the truncated,
  penalised target (chi-square, fixed seeds);
* no truncation and no penalties reduce to accept_sample exactly.
"""
import numpy as np
import pytest
from scipy import stats

import oracle
from oracle import dspk_oracle


def _order(w):
    return sorted(range(len(w)), key=lambda i: (-w[i], i))


@pytest.mark.parametrize("seed", range(40))
def test_truncate_properties(seed):
    g = np.random.default_rng(seed)
    v = int(g.integers(1, 9))
    w = g.integers(0, 4, size=v).astype(np.float64)     # small integers: many ties
    if w.sum() == 0:
        w[0] = 1
    w = w / w.sum()
    for k in (0, 1, 2, 3, v, v + 3):
        for top_p in (1.0, 0.999, 0.75, 0.5, 0.3, 1e-9):
            keep = oracle.truncate(w, k, top_p)
            order = _order(w)
            kept = [i for i in order if keep[i]]
            # a leading set of the order
            assert kept == order[:len(kept)]
            kk = v if k <= 0 else min(k, v)
            mk = sum(w[i] for i in order[:kk])
            if top_p >= 1.0:
                assert len(kept) == kk
            else:
                target = top_p * mk
                assert len(kept) <= kk
                assert sum(w[i] for i in kept) >= target - 1e-15           # reaches top_p
                assert sum(w[i] for i in kept[:-1]) < target               # and is the smallest such


def test_truncate_boundary_hand_cases():
    # mass before the second entry equals the target: it is not needed
    assert oracle.truncate([0.5, 0.5], 0, 0.5).tolist() == [True, False]
    # ties at the top-k boundary go to the smaller index
    assert oracle.truncate([0.2, 0.3, 0.3, 0.2], 1, 1.0).tolist() == [False, True, False, False]
    assert oracle.truncate([0.25, 0.25, 0.25, 0.25], 2, 1.0).tolist() == [True, True, False, False]
    # top-p inside the top-k distribution: top-2 mass 0.7, target 0.35 -> the first entry (0.4) suffices
    assert oracle.truncate([0.4, 0.3, 0.2, 0.1], 2, 0.5).tolist() == [True, False, False, False]


def _toy_model(steps, v, seed):
    g = np.random.default_rng(seed)
    return g.normal(0, 1.0, size=(steps, v))


def _sequential_penalised_greedy(z, counts, presence, frequency):
    c = np.array(counts, dtype=np.float64)
    out = []
    for t in range(z.shape[0]):
        zt = z[t] - presence * (c > 0) - frequency * c
        tok = int(np.argmax(zt))
        out.append(tok)
        c[tok] += 1
    return out


@pytest.mark.parametrize("presence,frequency", [(0.0, 0.0), (0.7, 0.0), (0.0, 0.4), (0.5, 0.9)])
def test_top1_rounds_reproduce_sequential_penalised_greedy(presence, frequency):
    steps, v, m = 40, 6, 4
    z = _toy_model(steps + m, v, 3)
    base = np.random.default_rng(9).integers(0, 3, size=v)
    want = _sequential_penalised_greedy(z[:steps], base, presence, frequency)
    g = np.random.default_rng(4)
    got, counts, t = [], base.astype(np.int64).copy(), 0
    while t < steps:
        rows = z[t:t + m + 1]
        # drafts: half of the time the true continuation, else a random token
        d = np.array([want[t + j] if (t + j < steps and g.random() < 0.6) else int(g.integers(0, v))
                      for j in range(m)])
        q = np.full((m, v), 0.01)
        q[np.arange(m), d] = 1.0             # the draft is its q's argmax, kept by top-1
        u = g.random(m + 1) * 0.999
        n, com = oracle.accept_sample_filtered(rows, q, d, u, 1.0, top_k=1, counts=counts,
                                               presence=presence, frequency=frequency)
        for tok in com[:n]:
            if t < steps:
                got.append(int(tok))
                counts[tok] += 1
                t += 1
    assert got == want


def test_penalty_without_draft_counts_is_caught(monkeypatch):
    """A row that ignores the drafts before it (counts fixed for the whole
    block) is not sequential decoding."""
    def flat(logits, counts, draft_ids, presence, frequency):
        z = np.asarray(logits, dtype=np.float64)
        c = np.zeros(z.shape[1]) if counts is None else np.asarray(counts, dtype=np.float64)
        return z - presence * (c > 0) - frequency * c
    monkeypatch.setattr(dspk_oracle, "penalized_logits", flat)
    with pytest.raises(AssertionError):
        test_top1_rounds_reproduce_sequential_penalised_greedy(0.5, 0.9)


def test_unfiltered_equals_accept_sample():
    g = np.random.default_rng(2)
    for _ in range(50):
        m, v = int(g.integers(2, 6)), int(g.integers(2, 30))
        z = g.normal(0, 2, (m, v))
        q = g.dirichlet(np.ones(v), size=m - 1)
        d = np.array([g.choice(v, p=q[j]) for j in range(m - 1)])
        u = g.random(m) * 0.999
        assert oracle.accept_sample_filtered(z, q, d, u, 0.8)[0] == oracle.accept_sample(z, q, d, u, 0.8)[0]
        assert np.array_equal(oracle.accept_sample_filtered(z, q, d, u, 0.8)[1],
                              oracle.accept_sample(z, q, d, u, 0.8)[1])


@pytest.mark.parametrize("top_k,top_p,pen", [(3, 1.0, 0.0), (0, 0.7, 0.0), (4, 0.8, 0.6)])
def test_first_token_is_the_truncated_target(top_k, top_p, pen):
    v, trials = 8, 60000
    g = np.random.default_rng(17)
    z = g.normal(0, 1.2, (2, v))
    counts = np.array([0, 2, 0, 1, 0, 0, 3, 0])
    q = g.dirichlet(np.ones(v) * 0.7, size=1)
    zp = oracle.penalized_logits(z, counts, [0], pen, pen / 2)
    p0 = oracle.softmax_t(zp[0], 1.0)
    p0 = np.where(oracle.truncate(p0, top_k, top_p), p0, 0.0)
    p0 /= p0.sum()
    qt = np.where(oracle.truncate(q[0], top_k, top_p), q[0], 0.0)
    qt /= qt.sum()
    hist = np.zeros(v)
    for _ in range(trials):
        d = g.choice(v, p=qt)
        u = g.random(2) * (1 - 1e-12)
        _, com = oracle.accept_sample_filtered(z, q, [d], u, 1.0, top_k, top_p, counts, pen, pen / 2)
        hist[com[0]] += 1
    sup = p0 > 0
    assert hist[~sup].sum() == 0                      # never outside the truncated support
    chi = stats.chisquare(hist[sup], p0[sup] * trials)
    assert chi.pvalue > 1e-3, chi


def _golden(name):
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")) as f:
        return json.load(f)[name]


@pytest.mark.parametrize("case", range(4))
def test_penalized_logits_hand_cases(case):
    """The penalty arithmetic against hand-worked values (tests/golden): the
    sign of each term, presence as an indicator, frequency per occurrence, and
    row j counting the history plus drafts 0..j-1 only."""
    c = _golden("penalties")[case]
    z = np.array(c["z"], dtype=np.float64)
    got = oracle.penalized_logits(z, c["counts"], np.array(c["d"], dtype=np.int64), c["presence"], c["frequency"])
    assert np.array_equal(got, np.array(c["expected"], dtype=np.float64)), (got, c["why"])


def test_top_k_at_least_v_is_no_truncation():
    """top_k >= v keeps every entry, so (with top_p = 1) truncation is off and
    q is used as supplied -- also when its rows do not sum to one, where a
    renormalisation would change the accept test."""
    g = np.random.default_rng(11)
    v, m = 7, 4
    for trial in range(200):
        z = g.normal(0, 2, size=(m, v))
        q = g.random((m - 1, v))
        q = q / q.sum(axis=1, keepdims=True) * g.uniform(0.6, 1.4, size=(m - 1, 1))   # rows not summing to 1
        d = g.integers(0, v, size=m - 1)
        u = (g.integers(0, 1 << 24, size=m) / float(1 << 24))
        want = oracle.accept_sample(z, q, d, u, 0.8) if np.all(np.abs(q.sum(axis=1) - 1) < 1e-5) else None
        for top_k in (v, v + 1, 1000):
            a = oracle.accept_sample_filtered(z, q, d, u, 0.8, top_k=top_k)
            b = oracle.accept_sample_filtered(z, q, d, u, 0.8, top_k=0)
            assert a[0] == b[0] and np.array_equal(a[1], b[1])
            if want is not None:
                assert a[0] == want[0]
        # with a real top-k (< v) the draft row is renormalised: results may differ, never fault
        r = oracle.accept_sample_filtered(z, q, d, u, 0.8, top_k=v - 1)
        assert 1 <= r[0] <= m
