"""Pins for stochastic acceptance (O6), the Leviathan/Chen rule.

* hand-worked cases (tests/golden): accept boundary, residual, q(d) = 0,
  temperature, data faults, inverse-CDF boundaries;
* special cases: q = p accepts every draft; disjoint supports always reject and
  resample from p; one-hot q and T -> 0 reduce to greedy acceptance;
* a deterministic grid over the final uniform reproduces p to within the grid
  step (the inverse CDF's direction and off-by-one);
* the acceptance rate of draft 0 equals sum_v min(p, q) (closed form of
  min(1, p/q));
* chi-square: the first committed token is distributed as p_0, and the first
  two tokens of a context-dependent toy target follow p_0(a) p_1(b | a) -- the
  theorem that speculative sampling samples the target exactly (pages:
  "Architecture" and the v0.0.2 release notes).
"""
import json
import os

import numpy as np
import pytest
from scipy import stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def _softmax(z, T=1.0):
    a = np.asarray(z, np.float64) / T
    e = np.exp(a - a.max())
    return e / e.sum()


def test_inverse_cdf_golden():
    for c in json.load(open(GOLDEN))["inverse_cdf"]:
        w = np.array(c["w"])
        for u, expect in c["cases"]:
            assert oracle.inverse_cdf(w, u * w.sum()) == expect, (c["w"], u)


def test_sample_golden():
    for c in json.load(open(GOLDEN))["sample"]:
        alen, com = oracle.accept_sample(np.array(c["z"], np.float64), np.array(c["q"]),
                                         np.array(c["d"]), np.array(c["u"]), c["T"])
        assert alen == c["accept_len"], c
        assert list(com) == c["committed"], c


def test_faults_nonfinite():
    z = np.zeros((3, 4))
    q = np.full((2, 4), 0.25)
    d = np.array([0, 1])
    u = np.array([0.1, 0.1, 0.1])
    assert oracle.accept_sample(z, q, d, u, 1.0)[0] == 3
    for bad in ("z_nan", "z_inf", "q_neg", "q_nan", "u_neg", "u_nan", "d_neg", "t_nan"):
        zz, qq, dd, uu, T = z.copy(), q.copy(), d.copy(), u.copy(), 1.0
        if bad == "z_nan": zz[2, 1] = np.nan
        if bad == "z_inf": zz[0, 0] = np.inf
        if bad == "q_neg": qq[1, 3] = -1e-9
        if bad == "q_nan": qq[0, 2] = np.nan
        if bad == "u_neg": uu[0] = -0.0 - 1e-30
        if bad == "u_nan": uu[2] = np.nan
        if bad == "d_neg": dd[1] = -1
        if bad == "t_nan": T = float("nan")
        alen, com = oracle.accept_sample(zz, qq, dd, uu, T)
        assert alen == -1 and (com == -1).all(), bad


def test_q_equal_p_accepts_everything():
    g = np.random.default_rng(1)
    for _ in range(200):
        v, m_rows, T = 6, 4, float(g.uniform(0.5, 2))
        z = g.normal(0, 2, size=(m_rows, v))
        q = np.array([_softmax(z[j], T) for j in range(m_rows - 1)])
        d = np.array([g.choice(v, p=q[j]) for j in range(m_rows - 1)])
        u = g.random(m_rows)
        alen, com = oracle.accept_sample(z, q, d, u, T)
        assert alen == m_rows
        assert list(com[:-1]) == list(d)


def test_disjoint_supports_always_reject_and_follow_p():
    """q puts all mass where p has none -> reject at draft 0, token ~ p_0."""
    v = 5
    z = np.array([[0.0, 1.0, 2.0, -np.inf, -np.inf]] * 3)
    z[:, 3:] = -1e300      # finite, but exp underflows to exactly 0
    q = np.zeros((2, v))
    q[:, 3] = 0.5
    q[:, 4] = 0.5
    p = _softmax(z[0])
    assert p[3] == 0 and p[4] == 0
    grid = (np.arange(4000) + 0.5) / 4000
    counts = np.zeros(v)
    for uf in grid:
        alen, com = oracle.accept_sample(z, q, np.array([3, 4]), np.array([0.0, 0.0, uf]), 1.0)
        assert alen == 1
        counts[com[0]] += 1
    assert np.abs(counts / len(grid) - p).max() <= 1.0 / len(grid) + 1e-12


def test_onehot_q_low_temperature_is_greedy():
    g = np.random.default_rng(2)
    for _ in range(300):
        v, m_rows = 7, 5
        z = g.normal(0, 1, size=(m_rows, v))
        t = np.argmax(z, axis=1)
        d = np.where(g.random(m_rows - 1) < 0.6, t[:-1], g.integers(0, v, m_rows - 1))
        q = np.zeros((m_rows - 1, v))
        q[np.arange(m_rows - 1), d] = 1.0
        u = g.random(m_rows) * 0.999
        alen, com = oracle.accept_sample(z, q, d, u, 1e-4)
        galen, gcom = oracle.accept_greedy(t[None, :], d[None, :])
        assert alen == galen[0]
        assert list(com) == list(gcom[0])


def test_bonus_grid_reproduces_p():
    """All drafts accepted (u_j = 0, q = p); the final uniform swept on a grid."""
    z = np.array([[0.3, -1.0, 2.0, 0.0, 1.1, -0.4]] * 3)
    T = 0.7
    p = _softmax(z[2], T)
    q = np.array([_softmax(z[j], T) for j in range(2)])
    n = 5000
    counts = np.zeros(6)
    for i in range(n):
        alen, com = oracle.accept_sample(z, q, np.array([2, 2]), np.array([0.0, 0.0, (i + 0.5) / n]), T)
        assert alen == 3
        counts[com[2]] += 1
    assert np.abs(counts / n - p).max() <= 1.0 / n + 1e-12


def test_acceptance_rate_closed_form():
    g = np.random.default_rng(3)
    v, trials = 8, 60000
    z = g.normal(0, 1.5, size=(2, v))
    qlog = g.normal(0, 1.5, size=v)
    q = _softmax(qlog)[None, :]
    p0 = _softmax(z[0])
    accepted = 0
    for _ in range(trials):
        d = g.choice(v, p=q[0])
        alen, _ = oracle.accept_sample(z, q, np.array([d]), g.random(2), 1.0)
        accepted += alen == 2
    rate = np.minimum(p0, q[0]).sum()
    sd = np.sqrt(rate * (1 - rate) / trials)
    assert abs(accepted / trials - rate) < 5 * sd


@pytest.mark.parametrize("v,m_rows,T", [(8, 2, 1.0), (8, 4, 0.8), (64, 2, 1.3)])
def test_first_token_distribution_chi2(v, m_rows, T):
    g = np.random.default_rng(v * 10 + m_rows)
    trials = 60000 if v == 8 else 80000
    z = g.normal(0, 1.2, size=(m_rows, v))
    q = np.array([_softmax(g.normal(0, 1.2, size=v), T) for _ in range(m_rows - 1)])
    p0 = _softmax(z[0], T)
    counts = np.zeros(v)
    for _ in range(trials):
        d = np.array([g.choice(v, p=q[j]) for j in range(m_rows - 1)])
        _, com = oracle.accept_sample(z, q, d, g.random(m_rows), T)
        counts[com[0]] += 1
    chi = stats.chisquare(counts, p0 * trials)
    assert chi.pvalue > 1e-3, chi


def test_two_token_joint_distribution_chi2():
    """Toy context-dependent target: row 1's logits depend on the input d_0."""
    g = np.random.default_rng(99)
    v, trials, T = 6, 60000, 1.0
    z0 = g.normal(0, 1.0, size=v)
    z1 = g.normal(0, 1.0, size=(v, v))             # row-1 logits given input token a
    q0 = _softmax(g.normal(0, 1.0, size=v))
    p0 = _softmax(z0)
    p1 = np.array([_softmax(z1[a]) for a in range(v)])
    joint = np.zeros((v, v))
    for _ in range(trials):
        d0 = g.choice(v, p=q0)
        z = np.stack([z0, z1[d0]])
        alen, com = oracle.accept_sample(z, q0[None, :], np.array([d0]), g.random(2), T)
        a = com[0]
        b = com[1] if alen == 2 else g.choice(v, p=p1[a])   # next round's first token ~ p
        joint[a, b] += 1
    expect = (p0[:, None] * p1) * trials
    chi = stats.chisquare(joint.ravel(), expect.ravel())
    assert chi.pvalue > 1e-3, chi
