"""Pins for the oracle's rejection-sampling verification of speculative drafts
(tinyserve README "How it works", Speculative decoding; PageServe "06
Development history", Next steps: rejection sampling).

Checked against what the method and the mathematics fix, not against the
oracle's own formula:
 * greedy special case: one-hot target and draft rows reduce verification
   to "keep the longest prefix of drafts that match the target's argmax,
   then emit the target's argmax";
 * the law of the first emitted token equals the target distribution p_0
   exactly (the sampler's defining property), measured by integrating the
   oracle over fine grids of both uniforms;
 * the acceptance probability equals sum_t min(p(t), q(t)) (one minus the
   total-variation distance);
 * a Monte Carlo chi-square test of the emitted tokens against the target
   law (the pages' statistical test of the sampler);
 * zero drafts (a plain decode row) draws from p_0; malformed sequences are
   flagged without disturbing the others; a residual without mass falls
   back to the target row.
"""
import numpy as np
import pytest
from scipy import stats

import oracle


def _dist(rng, v, zeros=0):
    x = rng.gamma(0.7, size=v)
    if zeros:
        x[rng.choice(v, zeros, replace=False)] = 0.0
    return (x / x.sum()).astype(np.float32)


def _batch(p_rows, q_rows, drafts, accept_u, sample_u):
    """Stack per-sequence rounds into the oracle's packed layout."""
    starts = np.concatenate([[0], np.cumsum([len(d) for d in drafts])]).astype(np.int32)
    V = p_rows[0].shape[1]
    tp = np.concatenate(p_rows).astype(np.float32)
    dp = np.concatenate(q_rows).astype(np.float32) if starts[-1] else np.zeros((0, V), np.float32)
    dt = np.concatenate([np.asarray(d, np.int32) for d in drafts]) if starts[-1] else np.zeros(0, np.int32)
    au = np.concatenate([np.asarray(a, np.float64) for a in accept_u]) if starts[-1] else np.zeros(0)
    return oracle.spec_verify(tp, dp, dt, starts, au, np.asarray(sample_u, np.float64))


def test_greedy_special_case():
    # one-hot rows: d_i is kept iff it is the target's argmax a_i; at the
    # first mismatch (or after the last draft) the target's argmax comes out
    rng = np.random.default_rng(0)
    V = 50
    p_rows, q_rows, drafts, au, su, expect = [], [], [], [], [], []
    for s in range(200):
        k = int(rng.integers(0, 7))
        a = rng.integers(0, V, k + 1)
        match = int(rng.integers(0, k + 1))
        d = a[:k].copy()
        for i in range(match, k):
            d[i] = (a[i] + 1 + rng.integers(0, V - 1)) % V  # != a[i]
        P = np.zeros((k + 1, V), np.float32)
        P[np.arange(k + 1), a] = 1
        Q = np.zeros((k, V), np.float32)
        Q[np.arange(k), d] = 1
        p_rows.append(P)
        q_rows.append(Q)
        drafts.append(d)
        au.append(rng.random(k))
        su.append(rng.random())
        expect.append((match, int(a[match])))
    na, nt = _batch(p_rows, q_rows, drafts, au, su)
    assert [(int(x), int(y)) for x, y in zip(na, nt)] == expect


def _grid(m):
    return (np.arange(m) + 0.5) / m


def _accept_prob(p, q, d, m):
    """Fraction of a u-grid for which draft d (k = 1) is kept."""
    u = _grid(m)
    n = len(u)
    na, _ = _batch([np.stack([p, p])] * n, [q[None]] * n, [[d]] * n, [[x] for x in u], [0.5] * n)
    return float((na == 1).mean())


def _draw_law(p, q, d, m):
    """Law of the token drawn after a rejection of d (u just below 1), over a v-grid."""
    v = _grid(m)
    n = len(v)
    na, nt = _batch([np.stack([p, p])] * n, [q[None]] * n, [[d]] * n, [[1 - 2 ** -40]] * n, v)
    assert np.all(na == 0)
    return np.bincount(nt, minlength=len(p)) / n


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_first_token_law_equals_target(seed):
    # P(x_0 = t) = sum_d q(d) [a(d) 1{t = d} + (1 - a(d)) r(t)], with the
    # acceptance a(d) and the post-rejection law r measured on the oracle
    # over grids of 2^14 points, must be p_0 (Leviathan et al. 2023).
    rng = np.random.default_rng(seed)
    V, M = 7, 1 << 14
    p = _dist(rng, V, zeros=1)
    q = _dist(rng, V, zeros=1)
    law = np.zeros(V)
    accept_total = 0.0
    for d in np.nonzero(q)[0]:
        a = _accept_prob(p, q, d, M)
        accept_total += q[d] * a
        law[d] += q[d] * a
        if a < 1:
            law += q[d] * (1 - a) * _draw_law(p, q, d, M)
    np.testing.assert_allclose(law, p, atol=4.0 / M)
    # acceptance probability: sum_t min(p, q) = 1 - total variation distance
    assert abs(accept_total - np.minimum(p, q).sum()) <= 2.0 / M


def test_statistical_law_of_emitted_tokens():
    # Monte Carlo over drafts and uniforms (the pages' statistical test):
    # the first emitted token follows p_0, and after an accepted first
    # draft the second follows p_1; acceptance rates are sum min(p_i, q_i)
    rng = np.random.default_rng(11)
    V, k, N = 8, 3, 100_000
    P = np.stack([_dist(rng, V) for _ in range(k + 1)])
    Q = np.stack([_dist(rng, V) for _ in range(k)])
    cdf = np.cumsum(Q.astype(np.float64), axis=1)
    d = np.stack([np.minimum(np.searchsorted(cdf[i], rng.random(N) * cdf[i, -1], side="right"), V - 1)
                  for i in range(k)], axis=1).astype(np.int32)
    starts = np.arange(N + 1, dtype=np.int32) * k
    na, nt = oracle.spec_verify(np.tile(P, (N, 1)), np.tile(Q, (N, 1)), d.reshape(-1), starts,
                                rng.random(N * k), rng.random(N))
    assert np.all((na >= 0) & (na <= k)) and np.all((nt >= 0) & (nt < V))
    law = P.astype(np.float64) / P.astype(np.float64).sum(axis=1, keepdims=True)
    x0 = np.where(na >= 1, d[:, 0], nt)
    assert stats.chisquare(np.bincount(x0, minlength=V), law[0] * N).pvalue > 1e-3
    one = na >= 1
    x1 = np.where(na[one] >= 2, d[one, 1], nt[one])
    assert stats.chisquare(np.bincount(x1, minlength=V), law[1] * one.sum()).pvalue > 1e-3
    for i in range(k):
        reached = na >= i
        kept = (na[reached] > i).mean()
        expect = np.minimum(P[i], Q[i]).astype(np.float64).sum()
        assert abs(kept - expect) < 5 * np.sqrt(expect * (1 - expect) / reached.sum())


def test_zero_drafts_draw_from_target():
    rng = np.random.default_rng(4)
    V, M = 9, 1 << 14
    p = _dist(rng, V, zeros=2)
    v = _grid(M)
    na, nt = _batch([p[None]] * M, [], [[]] * M, [[]] * M, v)
    assert np.all(na == 0)
    np.testing.assert_allclose(np.bincount(nt, minlength=V) / M, p, atol=1.0 / M)


def test_malformed_sequences_are_flagged_alone():
    rng = np.random.default_rng(5)
    V = 6
    p, q = _dist(rng, V), _dist(rng, V)
    good = ([np.stack([p, p])], [q[None]], [[2]], [[0.0]], [0.3])
    na, nt = _batch(good[0] * 3, good[1] * 3, [[2], [V], [-1]], [[0.0]] * 3, [0.3] * 3)
    assert na[1] == nt[1] == -1 and na[2] == nt[2] == -1
    assert na[0] == 1 and 0 <= nt[0] < V
    # a negative draft count
    na, nt = oracle.spec_verify(np.stack([p, p]), q[None], [2], [0, 1, 0], [0.0], [0.3, 0.3])
    assert na[1] == nt[1] == -1 and na[0] == 1


def test_residual_without_mass_falls_back_to_target():
    # p = q / 2 (a target row that does not sum to one): rejection is
    # possible, but max(p - q, 0) is zero everywhere; the draw then comes
    # from p itself
    rng = np.random.default_rng(6)
    V, M = 5, 1 << 12
    q = _dist(rng, V)
    p = (q / 2).astype(np.float32)
    law = _draw_law(p, q, 0, M)
    np.testing.assert_allclose(law, p / p.sum(), atol=1.0 / M)


def test_degenerate_uniforms_stay_in_range():
    rng = np.random.default_rng(7)
    V = 6
    p, q = _dist(rng, V), _dist(rng, V)
    vs = [0.0, -1.0, float("nan"), 1.0, 2.0, 1 - 2 ** -53]
    na, nt = _batch([np.stack([p, p])] * len(vs), [q[None]] * len(vs), [[1]] * len(vs),
                    [[0.5]] * len(vs), vs)
    assert np.all((nt >= 0) & (nt < V))
    # v <= 0 (or NaN) takes the first token with mass, v >= 1 the last
    assert nt[0] == nt[1] == nt[2] and nt[3] == nt[4] == nt[5]


def test_inverse_cdf_boundaries_are_exact():
    # the draw is the smallest t with F(t) > v (F the normalised running
    # sum): with dyadic weights every boundary is exact, a token without
    # mass is never drawn, and v on a step of F moves to the next token
    p = np.array([0, 0.25, 0, 0.25, 0.5, 0], np.float32)
    cases = {0.0: 1, 0.1: 1, 0.25 - 2 ** -30: 1, 0.25: 3, 0.4: 3, 0.5 - 2 ** -40: 3, 0.5: 4,
             0.75: 4, 1 - 2 ** -53: 4}
    vs = list(cases)
    na, nt = _batch([p[None]] * len(vs), [], [[]] * len(vs), [[]] * len(vs), vs)
    assert [int(t) for t in nt] == [cases[v] for v in vs]
