"""Statistical pins for the oracle (CPU only).

* The closed form of the expected number of tokens per round,
  E[tau] = (1 - Acc^(k+1)) / (1 - Acc), Acc = E_{x~q}[min(1, p(x)/q(x))]
  (AdaFlash paper, Section 2.1; restated in the reading notes), on inputs where
  every position has the same (p, q) pair; plus a chi-square test of the
  accept-length histogram against the truncated geometric law it implies.
* Losslessness: the emitted token's law equals the target distribution (paper,
  Section 2.1; DFlash notes, Section 5.2) -- exactly, by enumerating draft ids and
  the intervals of u that the oracle's sampler maps to each id, and by Monte Carlo
  chi-square through the whole oracle.
* Mutation checks: a residual taken the wrong way round, or an inverted
  acceptance ratio, planted in the oracle, must make these pins fail.
"""

import math

import numpy as np
import pytest
from scipy.special import softmax
from scipy.stats import chisquare

import oracle.verify as ov
from oracle import acceptance, final_token_distribution, inverse_cdf, log_softmax, verify_request


# ----------------------------------------------------------------------------- helpers
def _pair(rng, V, scale=2.0, sigma=1.0):
    lp = scale * rng.standard_normal(V)
    lq = lp + sigma * rng.standard_normal(V)
    return lp, lq


def _acc(lp, lq, T):
    return float(np.minimum(softmax(lp / T), softmax(lq / T)).sum())


def _tau_law(acc, k):
    """P(a = j), j = 0..k, for i.i.d. per-position survival probability acc."""
    p = np.array([acc**j * (1 - acc) for j in range(k)] + [acc**k])
    return p


def _run_iid(rng, lp, lq, k, T, n):
    """n rounds where every position uses the same (p, q) pair; x_i ~ q_T i.i.d."""
    q = softmax(lq / T)
    target = np.repeat(lp[None, :], k + 1, axis=0)
    draft = np.repeat(lq[None, :], k, axis=0)
    a = np.empty(n, dtype=np.int64)
    for t in range(n):
        x = rng.choice(lq.shape[0], size=k, p=q)
        u = rng.random(k + 1)
        a[t] = verify_request(target, draft, x, u, T, 1.0, with_rkl=False)["accept_len"]
    return a


def _tau_check(rng, lp, lq, k, T, n):
    acc = _acc(lp, lq, T)
    a = _run_iid(rng, lp, lq, k, T, n)
    law = _tau_law(acc, k)
    e_tau = (1 - acc ** (k + 1)) / (1 - acc)  # the page's closed form
    mean_law = float(np.sum(law * (np.arange(k + 1) + 1)))
    assert mean_law == pytest.approx(e_tau, rel=1e-12)
    var = float(np.sum(law * (np.arange(k + 1) + 1) ** 2)) - mean_law**2
    z = (np.mean(a + 1) - e_tau) / math.sqrt(var / n)
    hist = np.bincount(a, minlength=k + 1)
    keep = law * n >= 5  # chi-square needs expected counts >= 5: pool the rest
    obs = np.append(hist[keep], hist[~keep].sum())
    exp = np.append(law[keep] * n, law[~keep].sum() * n)
    if exp[-1] == 0:
        obs, exp = obs[:-1], exp[:-1]
    pval = chisquare(obs, exp).pvalue
    return z, pval


# ----------------------------------------------------------------------------- E[tau]
@pytest.mark.parametrize("k,T,seed", [(4, 1.0, 0), (15, 1.0, 1), (6, 0.7, 2)])
def test_expected_tau_closed_form(k, T, seed):
    rng = np.random.default_rng(seed)
    lp, lq = _pair(rng, 32)
    z, pval = _tau_check(rng, lp, lq, k, T, 3000)
    assert abs(z) < 4.0
    assert pval > 1e-4


def test_expected_tau_ragged_lengths():
    rng = np.random.default_rng(3)
    lp, lq = _pair(rng, 24)
    for k in (1, 3, 7):
        z, pval = _tau_check(rng, lp, lq, k, 1.0, 1500)
        assert abs(z) < 4.0 and pval > 1e-4


def test_oracle_expected_tau_matches_closed_form():
    acc = 0.45
    assert ov.expected_tau([acc] * 15) == pytest.approx((1 - acc**16) / (1 - acc), rel=1e-14)
    assert ov.expected_tau([]) == 1.0


# ----------------------------------------------------------------------------- losslessness
def _sampler_law(mass, V):
    """Exact measure of u in [0, 1) that the oracle's inverse_cdf maps to each id,
    found by bisecting the change points of the (monotone) map u -> id."""
    law = np.zeros(V)
    grid = (np.arange(4096) + 0.5) / 4096
    ids = [inverse_cdf(mass, float(u))[0] for u in grid]
    edges = [0.0]
    for g in range(1, len(grid)):
        if ids[g] != ids[g - 1]:
            lo, hi = grid[g - 1], grid[g]
            for _ in range(60):
                mid = 0.5 * (lo + hi)
                if inverse_cdf(mass, mid)[0] == ids[g - 1]:
                    lo = mid
                else:
                    hi = mid
            edges.append(hi)
    edges.append(1.0)
    owners = [ids[0]] + [ids[g] for g in range(1, len(grid)) if ids[g] != ids[g - 1]]
    for j, y in enumerate(owners):
        law[y] += edges[j + 1] - edges[j]
    return law


def _emitted_law(lp, lq, T):
    """P(first emitted token = y | slot reached), enumerated through the oracle's own
    acceptance test and sampler: sum_x q(x) [1(x=y) P_acc(x) + (1 - P_acc(x)) R(y)]."""
    V = lp.shape[0]
    log_p, _ = log_softmax(lp, T)
    log_q, _ = log_softmax(lq, T)
    p, q = np.exp(log_p), np.exp(log_q)
    resid = _sampler_law(final_token_distribution(p, q), V)
    law = np.zeros(V)
    for x in range(V):
        pacc = acceptance(log_p[x], log_q[x], 0.0)[1]  # P(u < r) = r for u ~ U[0, 1)
        law[x] += q[x] * pacc
        law += q[x] * (1 - pacc) * resid
    return law, p


@pytest.mark.parametrize("V,T,seed", [(8, 1.0, 10), (16, 1.0, 11), (16, 0.7, 12), (8, 2.0, 13)])
def test_lossless_exact_enumeration(V, T, seed):
    rng = np.random.default_rng(seed)
    lp, lq = _pair(rng, V, scale=1.5, sigma=1.2)
    law, p = _emitted_law(lp, lq, T)
    np.testing.assert_allclose(law, p, atol=1e-12)
    # the bonus draw: the sampler's law on p itself is p
    np.testing.assert_allclose(_sampler_law(final_token_distribution(p, None), V), p, atol=1e-12)


def _mc_slots(rng, V, k, T, n):
    lp = 1.5 * rng.standard_normal((k + 1, V))
    lq = lp[:k] + 1.2 * rng.standard_normal((k, V))
    qs = [softmax(lq[i] / T) for i in range(k)]
    counts = np.zeros((k + 1, V))
    for _ in range(n):
        x = np.array([rng.choice(V, p=qs[i]) for i in range(k)])
        r = verify_request(lp, lq, x, rng.random(k + 1), T, 1.0, with_rkl=False)
        for j in range(r["accept_len"] + 1):
            counts[j, r["tokens"][j]] += 1
    pvals = []
    for j in range(k + 1):
        n_j = counts[j].sum()
        if n_j < 50:
            continue
        exp = softmax(lp[j] / T) * n_j
        pvals.append(chisquare(counts[j], exp).pvalue)
    return pvals


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_lossless_monte_carlo(T):
    rng = np.random.default_rng(20 if T == 1.0 else 21)
    pvals = _mc_slots(rng, 8, 3, T, 20000)
    assert len(pvals) >= 3
    assert min(pvals) > 1e-4 / len(pvals)


# ----------------------------------------------------------------------------- mutations
def test_mutation_reversed_residual_is_caught(monkeypatch):
    def wrong(p, q=None):
        if q is None:
            return np.array(p)
        r = np.maximum(0.0, q - p)  # residual taken the wrong way round
        return r if np.any(r > 0) else np.array(p)

    monkeypatch.setattr(ov, "final_token_distribution", wrong)
    rng = np.random.default_rng(10)
    lp, lq = _pair(rng, 8, scale=1.5, sigma=1.2)
    p = np.exp(log_softmax(lp, 1.0)[0])
    q = np.exp(log_softmax(lq, 1.0)[0])
    resid = _sampler_law(ov.final_token_distribution(p, q), 8)
    law = np.zeros(8)
    for x in range(8):
        pacc = min(1.0, p[x] / q[x])
        law[x] += q[x] * pacc
        law += q[x] * (1 - pacc) * resid
    assert np.max(np.abs(law - p)) > 1e-3
    pvals = _mc_slots(np.random.default_rng(20), 8, 3, 1.0, 4000)
    assert min(pvals) < 1e-4


def test_mutation_inverted_ratio_is_caught(monkeypatch):
    def wrong(log_p_x, log_q_x, u):
        r = min(1.0, math.exp(log_q_x - log_p_x))  # q/p instead of p/q
        return (u < r), r, abs(u - r)

    monkeypatch.setattr(ov, "acceptance", wrong)
    rng = np.random.default_rng(0)
    lp, lq = _pair(rng, 32)
    z, pval = _tau_check(rng, lp, lq, 4, 1.0, 3000)
    assert abs(z) > 4.0 or pval < 1e-4
