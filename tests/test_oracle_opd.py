"""Pins for the oracle's hard-label cross-entropy and mixture OPD loss (CPU only).

Pinned against: the toy position the AdaFlash reading notes work through
(tests/golden/adaflash_notes_toy_opd.json: hard-label CE 0.598, OPD value 0.5132 at
alpha = 0.8, built there from the rounded parts), closed forms of the definition
(alpha = 0 and 1, identical rows, a uniform drafter), scipy's rel_entr for the
unclipped reverse KL and softmax for the cross-entropy, and the lowest-id tie rule.
"""

import json
import math
import os

import numpy as np
import pytest
from scipy.special import log_softmax as sp_log_softmax
from scipy.special import rel_entr

from oracle import hard_ce_row, opd_loss


@pytest.fixture(scope="module")
def toy(golden_dir):
    with open(os.path.join(golden_dir, "adaflash_notes_toy_opd.json")) as f:
        return json.load(f)


def _toy_logits(toy):
    return np.log(np.array(toy["p_target"])), np.log(np.array(toy["q_draft"]))


def test_toy_hard_ce_and_opd_match_printed_values(toy):
    lp, lq = _toy_logits(toy)
    h, x = hard_ce_row(lp, lq)
    assert x == 0  # token A, the target's top-1
    assert abs(h - toy["printed_hard_ce"]) <= 10 ** -toy["printed_decimals"]
    assert h == pytest.approx(-math.log(toy["q_draft"][0]), rel=1e-14)
    out = opd_loss(lp[None, :], lq[None, :], [1], delta=math.inf, alpha=toy["printed_opd_alpha"])
    # the page combines the rounded 0.598 and 0.174; exact arithmetic agrees to ~5e-4
    assert abs(out["opd"][0] - toy["printed_opd"]) <= 5e-4
    kl = float(np.sum(rel_entr(np.array(toy["q_draft"]), np.array(toy["p_target"]))))
    assert out["opd"][0] == pytest.approx(0.8 * -math.log(0.55) + 0.2 * kl, rel=1e-13)


def test_toy_clipped_opd_follows_the_entrywise_min(toy):
    # delta = 0.01 clips the three positive terms and keeps the negative one (reading of
    # the notes' remark: see the fixture's note)
    lp, lq = _toy_logits(toy)
    q, p = np.array(toy["q_draft"]), np.array(toy["p_target"])
    first = q[0] * math.log(q[0] / p[0])
    out = opd_loss(lp[None, :], lq[None, :], [1], delta=0.01, alpha=0.8)
    assert out["rkl"][0] == pytest.approx(first + 3 * 0.01, rel=1e-13)
    assert out["opd"][0] == pytest.approx(0.8 * -math.log(0.55) + 0.2 * (first + 0.03), rel=1e-13)


def test_alpha_limits_and_means_over_positions():
    rng = np.random.default_rng(3)
    lp = rng.normal(size=(7, 50)) * 2
    lq = lp + rng.normal(size=(7, 50))
    k = [3, 4]
    a1 = opd_loss(lp, lq, k, delta=0.3, alpha=1.0)
    a0 = opd_loss(lp, lq, k, delta=0.3, alpha=0.0)
    for b, (lo, hi) in enumerate(((0, 3), (3, 7))):
        ce = [-sp_log_softmax(lq[r])[np.argmax(lp[r])] for r in range(lo, hi)]
        assert a1["opd"][b] == pytest.approx(np.mean(ce), rel=1e-13)
        assert a0["opd"][b] == pytest.approx(np.mean(a0["rkl"][lo:hi]), rel=1e-13)


def test_identical_rows_give_alpha_times_target_entropy_of_top1():
    lp = np.array([[0.3, 2.0, -1.0, 0.7], [1.0, 1.0, 0.0, -3.0]])
    out = opd_loss(lp, lp.copy(), [2], delta=1.0, alpha=0.8)
    assert np.all(out["rkl"] == 0.0)
    ce = [-sp_log_softmax(lp[0])[1], -sp_log_softmax(lp[1])[0]]
    assert out["opd"][0] == pytest.approx(0.8 * np.mean(ce), rel=1e-14)


def test_uniform_drafter_costs_log_v():
    V = 37
    lp = np.linspace(-2, 3, V)
    h, x = hard_ce_row(lp, np.zeros(V))
    assert x == V - 1 and h == pytest.approx(math.log(V), rel=1e-14)


def test_ties_go_to_the_lowest_id():
    lp = np.array([0.0, 5.0, 1.0, 5.0])
    lq = np.array([0.0, -1.0, 0.0, 2.0])
    h, x = hard_ce_row(lp, lq)
    assert x == 1
    assert h == pytest.approx(-sp_log_softmax(lq)[1], rel=1e-14)


def test_p_row_index_pairs_rows():
    rng = np.random.default_rng(4)
    lp = rng.normal(size=(5, 20))
    lq = rng.normal(size=(3, 20))
    idx = [4, 0, 2]
    out = opd_loss(lp, lq, [3], delta=0.5, alpha=0.8, p_row_index=idx)
    for r, t in enumerate(idx):
        assert out["hard"][r] == pytest.approx(hard_ce_row(lp[t], lq[r])[0], rel=1e-15)


# ----------------------------------------------------------------------------- gradient
from oracle import clipped_rkl_grad_row, opd_grad  # noqa: E402


def _fd_grad(f, a, h=1e-6):
    g = np.empty_like(a)
    for z in range(a.shape[0]):
        e = np.zeros_like(a)
        e[z] = h
        g[z] = (f(a + e) - f(a - e)) / (2 * h)
    return g


def _R(lp, lq, delta):
    from oracle import clipped_rkl_row

    return clipped_rkl_row(lp, lq, delta)["R"]


@pytest.mark.parametrize("delta", [math.inf, 0.05, 0.01])
def test_rkl_gradient_matches_finite_differences(delta):
    rng = np.random.default_rng(7)
    for V in (3, 8, 16):
        lp = rng.normal(size=V) * 2
        lq = lp + rng.normal(size=V)
        g = clipped_rkl_grad_row(lp, lq, delta)
        # stay away from the kink: no entry within the difference step of delta
        lpq = sp_log_softmax(lq) - sp_log_softmax(lp)
        t = np.exp(sp_log_softmax(lq)) * lpq
        assert np.all(np.abs(t - delta) > 1e-3)
        fd = _fd_grad(lambda a: _R(lp, a, delta), lq)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-9)
        assert abs(g.sum()) < 1e-12  # logits are shift-invariant


def test_rkl_gradient_equals_autograd_of_the_definition():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(8)
    lp = rng.normal(size=40) * 3
    lq = lp + rng.normal(size=40) * 1.5
    for delta in (math.inf, 0.02):
        a = torch.tensor(lq, dtype=torch.float64, requires_grad=True)
        log_q = torch.log_softmax(a, 0)
        log_p = torch.log_softmax(torch.tensor(lp, dtype=torch.float64), 0)
        terms = log_q.exp() * (log_q - log_p)
        loss = torch.clamp(terms, max=delta).sum() if math.isfinite(delta) else terms.sum()
        loss.backward()
        np.testing.assert_allclose(clipped_rkl_grad_row(lp, lq, delta), a.grad.numpy(),
                                   rtol=1e-12, atol=1e-15)


def test_unclipped_gradient_is_the_kl_gradient():
    # delta -> inf: dKL(q||p)/da_z = q_z (L_z - KL)
    rng = np.random.default_rng(9)
    lp, lq = rng.normal(size=25), rng.normal(size=25)
    q = np.exp(sp_log_softmax(lq))
    L = sp_log_softmax(lq) - sp_log_softmax(lp)
    kl = float(np.sum(rel_entr(q, np.exp(sp_log_softmax(lp)))))
    np.testing.assert_allclose(clipped_rkl_grad_row(lp, lq, math.inf), q * (L - kl),
                               rtol=1e-12, atol=1e-16)


def test_clip_cuts_the_gradient_of_every_positive_term():
    # delta below every positive term: those entries pass no gradient, the negative ones do
    lp = np.log(np.array([0.1, 0.2, 0.3, 0.4]))
    lq = np.log(np.array([0.4, 0.3, 0.2, 0.1]))
    t = np.array([0.4, 0.3, 0.2, 0.1]) * (lq - lp)
    g = clipped_rkl_grad_row(lp, lq, delta=1e-9)
    neg = t < 0
    assert np.any(neg)  # negative terms keep a gradient; positives are cut
    q = np.exp(lq)
    gy = np.where(neg, (lq - lp) + 1.0, 0.0)
    np.testing.assert_allclose(g, q * (gy - np.sum(q * gy)), rtol=1e-13)


def test_opd_gradient_matches_finite_differences_of_the_loss():
    rng = np.random.default_rng(10)
    lp = rng.normal(size=(5, 12)) * 2
    lq = lp + rng.normal(size=(5, 12))
    k = [2, 3]
    delta, alpha = 0.05, 0.8
    g = opd_grad(lp, lq, k, delta, alpha)
    off = [0, 2, 5]
    for b in range(2):
        for r in range(off[b], off[b + 1]):
            def f(a, r=r, b=b):
                rows = lq[off[b]:off[b + 1]].copy()
                rows[r - off[b]] = a
                return opd_loss(lp[off[b]:off[b + 1]], rows, [k[b]], delta, alpha)["opd"][0]
            np.testing.assert_allclose(g[r], _fd_grad(f, lq[r]), rtol=1e-6, atol=1e-9)
