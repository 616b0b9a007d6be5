"""Pins for the oracle's entry-wise clipped reverse-KL (CPU only).

Pinned against: the worked toy example the AdaFlash reading notes print
(tests/golden/adaflash_notes_toy_opd.json), scipy's rel_entr for the unclipped
limit, and invariants that follow from the definition.
"""

import json
import math
import os

import numpy as np
import pytest
from scipy.special import rel_entr, softmax

from oracle import clipped_rkl, clipped_rkl_row, log_softmax


@pytest.fixture(scope="module")
def toy(golden_dir):
    with open(os.path.join(golden_dir, "adaflash_notes_toy_opd.json")) as f:
        return json.load(f)


def _toy_logits(toy):
    return np.log(np.array(toy["p_target"])), np.log(np.array(toy["q_draft"]))


def test_toy_terms_match_printed_values(toy):
    lp, lq = _toy_logits(toy)
    r = clipped_rkl_row(lp, lq, delta=math.inf)
    tol = 10 ** -toy["printed_decimals"] + 1e-12  # the page truncates some values (-0.3747 -> -0.374)
    np.testing.assert_allclose(r["terms"], toy["printed_terms"], atol=tol)
    assert abs(r["KL"] - toy["printed_rkl_sum"]) <= tol
    assert abs(r["R"] - toy["printed_rkl_sum"]) <= tol  # nothing is clipped with delta = inf
    # the per-entry log ratios the page prints before multiplying by q
    q = np.array(toy["q_draft"])
    np.testing.assert_allclose(r["terms"] / q, toy["printed_log_ratio"], atol=tol)


def test_toy_hard_label_term_pins_log_softmax(toy):
    # -log q(A) where A is the target's top-1 token; the page prints 0.598
    lp, lq = _toy_logits(toy)
    top1 = int(np.argmax(lp))
    log_q, _ = log_softmax(lq, 1.0)
    assert abs(-log_q[top1] - toy["printed_hard_ce"]) <= 5e-4
    # and the mixture value the page builds from its rounded numbers
    a = toy["printed_opd_alpha"]
    kl = clipped_rkl_row(lp, lq, math.inf)["KL"]
    assert abs(a * -log_q[top1] + (1 - a) * kl - toy["printed_opd"]) <= 5e-4


def test_toy_clipping_is_entrywise(toy):
    lp, lq = _toy_logits(toy)
    terms = clipped_rkl_row(lp, lq, math.inf)["terms"]
    for delta in (1.0, 0.1, 0.01):
        r = clipped_rkl_row(lp, lq, delta)
        assert r["R"] == pytest.approx(float(np.sum(np.minimum(terms, delta))), abs=1e-15)
    # delta = 0.01: the three positive entries are capped, the negative one passes unchanged
    r = clipped_rkl_row(lp, lq, 0.01)
    assert r["n_clipped"] == 3
    assert r["R"] == pytest.approx(toy["printed_terms"][0] + 3 * 0.01, abs=5e-4)
    assert r["R"] < 0.0
    # delta = 0.1: only B (0.2079) is capped
    assert clipped_rkl_row(lp, lq, 0.1)["n_clipped"] == 1


def test_rare_token_term(toy):
    rt = toy["printed_rare_token"]
    q = np.array([rt["q"], 1.0 - rt["q"]])
    p = np.array([rt["p"], 1.0 - rt["p"]])
    term = clipped_rkl_row(np.log(p), np.log(q), math.inf)["terms"][0]
    assert abs(term - rt["term"]) <= 5e-4
    assert term == pytest.approx(0.02 * math.log(20000.0), rel=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_unclipped_limit_is_scipy_kl(seed):
    rng = np.random.default_rng(seed)
    V = 257
    lp = 3.0 * rng.standard_normal(V)
    lq = lp + rng.standard_normal(V)
    q, p = softmax(lq), softmax(lp)
    ref = math.fsum(rel_entr(q, p).tolist())
    r = clipped_rkl_row(lp, lq, math.inf)
    assert r["R"] == pytest.approx(ref, rel=1e-12, abs=1e-15)
    assert r["KL"] >= 0.0


@pytest.mark.parametrize("seed", [3, 4, 5, 6])
def test_invariants(seed):
    rng = np.random.default_rng(seed)
    V = 1000
    lp = 4.0 * rng.standard_normal(V)
    lq = lp + 2.0 * rng.standard_normal(V)
    lp[rng.choice(V, 100, replace=False)] -= 20.0  # a few entries the target all but forbids
    p, q = softmax(lp), softmax(lq)
    tv = 0.5 * float(np.abs(p - q).sum())
    prev = -math.inf
    kl = clipped_rkl_row(lp, lq, math.inf)["KL"]
    for delta in (1e-4, 1e-3, 1e-2, 0.1, 1.0, 10.0):
        r = clipped_rkl_row(lp, lq, delta)
        assert r["R"] <= kl + 1e-12  # clipping only lowers the sum
        assert r["R"] >= prev - 1e-12  # non-decreasing in delta
        assert r["R"] >= -tv - 1e-12  # each negative term q log(q/p) >= q - p
        prev = r["R"]


def test_identical_rows_give_exact_zero():
    rng = np.random.default_rng(7)
    lp = 4.0 * rng.standard_normal(4096)
    for delta in (1e-3, 1.0, math.inf):
        r = clipped_rkl_row(lp, lp.copy(), delta)
        assert r["R"] == 0.0 and r["KL"] == 0.0


def test_batch_uses_row_index():
    rng = np.random.default_rng(8)
    t = rng.standard_normal((5, 64))
    d = rng.standard_normal((3, 64))
    idx = np.array([4, 0, 2])
    got = clipped_rkl(t, d, 0.05, p_row_index=idx)
    for r in range(3):
        assert got[r] == clipped_rkl_row(t[idx[r]], d[r], 0.05)["R"]
