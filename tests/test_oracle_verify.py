"""Pins for the oracle's verification steps (CPU only): library routines, closed forms,
hand cases and the worked examples the pages print."""

import json
import math
import os

import numpy as np
import pytest
from scipy.special import log_softmax as sp_log_softmax
from scipy.special import logsumexp

from oracle import (acceptance, final_token_distribution, greedy_argmax, inverse_cdf,
                    log_softmax, verify_block, verify_request, widen_logits)


# ----------------------------------------------------------------------------- step 1
@pytest.mark.parametrize("T", [0.7, 1.0, 2.5])
def test_log_softmax_matches_scipy(T):
    rng = np.random.default_rng(1)
    l = 4.0 * rng.standard_normal(5000) - 3.0
    lp, lse = log_softmax(l, T)
    np.testing.assert_allclose(lp, sp_log_softmax(l / T), rtol=0, atol=1e-12)
    assert lse == pytest.approx(logsumexp(l / T), rel=1e-14)


@pytest.mark.parametrize("V", [1, 7, 1000, 151936])
def test_uniform_row_closed_form(V):
    c = -3.25
    _, lse = log_softmax(np.full(V, c), 1.0)
    assert lse == pytest.approx(c + math.log(V), rel=1e-14, abs=1e-14)


def test_bf16_widening_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F7F, 0x0001], dtype=np.uint16)
    want = [1.0, -1.0, 3.140625, 0.0, -0.0, 3.3895313892515355e38, 9.183549615799121e-41]
    np.testing.assert_array_equal(widen_logits(bits, "bf16"), np.array(want))


def test_argmax_ties_go_to_lowest_id():
    assert greedy_argmax(np.array([1.0, 3.0, 2.0, 3.0, 3.0])) == 1
    assert greedy_argmax(np.array([-5.0, -5.0])) == 0


# ----------------------------------------------------------------------------- step 2 (toy)
@pytest.fixture(scope="module")
def toy(golden_dir):
    with open(os.path.join(golden_dir, "adaflash_notes_toy_opd.json")) as f:
        return json.load(f)


def test_toy_acceptance(toy):
    lp = np.log(np.array(toy["p_target"]))
    lq = np.log(np.array(toy["q_draft"]))
    log_p, _ = log_softmax(lp, 1.0)
    log_q, _ = log_softmax(lq, 1.0)
    # B: p/q = 0.15/0.30 = 0.5
    assert acceptance(log_p[1], log_q[1], 0.49)[0]
    assert not acceptance(log_p[1], log_q[1], 0.51)[0]
    assert acceptance(log_p[1], log_q[1], 0.51)[1] == pytest.approx(0.5, rel=1e-12)
    # A: p/q = 0.80/0.55 > 1 -> always accepted
    assert acceptance(log_p[0], log_q[0], 1.0 - 2.0**-24)[0]
    # u = 0 accepts anything the target gives positive mass; equality rejects
    assert acceptance(log_p[3], log_q[3], 0.0)[0]
    assert not acceptance(0.0, 0.0, 1.0)[0]


def test_toy_rejection_resamples_the_residual(toy):
    # residual max(0, p - q) = (0.25, 0, 0, 0): any rejection emits A
    lp = np.log(np.array(toy["p_target"]))
    lq = np.log(np.array(toy["q_draft"]))
    mass = final_token_distribution(np.exp(log_softmax(lp, 1)[0]), np.exp(log_softmax(lq, 1)[0]))
    np.testing.assert_allclose(mass, [0.25, 0, 0, 0], atol=1e-15)
    target = np.stack([lp, lp])
    for u_fin in (0.0, 0.3, 0.999):
        r = verify_request(target, lq[None, :], np.array([1]), np.array([0.9, u_fin]), 1.0, 1.0)
        assert r["accept_len"] == 0
        assert list(r["tokens"]) == [0, -1]


# ----------------------------------------------------------------------------- step 4
def test_inverse_cdf_uniform_row_is_floor():
    rng = np.random.default_rng(2)
    V = 1000
    for u in rng.random(200):
        if abs(u * V - round(u * V)) < 1e-6:
            continue
        tok, margin = inverse_cdf(np.full(V, 1.0 / V), float(u))
        assert tok == int(math.floor(u * V))
        assert margin > 0


def test_inverse_cdf_bin_edges():
    mass = np.array([0.1, 0.2, 0.0, 0.3, 0.4])
    C = np.cumsum(mass)
    for j, c in enumerate(C[:-1]):
        below = inverse_cdf(mass, c - 1e-9)[0]
        above = inverse_cdf(mass, c + 1e-9)[0]
        assert below <= j < above
        assert mass[above] > 0 and mass[below] > 0  # zero-mass ids are never chosen
    assert inverse_cdf(mass, 0.0)[0] == 0
    assert inverse_cdf(mass, 1.0 - 2.0**-24)[0] == 4


def test_zero_residual_falls_back_to_p():
    p = np.array([0.5, 0.5])
    np.testing.assert_array_equal(final_token_distribution(p, p.copy()), p)
    np.testing.assert_array_equal(final_token_distribution(p, None), p)


# ----------------------------------------------------------------------------- whole request
def _rows(rng, k, V, scale=3.0, sigma=0.7):
    lp = scale * rng.standard_normal((k + 1, V))
    lq = lp[:k] + sigma * rng.standard_normal((k, V))
    return lp, lq


def test_greedy_trace_worked_example(golden_dir):
    with open(os.path.join(golden_dir, "dflash_notes_greedy_trace.json")) as f:
        g = json.load(f)
    rng = np.random.default_rng(3)
    k, V = g["block_drafts"], 64
    lp, lq = _rows(rng, k, V)
    argmax_p = np.array([greedy_argmax(r) for r in lp])
    x = argmax_p[:k].copy()
    for i, match in enumerate(g["match_pattern_prefix"]):
        if not match:
            x[i] = (argmax_p[i] + 1) % V
    u = rng.random(k + 1)
    r = verify_request(lp, lq, x, u, 0.0, 1.0)
    assert r["accept_len"] == g["expected_accept_len"]
    n_emitted = int(np.count_nonzero(r["tokens"] >= 0))
    assert n_emitted == g["expected_tokens_emitted"]
    assert list(r["tokens"][:4]) == list(x[:4])
    assert r["tokens"][4] == argmax_p[4]  # the replacement is the target argmax
    # every draft matching gives a = k and the bonus argmax of target row k
    r2 = verify_request(lp, lq, argmax_p[:k], u, 0.0, 1.0)
    assert r2["accept_len"] == k and r2["tokens"][k] == argmax_p[k]


@pytest.mark.parametrize("T", [0.7, 1.0])
def test_all_accept_when_drafter_equals_target(T):
    rng = np.random.default_rng(4)
    k, V = 6, 50
    lp, _ = _rows(rng, k, V)
    lq = lp[:k].copy()
    x = rng.integers(0, V, size=k)
    u = rng.random(k + 1) * (1 - 1e-9)
    r = verify_request(lp, lq, x, u, T, 1.0)
    assert r["accept_len"] == k
    assert list(r["tokens"][:k]) == list(x)
    # the bonus is the inverse CDF of p_T on target row k
    p_bonus = np.exp(log_softmax(lp[k], T)[0])
    assert r["tokens"][k] == inverse_cdf(p_bonus, u[k])[0]
    assert np.all(r["rkl"] == 0.0)


def test_first_position_reject():
    rng = np.random.default_rng(5)
    k, V = 5, 40
    lp, lq = _rows(rng, k, V)
    lp[0, 7] -= 30.0  # the target all but forbids id 7 at position 0
    lq[0, 7] = lq[0].max() + 2.0  # the drafter likes it
    x = np.full(k, 7)
    u = np.full(k + 1, 0.9)
    r = verify_request(lp, lq, x, u, 1.0, 1.0)
    assert r["accept_len"] == 0 and r["tokens"][0] != 7 and np.all(r["tokens"][1:] == -1)
    p0 = np.exp(log_softmax(lp[0], 1)[0])
    q0 = np.exp(log_softmax(lq[0], 1)[0])
    assert r["tokens"][0] == inverse_cdf(np.maximum(0, p0 - q0), 0.9)[0]


def test_temperature_changes_ratio_not_rkl():
    rng = np.random.default_rng(6)
    k, V = 3, 100
    lp, lq = _rows(rng, k, V)
    x = np.array([3, 4, 5])
    u = np.full(k + 1, 0.5)
    a = verify_request(lp, lq, x, u, 0.7, 1.0)
    b = verify_request(lp, lq, x, u, 1.0, 1.0)
    p07 = np.exp(sp_log_softmax(lp[0] / 0.7))[3]
    assert a["p_at_draft"][0] == pytest.approx(p07, rel=1e-12)
    assert a["p_at_draft"][0] != pytest.approx(b["p_at_draft"][0], rel=1e-6)
    np.testing.assert_array_equal(a["rkl"], b["rkl"])


def test_invalid_token_flags_request():
    rng = np.random.default_rng(7)
    lp, lq = _rows(rng, 2, 10)
    r = verify_request(lp, lq, np.array([1, 10]), np.full(3, 0.5), 1.0, 1.0)
    assert r["accept_len"] == -1 and np.all(r["tokens"] == -1)
    assert np.all(np.isfinite(r["rkl"]))


def test_packed_batch_equals_per_request_calls():
    rng = np.random.default_rng(8)
    V, ks, temps = 300, [1, 4, 2, 15], [1.0, 0.0, 0.7, 1.0]
    tgt, drf, xs, us = [], [], [], []
    for kb, T in zip(ks, temps):
        lp, lq = _rows(rng, kb, V)
        tgt.append(lp)
        drf.append(lq)
        xs.append(rng.integers(0, V, size=kb))
        us.append(rng.random(kb + 1))
    res = verify_block(target=np.concatenate(tgt).astype(np.float32),
                       draft=np.concatenate(drf).astype(np.float32), dtype="f32", V=V, k=ks,
                       draft_tokens=np.concatenate(xs), uniforms=np.concatenate(us),
                       temperature=np.array(temps, np.float32), delta=0.5)
    t0 = d0 = 0
    for b, (kb, T) in enumerate(zip(ks, temps)):
        r = verify_request(np.float32(tgt[b]).astype(np.float64),
                           np.float32(drf[b]).astype(np.float64), xs[b], us[b], T, 0.5)
        assert res["accept_len"][b] == r["accept_len"]
        np.testing.assert_array_equal(res["out_tokens"][t0:t0 + kb + 1], r["tokens"])
        np.testing.assert_array_equal(res["rkl"][d0:d0 + kb], r["rkl"])
        t0 += kb + 1
        d0 += kb
