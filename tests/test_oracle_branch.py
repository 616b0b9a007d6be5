"""Pins of the branch-lookup oracle (D3D review page, Methodology, inference paragraph: a
verified prefix matching a prepared successor block is a cache hit).  Pinned by the DFlash
notes' greedy trace (Section 5.2, worked example #4) read through the lookup, the
full-acceptance wildcard, invalid requests, and an independent vectorised formulation on
random keys; a planted off-by-one in the accept length is caught."""

import json
import os

import numpy as np

from oracle import branch_lookup, final_tokens

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _trace():
    with open(os.path.join(GOLDEN, "dflash_notes_greedy_trace.json")) as f:
        return json.load(f)


def test_greedy_trace_hits_the_replacement_branch():
    g = _trace()
    k, a = g["block_drafts"], g["expected_accept_len"]
    # the round's packed output: four accepted drafts, the replacement, then -1 (5 tokens)
    drafts = [11, 12, 13, 14]
    replacement = 99
    out = np.full(k + 1, -1)
    out[:a] = drafts
    out[a] = replacement
    assert int(np.sum(out >= 0)) == g["expected_tokens_emitted"]
    y = final_tokens(out, [a], [k])
    assert y.tolist() == [replacement]
    pos = np.array([[3, 4, 4, 4, k]])
    tok = np.array([[replacement, 7, replacement, -1, -1]])
    assert branch_lookup([a], y, pos, tok).tolist() == [2]  # the first matching key wins
    # a branch for the same position but another token, and one a position later, miss
    assert branch_lookup([a], y, np.array([[4, 5]]), np.array([[7, replacement]])).tolist() == [-1]


def test_full_acceptance_wildcard_and_invalid_requests():
    k = 15
    pos = np.array([[0, 5, k], [0, 5, k], [k, k, k]])
    tok = np.array([[3, 3, -1], [3, 3, -1], [-1, -1, -1]])
    hit = branch_lookup([k, 5, -1], [42, 3, 7], pos, tok)
    assert hit.tolist() == [2, 1, -1]
    assert final_tokens(np.arange(2 * (k + 1)), [k, -1], [k, k]).tolist() == [k, -1]


def _vectorised(accept_len, final_token, pos, tok):
    accept_len = np.asarray(accept_len)[:, None]
    match = (pos == accept_len) & ((tok == np.asarray(final_token)[:, None]) | (tok == -1))
    match &= accept_len >= 0
    first = np.where(match.any(axis=1), match.argmax(axis=1), -1)
    return first


def test_lookup_equals_a_vectorised_formulation():
    rng = np.random.default_rng(7)
    for _ in range(20):
        B, n, k = 64, int(rng.integers(1, 30)), int(rng.integers(1, 16))
        al = rng.integers(-1, k + 1, size=B)
        y = rng.integers(0, 6, size=B)
        pos = rng.integers(0, k + 1, size=(B, n))
        tok = rng.integers(-1, 6, size=(B, n))
        np.testing.assert_array_equal(branch_lookup(al, y, pos, tok), _vectorised(al, y, pos, tok))


def test_planted_off_by_one_is_caught():
    def shifted(accept_len, final_token, branch_pos, branch_tok):
        return branch_lookup(np.asarray(accept_len) + 1, final_token, branch_pos, branch_tok)

    g = _trace()
    a = g["expected_accept_len"]
    pos = np.array([[3, 4, 5]])
    tok = np.array([[99, 99, 99]])
    assert branch_lookup([a], [99], pos, tok).tolist() == [1]
    assert shifted([a], [99], pos, tok).tolist() != [1]
