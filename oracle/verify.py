"""Oracle: batched verification of a one-pass diffusion draft block (test infrastructure only).

The algorithm, per request b with k_b draft tokens (AdaFlash paper, Section 2.1
"Speculative Decoding and Diffusion Drafters"; reading notes, steps 3-4 of the
basic recipe; DFlash notes, Section 3.1 step 6 and Section 5.2):

1. Distributions.  Target row i (i = 0..k_b) and draft row i (i < k_b) are
   turned into p_T = softmax(l_p / T_b) and q_T = softmax(l_q / T_b).  The
   drafter's rows are per-position marginals from one forward pass; the test is
   applied to each position independently with those marginals (DFlash notes,
   Section 5.2).
2. Acceptance.  Draft x_i is accepted with probability min(1, p_T(x_i) / q_T(x_i)),
   realised with the given uniform as u_i < min(1, ratio).  For T_b = 0 (greedy,
   the paper's default decoding, Appendix B.1) the draft is accepted iff it equals
   the target argmax (DFlash notes, Section 5.2, worked example #4).
3. First-rejection scan.  Everything before the first rejection is kept:
   a_b = first rejected position, or k_b if none.  Positions >= k_b do not exist:
   the per-request length came from the length head (paper, Section 3.2).
4. Final token.  At a rejection the token is drawn from the normalised residual
   max(0, p_T - q_T) of that position (paper, Section 2.1; reading notes step 4);
   if every draft was accepted it is a bonus token drawn from p_T of target row
   k_b (DFlash notes, Section 3.1 step 6).  Greedy takes the target argmax.
5. Emit.  a_b accepted drafts followed by the final token: a_b + 1 tokens.

Plus the per-position clipped reverse-KL from ``oracle.rkl`` for every draft row.

Parity unpinned: the fallback of step 4 for a residual of zero total mass (draw from
p_T of the same row).  In exact arithmetic that mass equals the rejection probability,
so the pages never reach the case; the fallback is a reading, and nothing on the pages
gives a value to check it against.
"""

from __future__ import annotations

import math

import numpy as np

from .rkl import clipped_rkl_row


# ----------------------------------------------------------------------------- inputs
def widen_logits(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of stored logits: bf16 bit patterns (uint16) or fp32."""
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------- step 1
def log_softmax(logits: np.ndarray, T: float):
    """log softmax(l / T) over the full vocabulary and its log-normaliser, T > 0."""
    z = np.asarray(logits, dtype=np.float64) / T
    m = np.max(z)
    lse = m + math.log(np.sum(np.exp(z - m)))
    return z - lse, lse


def greedy_argmax(logits: np.ndarray) -> int:
    """Argmax with ties going to the lowest id (np.argmax returns the first maximum)."""
    return int(np.argmax(np.asarray(logits)))


# ----------------------------------------------------------------------------- step 2
def acceptance(log_p_x: float, log_q_x: float, u: float):
    """u < min(1, p(x)/q(x)).  Returns (accepted, min(1, ratio), |u - min(1, ratio)|)."""
    r = min(1.0, math.exp(log_p_x - log_q_x))
    return (u < r), r, abs(u - r)


# ----------------------------------------------------------------------------- step 4
def final_token_distribution(p: np.ndarray, q=None) -> np.ndarray:
    """Unnormalised mass the final token is drawn from.

    Rejection at a position: max(0, p - q).  Bonus (q is None): p itself.  A residual
    of zero total mass can only come from rounding (its exact mass equals the
    rejection probability), and then p is used.
    """
    if q is None:
        return np.array(p, dtype=np.float64)
    r = np.maximum(0.0, p - q)
    if not np.any(r > 0.0):
        return np.array(p, dtype=np.float64)
    return r


def inverse_cdf(mass: np.ndarray, u: float):
    """Smallest id j with (sum_{y<=j} mass_y) > u * Z, Z = total mass; ascending id order.

    Returns (token, margin): margin is the distance of u*Z to the nearer edge of the
    chosen id's cumulative interval, divided by Z.  If rounding leaves no such id,
    the largest id with positive mass is taken (margin 0).
    """
    C = np.cumsum(np.asarray(mass, dtype=np.float64))
    Z = C[-1]
    thr = u * Z
    j = int(np.searchsorted(C, thr, side="right"))
    if j >= C.shape[0]:
        return int(np.flatnonzero(mass > 0.0)[-1]), 0.0
    lo = C[j - 1] if j > 0 else 0.0
    return j, min(C[j] - thr, thr - lo) / Z


# ----------------------------------------------------------------------------- one request
def verify_request(target_logits: np.ndarray, draft_logits: np.ndarray, x: np.ndarray,
                   u: np.ndarray, T: float, delta: float, with_rkl: bool = True) -> dict:
    """One request: ``target_logits`` [k+1, V], ``draft_logits`` [k, V] (float64),
    ``x`` [k] draft ids, ``u`` [k+1] uniforms, temperature ``T``, clip threshold ``delta``."""
    k = draft_logits.shape[0]
    V = target_logits.shape[1]
    assert target_logits.shape[0] == k + 1 and x.shape == (k,) and u.shape == (k + 1,)
    out = {
        "k": k,
        "accepted": np.zeros(k, dtype=bool),
        "ratio": np.full(k, np.nan),
        "accept_margin": np.full(k, np.inf),
        "p_at_draft": np.full(k, np.nan),
        "q_at_draft": np.full(k, np.nan),
        "acc_rate": np.full(k, np.nan),  # Acc_i = sum_y min(p_T, q_T)
    }
    if np.any((x < 0) | (x >= V)):
        out.update(accept_len=-1, tokens=np.full(k + 1, -1, dtype=np.int64), token_margin=np.inf,
                   invalid=True)
    else:
        out["invalid"] = False
    Tm = 1.0 if T == 0.0 else T  # greedy requests report temperature-1 probabilities

    # step 1 (+ the reported probabilities at the draft tokens)
    log_pT = [log_softmax(target_logits[i], Tm)[0] for i in range(k + 1)]
    log_qT = [log_softmax(draft_logits[i], Tm)[0] for i in range(k)]
    for i in range(k):
        out["acc_rate"][i] = float(np.sum(np.minimum(np.exp(log_pT[i]), np.exp(log_qT[i]))))
        if not out["invalid"]:
            out["p_at_draft"][i] = math.exp(log_pT[i][x[i]])
            out["q_at_draft"][i] = math.exp(log_qT[i][x[i]])

    if not out["invalid"]:
        # steps 2-3: acceptance and first-rejection scan
        a = k
        for i in range(k):
            if T == 0.0:
                ok = int(x[i]) == greedy_argmax(target_logits[i])
                out["accepted"][i] = ok
            else:
                ok, r, margin = acceptance(log_pT[i][x[i]], log_qT[i][x[i]], float(u[i]))
                out["accepted"][i], out["ratio"][i], out["accept_margin"][i] = ok, r, margin
            if not ok:
                a = i
                break
        # step 4: final token
        if T == 0.0:
            tok, tmargin = greedy_argmax(target_logits[a]), np.inf
        else:
            p = np.exp(log_pT[a])
            mass = final_token_distribution(p, None if a == k else np.exp(log_qT[a]))
            tok, tmargin = inverse_cdf(mass, float(u[k]))
        # step 5: emit a accepted drafts then the final token
        tokens = np.full(k + 1, -1, dtype=np.int64)
        tokens[:a] = x[:a]
        tokens[a] = tok
        out.update(accept_len=a, tokens=tokens, token_margin=tmargin)

    if with_rkl:
        rows = [clipped_rkl_row(target_logits[i], draft_logits[i], delta) for i in range(k)]
        out["rkl"] = np.array([r["R"] for r in rows])
        out["kl"] = np.array([r["KL"] for r in rows])
        out["rkl_l1"] = np.array([r["L1"] for r in rows])
        out["n_clipped"] = np.array([r["n_clipped"] for r in rows])
    return out


def expected_tau(acc_rates) -> float:
    """E[tau] = sum_{j=0}^{k} prod_{i<j} Acc_i: expected tokens emitted per round when
    position i survives with probability Acc_i.  With equal Acc_i this is the
    paper's (1 - Acc^(k+1)) / (1 - Acc) (Section 2.1)."""
    total, prod = 1.0, 1.0
    for a in acc_rates:
        prod *= a
        total += prod
    return total


# ----------------------------------------------------------------------------- batch
def verify_block(*, target, draft, dtype, V, k, draft_tokens, uniforms, temperature, delta,
                 requests=None, with_rkl: bool = True) -> dict:
    """Packed batch: request b owns target rows off_t[b] .. off_t[b]+k_b and draft rows
    off_d[b] .. off_d[b]+k_b-1 (one verification batch of total length sum k_b, paper
    Section 3.3).  ``requests`` restricts the work to a subset (outputs for the others
    are left as -1 / NaN)."""
    k = np.asarray(k, dtype=np.int64)
    B = k.shape[0]
    off_t = np.concatenate([[0], np.cumsum(k + 1)])
    off_d = np.concatenate([[0], np.cumsum(k)])
    n_t, n_d = int(off_t[-1]), int(off_d[-1])
    res = {
        "accept_len": np.full(B, -1, dtype=np.int64),
        "out_tokens": np.full(n_t, -1, dtype=np.int64),
        "rkl": np.full(n_d, np.nan),
        "kl": np.full(n_d, np.nan),
        "rkl_l1": np.full(n_d, np.nan),
        "p_at_draft": np.full(n_d, np.nan),
        "q_at_draft": np.full(n_d, np.nan),
        "accept_margin": np.full(n_d, np.inf),
        "token_margin": np.full(B, np.inf),
        "acc_rate": np.full(n_d, np.nan),
        "expected_tau": np.full(B, np.nan),
        "done": np.zeros(B, dtype=bool),
    }
    todo = range(B) if requests is None else requests
    for b in todo:
        kb = int(k[b])
        tl = widen_logits(target[off_t[b]: off_t[b + 1], :V], dtype)
        dl = widen_logits(draft[off_d[b]: off_d[b + 1], :V], dtype)
        r = verify_request(tl, dl, np.asarray(draft_tokens[off_d[b]: off_d[b + 1]], dtype=np.int64),
                           np.asarray(uniforms[off_t[b]: off_t[b + 1]], dtype=np.float64),
                           float(temperature[b]), float(delta), with_rkl=with_rkl)
        res["accept_len"][b] = r["accept_len"]
        res["out_tokens"][off_t[b]: off_t[b + 1]] = r["tokens"]
        res["token_margin"][b] = r["token_margin"]
        sl = slice(off_d[b], off_d[b + 1])
        res["p_at_draft"][sl] = r["p_at_draft"]
        res["q_at_draft"][sl] = r["q_at_draft"]
        res["accept_margin"][sl] = r["accept_margin"]
        res["acc_rate"][sl] = r["acc_rate"]
        res["expected_tau"][b] = expected_tau(r["acc_rate"])
        if with_rkl:
            res["rkl"][sl] = r["rkl"]
            res["kl"][sl] = r["kl"]
            res["rkl_l1"][sl] = r["rkl_l1"]
        res["done"][b] = True
        assert kb == r["k"]
    return res
