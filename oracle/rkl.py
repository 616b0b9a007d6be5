"""Oracle: entry-wise clipped reverse-KL (test infrastructure only).

Definition (AdaFlash paper, Section 3.1, "Entry-wise Divergence Clipping"; the
reading notes' Algorithm 2 restates it): for draft position i,

    R_i = sum over the whole vocabulary y of  min( q_i(y) * log(q_i(y) / p_i(y)),  delta )

with q_i the drafter's distribution at position i and p_i the target's, the
minimum taken per (i, y) entry before the sum.  The paper's loss also divides by
k; that factor is left to the caller.  Appendix B.1 fixes the reverse-KL
temperature at 1, so both distributions are plain softmaxes of the logits.

The term is evaluated in the log domain, q * (log q - log p), so an underflowed
q contributes exactly 0 and finite logits never give NaN.
"""

from __future__ import annotations

import math

import numpy as np


def _log_softmax_t1(logits: np.ndarray) -> np.ndarray:
    l = np.asarray(logits, dtype=np.float64)
    m = np.max(l)
    return l - (m + np.log(np.sum(np.exp(l - m))))


def clipped_rkl_row(target_logits: np.ndarray, draft_logits: np.ndarray, delta: float) -> dict:
    """One draft position: R (clipped), KL (unclipped) and diagnostics, in float64.

    ``delta = inf`` gives the plain reverse KL(q || p).
    """
    log_p = _log_softmax_t1(target_logits)
    log_q = _log_softmax_t1(draft_logits)
    q = np.exp(log_q)
    terms = q * (log_q - log_p)
    clipped = np.minimum(terms, delta)
    return {
        "R": math.fsum(clipped.tolist()),
        "KL": math.fsum(terms.tolist()),
        "L1": math.fsum(np.abs(clipped).tolist()),  # mass of the summands, the scale for tolerances
        "n_clipped": int(np.count_nonzero(terms > delta)),
        "terms": terms,
    }


def clipped_rkl(target_rows: np.ndarray, draft_rows: np.ndarray, delta: float,
                p_row_index=None) -> np.ndarray:
    """R for every draft row r, against target row ``p_row_index[r]`` (identity if None)."""
    n = draft_rows.shape[0]
    idx = np.arange(n) if p_row_index is None else np.asarray(p_row_index)
    return np.array([clipped_rkl_row(target_rows[idx[r]], draft_rows[r], delta)["R"]
                     for r in range(n)], dtype=np.float64)
