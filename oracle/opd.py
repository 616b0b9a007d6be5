"""Oracle: hard-label cross-entropy and the mixture on-policy-distillation loss
(test infrastructure only).

Definitions (AdaFlash paper, Section 3.1, "Mixture OPD Loss with Reverse-KL" and the
final OPD loss that combines it with "Entry-wise Divergence Clipping"; Appendix B.1
fixes the distillation temperature at 1, so both distributions are plain softmaxes):

    x*_i        = argmax_x p_i(x)                  the target's top-1 token at position i
    l_hard      = -(1/k) sum_i log q_i(x*_i)       hard-label cross-entropy
    l_rkl^clip  = (1/k) sum_i R_i                  R_i as in ``oracle.rkl``
    l_OPD       = alpha l_hard + (1 - alpha) l_rkl^clip

for one request whose drafter proposed k positions (after the length head's truncation,
Section 3.2, k is that request's k_b).  Ties in the argmax go to the lowest id.

The gradient of l_OPD with respect to the drafter's logits (the signal OPD trains with;
the paper motivates the clip by the outlier gradients it removes, Section 3.1 and
Figure 3) is derived here from these definitions; where an entry sits exactly on the
clip (t = delta) the clipped side's derivative, 0, is taken.
"""

from __future__ import annotations

import math

import numpy as np

from .rkl import clipped_rkl_row


def _log_softmax_t1(logits: np.ndarray) -> np.ndarray:
    l = np.asarray(logits, dtype=np.float64)
    m = np.max(l)
    return l - (m + np.log(np.sum(np.exp(l - m))))


def hard_ce_row(target_logits: np.ndarray, draft_logits: np.ndarray):
    """(-log q(x*), x*) for one position, x* the first id where the target logit is largest."""
    x = int(np.argmax(np.asarray(target_logits, dtype=np.float64)))  # first maximum
    return float(-_log_softmax_t1(draft_logits)[x]), x


def opd_loss(target_rows: np.ndarray, draft_rows: np.ndarray, k, delta: float, alpha: float,
             p_row_index=None) -> dict:
    """Per draft row: R_i, -log q_i(x*_i), x*_i; per request (rows packed, k[b] each): the
    means of both and l_OPD.  Draft row r pairs with target row p_row_index[r] (identity if
    None)."""
    n = draft_rows.shape[0]
    idx = np.arange(n) if p_row_index is None else np.asarray(p_row_index)
    R = np.empty(n)
    hard = np.empty(n)
    top1 = np.empty(n, dtype=np.int64)
    for r in range(n):
        R[r] = clipped_rkl_row(target_rows[idx[r]], draft_rows[r], delta)["R"]
        hard[r], top1[r] = hard_ce_row(target_rows[idx[r]], draft_rows[r])
    k = np.asarray(k, dtype=np.int64)
    assert int(k.sum()) == n
    off = np.concatenate([[0], np.cumsum(k)])
    hard_mean = np.array([math.fsum(hard[off[b]:off[b + 1]]) / k[b] for b in range(k.shape[0])])
    rkl_mean = np.array([math.fsum(R[off[b]:off[b + 1]]) / k[b] for b in range(k.shape[0])])
    return {
        "rkl": R,
        "hard": hard,
        "top1": top1,
        "hard_mean": hard_mean,
        "rkl_mean": rkl_mean,
        "opd": alpha * hard_mean + (1.0 - alpha) * rkl_mean,
    }


def clipped_rkl_grad_row(target_logits: np.ndarray, draft_logits: np.ndarray,
                         delta: float) -> np.ndarray:
    """d R / d a_z for one position, a the drafter's logits (temperature 1).

    With L_y = log q_y - log p_y, t_y = q_y L_y and dq_y/da_z = q_y (1[y = z] - q_z):
        dt_y/da_z = q_y (1[y = z] - q_z) (L_y + 1),
    and min(delta, t) passes the derivative where t < delta and stops it where the clip is
    active (at t = delta exactly the clipped side, 0, is taken), so
        dR/da_z = q_z (g_z - sum_y q_y g_y),   g_y = 1[t_y < delta] (L_y + 1).
    """
    log_p = _log_softmax_t1(target_logits)
    log_q = _log_softmax_t1(draft_logits)
    q = np.exp(log_q)
    L = log_q - log_p
    g = np.where(q * L < delta, L + 1.0, 0.0)
    return q * (g - math.fsum((q * g).tolist()))


def opd_grad(target_rows: np.ndarray, draft_rows: np.ndarray, k, delta: float, alpha: float,
             p_row_index=None) -> np.ndarray:
    """d l_OPD,b / d a_r for every draft row r of request b (rows packed, k[b] each):
        (alpha / k_b) (q_r - e_{x*_r}) + ((1 - alpha) / k_b) dR_r/da_r,
    the first term the gradient of -log q_r(x*_r), x*_r the target's top-1."""
    n = draft_rows.shape[0]
    idx = np.arange(n) if p_row_index is None else np.asarray(p_row_index)
    k = np.asarray(k, dtype=np.int64)
    assert int(k.sum()) == n
    req = np.repeat(np.arange(k.shape[0]), k)
    out = np.empty(draft_rows.shape, dtype=np.float64)
    for r in range(n):
        kb = float(k[req[r]])
        q = np.exp(_log_softmax_t1(draft_rows[r]))
        _, x = hard_ce_row(target_rows[idx[r]], draft_rows[r])
        ce = q.copy()
        ce[x] -= 1.0
        out[r] = (alpha / kb) * ce + ((1.0 - alpha) / kb) * clipped_rkl_grad_row(
            target_rows[idx[r]], draft_rows[r], delta)
    return out
