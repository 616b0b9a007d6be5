"""Oracle: the adaptive length head, its truncation, the packed layout and its loss
(test infrastructure only).

Definitions (AdaFlash paper, Section 3.2 "Design of the Adaptive Length Head" and "Online
Update of the Length Head"; Section 3.3 "Adaptive Request Scheduling" for the packing):

    h'_i   = SiLU(W1 h_i + b1),  i = 1..k         per-position features in R^{H'}, H' < H
    h_bar  = (1/k) sum_i h'_i                     mean pooling over the draft positions
    a_hat  = sigmoid(w2 . h_bar + b2)             predicted acceptance rate in [0, 1]
    k_hat  = clamp(floor(a_hat * gamma * k), 1, k)   (the pages' gamma scales a_hat; it is
                                                      applied before the floor, in float64)
    l_len  = (a_hat - a*)^2,  a* = a_b / k_hat_b  the fraction of the verified drafts accepted

The pages state a linear projection and a final linear layer without saying whether they
carry biases; both biases are taken as inputs here (zeros reproduce a bias-free head).
The verification batch is packed to total length sum_b k_hat_b: request b's target rows start
at off_t[b] = sum_{c<b} (k_hat_c + 1) and its draft rows at off_t[b] - b.
"""

from __future__ import annotations

import math

import numpy as np


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x * _sigmoid(x)


def length_head(h: np.ndarray, W1: np.ndarray, b1, w2: np.ndarray, b2: float) -> np.ndarray:
    """a_hat for every request: h [B, k, H], W1 [H', H], b1 [H'] (or None), w2 [H'], b2."""
    h = np.asarray(h, dtype=np.float64)
    W1 = np.asarray(W1, dtype=np.float64)
    b1 = np.zeros(W1.shape[0]) if b1 is None else np.asarray(b1, dtype=np.float64)
    feats = silu(np.einsum("bkh,nh->bkn", h, W1) + b1)  # per-position features
    pooled = feats.mean(axis=1)
    return _sigmoid(pooled @ np.asarray(w2, dtype=np.float64) + float(b2))


def truncate(a_hat, k: int, gamma: float = 1.0) -> np.ndarray:
    """k_hat = clamp(floor(a_hat * gamma * k), 1, k)."""
    a = np.asarray(a_hat, dtype=np.float64)
    return np.clip(np.floor(a * float(gamma) * k), 1, k).astype(np.int64)


def truncation_margin(a_hat, k: int, gamma: float = 1.0) -> np.ndarray:
    """Distance of a_hat * gamma * k to the nearest integer (the floor's decision margin)."""
    x = np.asarray(a_hat, dtype=np.float64) * float(gamma) * k
    return np.abs(x - np.round(x))


def packed_offsets(k_hat) -> dict:
    """Target-row and draft-row offsets of the packed verification batch."""
    k_hat = np.asarray(k_hat, dtype=np.int64)
    off_t = np.concatenate([[0], np.cumsum(k_hat + 1)])
    return {"off_t": off_t, "off_d": off_t[:-1] - np.arange(k_hat.shape[0]),
            "n_draft_rows": int(k_hat.sum()), "n_target_rows": int(off_t[-1])}


def length_loss(a_hat, accept_len, k_hat) -> np.ndarray:
    """(a_hat - a*)^2 with a* = accept_len / k_hat."""
    a_star = np.asarray(accept_len, dtype=np.float64) / np.asarray(k_hat, dtype=np.float64)
    return (np.asarray(a_hat, dtype=np.float64) - a_star) ** 2
