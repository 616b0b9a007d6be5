"""Pins for the oracle's adaptive length head, truncation, packing and loss (CPU only).

Pinned against: the truncation cases worked from the paper's formula (a_hat = 0.73, k = 15
gives 10; a tiny a_hat is clamped to 1; gamma = 1.2 at a_hat = 1 is clamped to k), closed
forms (zero inputs reduce the head to sigmoid(w2 . SiLU(b1) + b2); one position, one
feature, no bias reduce it to sigmoid(w2 SiLU(w1 h))), library routines (scipy's expit for
the sigmoid inside SiLU, torch's linear + silu + mean in float64 for the whole head), and
invariants (mean pooling ignores position order; the loss vanishes when the prediction is
the realised rate).
"""

import numpy as np
import pytest
from scipy.special import expit

from oracle import length_head, length_loss, packed_offsets, silu, truncate, truncation_margin


def test_truncation_cases():
    assert int(truncate(0.73, 15)) == 10
    assert int(truncate(0.05, 15)) == 1
    assert int(truncate(1.0, 15, gamma=1.2)) == 15
    assert int(truncate(0.0, 15)) == 1
    assert list(truncate([0.2, 0.5, 0.99], 16)) == [3, 8, 15]
    assert truncation_margin(0.5, 16)[()] == 0.0 and truncation_margin(0.53, 10)[()] == pytest.approx(0.3)


def test_silu_is_x_times_expit():
    x = np.linspace(-8, 8, 33)
    np.testing.assert_allclose(silu(x), x * expit(x), rtol=1e-15)


def test_zero_input_closed_form():
    rng = np.random.default_rng(1)
    Hp, H = 6, 10
    W1 = rng.normal(size=(Hp, H))
    b1, w2, b2 = rng.normal(size=Hp), rng.normal(size=Hp), 0.3
    a = length_head(np.zeros((2, 4, H)), W1, b1, w2, b2)
    ref = expit(w2 @ (b1 * expit(b1)) + b2)
    np.testing.assert_allclose(a, [ref, ref], rtol=1e-14)


def test_scalar_head_closed_form():
    a = length_head(np.array([[[2.0]]]), np.array([[0.5]]), None, np.array([3.0]), 0.0)
    z = 0.5 * 2.0
    assert a[0] == pytest.approx(expit(3.0 * z * expit(z)), rel=1e-15)


def test_head_equals_torch_modules_in_float64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(2)
    B, k, H, Hp = 3, 5, 16, 8
    h = rng.normal(size=(B, k, H))
    W1, b1 = rng.normal(size=(Hp, H)) / 4, rng.normal(size=Hp)
    w2, b2 = rng.normal(size=Hp), -0.2
    t = torch.nn.functional.linear(torch.tensor(h), torch.tensor(W1), torch.tensor(b1))
    ref = torch.sigmoid(torch.nn.functional.silu(t).mean(dim=1) @ torch.tensor(w2) + b2).numpy()
    np.testing.assert_allclose(length_head(h, W1, b1, w2, b2), ref, rtol=1e-13)


def test_mean_pooling_ignores_position_order():
    rng = np.random.default_rng(3)
    h = rng.normal(size=(1, 7, 12))
    W1, w2 = rng.normal(size=(5, 12)), rng.normal(size=5)
    a = length_head(h, W1, None, w2, 0.0)
    b = length_head(h[:, rng.permutation(7)], W1, None, w2, 0.0)
    assert a[0] == pytest.approx(b[0], rel=1e-14)


def test_packed_offsets_and_loss():
    off = packed_offsets([3, 1, 4])
    assert list(off["off_t"]) == [0, 4, 6, 11]
    assert list(off["off_d"]) == [0, 3, 4]
    assert off["n_draft_rows"] == 8 and off["n_target_rows"] == 11
    np.testing.assert_allclose(length_loss([0.5, 0.25], [2, 1], [4, 4]), [0.0, 0.0], atol=0)
    np.testing.assert_allclose(length_loss([1.0], [0], [5]), [1.0])
