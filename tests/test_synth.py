"""The seeded input generator: determinism and the structure of each workload (CPU only)."""

import numpy as np
import pytest

from synth import bf16_bits_from_f64, bf16_bits_to_f32, make_workload, workload


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-8 + 2**-20, -3.0, 0.0])
    np.testing.assert_array_equal(bf16_bits_to_f32(bf16_bits_from_f64(x)),
                                  np.array([1.0, 1.0 + 4 * 2**-8, 1.0 + 2 * 2**-8, -3.0, 0.0],
                                           dtype=np.float32))


def test_same_seed_same_bytes():
    a = workload("ragged", rep=0, B=4)
    b = workload("ragged", rep=0, B=4)
    c = workload("ragged", rep=1, B=4)
    for f in ("k", "temperature", "target", "draft", "draft_tokens", "uniforms"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    assert not np.array_equal(a.target, c.target)


def test_tiny_shape_and_ranges():
    w = workload("tiny")
    assert w.dtype == "f32" and w.B == 1 and list(w.k) == [4] and w.V == 1000
    assert w.target.shape == (5, 1000) and w.draft.shape == (4, 1000)
    assert np.all((w.uniforms >= 0) & (w.uniforms < 1))
    assert np.all((w.draft_tokens >= 0) & (w.draft_tokens < 1000))


def test_ragged_mix():
    w = workload("ragged", B=12)
    assert w.k.min() >= 1 and w.k.max() <= 15
    assert set(np.unique(w.temperature)).issubset({0.0, np.float32(0.7), 1.0})
    do = w.draft_offsets
    for b in range(w.B):  # greedy requests draft the drafter's argmax
        if w.temperature[b] == 0.0:
            for i in range(w.k[b]):
                row = bf16_bits_to_f32(w.draft[do[b] + i])
                assert w.draft_tokens[do[b] + i] == int(np.argmax(row))


def test_large_vocab_forced_cases():
    w = workload("large_vocab", B=20)  # floor(5% of 20) = 1 forced request of each kind
    assert len(w.meta["all_accept"]) == 1 and len(w.meta["first_reject"]) == 1
    to, do = w.target_offsets, w.draft_offsets
    for b in w.meta["all_accept"]:
        for i in range(w.k[b]):
            np.testing.assert_array_equal(w.draft[do[b] + i], w.target[to[b] + i])
    for b in w.meta["first_reject"]:
        assert w.uniforms[to[b]] >= 0.5


def test_padding_columns_are_poisoned():
    w = make_workload(B=2, k=[1, 2], V=37, ld=48, dtype="bf16", seed=(5,))
    assert np.all(w.target[:, 37:] == 0x42C8) and np.all(w.draft[:, 37:] == 0x42C8)
    assert w.target.shape == (5, 48)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_subset_repacks_requests(dtype):
    w = make_workload(B=4, k=[3, 1, 2, 4], V=50, dtype=dtype, seed=(6,))
    s = w.subset([2, 0])
    assert list(s.k) == [2, 3]
    np.testing.assert_array_equal(s.target[:3], w.target[6:9])
    np.testing.assert_array_equal(s.draft_tokens[:2], w.draft_tokens[4:6])
