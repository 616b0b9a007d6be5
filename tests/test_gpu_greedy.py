"""GPU parity of sv_verify_block_greedy (every request greedy: accept iff the draft equals the
target argmax; DFlash notes, Section 5.2, worked example #4) against the CPU oracle and against
sv_verify_block with T_b = 0.  Needs an MI355X and the built library."""

import json
import os

import numpy as np
import pytest

from synth import bf16_bits_from_f64, make_workload, workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_util import run_gpu, run_oracle, to_device  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_block_verification_sv_amd as pkg

    pkg.lib()


def _greedy(w, d=None, **kw):
    import draft_block_verification_sv_amd as pkg

    d = to_device(w) if d is None else d
    out = pkg.verify_block_greedy(d["target"], d["k"], d["draft_tokens"], k_max=w.k_max, **kw)
    torch.cuda.synchronize()
    return {k_: v.cpu().numpy() for k_, v in out.items()}


def _exact(w, got, ref, requests=None):
    to = w.target_offsets
    for b in (range(w.B) if requests is None else requests):
        assert int(got["accept_len"][b]) == int(ref["accept_len"][b]), b
        sl = slice(int(to[b]), int(to[b + 1]))
        np.testing.assert_array_equal(got["out_tokens"][sl].astype(np.int64), ref["out_tokens"][sl])


@pytest.mark.parametrize("dtype,V,ld", [("bf16", 5003, None), ("f32", 4093, 4100), ("bf16", 7, None)])
def test_ragged_greedy_batch_matches_oracle(dtype, V, ld):
    w = make_workload(B=6, k=[1, 9, 4, 15, 2, 6], V=V, ld=ld, dtype=dtype, s=3.0,
                      sigma=[0.1, 0.3, 0.5, 0.2, 1.0, 0.05], temperature=0.0, seed=(41, V))
    got = _greedy(w)
    assert int(got["device_status"][0]) == 0
    _exact(w, got, run_oracle(w, with_rkl=False))


def test_golden_greedy_trace(golden_dir):
    with open(os.path.join(golden_dir, "dflash_notes_greedy_trace.json")) as f:
        g = json.load(f)
    w = make_workload(B=1, k=[g["block_drafts"]], V=3001, dtype="bf16", temperature=0.0,
                      seed=(6,))
    tgt = w.rows_f32("target", slice(0, 16)).astype(np.float64)
    argmax_p = np.argmax(tgt, axis=1)
    x = argmax_p[:15].copy()
    for i, match in enumerate(g["match_pattern_prefix"]):
        if not match:
            x[i] = (argmax_p[i] + 1) % w.V
    w.draft_tokens[:] = x
    got = _greedy(w)
    assert got["accept_len"][0] == g["expected_accept_len"]
    assert int(np.count_nonzero(got["out_tokens"] >= 0)) == g["expected_tokens_emitted"]
    assert got["out_tokens"][g["expected_accept_len"]] == argmax_p[g["expected_accept_len"]]


def test_ties_go_to_the_lowest_id():
    w = make_workload(B=1, k=[2], V=4096, dtype="bf16", temperature=0.0, seed=(42,))
    row = np.full(w.V, -5.0)
    row[[3000, 700, 2500]] = 7.0  # three equal maxima in different slices and lanes
    for r in range(3):
        w.target[r, : w.V] = bf16_bits_from_f64(row)
    w.draft_tokens[:] = [700, 3000]
    got = _greedy(w)
    assert list(got["accept_len"]) == [1]
    assert list(got["out_tokens"]) == [700, 700, -1]


def test_full_size_equals_verify_with_zero_temperature():
    w = workload("high_concurrency")
    w.temperature[:] = 0.0
    d = to_device(w)
    got = _greedy(w, d)
    assert int(got["device_status"][0]) == 0
    ver = run_gpu(w, d)  # the general path with T_b = 0
    np.testing.assert_array_equal(got["accept_len"], ver["accept_len"])
    np.testing.assert_array_equal(got["out_tokens"], ver["out_tokens"])
    sample = [0, 5, 64, 127]
    _exact(w, got, run_oracle(w, requests=sample, with_rkl=False), requests=sample)


def test_large_batch_uses_the_plan():
    # more than 2048 requests: descriptors come from the plan kernel
    B = 2100
    w = make_workload(B=B, k=np.where(np.arange(B) % 3 == 0, 2, 1), V=300, dtype="bf16",
                      sigma=0.2, temperature=0.0, seed=(43,))
    got = _greedy(w)
    assert int(got["device_status"][0]) == 0
    _exact(w, got, run_oracle(w, with_rkl=False))


def test_bad_token_and_void_calls():
    w = make_workload(B=3, k=[2, 3, 1], V=500, dtype="f32", temperature=0.0, seed=(44,))
    w.draft_tokens[3] = 999  # request 1
    got = _greedy(w)
    assert int(got["device_status"][0]) & 4
    assert got["accept_len"][1] == -1 and got["accept_len"][0] >= 0 and got["accept_len"][2] >= 0
    d = to_device(w)
    d["k"] = torch.tensor([2, 0, 4], dtype=torch.int32).cuda()
    got = _greedy(w, d)
    assert int(got["device_status"][0]) & 1
    assert np.all(got["accept_len"] == -1) and np.all(got["out_tokens"] == -1)


def test_maximum_draft_length():
    # k_b = k_max = 64: the bonus row of an all-accepted request is row 64
    w = make_workload(B=3, k=[64, 64, 3], V=2001, dtype="bf16", temperature=0.0, all_accept=(0,),
                      k_max=64, seed=(45,))
    got = _greedy(w)
    assert int(got["device_status"][0]) == 0 and int(got["accept_len"][0]) == 64
    _exact(w, got, run_oracle(w, with_rkl=False))
