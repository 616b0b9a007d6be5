"""GPU parity of sv_opd_loss (hard-label cross-entropy, clipped reverse-KL and the
mixture OPD loss of the AdaFlash paper, Section 3.1) against the CPU oracle.  Needs an
MI355X and the built library."""

import json
import math
import os

import numpy as np
import pytest

from synth import make_workload, workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from gpu_util import RKL_ABS, RTOL, to_device  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_block_verification_sv_amd as pkg

    pkg.lib()


def _pairing(w):
    # draft row of request b, position i -> target row off_t[b] + i (the verification layout)
    return np.concatenate([np.arange(w.target_offsets[b], w.target_offsets[b] + w.k[b])
                           for b in range(w.B)]).astype(np.int32)


def _check(w, got, delta, alpha, idx, rows=None, requests=None):
    tl = oracle.widen_logits(w.target[:, : w.V], w.dtype)
    dl = oracle.widen_logits(w.draft[:, : w.V], w.dtype)
    rows = range(w.n_draft_rows) if rows is None else rows
    hard = got["hard_ce"].cpu().numpy().astype(np.float64)
    rkl = got["rkl"].cpu().numpy().astype(np.float64)
    top1 = got["top1"].cpu().numpy()
    worst = 0.0
    tol_h, tol_r = {}, {}
    for r in rows:
        ref = oracle.clipped_rkl_row(tl[idx[r]], dl[r], delta)
        h, x = oracle.hard_ce_row(tl[idx[r]], dl[r])
        assert top1[r] == x, (r, top1[r], x)  # first argmax, exact
        tol_h[r] = RTOL * abs(h) + RKL_ABS
        assert abs(hard[r] - h) <= tol_h[r], (r, hard[r], h)
        tol_r[r] = RTOL * max(abs(ref["R"]), ref["L1"]) + RKL_ABS
        assert abs(rkl[r] - ref["R"]) <= tol_r[r], (r, rkl[r], ref["R"])
        worst = max(worst, abs(hard[r] - h) / max(abs(h), 1e-30))
    if got.get("opd") is not None:
        opd = got["opd"].cpu().numpy().astype(np.float64)
        off = np.concatenate([[0], np.cumsum(w.k)])
        for b in (range(w.B) if requests is None else requests):
            sl = slice(off[b], off[b + 1])
            ref = oracle.opd_loss(tl[idx[sl]], dl[sl], [w.k[b]], delta, alpha)
            # the mean of the rows' tolerances, plus the fp32 rounding of the output itself
            rr = range(off[b], off[b + 1])
            tol = (alpha * np.mean([tol_h[r] for r in rr]) +
                   (1 - alpha) * np.mean([tol_r[r] for r in rr]) + 2.0**-23 * abs(ref["opd"][0]))
            assert abs(opd[b] - ref["opd"][0]) <= tol, (b, opd[b], ref["opd"][0])
    return worst


def test_toy_position_through_the_kernel(golden_dir):
    import draft_block_verification_sv_amd as pkg

    with open(os.path.join(golden_dir, "adaflash_notes_toy_opd.json")) as f:
        toy = json.load(f)
    lp = torch.tensor(np.log(toy["p_target"]), dtype=torch.float32).cuda()[None, :]
    lq = torch.tensor(np.log(toy["q_draft"]), dtype=torch.float32).cuda()[None, :]
    k = torch.tensor([1], dtype=torch.int32).cuda()
    for delta in (1e30, 0.01):
        got = pkg.opd_loss(lp, lq, k, delta=delta, alpha=0.8)
        torch.cuda.synchronize()
        assert int(got["device_status"].item()) == 0
        ref = oracle.opd_loss(lp.cpu().double().numpy(), lq.cpu().double().numpy(), [1], delta, 0.8)
        assert int(got["top1"].item()) == 0
        assert float(got["hard_ce"].item()) == pytest.approx(ref["hard"][0], rel=1e-6)
        assert float(got["opd"].item()) == pytest.approx(ref["opd"][0], rel=1e-6, abs=1e-6)
    # the notes' printed OPD value (built from rounded parts) at delta = inf
    got = pkg.opd_loss(lp, lq, k, delta=1e30, alpha=toy["printed_opd_alpha"])
    assert abs(float(got["opd"].item()) - toy["printed_opd"]) <= 5e-4


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_batch_packed_pairing(dtype):
    import draft_block_verification_sv_amd as pkg

    w = make_workload(B=5, k=[1, 7, 3, 15, 2], V=5003, dtype=dtype, s=3.0,
                      sigma=[0.3, 1.0, 2.0, 0.7, 1.5], outlier_frac=0.05, seed=(21, dtype == "f32"))
    d = to_device(w)
    idx = _pairing(w)
    k = torch.from_numpy(w.k.astype(np.int32)).cuda()
    for delta, alpha in ((1.0, 0.8), (0.02, 0.5)):
        got = pkg.opd_loss(d["target"], d["draft"], k, delta=delta, alpha=alpha,
                           p_row_index=torch.from_numpy(idx).cuda())
        torch.cuda.synchronize()
        assert int(got["device_status"].item()) == 0
        worst = _check(w, got, delta, alpha, idx)
        print(f"[opd] {dtype} delta={delta}: max hard-CE rel err {worst:.2e}", flush=True)


def test_identity_pairing_padded_rows():
    import draft_block_verification_sv_amd as pkg

    w = make_workload(B=2, k=[4, 3], V=4093, ld=4100, dtype="f32", s=4.0, sigma=1.0, seed=(22,))
    d = to_device(w)
    # identity pairing: draft row r against target row r
    got = pkg.opd_loss(d["target"], d["draft"], torch.from_numpy(w.k).cuda(), delta=0.5,
                       alpha=0.8)
    torch.cuda.synchronize()
    assert int(got["device_status"].item()) == 0
    _check(w, got, 0.5, 0.8, np.arange(w.n_draft_rows))


def test_equal_rows_give_zero_rkl_and_target_top1():
    import draft_block_verification_sv_amd as pkg

    w = make_workload(B=1, k=[3], V=3000, dtype="bf16", all_accept=(0,), seed=(23,))
    d = to_device(w)
    idx = _pairing(w)
    got = pkg.opd_loss(d["target"], d["draft"], torch.from_numpy(w.k).cuda(), delta=1.0,
                       alpha=0.8, p_row_index=torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    assert np.all(got["rkl"].cpu().numpy() == 0.0)
    _check(w, got, 1.0, 0.8, idx)


def test_full_size_sampled():
    import draft_block_verification_sv_amd as pkg

    w = workload("high_concurrency")
    d = to_device(w)
    idx = _pairing(w)
    got = pkg.opd_loss(d["target"], d["draft"], torch.from_numpy(w.k).cuda(), delta=w.delta,
                       alpha=0.8, p_row_index=torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    assert int(got["device_status"].item()) == 0
    requests = [0, 63, 127]
    rows = [r for b in requests for r in range(int(w.draft_offsets[b]), int(w.draft_offsets[b + 1]))]
    _check(w, got, w.delta, 0.8, idx, rows=rows, requests=requests)
    # every row finite, every x* in range
    assert np.all(np.isfinite(got["hard_ce"].cpu().numpy()))
    t1 = got["top1"].cpu().numpy()
    assert np.all((t1 >= 0) & (t1 < w.V))
    # the fused verification path (whose heavy lanes are summed by the draw launch) meets the
    # same bar on the same rows
    from gpu_util import run_gpu

    ver = run_gpu(w, d)
    tl = oracle.widen_logits(w.target[:, : w.V], w.dtype)
    dl = oracle.widen_logits(w.draft[:, : w.V], w.dtype)
    for r in rows:
        ref = oracle.clipped_rkl_row(tl[idx[r]], dl[r], w.delta)
        tol = RTOL * max(abs(ref["R"]), ref["L1"]) + RKL_ABS
        assert abs(float(ver["rkl"][r]) - ref["R"]) <= tol, (r, ver["rkl"][r], ref["R"])


def test_bad_lengths_and_pairing_are_flagged():
    import draft_block_verification_sv_amd as pkg

    w = make_workload(B=3, k=[2, 2, 2], V=700, dtype="bf16", seed=(24,))
    d = to_device(w)
    idx = _pairing(w)
    bad_k = torch.tensor([2, 3, 2], dtype=torch.int32).cuda()  # sums to 7, rows are 6
    got = pkg.opd_loss(d["target"], d["draft"], bad_k, p_row_index=torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    assert int(got["device_status"].item()) & 2
    assert np.all(np.isnan(got["opd"].cpu().numpy()))
    zero_k = torch.tensor([2, 0, 4], dtype=torch.int32).cuda()
    got = pkg.opd_loss(d["target"], d["draft"], zero_k, p_row_index=torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    assert int(got["device_status"].item()) & 1
    idx2 = idx.copy()
    idx2[1] = w.n_target_rows
    got = pkg.opd_loss(d["target"], d["draft"], torch.from_numpy(w.k).cuda(),
                       p_row_index=torch.from_numpy(idx2).cuda())
    torch.cuda.synchronize()
    assert int(got["device_status"].item()) & 2
    h = got["hard_ce"].cpu().numpy()
    assert np.isnan(h[1]) and np.all(np.isfinite(np.delete(h, 1)))
    assert int(got["top1"].cpu().numpy()[1]) == -1


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_split_rows(dtype):
    # 10 rows of 60 slices: each row is streamed in parts and folded by the part that arrives last;
    # the hard-label cross-entropy needs the first argmax across parts
    import draft_block_verification_sv_amd as pkg

    w = make_workload(B=3, k=[4, 1, 5], V=61001, dtype=dtype, s=3.0, sigma=[0.4, 1.2, 2.0],
                      outlier_frac=0.05, seed=(25, dtype == "f32"))
    d = to_device(w)
    idx = _pairing(w)
    k = torch.from_numpy(w.k.astype(np.int32)).cuda()
    for delta, alpha in ((1.0, 0.8), (0.01, 0.5)):
        got = pkg.opd_loss(d["target"], d["draft"], k, delta=delta, alpha=alpha,
                           p_row_index=torch.from_numpy(idx).cuda())
        torch.cuda.synchronize()
        assert int(got["device_status"].item()) == 0
        worst = _check(w, got, delta, alpha, idx)
        print(f"[opd] split rows {dtype} delta={delta}: max hard-CE rel err {worst:.2e}", flush=True)


@pytest.mark.parametrize("dtype,k", [("bf16", [4, 1, 5]), ("f32", [4, 1, 5]), ("bf16", [9, 8, 7])])
def test_folded_split_rows(dtype, k):
    # 137 slices a row: split into 16 parts that fold their waves into 64 lanes (10 rows: 160
    # workgroups; 24 rows: 384), the part arriving last finishing each row.
    # Without a draw launch every heavy or clipped lane is summed again in the finalize, in
    # four blocks.
    import draft_block_verification_sv_amd as pkg

    w = make_workload(B=3, k=k, V=140001, dtype=dtype, s=3.0, sigma=[0.3, 1.2, 2.0],
                      outlier_frac=0.05, seed=(26, dtype == "f32", len(k)))
    d = to_device(w)
    idx = _pairing(w)
    kt = torch.from_numpy(w.k.astype(np.int32)).cuda()
    for delta, alpha in ((1.0, 0.8), (0.01, 0.5)):
        got = pkg.opd_loss(d["target"], d["draft"], kt, delta=delta, alpha=alpha,
                           p_row_index=torch.from_numpy(idx).cuda())
        torch.cuda.synchronize()
        assert int(got["device_status"].item()) == 0
        worst = _check(w, got, delta, alpha, idx)
        print(f"[opd] folded split rows {dtype} k={k} delta={delta}: max hard-CE rel err {worst:.2e}",
              flush=True)
