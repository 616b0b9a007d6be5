"""GPU parity of sv_opd_loss_grad (gradient of the mixture OPD loss of the AdaFlash paper,
Section 3.1, with respect to the drafter logits) against the CPU oracle.  Needs an MI355X
and the built library."""

import math

import numpy as np
import pytest

from synth import make_workload, workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from gpu_util import to_device  # noqa: E402

RTOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_block_verification_sv_amd as pkg

    pkg.lib()


def _pairing(w):
    return np.concatenate([np.arange(w.target_offsets[b], w.target_offsets[b] + w.k[b])
                           for b in range(w.B)]).astype(np.int32)


def _grad_tolerance(lp, lq, delta, ch, cr, x):
    """Per element: 1e-5 of the magnitude of each part of the gradient.  Rows with an entry
    whose term sits within 1e-5 of the clip are reported (the clip indicator is a decision)."""
    log_p = lp - (lp.max() + np.log(np.sum(np.exp(lp - lp.max()))))
    log_q = lq - (lq.max() + np.log(np.sum(np.exp(lq - lq.max()))))
    q = np.exp(log_q)
    L = log_q - log_p
    t = q * L
    near = np.abs(t - delta) <= 1e-5 * max(delta, 1e-30)
    g = np.where(t < delta, L + 1.0, 0.0)
    sg = float(np.sum(q * g))
    onehot = np.zeros_like(q)
    onehot[x] = 1.0
    tol = RTOL * (ch * (q + onehot) + cr * q * (np.abs(L) + 1.0 + abs(sg))) + 1e-30
    return tol, bool(near.any())


def _compare(w, got, delta, alpha, idx, rows, bf16_out=False):
    tl = oracle.widen_logits(w.target[:, : w.V], w.dtype)
    dl = oracle.widen_logits(w.draft[:, : w.V], w.dtype)
    k = np.asarray(w.k)
    req = np.repeat(np.arange(w.B), k)
    G = got["grad"].float().cpu().numpy().astype(np.float64)
    worst = 0.0
    for r in rows:
        b = req[r]
        off = int(w.draft_offsets[b])
        ref = oracle.opd_grad(tl[idx[off: off + k[b]]], dl[off: off + k[b]], [k[b]], delta,
                              alpha)[r - off]
        _, x = oracle.hard_ce_row(tl[idx[r]], dl[r])
        tol, near = _grad_tolerance(tl[idx[r]], dl[r], delta, alpha / k[b], (1 - alpha) / k[b], x)
        assert not near, f"row {r}: an entry sits on the clip; choose another delta"
        if bf16_out:
            tol = tol + 2.0**-8 * np.abs(ref)  # round to nearest bf16: half an 8-bit ulp
        err = np.abs(G[r] - ref)
        bad = np.flatnonzero(err > tol)
        assert bad.size == 0, (r, bad[:5], G[r][bad[:5]], ref[bad[:5]])
        worst = max(worst, float(np.max(err / np.maximum(np.abs(ref), 1e-30))))
    return worst


def test_tiny_vocabulary_full_gradient():
    import draft_block_verification_sv_amd as pkg

    w = make_workload(B=2, k=[2, 3], V=16, dtype="f32", s=2.0, sigma=1.0, seed=(31,))
    d = to_device(w)
    idx = _pairing(w)
    for delta, alpha in ((0.05, 0.8), (1e30, 0.3)):
        got = pkg.opd_loss_grad(d["target"], d["draft"], torch.from_numpy(w.k).cuda(),
                                delta=delta, alpha=alpha, p_row_index=torch.from_numpy(idx).cuda())
        torch.cuda.synchronize()
        assert int(got["device_status"].item()) == 0
        _compare(w, got, delta, alpha, idx, range(w.n_draft_rows))


@pytest.mark.parametrize("dtype,gdt", [("bf16", "f32"), ("bf16", "bf16"), ("f32", "f32")])
def test_ragged_batch(dtype, gdt):
    import draft_block_verification_sv_amd as pkg

    w = make_workload(B=4, k=[1, 6, 3, 9], V=5003, dtype=dtype, s=3.0, sigma=[0.3, 1.0, 2.0, 0.7],
                      outlier_frac=0.05, seed=(32, dtype == "f32"))
    d = to_device(w)
    idx = _pairing(w)
    g_dtype = torch.bfloat16 if gdt == "bf16" else torch.float32
    got = pkg.opd_loss_grad(d["target"], d["draft"], torch.from_numpy(w.k).cuda(), delta=0.3,
                            alpha=0.8, p_row_index=torch.from_numpy(idx).cuda(), grad_dtype=g_dtype)
    torch.cuda.synchronize()
    assert int(got["device_status"].item()) == 0
    worst = _compare(w, got, 0.3, 0.8, idx, range(w.n_draft_rows), bf16_out=(gdt == "bf16"))
    print(f"[grad] {dtype}->{gdt}: max rel err {worst:.2e}", flush=True)
    # the forward outputs are those of sv_opd_loss, bit for bit
    fwd = pkg.opd_loss(d["target"], d["draft"], torch.from_numpy(w.k).cuda(), delta=0.3,
                       alpha=0.8, p_row_index=torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    for key in ("rkl", "hard_ce", "top1", "opd"):
        np.testing.assert_array_equal(got[key].cpu().numpy(), fwd[key].cpu().numpy())


def test_full_size_sampled_rows_and_invariants():
    import draft_block_verification_sv_amd as pkg

    w = workload("high_concurrency")
    d = to_device(w)
    idx = _pairing(w)
    got = pkg.opd_loss_grad(d["target"], d["draft"], torch.from_numpy(w.k).cuda(), delta=w.delta,
                            alpha=0.8, p_row_index=torch.from_numpy(idx).cuda(),
                            grad_dtype=torch.float32)
    torch.cuda.synchronize()
    assert int(got["device_status"].item()) == 0
    rows = [0, 7, 14, 15 * 64, 15 * 64 + 9, 15 * 127 + 14]
    _compare(w, got, w.delta, 0.8, idx, rows)
    # every row: finite, and it sums to zero (the loss does not change when a logit row shifts)
    G = got["grad"]
    assert bool(torch.isfinite(G).all())
    s = G.double().sum(dim=1).abs().max().item()
    assert s < 1e-6, s


def test_void_lengths_and_bad_pairing_give_nan():
    import draft_block_verification_sv_amd as pkg

    w = make_workload(B=2, k=[2, 3], V=900, dtype="bf16", seed=(33,))
    d = to_device(w)
    idx = _pairing(w)
    bad_k = torch.tensor([2, 2], dtype=torch.int32).cuda()  # 4 != 5 rows
    got = pkg.opd_loss_grad(d["target"], d["draft"], bad_k, p_row_index=torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    assert int(got["device_status"].item()) & 2
    assert bool(torch.isnan(got["grad"].float()).all())
    idx2 = idx.copy()
    idx2[3] = -1
    got = pkg.opd_loss_grad(d["target"], d["draft"], torch.from_numpy(w.k).cuda(),
                            p_row_index=torch.from_numpy(idx2).cuda(), grad_dtype=torch.float32)
    torch.cuda.synchronize()
    assert int(got["device_status"].item()) & 2
    G = got["grad"].cpu().numpy()
    assert np.all(np.isnan(G[3])) and np.all(np.isfinite(np.delete(G, 3, axis=0)))


@pytest.mark.parametrize("dtype,ld", [("bf16", 40000), ("f32", 40003)])
def test_many_clipped_lanes(dtype, ld):
    # a small delta fails the no-clip bound on most lanes, so the row statistic of the gradient
    # comes from the entry-by-entry re-read, over several rounds of pieces; the split-row path
    # (9 rows of 40 slices) is taken as well
    import draft_block_verification_sv_amd as pkg

    w = make_workload(B=3, k=[2, 4, 3], V=40000, ld=ld, dtype=dtype, s=3.0, sigma=[0.5, 1.5, 1.0],
                      outlier_frac=0.05, seed=(34, ld))
    d = to_device(w)
    idx = _pairing(w)
    got = pkg.opd_loss_grad(d["target"], d["draft"], torch.from_numpy(w.k).cuda(), delta=0.004,
                            alpha=0.8, p_row_index=torch.from_numpy(idx).cuda(),
                            grad_dtype=torch.float32)
    torch.cuda.synchronize()
    assert int(got["device_status"].item()) == 0
    worst = _compare(w, got, 0.004, 0.8, idx, range(w.n_draft_rows))
    print(f"[grad] many clipped lanes {dtype} ld={ld}: max rel err {worst:.2e}", flush=True)


def test_many_clipped_folded_lanes():
    # rows of 137 slices split into 16 parts folded into 64 lanes (9 rows: finished by the last
    # part in the streaming launch); the small delta fails the bound on most folded lanes, whose
    # columns are then re-read in four blocks, one per wave
    import draft_block_verification_sv_amd as pkg

    w = make_workload(B=3, k=[2, 4, 3], V=140001, dtype="bf16", s=3.0, sigma=[0.5, 1.5, 1.0],
                      outlier_frac=0.05, seed=(35,))
    d = to_device(w)
    idx = _pairing(w)
    got = pkg.opd_loss_grad(d["target"], d["draft"], torch.from_numpy(w.k).cuda(), delta=0.004,
                            alpha=0.8, p_row_index=torch.from_numpy(idx).cuda(),
                            grad_dtype=torch.float32)
    torch.cuda.synchronize()
    assert int(got["device_status"].item()) == 0
    worst = _compare(w, got, 0.004, 0.8, idx, range(w.n_draft_rows))
    print(f"[grad] many clipped folded lanes: max rel err {worst:.2e}", flush=True)
