"""Statistical checks of the HIP path itself (MI355X): the closed form of the expected
number of tokens per round (AdaFlash paper, Section 2.1) and losslessness (the emitted
token follows the target distribution; paper Section 2.1, DFlash notes Section 5.2),
both with large sample counts that only the GPU makes cheap."""

import math

import numpy as np
import pytest
from scipy.special import softmax
from scipy.stats import chisquare

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _uniforms(rng, n):
    return ((rng.integers(0, 2**32, size=n, dtype=np.uint64) >> 8).astype(np.float64)
            * 2.0**-24).astype(np.float32)


def _run(lp_rows, lq_rows, k, B, T, rng):
    """B requests of k drafts; request b uses target rows lp_rows[0..k], draft rows
    lq_rows[0..k-1]; x_i ~ q_T(row i) independently; fresh uniforms."""
    import draft_block_verification_sv_amd as pkg

    V = lp_rows.shape[1]
    dev = "cuda"
    tgt = torch.from_numpy(np.ascontiguousarray(lp_rows, dtype=np.float32)).to(dev)
    drf = torch.from_numpy(np.ascontiguousarray(lq_rows, dtype=np.float32)).to(dev)
    target = tgt.unsqueeze(0).expand(B, k + 1, V).reshape(B * (k + 1), V).contiguous()
    draft = drf.unsqueeze(0).expand(B, k, V).reshape(B * k, V).contiguous()
    qs = [softmax(lq_rows[i].astype(np.float64) / T) for i in range(k)]
    x = np.stack([rng.choice(V, size=B, p=qs[i]) for i in range(k)], axis=1).astype(np.int32)
    u = _uniforms(rng, B * (k + 1))
    out = pkg.verify_block(target, draft, torch.full((B,), k, dtype=torch.int32, device=dev),
                           torch.from_numpy(x.reshape(-1)).to(dev), torch.from_numpy(u).to(dev),
                           torch.full((B,), T, dtype=torch.float32, device=dev), 1.0, k_max=k,
                           with_rkl=False, with_probs=False)
    torch.cuda.synchronize()
    assert int(out["device_status"].item()) == 0
    return out["accept_len"].cpu().numpy(), out["out_tokens"].cpu().numpy().reshape(B, k + 1)


@pytest.mark.parametrize("k,T", [(4, 1.0), (15, 1.0), (6, 0.7)])
def test_expected_tau_closed_form_through_kernel(k, T):
    rng = np.random.default_rng(100 + k)
    V, B = 1000, 16384
    lp = (2.0 * rng.standard_normal(V)).astype(np.float32)
    lq = (lp + rng.standard_normal(V)).astype(np.float32)
    acc = float(np.minimum(softmax(lp.astype(np.float64) / T),
                           softmax(lq.astype(np.float64) / T)).sum())
    a, _ = _run(np.repeat(lp[None], k + 1, 0), np.repeat(lq[None], k, 0), k, B, T, rng)
    e_tau = (1 - acc ** (k + 1)) / (1 - acc)
    law = np.array([acc**j * (1 - acc) for j in range(k)] + [acc**k])
    var = float(np.sum(law * (np.arange(k + 1) + 1) ** 2)) - e_tau**2
    z = (np.mean(a + 1) - e_tau) / math.sqrt(var / B)
    hist = np.bincount(a, minlength=k + 1)
    keep = law * B >= 5
    obs = np.append(hist[keep], hist[~keep].sum())
    exp = np.append(law[keep] * B, law[~keep].sum() * B)
    if exp[-1] == 0:
        obs, exp = obs[:-1], exp[:-1]
    pval = chisquare(obs, exp).pvalue
    print(f"[stats] k={k} T={T}: Acc={acc:.4f} E[tau]={e_tau:.4f} mean={np.mean(a + 1):.4f} "
          f"z={z:.2f} chi2 p={pval:.3g}", flush=True)
    assert abs(z) < 4.0
    assert pval > 1e-4


@pytest.mark.parametrize("V,T", [(16, 1.0), (16, 0.7), (8, 1.0)])
def test_lossless_through_kernel(V, T):
    rng = np.random.default_rng(200 + V)
    k, B, calls = 3, 65536, 4
    lp = (1.5 * rng.standard_normal((k + 1, V))).astype(np.float32)
    lq = (lp[:k] + 1.2 * rng.standard_normal((k, V))).astype(np.float32)
    counts = np.zeros((k + 1, V))
    for _ in range(calls):
        a, toks = _run(lp, lq, k, B, T, rng)
        for j in range(k + 1):
            reached = a >= j
            counts[j] += np.bincount(toks[reached, j], minlength=V)
    pvals = []
    for j in range(k + 1):
        n = counts[j].sum()
        if n < 1000:
            continue
        p = softmax(lp[j].astype(np.float64) / T)
        pvals.append(chisquare(counts[j], p * n).pvalue)
    print(f"[stats] lossless V={V} T={T}: slot p-values {[f'{x:.3g}' for x in pvals]}", flush=True)
    assert len(pvals) >= 3
    assert min(pvals) > 1e-4 / len(pvals)
