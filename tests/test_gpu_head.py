"""GPU parity of the adaptive length head (AdaFlash paper, Section 3.2) on the matrix cores,
its truncation and packing (Section 3.3) and its loss, against the CPU oracle.  Weights are
seeded random (no trained head is available).  Needs an MI355X and the built library."""

import numpy as np
import pytest

from synth import bf16_bits_from_f64, bf16_bits_to_f32, make_workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_block_verification_sv_amd as pkg

    pkg.lib()


def _bf16_tensor(x):
    bits = bf16_bits_from_f64(np.asarray(x, dtype=np.float64))
    t = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    return t, bf16_bits_to_f32(bits).astype(np.float64)


def _case(B, k, H, Hf, seed, bias=True, scale=1.0, ld_pad=0):
    rng = np.random.default_rng(seed)
    h_t, h = _bf16_tensor(rng.normal(size=(B, k, H + ld_pad)))
    W_t, W = _bf16_tensor(rng.normal(size=(Hf, H + ld_pad)) * scale / np.sqrt(H))
    h_t, h = h_t[:, :, :H], h[:, :, :H]
    W_t, W = W_t[:, :H], W[:, :H]
    b1 = (rng.normal(size=Hf) * 0.5).astype(np.float32) if bias else None
    w2 = (rng.normal(size=Hf) * 3.0 / np.sqrt(Hf)).astype(np.float32)
    b2 = float(rng.normal())
    return h_t, h, W_t, W, b1, w2, b2


def _tolerance(h, W, b1, w2):
    """Per request: a bound on |a_hat_gpu - a_hat| from fp32 accumulation of the K = H
    products (1e-5 of the sum of their magnitudes), the fp32 SiLU (2e-7 relative) and the
    pooled features' fp32 rounding, carried through the mean, the dot with w2 and the sigmoid."""
    z = np.einsum("bkh,nh->bkn", h, W) + (0.0 if b1 is None else b1)
    zabs = np.einsum("bkh,nh->bkn", np.abs(h), np.abs(W))
    sig = 1.0 / (1.0 + np.exp(-z))
    dsilu = np.abs(sig * (1.0 + z * (1.0 - sig)))
    silu = z * sig
    dz = 1e-5 * zabs + 1e-7
    dpool = (dsilu * dz + 2e-7 * np.abs(silu)).mean(axis=1) + 2**-24 * np.abs(silu.mean(axis=1))
    ddot = dpool @ np.abs(w2.astype(np.float64))
    return ddot, z


def _check(h_t, h, W_t, W, b1, w2, b2, k, gamma=1.0):
    import draft_block_verification_sv_amd as pkg

    out = pkg.length_head(h_t, W_t, torch.from_numpy(w2).cuda(),
                          None if b1 is None else torch.from_numpy(b1).cuda(), b2=b2, gamma=gamma)
    torch.cuda.synchronize()
    ref = oracle.length_head(h, W, b1, w2.astype(np.float64), b2)
    ddot, _ = _tolerance(h, W, b1, w2)
    tol = ref * (1 - ref) * ddot + 1e-7
    got = out["a_hat"].cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= tol), (got, ref, tol)
    kh = out["k_hat"].cpu().numpy()
    kref = oracle.truncate(ref, k, gamma)
    margin = oracle.truncation_margin(ref, k, gamma)
    sure = margin > tol * gamma * k  # the floor is a decision: compare where it is not marginal
    np.testing.assert_array_equal(kh[sure], kref[sure])
    assert np.all((kh >= 1) & (kh <= k))
    off = oracle.packed_offsets(kh)
    np.testing.assert_array_equal(out["off_t"].cpu().numpy(), off["off_t"])
    return out, ref, float(np.max(np.abs(got - ref)))


def test_head_at_the_drafter_shape():
    # B = 128 requests, k = 15 positions, H = 4096 (the Qwen3-8B hidden size), H' = 256
    h_t, h, W_t, W, b1, w2, b2 = _case(128, 15, 4096, 256, seed=51)
    _, ref, err = _check(h_t, h, W_t, W, b1, w2, b2, k=15, gamma=1.0)
    print(f"[head] B=128 k=15 H=4096 H'=256: max |a_hat err| {err:.2e}; "
          f"a_hat range {ref.min():.3f}..{ref.max():.3f}", flush=True)
    assert ref.min() < 0.3 and ref.max() > 0.7  # the weights spread the predictions


@pytest.mark.parametrize("B,k,H,Hf,bias,pad", [(3, 1, 32, 16, True, 0), (5, 16, 256, 100, False, 8),
                                               (4, 20, 512, 64, True, 16), (2, 64, 96, 300, True, 0)])
def test_head_odd_shapes(B, k, H, Hf, bias, pad):
    h_t, h, W_t, W, b1, w2, b2 = _case(B, k, H, Hf, seed=52 + B + k, bias=bias, ld_pad=pad)
    _check(h_t, h, W_t, W, b1, w2, b2, k=k, gamma=1.3)


def test_zero_hidden_states_reduce_to_the_bias_path():
    import draft_block_verification_sv_amd as pkg

    Hf = 64
    rng = np.random.default_rng(53)
    b1 = rng.normal(size=Hf).astype(np.float32)
    w2 = rng.normal(size=Hf).astype(np.float32)
    h_t = torch.zeros(4, 8, 128, dtype=torch.bfloat16).cuda()
    W_t, _ = _bf16_tensor(rng.normal(size=(Hf, 128)))
    out = pkg.length_head(h_t, W_t, torch.from_numpy(w2).cuda(), torch.from_numpy(b1).cuda(), b2=0.1)
    torch.cuda.synchronize()
    b1d = b1.astype(np.float64)
    ref = 1.0 / (1.0 + np.exp(-(w2.astype(np.float64) @ (b1d / (1.0 + np.exp(-b1d))) + 0.1)))
    np.testing.assert_allclose(out["a_hat"].cpu().numpy(), ref, rtol=2e-6)


def test_length_loss_and_the_loop_through_verification():
    import draft_block_verification_sv_amd as pkg
    from gpu_util import run_gpu, to_device

    h_t, h, W_t, W, b1, w2, b2 = _case(6, 15, 512, 64, seed=54)
    out = pkg.length_head(h_t, W_t, torch.from_numpy(w2).cuda(), torch.from_numpy(b1).cuda(), b2=b2)
    torch.cuda.synchronize()
    kh = out["k_hat"].cpu().numpy()
    # pack a verification batch with the predicted lengths and verify it
    w = make_workload(B=6, k=kh, V=3000, dtype="bf16", sigma=0.8, seed=(55,), k_max=15)
    np.testing.assert_array_equal(out["off_t"].cpu().numpy(), w.target_offsets)
    got = run_gpu(w, to_device(w))
    al = torch.from_numpy(got["accept_len"].astype(np.int32)).cuda()
    loss, dloss = pkg.length_loss(out["a_hat"], al, out["k_hat"])
    torch.cuda.synchronize()
    ref = oracle.length_loss(out["a_hat"].cpu().numpy(), got["accept_len"], kh)
    np.testing.assert_allclose(loss.cpu().numpy(), ref, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(dloss.cpu().numpy(),
                               2 * (out["a_hat"].cpu().numpy() - got["accept_len"] / kh), rtol=1e-6,
                               atol=1e-7)
    bad = torch.tensor([-1, 3], dtype=torch.int32).cuda()
    loss, _ = pkg.length_loss(out["a_hat"][:2].contiguous(), bad,
                              torch.tensor([4, 2], dtype=torch.int32).cuda())
    torch.cuda.synchronize()
    assert np.all(np.isnan(loss.cpu().numpy()))  # invalid request; accepted more than verified
