"""sv_verify_block_noalloc (the library's fixed scratch in place of a caller workspace) against
sv_verify_block on the same inputs, two calls in a row, the second smaller.  Both go through
the C ABI; the outputs must agree bit for bit (the same kernels run), and the first call's
outputs are also held to the oracle."""

import numpy as np
import pytest

from synth import make_workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_util import compare, run_oracle, to_device  # noqa: E402


def _outputs(w, dev):
    n_d, B = w.n_draft_rows, w.B
    return {
        "accept_len": torch.full((B,), -7, dtype=torch.int32, device=dev),
        "out_tokens": torch.full((n_d + B,), -7, dtype=torch.int32, device=dev),
        "rkl": torch.full((n_d,), 7.0, dtype=torch.float32, device=dev),
        "p_at_draft": torch.full((n_d,), 7.0, dtype=torch.float32, device=dev),
        "q_at_draft": torch.full((n_d,), 7.0, dtype=torch.float32, device=dev),
        "device_status": torch.full((1,), -7, dtype=torch.int32, device=dev),
    }


def test_noalloc_matches_workspace_entry_point():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_block_verification_sv_amd as pkg

    big = make_workload(B=9, k=[1, 15, 3, 7, 2, 5, 1, 9, 15], V=70001, dtype="bf16", s=3.0,
                        sigma=[0.3, 0.8, 1.5, 0.5, 2.0, 1.0, 0.7, 1.2, 0.4],
                        temperature=[1.0, 0.0, 0.7, 1.3, 0.0, 0.5, 2.0, 1.0, 1.0], delta=0.5,
                        seed=(31,))
    small = make_workload(B=3, k=[2, 4, 1], V=5003, dtype="f32", temperature=[1.0, 0.7, 0.0],
                          seed=(32,))
    for i, w in enumerate((big, small)):
        print(f"[noalloc] call {i}: B={w.B} V={w.V} {w.dtype}", flush=True)
        d = to_device(w)
        ref = pkg.verify_block(d["target"], d["draft"], d["k"], d["draft_tokens"], d["uniforms"],
                               d["temperature"], w.delta, k_max=w.k_max)
        out = _outputs(w, torch.device("cuda:0"))
        pkg.verify_block_noalloc(d["target"], d["draft"], d["k"], d["draft_tokens"],
                                 d["uniforms"], d["temperature"], w.delta, out, k_max=w.k_max)
        torch.cuda.synchronize()
        for key in ("accept_len", "out_tokens", "rkl", "p_at_draft", "q_at_draft",
                    "device_status"):
            np.testing.assert_array_equal(out[key].cpu().numpy(), ref[key].cpu().numpy(), key)
        assert int(out["device_status"].item()) == 0
        got = {k_: v.cpu().numpy() for k_, v in out.items()}
        s = compare(w, got, run_oracle(w))
        assert s["exact"] + len(s["flips"]) == w.B


def test_noalloc_split_rows_in_one_launch():
    # Rows split into 16 parts that fold their waves (a single request of 16 rows, and 19
    # rows), finished by the part of each row that arrives last (arrival flags in the scratch).
    # The fixed scratch holds their records, so both entry points split alike and agree bit
    # for bit.
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_block_verification_sv_amd as pkg

    one = make_workload(B=1, k=[15], V=140001, dtype="bf16", s=4.0, sigma=[1.0], delta=1.0,
                        seed=(33,))
    two = make_workload(B=2, k=[9, 8], V=140001, dtype="bf16", s=3.0, sigma=[0.5, 1.5],
                        temperature=[1.0, 0.7], delta=0.05, seed=(34,))
    for i, w in enumerate((one, two, one)):
        print(f"[noalloc split] call {i}: B={w.B} V={w.V}", flush=True)
        d = to_device(w)
        ref = pkg.verify_block(d["target"], d["draft"], d["k"], d["draft_tokens"], d["uniforms"],
                               d["temperature"], w.delta, k_max=w.k_max)
        out = _outputs(w, torch.device("cuda:0"))
        pkg.verify_block_noalloc(d["target"], d["draft"], d["k"], d["draft_tokens"],
                                 d["uniforms"], d["temperature"], w.delta, out, k_max=w.k_max)
        torch.cuda.synchronize()
        for key in ("accept_len", "out_tokens", "rkl", "p_at_draft", "q_at_draft",
                    "device_status"):
            np.testing.assert_array_equal(out[key].cpu().numpy(), ref[key].cpu().numpy(), key)
        assert int(out["device_status"].item()) == 0
    got = {k_: v.cpu().numpy() for k_, v in out.items()}
    s = compare(one, got, run_oracle(one))
    assert s["exact"] + len(s["flips"]) == one.B
