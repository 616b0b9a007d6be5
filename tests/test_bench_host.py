"""Host logic of bench.py (no GPU): the parity summary it prints beside the oracle baseline."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import bench  # noqa: E402
import oracle  # noqa: E402
from synth import make_workload  # noqa: E402


def _case():
    w = make_workload(B=4, k=[3, 2, 4, 1], V=500, dtype="bf16", temperature=[1.0, 0.0, 0.7, 1.0],
                      seed=(1,))
    bench._W = w
    refs = [bench._oracle_request(b) for b in range(w.B)]
    full = oracle.verify_block(target=w.target, draft=w.draft, dtype=w.dtype, V=w.V, k=w.k,
                               draft_tokens=w.draft_tokens, uniforms=w.uniforms,
                               temperature=w.temperature, delta=w.delta)
    out = {"accept_len": torch.from_numpy(full["accept_len"].astype(np.int32)),
           "out_tokens": torch.from_numpy(full["out_tokens"].astype(np.int32)),
           "rkl": torch.from_numpy(full["rkl"].astype(np.float32)),
           "p_at_draft": torch.from_numpy(full["p_at_draft"].astype(np.float32))}
    return w, refs, out


def test_parity_sample_of_the_oracles_own_outputs():
    w, refs, out = _case()
    s = bench.parity_sample(w, out, refs)
    assert s["requests"] == 4 and s["exact"] == 4 and s["mismatches"] == 0
    assert s["max_rkl_err_over_bar"] < 0.1  # fp32 rounding of the stored values only


def test_parity_sample_counts_a_changed_decision():
    w, refs, out = _case()
    b = next(b for b, r in refs if r["accept_len"] < int(w.k[b]))  # a request with a rejection
    out["accept_len"][b] += 1
    s = bench.parity_sample(w, out, refs)
    assert s["exact"] == 3 and s["mismatches"] + s["boundary_flips"] == 1
    out["rkl"][0] += 1e-3
    assert bench.parity_sample(w, out, refs)["max_rkl_err_over_bar"] > 1.0
