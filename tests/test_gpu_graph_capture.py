"""Calls captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.  A captured launch keeps
the arguments it was captured with, among them the epoch its split rows' arrival flags carry;
the part that finishes a row clears them, so every replay starts from cleared flags.  Replays
back to back on new inputs copied into the captured buffers, with eager calls on the same
workspace (and the same fixed scratch) between rounds, must give the eager outputs for those
inputs bit for bit."""

import numpy as np
import pytest

from synth import make_workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_util import to_device  # noqa: E402

KEYS = ("accept_len", "out_tokens", "rkl", "p_at_draft", "q_at_draft", "device_status")
INPUTS = ("target", "draft", "k", "draft_tokens", "uniforms", "temperature")


def _outputs(w, dev):
    n_d, B = w.n_draft_rows, w.B
    return {
        "accept_len": torch.empty(B, dtype=torch.int32, device=dev),
        "out_tokens": torch.empty(n_d + B, dtype=torch.int32, device=dev),
        "rkl": torch.empty(n_d, dtype=torch.float32, device=dev),
        "p_at_draft": torch.empty(n_d, dtype=torch.float32, device=dev),
        "q_at_draft": torch.empty(n_d, dtype=torch.float32, device=dev),
        "device_status": torch.empty(1, dtype=torch.int32, device=dev),
    }


def _snapshot(out):
    return {k: out[k].cpu().numpy().copy() for k in KEYS}


@pytest.mark.parametrize("entry", ["workspace", "noalloc"])
def test_split_call_replays_in_a_graph(entry):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_block_verification_sv_amd as pkg

    dev = torch.device("cuda:0")
    # one request of 16 rows, each split into 16 parts finished in the streaming launch; two
    # input sets of that shape, and a third workload run eagerly between rounds
    wa = make_workload(B=1, k=[15], V=139264, dtype="bf16", s=4.0, sigma=[1.0], seed=(41,))
    wb = make_workload(B=1, k=[15], V=139264, dtype="bf16", s=3.0, sigma=[0.6], seed=(43,))
    w2 = make_workload(B=2, k=[9, 8], V=139264, dtype="bf16", s=3.0, sigma=[0.5, 1.5], seed=(42,))
    da, db, d2 = to_device(wa), to_device(wb), to_device(w2)
    ws = pkg.alloc_workspace(pkg.workspace_size(wa.B, wa.k_max, wa.V, pkg.SV_BF16), dev)
    ws2 = pkg.alloc_workspace(pkg.workspace_size(w2.B, w2.k_max, w2.V, pkg.SV_BF16), dev)

    def call(dd, ww, out, wsp):
        args = tuple(dd[key] for key in INPUTS) + (ww.delta,)
        if entry == "noalloc":
            pkg.verify_block_noalloc(*args, out, k_max=ww.k_max)
        else:
            pkg.verify_block(*args, k_max=ww.k_max, workspace=wsp, out=out)

    # eager references (outside any capture; the scratch's address is looked up here)
    refs = []
    for dd, ww in ((da, wa), (db, wb)):
        o = _outputs(ww, dev)
        call(dd, ww, o, ws)
        torch.cuda.synchronize()
        refs.append(_snapshot(o))
        assert int(refs[-1]["device_status"][0]) == 0
    assert not np.array_equal(refs[0]["rkl"], refs[1]["rkl"])

    # the captured call reads its inputs from these buffers
    buf = {key: da[key].clone() for key in INPUTS}
    out = _outputs(wa, dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(buf, wa, out, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(buf, wa, out, ws)
    torch.cuda.synchronize()

    out2 = _outputs(w2, dev)
    for r in range(2):
        # back-to-back replays on alternating inputs: each finds the flags the one before left,
        # under the same epoch
        for rr, which in enumerate((0, 1, 0, 1)):
            print(f"[graph] {entry}: round {r}, replay {rr}, inputs {which}", flush=True)
            src = da if which == 0 else db
            for key in INPUTS:
                buf[key].copy_(src[key])
            for key in KEYS:
                out[key].fill_(-7)
            g.replay()
            torch.cuda.synchronize()
            got = _snapshot(out)
            for key in KEYS:
                np.testing.assert_array_equal(got[key], refs[which][key], f"round {r} replay {rr}: {key}")
        # eager calls between rounds, on the same workspace or scratch
        call(d2, w2, out2, ws2 if entry == "workspace" else None)
        call(da, wa, _outputs(wa, dev), ws)
        torch.cuda.synchronize()
