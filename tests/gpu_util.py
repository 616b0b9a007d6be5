"""Helpers for the GPU parity tests: upload a workload, run the library through its
C ABI (via the binding), and compare with the oracle.

Comparison rules (fp32 GPU against the float64 oracle):
* accept lengths and emitted tokens are compared decision by decision in request
  order.  The first decision where the two differ must be one whose oracle margin
  (|u - min(1, ratio)| for an acceptance, distance of u*Z to the chosen id's CDF
  edges over Z for a draw) is at most 1e-5: that is a boundary flip, counted and
  reported, and the rest of that request is not compared.  Greedy decisions have
  infinite margin and must always match.
* p_T(x_i), q_T(x_i): |got - ref| <= 1e-5 |ref|.
* clipped reverse-KL: |got - ref| <= 1e-5 max(|ref|, sum_y |min(delta, t_y)|) + 1e-12.
  The relative bar is the one the verification path is built to (fp32 accumulation,
  lanes that hold most of a row's mass summed again in fp64).  The absolute floor covers
  only the fp64 rounding of the finalize, which forms R from per-lane terms of up to
  ~100 (log2 units times mass) that cancel: ~1e-14.  It matters only where the scale is
  0 or nearly so (q equal to p up to a constant, V = 1).
"""

from __future__ import annotations

import numpy as np
import torch

import oracle

MARGIN = 1e-5
RTOL = 1e-5
RKL_ABS = 1e-12


def to_device(w, dev="cuda:0"):
    def logits(a):
        if w.dtype == "bf16":
            t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        return t[:, : w.V]  # row stride stays ld

    return dict(
        target=logits(w.target),
        draft=logits(w.draft),
        k=torch.from_numpy(w.k.astype(np.int32)).to(dev),
        draft_tokens=torch.from_numpy(w.draft_tokens.astype(np.int32)).to(dev),
        uniforms=torch.from_numpy(w.uniforms.astype(np.float32)).to(dev),
        temperature=torch.from_numpy(w.temperature.astype(np.float32)).to(dev),
    )


def run_gpu(w, dev_inputs=None, *, with_rkl=True, delta=None, k_max=None, **kw):
    import draft_block_verification_sv_amd as pkg

    d = dev_inputs if dev_inputs is not None else to_device(w)
    out = pkg.verify_block(d["target"], d["draft"], d["k"], d["draft_tokens"], d["uniforms"],
                           d["temperature"], w.delta if delta is None else delta,
                           k_max=w.k_max if k_max is None else k_max, with_rkl=with_rkl, **kw)
    torch.cuda.synchronize()
    return {k_: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for k_, v in out.items()}


def run_oracle(w, requests=None, delta=None, with_rkl=True):
    return oracle.verify_block(target=w.target, draft=w.draft, dtype=w.dtype, V=w.V, k=w.k,
                               draft_tokens=w.draft_tokens, uniforms=w.uniforms,
                               temperature=w.temperature,
                               delta=w.delta if delta is None else delta, requests=requests,
                               with_rkl=with_rkl)


def compare(w, got, ref, requests=None, check_rkl=True):
    """Asserts parity on the given requests; returns a summary dict."""
    reqs = range(w.B) if requests is None else requests
    to, do = w.target_offsets, w.draft_offsets
    flips, exact = [], 0
    max_p_rel = max_rkl_rel = 0.0
    for b in reqs:
        kb = int(w.k[b])
        t0, d0 = int(to[b]), int(do[b])
        ga, ra = int(got["accept_len"][b]), int(ref["accept_len"][b])
        gt = got["out_tokens"][t0: t0 + kb + 1].astype(np.int64)
        rt = ref["out_tokens"][t0: t0 + kb + 1]
        if ga == ra and np.array_equal(gt, rt):
            exact += 1
        else:
            if ga != ra:
                pos = min(ga, ra)
                margin = ref["accept_margin"][d0 + pos]
                what = f"acceptance at position {pos}"
            else:
                margin = ref["token_margin"][b]
                what = "final token"
            assert margin <= MARGIN, (
                f"request {b}: {what} differs (gpu a={ga} tokens={gt.tolist()}, oracle a={ra} "
                f"tokens={rt.tolist()}) with oracle margin {margin:.3g} > {MARGIN}")
            flips.append((b, what, float(margin)))
        if ra >= 0:
            # structure of the GPU output: a accepted drafts, one final token, then -1
            assert 0 <= ga <= kb
            np.testing.assert_array_equal(gt[:ga], w.draft_tokens[d0: d0 + ga])
            assert 0 <= gt[ga] < w.V
            assert np.all(gt[ga + 1:] == -1)
        sl = slice(d0, d0 + kb)
        if ref["accept_len"][b] >= 0 and got.get("p_at_draft") is not None:
            for name in ("p_at_draft", "q_at_draft"):
                r = ref[name][sl]
                g = got[name][sl].astype(np.float64)
                err = np.abs(g - r)
                assert np.all(err <= RTOL * np.abs(r) + 1e-37), (b, name, g, r)
                max_p_rel = max(max_p_rel, float(np.max(err / np.maximum(np.abs(r), 1e-300))))
        if check_rkl and got.get("rkl") is not None:
            r = ref["rkl"][sl]
            g = got["rkl"][sl].astype(np.float64)
            scale = np.maximum(np.abs(r), ref["rkl_l1"][sl])
            err = np.abs(g - r)
            assert np.all(err <= RTOL * scale + RKL_ABS), (b, g, r, err / scale)
            max_rkl_rel = max(max_rkl_rel, float(np.max(err / np.maximum(scale, 1e-30))))
    return dict(exact=exact, flips=flips, max_p_rel=max_p_rel, max_rkl_rel=max_rkl_rel)
