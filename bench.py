#!/usr/bin/env python3
"""Throughput of batched draft-block verification with the fused clipped reverse-KL.

One step = one sv_verify_block call over one packed batch resident in HBM: the
streaming pass over every target and draft logit row, the per-row finalize (rKL,
acceptance test), the first-rejection scan and the residual / bonus draw.

Workload (default): B=128 requests, k=15 drafts each (16-position blocks),
V=151936, bf16 logits, drafter noise sigma_b in {0.5, 1, 2}, delta=1, seeded
synthetic inputs (see synth/workloads.py).  Prints one JSON line on stdout;
progress goes to stderr.

  python bench.py [--steps K] [--warmup W] [--workload high_concurrency] [--no-cpu-baseline]

With --op opd the step is instead one sv_opd_loss call (hard-label cross-entropy, clipped
reverse-KL and the per-request OPD loss) over the same workload's draft rows, each paired
with the target row that scores it.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "verified draft positions/sec and achieved HBM GB/s (% of peak), B=128 k=15 V=151936"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "sv_rowpair_b128_k15_v151936_counters.json")
STREAM_KERNEL = "sv_rowpair"  # the kernel that streams the logits: the roofline kernel
# the sources the streaming kernel is compiled from (its counters are void once they change)
KERNEL_SOURCES = [os.path.join(ROOT, "draft_block_verification_sv_amd", "csrc", f)
                  for f in ("sv_rowpair.hip", "sv_kernels.hip", "sv_device.h", "sv_lanes.h", "sv_layout.h", "sv_launch.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


_W = None  # the workload, inherited by the forked cpu_baseline workers


def _oracle_request(b):
    # cpu_baseline worker: the oracle, unchanged, on one request; returns that request's outputs
    import oracle

    w = _W
    r = oracle.verify_block(target=w.target, draft=w.draft, dtype=w.dtype, V=w.V, k=w.k,
                            draft_tokens=w.draft_tokens, uniforms=w.uniforms,
                            temperature=w.temperature, delta=w.delta, requests=[b])
    ot, od, kb = int(w.target_offsets[b]), int(w.draft_offsets[b]), int(w.k[b])
    sl = slice(od, od + kb)
    return b, {"accept_len": int(r["accept_len"][b]), "tokens": r["out_tokens"][ot: ot + kb + 1],
               "rkl": r["rkl"][sl], "rkl_l1": r["rkl_l1"][sl], "p_at": r["p_at_draft"][sl],
               "accept_margin": r["accept_margin"][sl], "token_margin": float(r["token_margin"][b])}


def parity_sample(w, out, refs) -> dict:
    """The GPU outputs of the timed call against the oracle's on the baseline's requests:
    accept lengths and tokens exact, or a boundary flip when the first differing decision had
    an oracle margin <= 1e-5; the clipped rKL's error relative to max(|R|, sum |min(delta, t)|)
    and as a fraction of the parity bar (<= 1 passes); p_T(x_i)'s relative error."""
    import numpy as np

    al = out["accept_len"].cpu().numpy()
    ot = out["out_tokens"].cpu().numpy()
    rkl = out["rkl"].cpu().numpy().astype(np.float64)
    pat = out["p_at_draft"].cpu().numpy().astype(np.float64)
    exact = flips = wrong = 0
    max_rkl = max_bar = max_p = 0.0
    for b, r in refs:
        o_t, o_d, kb = int(w.target_offsets[b]), int(w.draft_offsets[b]), int(w.k[b])
        if int(al[b]) == r["accept_len"] and np.array_equal(ot[o_t: o_t + kb + 1], r["tokens"]):
            exact += 1
        else:
            n = min(int(al[b]), r["accept_len"])  # the first position the two decided apart
            margin = (r["accept_margin"][n] if int(al[b]) != r["accept_len"] and 0 <= n < kb
                      else r["token_margin"])
            if margin <= 1e-5:
                flips += 1
            else:
                wrong += 1
        g = rkl[o_d: o_d + kb]
        scale = np.maximum(np.abs(r["rkl"]), r["rkl_l1"])
        max_rkl = max(max_rkl, float(np.max(np.abs(g - r["rkl"]) / scale)))
        # against the parity bar: 1e-5 of the scale plus the fp64 rounding floor of the finalize
        max_bar = max(max_bar, float(np.max(np.abs(g - r["rkl"]) / (1e-5 * scale + 1e-12))))
        ok = np.isfinite(r["p_at"]) & (r["p_at"] > 0)
        if np.any(ok):
            max_p = max(max_p, float(np.max(np.abs(pat[o_d: o_d + kb][ok] - r["p_at"][ok]) / r["p_at"][ok])))
    return {"requests": len(refs), "exact": exact, "boundary_flips": flips, "mismatches": wrong,
            "max_rkl_rel": max_rkl, "max_rkl_err_over_bar": max_bar, "max_p_rel": max_p}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, n_requests: int) -> dict:
    """Runs before anything touches the GPU, so the forked workers inherit no device state."""
    import multiprocessing as mp

    global _W
    _W = w
    # the GPU machine gives one GPU's jobs a 16-core share, whatever os.cpu_count() reports there
    cores = max(1, min(16, os.cpu_count() or 1))
    reqs = list(range(min(n_requests, w.B)))
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        refs = pool.map(_oracle_request, reqs, chunksize=1)
    dt = time.perf_counter() - t0
    positions = sum(int(w.k[b]) for b, _ in refs)
    return refs, {"value": positions / dt, "unit": "positions/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpu_count": os.cpu_count(),
            "cores_note": "worker processes capped at the 16-core share one GPU's jobs get",
            "sample": f"{len(reqs)} of {w.B} requests ({positions} verified positions, all "
                      f"outputs incl. the clipped rKL), float64 NumPy, {cores} worker processes, "
                      f"{dt:.2f} s wall"}


_OPD = None  # (target rows, draft rows, pairing, delta), inherited by forked workers


def _oracle_opd_request(b):
    import oracle

    tl, dl, idx, off, k, delta, grad = _OPD
    sl = slice(int(off[b]), int(off[b + 1]))
    oracle.opd_loss(tl[idx[sl]], dl[sl], [int(k[b])], delta, 0.8)
    if grad:
        oracle.opd_grad(tl[idx[sl]], dl[sl], [int(k[b])], delta, 0.8)
    return int(k[b])


def cpu_baseline_opd(w, idx, n_requests: int, grad: bool = False) -> dict:
    import multiprocessing as mp

    import oracle

    global _OPD
    tl = oracle.widen_logits(w.target[:, : w.V], w.dtype)
    dl = oracle.widen_logits(w.draft[:, : w.V], w.dtype)
    _OPD = (tl, dl, idx, w.draft_offsets, w.k, w.delta, grad)
    # the GPU machine gives one GPU's jobs a 16-core share, whatever os.cpu_count() reports there
    cores = max(1, min(16, os.cpu_count() or 1))
    reqs = list(range(min(n_requests, w.B)))
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(cores) as pool:
        rows = sum(pool.map(_oracle_opd_request, reqs, chunksize=1))
    dt = time.perf_counter() - t0
    what = "hard CE, clipped rKL, OPD loss" + (" and its gradient rows" if grad else "")
    return {"value": rows / dt, "unit": "rows/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(reqs)} of {w.B} requests ({rows} row pairs: {what}), float64 NumPy, "
                      f"{cores} worker processes, {dt:.2f} s wall"}


def _oracle_greedy_request(b):
    import numpy as np

    import oracle

    w = _W
    oracle.verify_block(target=w.target, draft=w.draft, dtype=w.dtype, V=w.V, k=w.k,
                        draft_tokens=w.draft_tokens, uniforms=w.uniforms,
                        temperature=np.zeros(w.B), delta=w.delta, requests=[b], with_rkl=False)
    return int(w.k[b])


def cpu_baseline_greedy(w, n_requests: int) -> dict:
    """The oracle at temperature 0, without the reverse-KL (it also forms the reported
    probabilities and per-position acceptance rates)."""
    import multiprocessing as mp

    global _W
    _W = w
    # the GPU machine gives one GPU's jobs a 16-core share, whatever os.cpu_count() reports there
    cores = max(1, min(16, os.cpu_count() or 1))
    reqs = list(range(min(n_requests, w.B)))
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(cores) as pool:
        positions = sum(pool.map(_oracle_greedy_request, reqs, chunksize=1))
    dt = time.perf_counter() - t0
    return {"value": positions / dt, "unit": "positions/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{len(reqs)} of {w.B} requests ({positions} verified positions at "
                      f"temperature 0, no rKL), float64 NumPy, {cores} worker processes, "
                      f"{dt:.2f} s wall"}


def bench_opd(args, w, grad=False):
    import numpy as np
    import torch

    import draft_block_verification_sv_amd as pkg

    idx_np = np.concatenate([np.arange(w.target_offsets[b], w.target_offsets[b] + w.k[b])
                             for b in range(w.B)]).astype(np.int32)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_opd(w, idx_np, args.cpu_requests, grad=grad)
        log(f"[bench] cpu baseline: {cpu['value']:.1f} rows/s")
    pkg.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")

    def up(a, dt=None):
        if dt is torch.bfloat16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(dt)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    bf = torch.bfloat16 if w.dtype == "bf16" else None
    target, draft = up(w.target, bf), up(w.draft, bf)
    idx, k = up(idx_np), up(w.k.astype(np.int32))
    n, V, B = w.n_draft_rows, w.V, w.B
    code = pkg.SV_BF16 if w.dtype == "bf16" else pkg.SV_F32
    size_fn = pkg.lib().sv_opd_grad_workspace_size if grad else pkg.lib().sv_rkl_workspace_size
    ws = pkg.alloc_workspace(int(size_fn(n, V, code)), dev)
    out = {"rkl": torch.empty(n, dtype=torch.float32, device=dev),
           "hard_ce": torch.empty(n, dtype=torch.float32, device=dev),
           "top1": torch.empty(n, dtype=torch.int32, device=dev),
           "opd": torch.empty(B, dtype=torch.float32, device=dev),
           "device_status": torch.empty(1, dtype=torch.int32, device=dev)}
    if grad:  # the gradient in the logits' dtype
        out["grad"] = torch.empty(n, V, dtype=target.dtype, device=dev)

    def step():
        if grad:
            pkg.opd_loss_grad(target, draft, k, delta=w.delta, alpha=0.8, p_row_index=idx,
                              workspace=ws, out=out)
        else:
            pkg.opd_loss(target, draft, k, delta=w.delta, alpha=0.8, p_row_index=idx,
                         workspace=ws, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert int(out["device_status"].item()) == 0
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = 1e3 * (time.perf_counter() - t_start) / args.steps
    pkg.profile_reset()
    pkg.profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = pkg.profile_read()
    pkg.profile_enable(False)
    kernels = {name: 1e3 * ms / cnt for name, (cnt, ms) in kt.items()}
    esize = 2 if w.dtype == "bf16" else 4
    if grad:  # the roofline kernel is the gradient pass: both rows read, the gradient written
        rows_bytes = 3 * n * V * esize
        roof_kernel = "sv_opd_grad"
        metric = "OPD loss + gradient row pairs/sec (forward pass, then gradient rows)"
    else:  # each draft row and its target row, once
        rows_bytes = 2 * n * V * esize
        roof_kernel = "sv_opd_rowpair"
        metric = "OPD loss row pairs/sec (hard CE + clipped rKL + per-request loss)"
    achieved = rows_bytes / (kernels[roof_kernel] * 1e-6) / 1e9
    res = {
        "metric": metric,
        "value": round(n / (ms_per_step * 1e-3), 1), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded logits shaped like the pages' workloads)",
        "config": {"workload": w.name, "op": args.op, "rows": n, "B": B, "V": V,
                   "input_dtype": w.dtype, "delta": w.delta, "alpha": 0.8,
                   "roofline_kernel": roof_kernel,
                   "roofline_kernel_bytes": rows_bytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None},
        "kernels_us": {kk: round(v, 2) for kk, v in kernels.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def bench_greedy(args, w):
    """Every request greedy (T_b = 0): sv_verify_block_greedy, target rows only."""
    import numpy as np
    import torch

    import draft_block_verification_sv_amd as pkg

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_greedy(w, args.cpu_requests)
        log(f"[bench] cpu baseline: {cpu['value']:.1f} positions/s")
    pkg.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    bf = torch.bfloat16 if w.dtype == "bf16" else None

    def up(a, dt=None):
        if dt is torch.bfloat16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(dt)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    target = up(w.target, bf)
    k, toks = up(w.k.astype(np.int32)), up(w.draft_tokens.astype(np.int32))
    code = pkg.SV_BF16 if w.dtype == "bf16" else pkg.SV_F32
    ws = pkg.alloc_workspace(pkg.workspace_size(w.B, w.k_max, w.V, code), dev)
    n_d, B, V = w.n_draft_rows, w.B, w.V
    out = {"accept_len": torch.empty(B, dtype=torch.int32, device=dev),
           "out_tokens": torch.empty(n_d + B, dtype=torch.int32, device=dev),
           "device_status": torch.empty(1, dtype=torch.int32, device=dev)}

    def step():
        pkg.verify_block_greedy(target, k, toks, k_max=w.k_max, workspace=ws, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert int(out["device_status"].item()) == 0
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = 1e3 * (time.perf_counter() - t_start) / args.steps
    pkg.profile_reset()
    pkg.profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = pkg.profile_read()
    pkg.profile_enable(False)
    kernels = {name: 1e3 * ms / cnt for name, (cnt, ms) in kt.items()}
    rows_bytes = (n_d + B) * V * (2 if w.dtype == "bf16" else 4)  # every target logit once
    achieved = rows_bytes / (kernels["sv_greedy"] * 1e-6) / 1e9
    res = {
        "metric": "verified draft positions/sec, greedy verification (target rows only)",
        "value": round(n_d / (ms_per_step * 1e-3), 1), "unit": "positions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded logits shaped like the pages' workloads)",
        "config": {"workload": w.name, "op": "greedy", "B": B, "k": int(w.k_max), "V": V,
                   "input_dtype": w.dtype, "algorithmic_bytes_per_step": rows_bytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None},
        "kernels_us": {kk: round(v, 2) for kk, v in kernels.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def bench_length_head(args):
    """The adaptive length head at the drafter's shape: B=128 requests, k=15 positions,
    H=4096, H'=256, seeded random bf16 weights and hidden states."""
    import numpy as np
    import torch

    import draft_block_verification_sv_amd as pkg

    B, k, H, Hf = 128, 15, 4096, 256
    g = torch.Generator(device="cpu").manual_seed(20261202)
    h_c = torch.randn(B, k, H, generator=g).to(torch.bfloat16)
    W1_c = (torch.randn(Hf, H, generator=g) / H ** 0.5).to(torch.bfloat16)
    b1_c = torch.randn(Hf, generator=g) * 0.5
    w2_c = torch.randn(Hf, generator=g) * 3 / Hf ** 0.5
    cpu = None
    if not args.no_cpu_baseline:  # the oracle, float64, on every request
        import oracle

        nb = B
        hh = h_c[:nb].float().numpy().astype(np.float64)
        WW = W1_c.float().numpy().astype(np.float64)
        t0 = time.perf_counter()
        oracle.length_head(hh, WW, b1_c.numpy().astype(np.float64), w2_c.numpy().astype(np.float64),
                           0.1)
        dt = time.perf_counter() - t0
        cpu = {"value": nb / dt, "unit": "requests/s", "cores": 1, "kind": "oracle",
               "sample": f"{nb} of {B} requests (projection, SiLU, pooling, a_hat), float64 "
                         f"NumPy, one process, {dt:.2f} s wall"}
        log(f"[bench] cpu baseline: {cpu['value']:.1f} requests/s")
    pkg.lib()
    dev = torch.device("cuda:0")
    h, W1, b1, w2 = h_c.to(dev), W1_c.to(dev), b1_c.to(dev), w2_c.to(dev)
    ws = pkg.alloc_workspace(int(pkg.lib().sv_length_head_workspace_size(B, k, H, Hf)), dev)
    out = {"a_hat": torch.empty(B, device=dev), "k_hat": torch.empty(B, dtype=torch.int32, device=dev),
           "off_t": torch.empty(B + 1, dtype=torch.int32, device=dev)}

    def step():
        pkg.length_head(h, W1, w2, b1, b2=0.1, gamma=1.0, workspace=ws, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = 1e3 * (time.perf_counter() - t_start) / args.steps
    pkg.profile_reset()
    pkg.profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = pkg.profile_read()
    pkg.profile_enable(False)
    kernels = {name: 1e3 * ms / cnt for name, (cnt, ms) in kt.items()}
    nbytes = (B * k * H + Hf * H) * 2  # hidden states and W1 once
    flops = 2.0 * B * k * H * Hf
    us = kernels["sv_head_feat"]
    res = {
        "metric": "length-head requests/sec (projection on MFMA, SiLU, pooling, k_hat, offsets)",
        "value": round(B / (ms_per_step * 1e-3), 1), "unit": "requests/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded random hidden states and head weights)",
        "config": {"workload": "length head: B=128 k=15 H=4096 H'=256 bf16", "op": "length_head",
                   "B": B, "k": k, "H": H, "H_feat": Hf, "bytes": nbytes, "flops": flops},
        "roofline": {"bound": "hbm", "achieved": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4), "traffic": None},
        "mfma_tflops": round(flops / (us * 1e-6) / 1e12, 2),
        "kernels_us": {kk: round(v, 2) for kk, v in kernels.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def bench_branch(args):
    """The prepared-branch lookup after verification at the high-concurrency shape (B=128,
    k=15) with D3D's main budget shape (coverage 12, fan-out 2: 24 keys per request), on
    seeded synthetic verification outcomes."""
    import numpy as np
    import torch

    import draft_block_verification_sv_amd as pkg

    B, k_max, n_branch = 128, 15, 24
    rng = np.random.default_rng(20261202)
    k = np.full(B, k_max, dtype=np.int32)
    al = rng.integers(0, k_max + 1, size=B).astype(np.int32)
    out = rng.integers(0, 151936, size=B * (k_max + 1)).astype(np.int32)
    pos = rng.integers(0, k_max + 1, size=(B, n_branch)).astype(np.int32)
    tok = rng.integers(-1, 151936, size=(B, n_branch)).astype(np.int32)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        t0 = time.perf_counter()
        reps = 20
        for _ in range(reps):
            oracle.branch_lookup(al, oracle.final_tokens(out, al, k), pos, tok)
        dt = (time.perf_counter() - t0) / reps
        cpu = {"value": B / dt, "unit": "requests/s", "cores": 1, "kind": "oracle",
               "sample": f"all {B} requests, {n_branch} keys each, {reps} repetitions, one "
                         f"process, {dt * 1e3:.2f} ms per call"}
    pkg.lib()
    dev = torch.device("cuda:0")
    t = {n: torch.from_numpy(v).to(dev) for n, v in
         (("k", k), ("al", al), ("out", out), ("pos", pos), ("tok", tok))}

    def step():
        pkg.branch_lookup(t["k"], t["al"], t["out"], t["pos"], t["tok"], k_max=k_max)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = 1e3 * (time.perf_counter() - t_start) / args.steps
    pkg.profile_reset()
    pkg.profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = pkg.profile_read()
    pkg.profile_enable(False)
    kernels = {name: 1e3 * ms / cnt for name, (cnt, ms) in kt.items()}
    nbytes = 4 * (2 * B + B + 2 * B * n_branch + B)  # k, a_b, the emitted token, keys, hit
    us = kernels["sv_branch"]
    res = {
        "metric": "prepared-branch lookups/sec after verification (requests)",
        "value": round(B / (ms_per_step * 1e-3), 1), "unit": "requests/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int32",
        "data": "synthetic (seeded verification outcomes and keys)",
        "config": {"workload": "branch lookup: B=128 k=15, 24 keys per request", "op": "branch",
                   "B": B, "k": k_max, "n_branch": n_branch, "bytes": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 6), "traffic": None},
        "kernels_us": {kk: round(v, 2) for kk, v in kernels.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def bench_tree(args):
    """Greedy verification of EAGLE-shaped draft trees (60 nodes each, the tree size the DFlash
    notes quote) for 32 requests at V=151936 bf16: the argmax of every target row (root and
    nodes), then the walk.  Seeded synthetic trees and logits whose row argmaxes follow a child's
    token with probability 0.7."""
    import numpy as np
    import torch

    import draft_block_verification_sv_amd as pkg
    from synth import bf16_bits_from_f64

    B, n_per, V = 32, 60, 151936
    rng = np.random.default_rng(20261202)
    parent, tokens, amax = [], [], []
    for b in range(B):
        par, tok = [], []
        for j in range(n_per):
            u = rng.random()
            p = (j - 1) if u < 0.5 else (int(rng.integers(-1, j)) if u < 0.9 else -1)
            used = {tok[i] for i in range(j) if par[i] == p}
            t = int(rng.integers(0, V))
            while t in used:
                t = int(rng.integers(0, V))
            par.append(p)
            tok.append(t)
        am = rng.integers(0, V, size=n_per + 1)
        for j in reversed(range(n_per)):  # the first child's token wins
            if rng.random() < 0.7:
                am[par[j] + 1] = tok[j]
        parent += par
        tokens += tok
        amax.append(am)
    rows = B * (n_per + 1)
    L = rng.normal(size=(rows, V)) * 2.0
    r = 0
    for am in amax:
        for a in am:
            L[r, a] = L[r].max() + 0.5
            r += 1
    bits = bf16_bits_from_f64(L)
    del L
    n = np.full(B, n_per, np.int32)
    parent = np.array(parent, np.int32)
    tokens = np.array(tokens, np.int32)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        nb = 8
        t0 = time.perf_counter()
        oracle.verify_tree_block(target=bits[: nb * (n_per + 1)], dtype="bf16", V=V,
                                 n_nodes=n[:nb], parent=parent[: nb * n_per],
                                 tokens=tokens[: nb * n_per])
        dt = time.perf_counter() - t0
        cpu = {"value": nb * n_per / dt, "unit": "tree nodes/s", "cores": 1, "kind": "oracle",
               "sample": f"{nb} of {B} requests ({nb * n_per} nodes), float64 NumPy, one process, "
                         f"{dt:.2f} s wall"}
        log(f"[bench] cpu baseline: {cpu['value']:.1f} nodes/s")
    pkg.lib()
    dev = torch.device("cuda:0")
    target = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    d = {k: torch.from_numpy(v).to(dev) for k, v in (("n", n), ("par", parent), ("tok", tokens))}
    ws = pkg.alloc_workspace(int(pkg.lib().sv_tree_workspace_size(B, int(n.sum()))), dev)
    out = {"accept_len": torch.empty(B, dtype=torch.int32, device=dev),
           "out_tokens": torch.empty(rows, dtype=torch.int32, device=dev),
           "out_nodes": torch.empty(B * n_per, dtype=torch.int32, device=dev),
           "device_status": torch.empty(1, dtype=torch.int32, device=dev)}

    def step():
        pkg.verify_tree_greedy(target, d["n"], d["par"], d["tok"], max_nodes=n_per, workspace=ws,
                               out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert int(out["device_status"].item()) == 0
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = 1e3 * (time.perf_counter() - t_start) / args.steps
    pkg.profile_reset()
    pkg.profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = pkg.profile_read()
    pkg.profile_enable(False)
    kernels = {name: 1e3 * ms / cnt for name, (cnt, ms) in kt.items()}
    nbytes = rows * V * 2  # every target logit once
    us = kernels["sv_tree_argmax"]
    mean_len = float(out["accept_len"].float().mean().item())
    res = {
        "metric": "draft-tree nodes verified/sec, greedy (target rows only)",
        "value": round(B * n_per / (ms_per_step * 1e-3), 1), "unit": "nodes/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded trees and logits)",
        "config": {"workload": "draft trees: B=32, 60 nodes each, V=151936 bf16", "op": "tree",
                   "B": B, "nodes": n_per, "V": V, "bytes": nbytes, "mean_accept_len": mean_len},
        "roofline": {"bound": "hbm", "achieved": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4), "traffic": None},
        "kernels_us": {kk: round(v, 2) for kk, v in kernels.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def bench_read_ceiling(args):
    """The practical read ceiling: the library's plain read kernel (1024 workgroups, each
    reading its contiguous share front to back with two 16-byte nontemporal loads per thread in
    flight) over the same number of bytes as a streaming launch."""
    import torch

    import draft_block_verification_sv_amd as pkg

    nbytes = args.read_ceiling // 16 * 16
    x = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda:0")
    out = torch.empty(pkg.binding.READ_PROBE_WORDS, dtype=torch.int32, device="cuda:0")
    for _ in range(args.warmup):
        pkg.read_probe(x, out)
    torch.cuda.synchronize()
    pkg.profile_reset()
    pkg.profile_enable(True)
    for _ in range(args.steps):
        pkg.read_probe(x, out)
    torch.cuda.synchronize()
    kt = pkg.profile_read()
    pkg.profile_enable(False)
    n, ms = kt["sv_read_probe"]
    us = 1e3 * ms / n
    gbs = nbytes / (us * 1e-6) / 1e9
    print(json.dumps({"read_ceiling": {"bytes": nbytes, "launches": n, "avg_us": round(us, 2),
                                       "GB/s": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}}),
          flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="high_concurrency")
    ap.add_argument("--op", choices=("verify", "greedy", "opd", "opd_grad", "length_head", "branch",
                                         "tree"),
                    default="verify")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-requests", type=int, default=128)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES (counter calibration)")
    ap.add_argument("--read-ceiling", type=int, default=0, metavar="BYTES",
                    help="only time the library's plain read kernel over BYTES of device memory")
    args = ap.parse_args()

    if args.read_ceiling:
        return bench_read_ceiling(args)
    if args.calibrate_copy:
        import torch

        n = args.calibrate_copy // 4
        x = torch.ones(n, dtype=torch.int32, device="cuda:0")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4, "launches": 3}), flush=True)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the verification path is per-GPU data-parallel "
              "(requests are independent), and this build runs on a single MI355X. "
              "Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import draft_block_verification_sv_amd as pkg
    from synth import workload

    if args.op == "length_head":
        return bench_length_head(args)
    if args.op == "branch":
        return bench_branch(args)
    if args.op == "tree":
        return bench_tree(args)
    t0 = time.perf_counter()
    w = workload(args.workload)
    log(f"[bench] generated {w.name} in {time.perf_counter() - t0:.1f}s")
    if args.op in ("opd", "opd_grad"):
        return bench_opd(args, w, grad=(args.op == "opd_grad"))
    if args.op == "greedy":
        return bench_greedy(args, w)
    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on {args.cpu_requests} requests")
        refs, cpu = cpu_baseline(w, args.cpu_requests)
        log(f"[bench] cpu baseline: {cpu['value']:.1f} positions/s")

    pkg.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")

    def up(a, dt=None):
        if dt is torch.bfloat16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(dt)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    bf = torch.bfloat16 if w.dtype == "bf16" else None
    target, draft = up(w.target, bf), up(w.draft, bf)
    k = up(w.k.astype(np.int32))
    toks = up(w.draft_tokens.astype(np.int32))
    uni = up(w.uniforms.astype(np.float32))
    temp = up(w.temperature.astype(np.float32))
    code = pkg.SV_BF16 if w.dtype == "bf16" else pkg.SV_F32
    ws = pkg.alloc_workspace(pkg.workspace_size(w.B, w.k_max, w.V, code), dev)
    n_d, B, V = w.n_draft_rows, w.B, w.V
    out = {
        "accept_len": torch.empty(B, dtype=torch.int32, device=dev),
        "out_tokens": torch.empty(n_d + B, dtype=torch.int32, device=dev),
        "rkl": torch.empty(n_d, dtype=torch.float32, device=dev),
        "p_at_draft": torch.empty(n_d, dtype=torch.float32, device=dev),
        "q_at_draft": torch.empty(n_d, dtype=torch.float32, device=dev),
        "device_status": torch.empty(1, dtype=torch.int32, device=dev),
    }

    def step():
        pkg.verify_block(target, draft, k, toks, uni, temp, w.delta, k_max=w.k_max,
                         workspace=ws, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert int(out["device_status"].item()) == 0
    log(f"[bench] warmup done ({args.warmup} steps)")

    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = 1e3 * elapsed / args.steps
    log(f"[bench] timed {args.steps} steps: {ms_per_step:.4f} ms/step")

    # per-kernel durations: HIP events the library records around each launch on the
    # call's stream, over a second pass of the same number of steps
    pkg.profile_reset()
    pkg.profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = pkg.profile_read()
    pkg.profile_enable(False)
    pkg.profile_reset()
    kernels = {name: {"launches": n, "avg_us": 1e3 * ms / n} for name, (n, ms) in kt.items()}
    log(f"[bench] kernels: {json.dumps(kernels)}")

    esize = 2 if w.dtype == "bf16" else 4
    rows_bytes = (w.n_target_rows + n_d) * V * esize  # every logit read once
    meta_bytes = 4 * (2 * (n_d + B) + B + n_d) + 4 * (B + (n_d + B) + 3 * n_d)
    # small launches split each row over several workgroups of one launch (timed under the
    # streaming kernel's name with a "_split" suffix), which still reads every logit once
    stream_name = STREAM_KERNEL if STREAM_KERNEL in kernels else STREAM_KERNEL + "_split"
    rows_us = kernels[stream_name]["avg_us"]
    kernel_gbs = rows_bytes / (rows_us * 1e-6) / 1e9
    traffic = None
    if os.path.exists(COUNTERS_FILE):
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
        if c.get("kernel_source_hash") == kernel_source_hash() and c.get("workload") == args.workload:
            traffic = c.get("hbm_bytes_per_call")
    roofline = {"bound": "hbm", "peak": PEAK_HBM_GBS, "unit": "GB/s", "traffic": traffic,
                "kernel": "sv_verify_block (every kernel of the call)",
                "kernels": sorted(kernels),
                "kernel_frac": {"kernel": stream_name, "achieved": round(kernel_gbs, 1),
                                "frac": round(kernel_gbs / PEAK_HBM_GBS, 4)}}

    # the practical read ceiling beside it: the library's plain read kernel over the same
    # number of bytes, timed the same way (after the measured passes)
    probe = torch.ones(rows_bytes // 4, dtype=torch.int32, device=dev)
    probe_out = torch.empty(pkg.binding.READ_PROBE_WORDS, dtype=torch.int32, device=dev)
    for _ in range(3):
        pkg.read_probe(probe, probe_out)
    torch.cuda.synchronize()
    pkg.profile_reset()
    pkg.profile_enable(True)
    for _ in range(args.steps):
        pkg.read_probe(probe, probe_out)
    torch.cuda.synchronize()
    n_probe, ms_probe = pkg.profile_read()["sv_read_probe"]
    pkg.profile_enable(False)
    pkg.profile_reset()
    del probe
    probe_gbs = (rows_bytes // 4 * 4) / (ms_probe / n_probe * 1e-3) / 1e9
    roofline["read_ceiling"] = {"kernel": "sv_read_probe", "achieved": round(probe_gbs, 1),
                                "frac": round(probe_gbs / PEAK_HBM_GBS, 4),
                                "kernel_over_ceiling": round(kernel_gbs / probe_gbs, 4)}

    if cpu is not None:  # the timed call's outputs against the oracle's on the sampled requests
        cpu["parity"] = parity_sample(w, out, refs)
        log(f"[bench] parity on the baseline's requests: {json.dumps(cpu['parity'])}")

    # device time of each call: HIP events around every call on the call's stream, in a pass
    # of its own (median, p10, p90)
    stream = torch.cuda.current_stream()
    call_us = []
    for _ in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        call_us.append((e0, e1))
    torch.cuda.synchronize()
    call_us = np.array([1e3 * a.elapsed_time(b) for a, b in call_us])
    call_stats = {"median": round(float(np.median(call_us)), 2),
                  "p10": round(float(np.percentile(call_us, 10)), 2),
                  "p90": round(float(np.percentile(call_us, 90)), 2)}
    # the call's rate: algorithmic bytes over the median device time of a whole call
    achieved = (rows_bytes + meta_bytes) / (float(np.median(call_us)) * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), **roofline}

    # realised acceptance: mean tokens per request-round and the per-position acceptance rate
    # (accepted at i among requests that reached i)
    al = out["accept_len"].cpu().numpy().astype(np.int64)
    kk = w.k.astype(np.int64)
    acc_profile = []
    for i in range(int(w.k_max)):
        reached = int(np.sum((al >= i) & (kk > i)))
        acc_profile.append(round(float(np.sum(al > i)) / reached, 4) if reached else None)
    realised = {"mean_tau": round(float(np.mean(al + 1)), 3), "acc_per_position": acc_profile}

    # inputs that fit the 256 MB last-level cache are also timed from HBM: the call rotates
    # through enough copies of the logits that each is evicted before it is read again
    cold = None
    in_bytes = (w.n_target_rows + w.n_draft_rows) * w.V * (2 if w.dtype == "bf16" else 4)
    if in_bytes < (512 << 20):
        n_sets = min(256, max(3, -(-(768 << 20) // in_bytes)))
        sets = [(target.clone(), draft.clone()) for _ in range(n_sets)]
        torch.cuda.synchronize()
        for j in range(args.warmup):
            tg, dr = sets[j % n_sets]
            pkg.verify_block(tg, dr, k, toks, uni, temp, w.delta, k_max=w.k_max, workspace=ws, out=out)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for j in range(args.steps):
            tg, dr = sets[j % n_sets]
            pkg.verify_block(tg, dr, k, toks, uni, temp, w.delta, k_max=w.k_max, workspace=ws, out=out)
        torch.cuda.synchronize()
        ms_cold = 1e3 * (time.perf_counter() - t0) / args.steps
        cold = {"ms_per_step": round(ms_cold, 5), "value": round(w.n_draft_rows / (ms_cold * 1e-3), 1),
                "input_sets": n_sets, "bytes_per_set": in_bytes}
        del sets
        log(f"[bench] rotating {n_sets} input sets: {ms_cold:.4f} ms/step")

    value = n_d / (ms_per_step * 1e-3)
    whole_gbs = (rows_bytes + meta_bytes) / (ms_per_step * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded logits shaped like the pages' workloads)",
        "config": {"workload": w.name, "B": B, "k": int(w.k_max), "V": V, "input_dtype": w.dtype,
                   "delta": w.delta, "verified_positions_per_step": n_d,
                   "algorithmic_bytes_per_step": rows_bytes + meta_bytes},
        "roofline": roofline,
        "step_hbm_gbs": round(whole_gbs, 1),
        "step_frac_of_peak": round(whole_gbs / PEAK_HBM_GBS, 4),
        "kernels_us": {n: round(v["avg_us"], 2) for n, v in kernels.items()},
        "call_us": call_stats,
        "inputs_from_hbm": cold,
        "realised": realised,
        "kernel_source_hash": kernel_source_hash(),
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
