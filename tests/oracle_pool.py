"""The oracle over many requests of one workload at once, for the GPU parity tests at full
batch size (test infrastructure only).

The worker processes are forked when the test session starts (``start``, called from
conftest), before anything touches the GPU, and live until it ends: they inherit no device
state and never use the GPU.  Each task carries one request's rows (``Workload.subset``), so no worker holds the
whole batch.  The results are assembled into the workload's own packed layout, in the form
``oracle.verify_block`` returns, so ``gpu_util.compare`` reads them unchanged.
"""

from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

_POOL = None


def start() -> None:
    global _POOL
    if _POOL is None:
        import atexit

        _POOL = mp.get_context("fork").Pool(workers())
        atexit.register(_POOL.terminate)


def workers() -> int:
    # the GPU machine gives one GPU's jobs 16 cores, whatever os.cpu_count() reports there
    return max(1, min(16, os.cpu_count() or 1))


def _one(args):
    import oracle

    sub, b, with_rkl = args
    r = oracle.verify_block(target=sub.target, draft=sub.draft, dtype=sub.dtype, V=sub.V, k=sub.k,
                            draft_tokens=sub.draft_tokens, uniforms=sub.uniforms,
                            temperature=sub.temperature, delta=sub.delta, with_rkl=with_rkl)
    return b, r


def oracle_refs(w, requests=None, with_rkl: bool = True) -> dict:
    """``oracle.verify_block``'s outputs for ``requests`` (all by default) of workload ``w``."""
    start()
    reqs = list(range(w.B)) if requests is None else [int(b) for b in requests]
    to, do = w.target_offsets, w.draft_offsets
    res = {
        "accept_len": np.full(w.B, -1, dtype=np.int64),
        "out_tokens": np.full(w.n_target_rows, -1, dtype=np.int64),
        "token_margin": np.full(w.B, np.inf),
        "expected_tau": np.full(w.B, np.nan),
        "done": np.zeros(w.B, dtype=bool),
    }
    for key in ("rkl", "kl", "rkl_l1", "p_at_draft", "q_at_draft", "acc_rate"):
        res[key] = np.full(w.n_draft_rows, np.nan)
    res["accept_margin"] = np.full(w.n_draft_rows, np.inf)
    tasks = ((w.subset([b]), b, with_rkl) for b in reqs)
    for b, r in _POOL.imap_unordered(_one, tasks, chunksize=1):
        st, sd = slice(to[b], to[b + 1]), slice(do[b], do[b + 1])
        res["accept_len"][b] = r["accept_len"][0]
        res["out_tokens"][st] = r["out_tokens"]
        res["token_margin"][b] = r["token_margin"][0]
        res["expected_tau"][b] = r["expected_tau"][0]
        res["done"][b] = r["done"][0]
        for key in ("rkl", "kl", "rkl_l1", "p_at_draft", "q_at_draft", "acc_rate",
                    "accept_margin"):
            res[key][sd] = r[key]
    return res
