"""Seeded synthetic draft-block verification workloads.

A workload is one verification batch in the packed layout the library takes:

* ``B`` requests; request ``b`` carries ``k[b]`` draft tokens (the per-request
  verification length after length-head truncation, AdaFlash paper, Section 3.2,
  equation for the verification length; packed into one batch of total length
  sum(k), Section 3.3 "Adaptive Request Scheduling").
* target logits: ``k[b] + 1`` rows per request, packed in request order.  Row
  ``i < k[b]`` scores draft token ``i``; row ``k[b]`` is the bonus row.
* draft logits: ``k[b]`` rows per request, packed in request order.
* draft tokens: one id per draft row.
* uniforms: one fp32 value per target row.  Slot ``i < k[b]`` is the acceptance
  uniform of draft ``i``; slot ``k[b]`` drives the single final-token draw.

Logit recipe (the pages print no logits, so this is a stand-in for the Qwen3
vocabularies the pages' experiments use):

    target row  = s * N(0, 1)^V + prior,   prior_y = -1.1 * ln(pi(y))
    draft row i = target row i + sigma * N(0, 1)^V

where ``pi`` is a seeded permutation of 1..V shared by every row (a Zipf(1.1)
log-prior).  Values are drawn in float64 and rounded to bf16 with
round-to-nearest-even (via fp32); those bits are the inputs of both the oracle
and the GPU path.  Draft tokens are drawn from the rounded draft logits at the
request temperature with the Gumbel-max trick (argmax for temperature 0), which
gives an exact sample of softmax(l / T) without evaluating it.  Uniforms are
``(r >> 8) * 2**-24`` for 32-bit random ``r``, so they lie in [0, 1) exactly in
fp32.

Nothing here evaluates a softmax, an acceptance test or a divergence.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

ROOT_SEED = 20261202

# name -> (seed stream id, description).  The stream id only separates the seeded streams.
WORKLOADS = {
    "tiny": (1, "tiny: B=1 k=4 V=1000 fp32"),
    "single": (2, "single request: B=1 k=15 V=151936 bf16, sigma rising 0.3->2.0 with position"),
    "ragged": (3, "ragged: B=32 k_b~U[1,15] V=151936 bf16, T_b in {0, 0.7, 1.0}"),
    "high_concurrency": (4, "high concurrency: B=128 k=15 V=151936 bf16, sigma_b in {0.5, 1, 2}, "
                            "fused rKL delta=1"),
    "large_vocab": (5, "large vocab stress: B=128 k=15 V=248320 bf16, 10% outlier ids shifted "
                       "-20, forced edge cases"),
}

_POISON_BF16 = 0x42C8  # bf16 bits of +100.0: fills columns in [V, ld) so reads past V are visible
_POISON_F32 = np.float32(100.0)


# ----------------------------------------------------------------------------- bf16 helpers
def bf16_bits_from_f64(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (fp32 first, then round-to-nearest-even on the top 16 bits)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return b.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _uniform_f32(rng: np.random.Generator, n: int) -> np.ndarray:
    r = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    return ((r >> 8).astype(np.float64) * 2.0**-24).astype(np.float32)


# ----------------------------------------------------------------------------- workload
@dataclasses.dataclass
class Workload:
    name: str
    dtype: str  # "bf16" or "f32"
    B: int
    V: int
    ld: int
    k_max: int
    k: np.ndarray  # int32[B]
    temperature: np.ndarray  # float32[B]
    delta: float
    target: np.ndarray  # uint16[n_t, ld] bf16 bits, or float32[n_t, ld]
    draft: np.ndarray  # same dtype, [n_d, ld]
    draft_tokens: np.ndarray  # int32[n_d]
    uniforms: np.ndarray  # float32[n_t]
    meta: dict = dataclasses.field(default_factory=dict)

    @property
    def n_draft_rows(self) -> int:
        return int(self.k.astype(np.int64).sum())

    @property
    def n_target_rows(self) -> int:
        return self.n_draft_rows + self.B

    @property
    def target_offsets(self) -> np.ndarray:
        """int64[B+1]: first target row of each request (packed layout bookkeeping)."""
        return np.concatenate([[0], np.cumsum(self.k.astype(np.int64) + 1)])

    @property
    def draft_offsets(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.k.astype(np.int64))])

    @property
    def esize(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def rows_f32(self, which: str, rows) -> np.ndarray:
        """Logit rows (first V columns) widened exactly to fp32."""
        a = self.target if which == "target" else self.draft
        a = a[rows, : self.V]
        return bf16_bits_to_f32(a) if self.dtype == "bf16" else np.asarray(a, dtype=np.float32)

    def subset(self, requests) -> "Workload":
        """A workload holding only the given requests (same bits, repacked)."""
        requests = np.asarray(requests, dtype=np.int64)
        to, do = self.target_offsets, self.draft_offsets
        t_rows = np.concatenate([np.arange(to[b], to[b + 1]) for b in requests])
        d_rows = np.concatenate([np.arange(do[b], do[b + 1]) for b in requests])
        return dataclasses.replace(
            self,
            name=self.name + f"[{len(requests)} requests]",
            B=len(requests),
            k=self.k[requests].copy(),
            temperature=self.temperature[requests].copy(),
            target=self.target[t_rows],
            draft=self.draft[d_rows],
            draft_tokens=self.draft_tokens[d_rows].copy(),
            uniforms=self.uniforms[t_rows].copy(),
            meta=dict(self.meta, parent_requests=requests.tolist()),
        )


def _generate(children, *, name, B, k, V, dtype, s, sigma, temperature, delta, ld,
              outlier_frac, outlier_shift, all_accept, first_reject, zipf_exponent,
              k_max) -> Workload:
    rng_perm, _rng_params, rng_t, rng_d, rng_out, rng_edge, rng_tok, rng_u = (
        np.random.Generator(np.random.PCG64(c)) for c in children
    )
    k = np.asarray(k, dtype=np.int32)
    temperature = np.asarray(temperature, dtype=np.float32)
    sigma = np.asarray(sigma, dtype=np.float64)
    assert k.shape == (B,) and temperature.shape == (B,) and sigma.shape[0] == B
    ld = V if ld is None else int(ld)
    assert ld >= V
    n_d = int(k.astype(np.int64).sum())
    n_t = n_d + B

    perm = rng_perm.permutation(V).astype(np.float64) + 1.0
    prior = -zipf_exponent * np.log(perm)

    if dtype == "bf16":
        target = np.full((n_t, ld), _POISON_BF16, dtype=np.uint16)
        draft = np.full((n_d, ld), _POISON_BF16, dtype=np.uint16)
    else:
        target = np.full((n_t, ld), _POISON_F32, dtype=np.float32)
        draft = np.full((n_d, ld), _POISON_F32, dtype=np.float32)

    def store(dst, row, vals):
        if dtype == "bf16":
            dst[row, :V] = bf16_bits_from_f64(vals)
        else:
            dst[row, :V] = vals.astype(np.float32)

    outlier_sets = {}
    t0 = d0 = 0
    for b in range(B):
        kb = int(k[b])
        for i in range(kb + 1):
            lp = s * rng_t.standard_normal(V) + prior
            if i < kb:
                lq = lp + sigma[b, i] * rng_d.standard_normal(V)
                if outlier_frac > 0.0:
                    ids = rng_out.choice(V, size=int(round(outlier_frac * V)), replace=False)
                    lp = lp.copy()
                    lp[ids] += outlier_shift
                    outlier_sets[(b, i)] = np.sort(ids)
                store(draft, d0 + i, lq)
            store(target, t0 + i, lp)
        t0 += kb + 1
        d0 += kb

    t_off = np.concatenate([[0], np.cumsum(k.astype(np.int64) + 1)])
    d_off = np.concatenate([[0], np.cumsum(k.astype(np.int64))])
    for b in all_accept:  # draft rows := target rows, bit for bit
        for i in range(int(k[b])):
            draft[d_off[b] + i] = target[t_off[b] + i]

    def widen(row):
        return (bf16_bits_to_f32(row[:V]) if dtype == "bf16" else row[:V]).astype(np.float64)

    tokens = np.empty(n_d, dtype=np.int32)
    for b in range(B):
        T = float(temperature[b])
        for i in range(int(k[b])):
            lq = widen(draft[d_off[b] + i])
            if T == 0.0:
                tokens[d_off[b] + i] = int(np.argmax(lq))
            else:
                tokens[d_off[b] + i] = int(np.argmax(lq / T + rng_tok.gumbel(size=V)))

    uniforms = _uniform_f32(rng_u, n_t)

    for b in first_reject:  # x_0 := the outlier id the drafter likes most; u_0 >= 0.5
        ids = outlier_sets[(b, 0)]
        lq = widen(draft[d_off[b]])
        tokens[d_off[b]] = int(ids[np.argmax(lq[ids])])
        uniforms[t_off[b]] = max(uniforms[t_off[b]], np.float32(0.5))

    return Workload(
        name=name, dtype=dtype, B=B, V=V, ld=ld, k_max=int(k_max), k=k,
        temperature=temperature, delta=float(delta), target=target, draft=draft,
        draft_tokens=tokens, uniforms=uniforms,
        meta=dict(s=s, sigma=sigma, outlier_frac=outlier_frac, outlier_shift=outlier_shift,
                  all_accept=sorted(int(x) for x in all_accept),
                  first_reject=sorted(int(x) for x in first_reject)),
    )


def make_workload(*, B, k, V, dtype="bf16", s=4.0, sigma=1.0, temperature=1.0, delta=1.0,
                  seed=(0,), ld=None, outlier_frac=0.0, outlier_shift=-20.0, all_accept=(),
                  first_reject=(), zipf_exponent=1.1, k_max=None, name="custom") -> Workload:
    """General generator used by tests: explicit per-request lengths, sigmas and temperatures.

    ``sigma`` may be a scalar, a per-request vector or a ``[B, max k]`` array (per position).
    """
    k = np.broadcast_to(np.asarray(k, dtype=np.int32), (B,)).copy()
    kmax_arr = int(k.max()) if B > 0 else 1
    sig = np.asarray(sigma, dtype=np.float64)
    if sig.ndim == 0:
        sig = np.full((B, kmax_arr), float(sig))
    elif sig.ndim == 1:
        sig = np.repeat(sig[:, None], kmax_arr, axis=1)
    temp = np.broadcast_to(np.asarray(temperature, dtype=np.float32), (B,)).copy()
    ss = np.random.SeedSequence([ROOT_SEED, 1000, *seed])
    return _generate(ss.spawn(8), name=name, B=B, k=k, V=V, dtype=dtype, s=s, sigma=sig,
                     temperature=temp, delta=delta, ld=ld, outlier_frac=outlier_frac,
                     outlier_shift=outlier_shift, all_accept=all_accept,
                     first_reject=first_reject, zipf_exponent=zipf_exponent,
                     k_max=k_max if k_max is not None else max(kmax_arr, 1))


def _position_sigma(n: int) -> np.ndarray:
    # token-level variance: drafter noise rising linearly from 0.3 to 2.0 over a 15-draft block
    return 0.3 + 1.7 * np.arange(n, dtype=np.float64) / 14.0


def workload(name: str, rep: int = 0, *, B: Optional[int] = None) -> Workload:
    """One of the named workloads (``B`` may be lowered for quick tests of the recipe)."""
    if name not in WORKLOADS:
        raise ValueError(f"unknown workload {name!r}; known: {', '.join(WORKLOADS)}")
    n, desc = WORKLOADS[name]
    ss = np.random.SeedSequence([ROOT_SEED, n, rep])
    children = ss.spawn(8)
    rng_params = np.random.Generator(np.random.PCG64(children[1]))
    common = dict(ld=None, outlier_frac=0.0, outlier_shift=-20.0, all_accept=(),
                  first_reject=(), zipf_exponent=1.1)
    if n == 1:
        Bn = 1
        return _generate(children, name=desc, B=Bn, k=[4], V=1000,
                         dtype="f32", s=3.0, sigma=np.full((1, 4), 0.5), temperature=[1.0],
                         delta=1.0, k_max=4, **common)
    if n == 2:
        return _generate(children, name=desc, B=1, k=[15], V=151936,
                         dtype="bf16", s=4.0, sigma=_position_sigma(15)[None, :],
                         temperature=[1.0], delta=1.0, k_max=15, **common)
    if n == 3:
        Bn = 32 if B is None else B
        k = rng_params.integers(1, 16, size=Bn).astype(np.int32)
        temp = rng_params.choice(np.array([0.0, 0.7, 1.0], dtype=np.float32), size=Bn)
        sig = np.repeat(_position_sigma(15)[None, :], Bn, axis=0)
        return _generate(children, name=desc, B=Bn, k=k, V=151936,
                         dtype="bf16", s=4.0, sigma=sig, temperature=temp, delta=1.0,
                         k_max=15, **common)
    if n in (4, 5):
        Bn = 128 if B is None else B
        V = 151936 if n == 4 else 248320
        sig_b = rng_params.choice(np.array([0.5, 1.0, 2.0]), size=Bn)
        sig = np.repeat(sig_b[:, None], 15, axis=1)
        extra = dict(common)
        if n == 5:
            n_edge = int(np.floor(0.05 * Bn))
            picks = rng_params.permutation(Bn)[: 2 * n_edge]
            extra.update(outlier_frac=0.10, all_accept=tuple(int(x) for x in picks[:n_edge]),
                         first_reject=tuple(int(x) for x in picks[n_edge:]))
        return _generate(children, name=desc, B=Bn,
                         k=np.full(Bn, 15, np.int32), V=V, dtype="bf16", s=4.0, sigma=sig,
                         temperature=np.ones(Bn, np.float32), delta=1.0, k_max=15, **extra)
    raise AssertionError(name)
