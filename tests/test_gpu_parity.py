"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same seeded
inputs.  Needs an MI355X and the built library."""

import json
import math
import os

import numpy as np
import pytest

from synth import make_workload, workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_util import RKL_ABS, RTOL, compare, run_gpu, run_oracle, to_device  # noqa: E402
from oracle_pool import oracle_refs  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_block_verification_sv_amd as pkg

    pkg.lib()  # fails loudly if the library is not built


def _report(name, s):
    print(f"[parity] {name}: exact={s['exact']} flips={len(s['flips'])} "
          f"max_p_rel={s['max_p_rel']:.2e} max_rkl_rel={s['max_rkl_rel']:.2e}", flush=True)


# ----------------------------------------------------------------------------- small cases
def test_tiny_fp32():
    w = workload("tiny")
    got = run_gpu(w)
    assert got["device_status"][0] == 0
    s = compare(w, got, run_oracle(w))
    _report("tiny", s)
    assert s["exact"] == 1


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_mixed_temperatures(dtype):
    # several slices and a ragged tail (V not a multiple of 8), every temperature mode
    w = make_workload(B=8, k=[1, 15, 3, 7, 2, 5, 1, 9], V=5003, dtype=dtype, s=3.0,
                      sigma=[0.3, 0.8, 1.5, 0.5, 2.0, 1.0, 0.7, 1.2],
                      temperature=[1.0, 0.0, 0.7, 1.3, 0.0, 0.5, 2.0, 1.0], delta=0.2,
                      seed=(1, dtype == "bf16"))
    got = run_gpu(w)
    assert got["device_status"][0] == 0
    s = compare(w, got, run_oracle(w))
    _report(f"ragged {dtype}", s)
    assert s["exact"] >= w.B - 1


@pytest.mark.parametrize("dtype,ld", [("bf16", 4104), ("bf16", 4097), ("f32", 4100), ("f32", 4099)])
def test_padded_rows(dtype, ld):
    # ld > V; padding columns hold +100 so a read past V would change every result
    w = make_workload(B=3, k=[4, 2, 6], V=4093, ld=ld, dtype=dtype, s=4.0, sigma=1.0,
                      temperature=[1.0, 0.7, 0.0], delta=0.5, seed=(2, ld))
    got = run_gpu(w)
    assert got["device_status"][0] == 0
    s = compare(w, got, run_oracle(w))
    _report(f"padded {dtype} ld={ld}", s)


@pytest.mark.parametrize("V", [1, 7, 64, 2048, 2049])
def test_tiny_and_boundary_vocab(V):
    w = make_workload(B=2, k=[1, 3], V=V, dtype="bf16", s=2.0, sigma=0.5, temperature=[1.0, 0.7],
                      delta=1.0, seed=(3, V))
    got = run_gpu(w)
    s = compare(w, got, run_oracle(w))
    _report(f"V={V}", s)


@pytest.mark.parametrize("dtype,ld", [("bf16", 40001), ("f32", 40000), ("f32", 40003)])
def test_small_delta_every_row_layout(dtype, ld):
    # nearly every lane fails the no-clip bound: several rounds of re-read pieces, for rows read
    # 16 bytes at a time and column by column
    w = make_workload(B=3, k=[5, 3, 4], V=40000, ld=ld, dtype=dtype, s=4.0, sigma=[0.5, 1.0, 2.0],
                      temperature=[1.0, 0.7, 0.0], delta=1e-3, outlier_frac=0.1, seed=(5, ld))
    got = run_gpu(w)
    assert got["device_status"][0] == 0
    s = compare(w, got, run_oracle(w))
    _report(f"delta=1e-3 {dtype} ld={ld}", s)


@pytest.mark.parametrize("delta", [1e-3, 1e-2, 0.1])
def test_small_delta_rereads_clipped_slices(delta):
    # small delta makes many slices fail the no-clip bound and take the direct path
    w = make_workload(B=3, k=[5, 3, 4], V=40000, dtype="bf16", s=4.0, sigma=[0.5, 1.0, 2.0],
                      temperature=1.0, delta=delta, outlier_frac=0.1, seed=(4,))
    got = run_gpu(w)
    s = compare(w, got, run_oracle(w))
    _report(f"delta={delta}", s)


# ----------------------------------------------------------------------------- heavy lanes
# Rows whose mass sits on a few tokens in distinct lanes of the streaming workgroup (column
# j 8 + (j % 4) 1024: slice j % 4, lane j), each shifted by one bf16 step between the target and
# the draft, so that the reverse-KL of each such lane cancels strongly.  Requests cycle through
# 12 such tokens (more heavy lanes than a row's record for the draw launch holds: summed in the
# finalize), 6 and 2 (summed by the draw launch) and 1 token holding most of the mass.  4
# requests split their rows over several workgroups; 40 do not.
def _heavy_lane_workload(dtype, B, seed, V=20000):
    from synth import bf16_bits_from_f64

    pattern = [12, 6, 2, 1]
    k = [3, 2, 3, 2] * (B // 4)
    w = make_workload(B=B, k=k, V=V, dtype=dtype, s=1.0, sigma=0.5, seed=seed)
    rng = np.random.default_rng(list(seed) + [99])
    to, do = w.target_offsets, w.draft_offsets

    def put(arr, row, vals):
        arr[row, :V] = bf16_bits_from_f64(vals) if dtype == "bf16" else vals.astype(np.float32)

    for b in range(B):
        n_tok = pattern[b % 4]
        cols = np.array([j * 8 + (j % 4) * 1024 for j in range(n_tok)])
        for i in range(int(w.k[b]) + 1):
            lp = rng.standard_normal(V)
            lp[cols] = (14.0 if n_tok > 1 else 12.0) + 0.25 * rng.standard_normal(n_tok)
            put(w.target, to[b] + i, lp)
            if i < w.k[b]:
                lq = lp.copy()
                lq[cols] += 0.0625
                lq += 1e-3 * rng.standard_normal(V)
                put(w.draft, do[b] + i, lq)
    return w


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B", [4, 40])
@pytest.mark.parametrize("delta", [1.0, 1e-3])
def test_heavy_lanes(dtype, B, delta):
    w = _heavy_lane_workload(dtype, B, (30, B, dtype == "f32"))
    got = run_gpu(w, delta=delta)
    assert got["device_status"][0] == 0
    s = compare(w, got, run_oracle(w, delta=delta))
    _report(f"heavy lanes {dtype} B={B} delta={delta}", s)


# The same rows long enough (137 slices) that a small launch splits them into 16 parts, which
# fold their four waves into 64 lanes: the heavy tokens' lanes stay distinct, now holding four
# times the columns, re-read in four blocks (finalize: 12 heavy lanes; draw launch: 6, 2, 1).
# B = 4 (14 rows): 224 streaming workgroups; B = 8 (28 rows): 448.  V = 140001 leaves bf16 rows
# unaligned (column by column loads); V = 139264 (136 slices) gives 16-byte rows.
@pytest.mark.parametrize("dtype,V", [("bf16", 140001), ("f32", 140001), ("bf16", 139264)])
@pytest.mark.parametrize("B", [4, 8])
def test_heavy_lanes_folded(dtype, V, B):
    w = _heavy_lane_workload(dtype, B, (31, B, dtype == "f32"), V=V)
    got = run_gpu(w, delta=1.0)
    assert got["device_status"][0] == 0
    s = compare(w, got, run_oracle(w, delta=1.0))
    _report(f"heavy lanes folded {dtype} V={V} B={B}", s)


@pytest.mark.parametrize("B", [1, 65])  # one request: split rows; 65 (130 rows): one WG per row
def test_clip_bound_when_lane_offset_trails_later_slices(B):
    # Regression for the no-clip bound.  Every logit is -30 except one token y that both rows
    # favour (l_q = l_p = 10, in a slice that is no lane's first) and a larger target token z
    # (l_p = 14).  Then c2 = LZ_p - LZ_q > 0 and t_y = ln2 q_y (L2E d_y + c2) with d_y = 0 is
    # about 4, clipped to delta = 1.  The lane's sum offset comes from its first slice (-30), so
    # E_y = 2^(l_q L2E - k_q) is about 2^57 against it: a bound that took max E_y <= 1 let this
    # lane through as unclipped and returned R near 4.
    from synth import bf16_bits_from_f64

    V = 151936
    w = make_workload(B=B, k=[1] * B, V=V, dtype="bf16", delta=1.0, temperature=1.0, seed=(11, B))
    lq = np.full(V, -30.0)
    lp = np.full(V, -30.0)
    y, z = 100 * 1024, 100
    lq[y] = lp[y] = 10.0
    lp[z] = 14.0
    to = w.target_offsets
    for b in range(B):
        w.target[to[b], :V] = bf16_bits_from_f64(lp)
        w.draft[b, :V] = bf16_bits_from_f64(lq)
    got = run_gpu(w)
    assert got["device_status"][0] == 0
    ref = run_oracle(w)
    assert np.all(np.abs(ref["rkl"] - 1.0) < 1e-3)  # the clipped term dominates
    s = compare(w, got, ref)
    _report(f"lane offset below a later slice, B={B}", s)


# ----------------------------------------------------------------------------- full-size workloads
def test_single_request_full_vocab():
    w = workload("single")
    dev = to_device(w)
    got = run_gpu(w, dev)
    assert got["device_status"][0] == 0
    s = compare(w, got, run_oracle(w))
    _report("single", s)
    # split rows fold their parts in a fixed order: bitwise deterministic too
    again = run_gpu(w, dev)
    for key in ("accept_len", "out_tokens", "rkl", "p_at_draft", "q_at_draft"):
        np.testing.assert_array_equal(got[key], again[key])


def test_ragged_batch_mixed_temperatures():
    w = workload("ragged")
    got = run_gpu(w)
    assert got["device_status"][0] == 0
    s = compare(w, got, run_oracle(w))
    _report("ragged B=32", s)
    assert len(s["flips"]) <= 2


@pytest.fixture(scope="module")
def high_concurrency():
    return workload("high_concurrency")


@pytest.fixture(scope="module")
def large_vocab():
    return workload("large_vocab")


def test_high_concurrency_full_size_all_requests(high_concurrency):
    w = high_concurrency
    dev = to_device(w)
    got = run_gpu(w, dev)
    assert got["device_status"][0] == 0
    assert np.all((got["accept_len"] >= 0) & (got["accept_len"] <= 15))
    # every request against the oracle (run in parallel worker processes)
    s = compare(w, got, oracle_refs(w))
    _report("high concurrency, all 128 requests", s)
    assert s["exact"] + len(s["flips"]) == w.B
    # bitwise determinism at full size
    again = run_gpu(w, dev)
    for key in ("accept_len", "out_tokens", "rkl", "p_at_draft", "q_at_draft"):
        np.testing.assert_array_equal(got[key], again[key])


def test_large_vocab_full_size_all_requests(large_vocab):
    w = large_vocab
    got = run_gpu(w)
    assert got["device_status"][0] == 0
    aa, fr = w.meta["all_accept"], w.meta["first_reject"]
    for b in aa:
        assert got["accept_len"][b] == 15
        d0 = int(w.draft_offsets[b])
        assert np.all(got["rkl"][d0: d0 + 15] == 0.0)
    for b in fr:
        assert got["accept_len"][b] == 0
    s = compare(w, got, oracle_refs(w))
    _report("large vocab, all 128 requests", s)
    assert s["exact"] + len(s["flips"]) == w.B


# ----------------------------------------------------------------------------- edge cases
def test_all_accept_and_bonus():
    w = make_workload(B=2, k=[6, 15], V=3000, dtype="bf16", temperature=[1.0, 0.7],
                      all_accept=(0, 1), seed=(5,))
    got = run_gpu(w)
    assert list(got["accept_len"]) == [6, 15]
    assert np.all(got["rkl"] == 0.0)
    compare(w, got, run_oracle(w))


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_residual_emptied_by_rounding(T):
    # A draft row equal to its target row except at the draft token, one bf16 step higher
    # at a logit of -30: the token is rejected (ratio e^(-0.125/T)), and the residual
    # max(0, p - q) is zero at every id in fp32 (the normalisers agree to the last bit),
    # so the draw falls back to p_T of the same row.  Four ids carry all of p's mass, so
    # the draw's outcome is fixed by the uniform; the oracle reaches the same id.
    from synth import bf16_bits_from_f64, bf16_bits_to_f32

    w = make_workload(B=1, k=[3], V=5003, dtype="bf16", s=3.0, sigma=0.0,
                      temperature=[T], seed=(12, int(T * 10)))
    V, rej, x = w.V, 1, 10
    row = np.full(V, -30.0)
    row[[100, 2000, 3500, 4900]] = [0.0, -0.5, -1.0, -2.0]
    w.target[rej, :V] = bf16_bits_from_f64(row)
    for i in range(3):
        w.draft[i, :V] = w.target[i, :V]  # equal rows: p_T(x)/q_T(x) = 1, accepted
    w.draft_tokens[rej] = x
    w.draft[rej, x] = bf16_bits_from_f64(np.array([-29.875]))[0]
    assert bf16_bits_to_f32(w.draft[rej, x:x + 1])[0] == -29.875
    got, ref = None, None
    for u in (0.05, 0.5, 0.8, 0.97):
        w.uniforms[:] = 0.5
        w.uniforms[rej] = 0.9999
        w.uniforms[3] = u  # slot k drives the final draw
        got = run_gpu(w)
        ref = run_oracle(w)
        assert got["device_status"][0] == 0
        assert got["accept_len"][0] == rej
        s = compare(w, got, ref)
        assert s["exact"] == 1, (u, got["out_tokens"])
        assert got["out_tokens"][rej] in (100, 2000, 3500, 4900)


def test_greedy_trace(golden_dir):
    with open(os.path.join(golden_dir, "dflash_notes_greedy_trace.json")) as f:
        g = json.load(f)
    w = make_workload(B=1, k=[g["block_drafts"]], V=3001, dtype="bf16", temperature=0.0,
                      seed=(6,))
    tgt = w.rows_f32("target", slice(0, 16)).astype(np.float64)
    argmax_p = np.argmax(tgt, axis=1)
    x = argmax_p[:15].copy()
    for i, match in enumerate(g["match_pattern_prefix"]):
        if not match:
            x[i] = (argmax_p[i] + 1) % w.V
    w.draft_tokens[:] = x
    got = run_gpu(w)
    assert got["accept_len"][0] == g["expected_accept_len"]
    toks = got["out_tokens"]
    assert int(np.count_nonzero(toks >= 0)) == g["expected_tokens_emitted"]
    assert toks[4] == argmax_p[4]


def test_invalid_requests_are_flagged_not_fatal():
    w = make_workload(B=4, k=[2, 3, 2, 1], V=500, dtype="f32", seed=(7,))
    w.draft_tokens[2] = 500  # request 1: token out of range
    w.temperature[2] = -1.0  # request 2: negative temperature
    w.uniforms[-1] = 1.0  # request 3: uniform out of range
    got = run_gpu(w)
    st = int(got["device_status"][0])
    assert st & 4 and st & 8 and st & 16 and not (st & 3)
    assert list(got["accept_len"][1:]) == [-1, -1, -1]
    ref = run_oracle(w, requests=[0])
    compare(w, got, ref, requests=[0])
    assert np.all(np.isfinite(got["rkl"]))  # the divergence does not depend on tokens


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_temperature_limits(dtype):
    # T_b = 2^-10, the smallest accepted temperature, against the oracle; positive
    # temperatures below it (1e-9, a subnormal) are flagged and only their request is void
    w = make_workload(B=4, k=[3, 4, 2, 5], V=3001, dtype=dtype, s=3.0, sigma=0.05,
                      temperature=[2.0**-10, 1e-9, 1.0, 1e-40], seed=(21, dtype == "bf16"))
    got = run_gpu(w)
    st = int(got["device_status"][0])
    assert st == 8, st
    assert got["accept_len"][1] == -1 and got["accept_len"][3] == -1
    s = compare(w, got, run_oracle(w, requests=[0, 2]), requests=[0, 2])
    _report(f"temperature limits {dtype}", s)
    assert s["exact"] + len(s["flips"]) == 2


def test_void_calls():
    w = make_workload(B=3, k=[2, 2, 2], V=300, dtype="bf16", seed=(8,))
    bad = w.k.copy()
    bad[1] = 0  # k_b outside [1, k_max]
    dev = to_device(w)
    dev["k"] = torch.from_numpy(bad).cuda()
    got = run_gpu(w, dev, k_max=4)
    assert int(got["device_status"][0]) & 1
    assert np.all(got["accept_len"] == -1) and np.all(got["out_tokens"] == -1)
    assert np.all(np.isnan(got["rkl"]))
    mism = w.k.copy()
    mism[1] = 3  # sum k_b != rows packed
    dev["k"] = torch.from_numpy(mism).cuda()
    got = run_gpu(w, dev, k_max=4)
    assert int(got["device_status"][0]) & 2
    assert np.all(got["accept_len"] == -1)


# One workspace through a call whose rows leave heavy lanes to the draw launch (records with
# lanes), a void call (every record must then read as empty, so that the draw's per-row
# workgroups leave the NaN outputs alone), and the first call again.  B = 4: split rows;
# B = 40: one workgroup per row.
@pytest.mark.parametrize("B", [4, 40])
def test_void_call_after_heavy_rows_on_one_workspace(B):
    import draft_block_verification_sv_amd as pkg

    w = _heavy_lane_workload("bf16", B, (32, B))
    ws = pkg.alloc_workspace(pkg.workspace_size(B, w.k_max, w.V, pkg.SV_BF16), "cuda")
    dev = to_device(w)
    ref = run_oracle(w, delta=1.0)
    first = run_gpu(w, dev, delta=1.0, workspace=ws)
    compare(w, first, ref)
    bad = w.k.copy()
    bad[1] = 0  # k_b outside [1, k_max]: the whole call is void
    dev_bad = dict(dev)
    dev_bad["k"] = torch.from_numpy(bad).cuda()
    got = run_gpu(w, dev_bad, delta=1.0, workspace=ws)
    assert int(got["device_status"][0]) & 1
    assert np.all(got["accept_len"] == -1) and np.all(got["out_tokens"] == -1)
    assert np.all(np.isnan(got["rkl"]))
    again = run_gpu(w, dev, delta=1.0, workspace=ws)
    compare(w, again, ref)
    assert np.array_equal(again["rkl"].view(np.uint32), first["rkl"].view(np.uint32))


def test_workspace_reuse_between_shapes():
    import draft_block_verification_sv_amd as pkg

    big = make_workload(B=4, k=[5, 5, 5, 5], V=6000, dtype="bf16", seed=(9,))
    small = make_workload(B=2, k=[1, 4], V=6000, dtype="bf16", seed=(10,))
    ws = pkg.alloc_workspace(pkg.workspace_size(4, 5, 6000, pkg.SV_BF16), "cuda")
    a = run_gpu(big, workspace=ws)
    b = run_gpu(small, workspace=ws)
    compare(big, a, run_oracle(big))
    compare(small, b, run_oracle(small))


# ----------------------------------------------------------------------------- standalone rKL
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_clipped_rkl_standalone(dtype):
    import draft_block_verification_sv_amd as pkg

    w = make_workload(B=3, k=[3, 2, 4], V=7001, dtype=dtype, sigma=1.5, outlier_frac=0.1,
                      seed=(11,))
    d = to_device(w)
    rng = np.random.default_rng(0)
    idx = rng.integers(0, w.n_target_rows, size=w.n_draft_rows).astype(np.int32)
    for delta in (1.0, 0.01):
        out, st = pkg.clipped_rkl(d["target"], d["draft"], delta,
                                  torch.from_numpy(idx).cuda())
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        got = out.cpu().numpy().astype(np.float64)
        import oracle

        tl = oracle.widen_logits(w.target[:, : w.V], dtype)
        dl = oracle.widen_logits(w.draft[:, : w.V], dtype)
        for r in range(w.n_draft_rows):
            ref = oracle.clipped_rkl_row(tl[idx[r]], dl[r], delta)
            tol = 1e-5 * max(abs(ref["R"]), ref["L1"]) + RKL_ABS
            assert abs(got[r] - ref["R"]) <= tol, (r, got[r], ref["R"])
    # out-of-range pairing is flagged and gives NaN for that row only
    idx[0] = w.n_target_rows
    out, st = pkg.clipped_rkl(d["target"], d["draft"], 1.0, torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    assert int(st.item()) & 2
    o = out.cpu().numpy()
    assert np.isnan(o[0]) and np.all(np.isfinite(o[1:]))


def _both_meet_the_bar(w, idx, delta, standalone, fused):
    import oracle

    tl = oracle.widen_logits(w.target[:, : w.V], w.dtype)
    dl = oracle.widen_logits(w.draft[:, : w.V], w.dtype)
    for r in range(len(idx)):
        ref = oracle.clipped_rkl_row(tl[idx[r]], dl[r], delta)
        tol = RTOL * max(abs(ref["R"]), ref["L1"]) + RKL_ABS
        for name, v in (("standalone", standalone), ("fused", fused)):
            assert abs(float(v[r]) - ref["R"]) <= tol, (name, r, float(v[r]), ref["R"])


def test_fused_rkl_and_standalone():
    import draft_block_verification_sv_amd as pkg

    w = make_workload(B=4, k=[3, 1, 5, 2], V=9000, dtype="bf16", seed=(12,))
    d = to_device(w)
    got = run_gpu(w, d)
    # standalone with the verification pairing: draft row of request b, position i -> target
    # row off_t[b] + i
    idx = np.concatenate([np.arange(w.target_offsets[b], w.target_offsets[b] + w.k[b])
                          for b in range(w.B)]).astype(np.int32)
    out, _ = pkg.clipped_rkl(d["target"], d["draft"], w.delta, torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    _both_meet_the_bar(w, idx, w.delta, out.cpu().numpy(), got["rkl"])


# ----------------------------------------------------------------------------- split rows
# Launches of a few rows split each row over several workgroups (parts); the part of a row
# that arrives last folds the parts' lane records.  V = 70001: 69 slices, so 8 parts per row,
# the last slice ragged.
@pytest.mark.parametrize("dtype,ld", [("bf16", 70001), ("f32", 70004)])
def test_split_rows_parity(dtype, ld):
    w = make_workload(B=4, k=[3, 1, 5, 2], V=70001, ld=ld, dtype=dtype, s=3.0,
                      sigma=[0.5, 1.0, 2.0, 0.8], temperature=[1.0, 0.0, 0.7, 1.3], delta=0.05,
                      outlier_frac=0.05, seed=(13, ld))
    got = run_gpu(w)
    assert got["device_status"][0] == 0
    s = compare(w, got, run_oracle(w))
    _report(f"split {dtype} ld={ld}", s)
    assert s["exact"] >= w.B - 1


# Small launches split their rows, by rows (n) and parts per row (P): more than 8 parts fold
# each part's four waves into 64 lanes, fewer keep 256; launches of up to about one and of
# about two workgroups per CU.  V = 70001 (69 slices, ragged): P = 8; V = 140001 (137 slices):
# P = 16.
@pytest.mark.parametrize("case", [
    ("folded, 13 rows", 140001, [6, 5], "bf16"),                # n = 13, P = 16: 208 WGs
    ("folded, 27 rows", 140001, [9, 7, 8], "bf16"),             # n = 27, P = 16: 432 WGs
    ("folded, 25 rows f32", 140004, [4, 9, 2, 6], "f32"),       # n = 25, P = 16
    ("unfolded, 40 rows", 70001, [7, 7, 7, 7, 7], "bf16"),      # n = 40, P = 8: 320 WGs
])
def test_split_regimes(case):
    name, V, k, dtype = case
    B = len(k)
    w = make_workload(B=B, k=k, V=V, dtype=dtype, s=3.0, sigma=[0.5, 1.0, 2.0, 0.8, 1.4][:B],
                      temperature=[1.0, 0.0, 0.7, 1.3, 1.0][:B], delta=0.05, outlier_frac=0.05,
                      seed=(15, V, B))
    got = run_gpu(w)
    assert got["device_status"][0] == 0
    s = compare(w, got, run_oracle(w))
    _report(f"split {name}", s)
    assert s["exact"] >= w.B - 1


def test_split_rows_standalone_and_fused():
    import draft_block_verification_sv_amd as pkg
    import oracle

    w = make_workload(B=4, k=[3, 1, 5, 2], V=70001, dtype="bf16", sigma=1.2, outlier_frac=0.1,
                      seed=(14,))
    d = to_device(w)
    got = run_gpu(w, d)
    idx = np.concatenate([np.arange(w.target_offsets[b], w.target_offsets[b] + w.k[b])
                          for b in range(w.B)]).astype(np.int32)
    out, st = pkg.clipped_rkl(d["target"], d["draft"], w.delta, torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    # the same pairing: both meet the bar (the verification call sums its heavy lanes in the
    # draw launch, the standalone call in its finalize)
    _both_meet_the_bar(w, idx, w.delta, out.cpu().numpy(), got["rkl"])
    tl = oracle.widen_logits(w.target[:, : w.V], "bf16")
    dl = oracle.widen_logits(w.draft[:, : w.V], "bf16")
    for delta in (1.0, 0.01):
        out, st = pkg.clipped_rkl(d["target"], d["draft"], delta, torch.from_numpy(idx[::-1].copy()).cuda())
        torch.cuda.synchronize()
        o = out.cpu().numpy().astype(np.float64)
        for r in range(w.n_draft_rows):
            ref = oracle.clipped_rkl_row(tl[idx[::-1][r]], dl[r], delta)
            tol = 1e-5 * max(abs(ref["R"]), ref["L1"]) + RKL_ABS
            assert abs(o[r] - ref["R"]) <= tol, (delta, r, o[r], ref["R"])
    # an out-of-range pairing gives NaN for that row only
    bad = idx.copy()
    bad[3] = -1
    out, st = pkg.clipped_rkl(d["target"], d["draft"], 1.0, torch.from_numpy(bad).cuda())
    torch.cuda.synchronize()
    assert int(st.item()) & 2
    o = out.cpu().numpy()
    assert np.isnan(o[3]) and np.all(np.isfinite(np.delete(o, 3)))


# ----------------------------------------------------------------------------- layouts
def test_large_batch_uses_the_plan():
    # more than 2048 requests: per-row descriptors come from the plan kernel
    B = 2100
    rng = np.random.default_rng(15)
    w = make_workload(B=B, k=rng.integers(1, 4, size=B), V=300, dtype="bf16", s=3.0,
                      sigma=0.8, temperature=rng.choice([0.0, 0.7, 1.0], size=B), delta=0.5,
                      seed=(15,))
    got = run_gpu(w)
    assert got["device_status"][0] == 0
    s = compare(w, got, run_oracle(w))
    _report("B=2100 (plan)", s)
    # a bad length voids the call on this path too
    dev = to_device(w)
    bad = w.k.copy()
    bad[B - 1] = 0
    dev["k"] = torch.from_numpy(bad).cuda()
    got = run_gpu(w, dev)
    assert int(got["device_status"][0]) & 1
    assert np.all(got["accept_len"] == -1) and np.all(np.isnan(got["rkl"]))


def test_invalid_token_in_split_rows():
    # 7 rows of 40 slices split into parts: the token check happens in the finalize
    w = make_workload(B=2, k=[3, 2], V=40000, dtype="bf16", temperature=[1.0, 0.7], seed=(16,))
    w.draft_tokens[1] = -5  # request 0
    got = run_gpu(w)
    st = int(got["device_status"][0])
    assert st & 4 and not (st & 3)
    assert got["accept_len"][0] == -1 and got["accept_len"][1] >= 0
    compare(w, got, run_oracle(w, requests=[1]), requests=[1])
    assert np.all(np.isfinite(got["rkl"]))


def test_workspace_without_split_records():
    # a workspace sized for B=128 has no room for the lane records of split rows: a one-request
    # call on it streams each row in one workgroup and still matches the oracle; the same holds
    # for the standalone reverse-KL on a workspace sized for 129 rows
    import draft_block_verification_sv_amd as pkg
    import oracle

    w = workload("single")
    big = pkg.workspace_size(128, 15, w.V, pkg.SV_BF16)
    assert big < pkg.workspace_size(1, 15, w.V, pkg.SV_BF16)
    ws = pkg.alloc_workspace(big, "cuda:0")
    d = to_device(w)
    got = run_gpu(w, d, workspace=ws)
    assert got["device_status"][0] == 0
    s = compare(w, got, run_oracle(w))
    _report("single on a B=128 workspace", s)
    n = w.n_draft_rows
    idx = torch.from_numpy(np.arange(n, dtype=np.int32)).cuda()
    wsr = pkg.alloc_workspace(int(pkg.lib().sv_rkl_workspace_size(129, w.V, pkg.SV_BF16)), "cuda:0")
    assert wsr.numel() < int(pkg.lib().sv_rkl_workspace_size(n, w.V, pkg.SV_BF16))
    out, st = pkg.clipped_rkl(d["target"], d["draft"], w.delta, idx, workspace=wsr)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    tl = oracle.widen_logits(w.target[:, : w.V], "bf16")
    dl = oracle.widen_logits(w.draft[:, : w.V], "bf16")
    o = out.cpu().numpy().astype(np.float64)
    for r in range(n):
        ref = oracle.clipped_rkl_row(tl[r], dl[r], w.delta)
        assert abs(o[r] - ref["R"]) <= 1e-5 * max(abs(ref["R"]), ref["L1"]) + RKL_ABS, r


# ----------------------------------------------------------------------------- maximum length
def test_maximum_draft_length():
    # k_b = k_max = 64: 65 target rows per request, one more than a wavefront has lanes.  An
    # all-accepted sampled request (its bonus row is row 64), an all-accepted greedy request, a
    # sampled request with rejections, and a short one
    w = make_workload(B=4, k=[64, 64, 64, 7], V=3001, dtype="bf16",
                      temperature=[1.0, 0.0, 0.7, 1.0], all_accept=(0, 1), k_max=64, seed=(17,))
    got = run_gpu(w)
    assert got["device_status"][0] == 0
    assert got["accept_len"][0] == 64 and got["accept_len"][1] == 64
    s = compare(w, got, run_oracle(w))
    _report("k_b = 64", s)


def test_maximum_draft_length_split_rows():
    # one request of 64 drafts at V=40000: 65 rows, streamed in parts
    w = make_workload(B=1, k=[64], V=40000, dtype="bf16", all_accept=(0,), k_max=64, seed=(18,))
    got = run_gpu(w)
    assert got["device_status"][0] == 0 and got["accept_len"][0] == 64
    compare(w, got, run_oracle(w))


def test_maximum_vocabulary():
    # V = 524288, the largest the library takes: 512 slices per row (split into 16 parts here),
    # 256 draw chunks, and with a small delta re-read rounds of four failing lanes
    w = make_workload(B=2, k=[2, 1], V=1 << 19, dtype="bf16", s=4.0, sigma=[0.5, 2.0],
                      temperature=[1.0, 0.7], delta=0.01, outlier_frac=0.02, seed=(19,))
    got = run_gpu(w)
    assert got["device_status"][0] == 0
    s = compare(w, got, run_oracle(w))
    _report("V = 524288", s)


def test_maximum_batch():
    # B = 65536 requests (the largest the library takes) of one draft over a tiny vocabulary:
    # 131072 row pairs and bonus rows laid out by the plan kernel
    B = 1 << 16
    rng = np.random.default_rng(20)
    w = make_workload(B=B, k=1, V=16, dtype="bf16", s=2.0, sigma=0.7,
                      temperature=rng.choice([0.0, 0.7, 1.0], size=B), delta=0.3, seed=(20,))
    got = run_gpu(w)
    assert got["device_status"][0] == 0
    s = compare(w, got, run_oracle(w))
    _report("B = 65536", s)
