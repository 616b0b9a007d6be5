"""The C ABI on the CPU: the library loads, exports every declared symbol, and rejects
host-checkable argument errors synchronously without touching the device."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    import draft_block_verification_sv_amd as pkg

    if not os.path.exists(pkg.library_path()):
        pytest.skip("libspecverify.so not built (run __graft_entry__.build())")
    return pkg.lib()


def test_header_declares_the_boundary():
    fns = _declared_functions()
    for f in ("sv_verify_block", "sv_clipped_rkl", "sv_workspace_size", "sv_status_string"):
        assert f in fns


def test_every_declared_symbol_is_exported(L):
    raw = ctypes.CDLL(L._name)
    missing = [f for f in _declared_functions() if not hasattr(raw, f)]
    assert not missing, missing


def test_status_strings(L):
    for s in range(7):
        assert L.sv_status_string(s)
    assert b"unknown" in L.sv_status_string(99)


def test_workspace_size(L):
    assert L.sv_workspace_size(128, 15, 151936, 0) > 0
    assert L.sv_workspace_size(0, 15, 100, 0) == 0
    assert L.sv_workspace_size(1, 0, 100, 0) == 0
    assert L.sv_workspace_size(1, 65, 100, 0) == 0
    assert L.sv_workspace_size(1, 4, 100, 7) == 0
    assert L.sv_rkl_workspace_size(10, 1000, 1) > 0
    assert L.sv_rkl_workspace_size(0, 1000, 1) == 0


NULL6 = [None] * 6


def _verify(L, dtype=0, B=1, k_max=4, V=100, ld_t=100, ld_d=100, n_d=1, ptrs=None, delta=1.0,
            outs=None, ws=None, ws_bytes=0):
    ptrs = ptrs if ptrs is not None else [8] * 5 + [None]  # fake, never dereferenced
    outs = outs if outs is not None else [8, 8, None, None, None, 8]
    return L.sv_verify_block(dtype, B, k_max, V, ld_t, ld_d, n_d, *ptrs, delta, *outs, ws,
                             ws_bytes, None)


def test_verify_argument_errors(L):
    big = 1 << 40
    assert _verify(L, dtype=3) == 3  # dtype
    assert _verify(L, B=0) == 2
    assert _verify(L, k_max=0) == 2
    assert _verify(L, k_max=65) == 2
    assert _verify(L, V=0) == 2
    assert _verify(L, ld_t=99) == 2
    assert _verify(L, ld_d=50) == 2
    assert _verify(L, n_d=0) == 2  # fewer draft rows than requests
    assert _verify(L, n_d=5) == 2  # more than B * k_max
    assert _verify(L, ptrs=[None, 8, 8, 8, 8, None]) == 1
    assert _verify(L, outs=[8, None, None, None, None, 8]) == 1
    assert _verify(L, outs=[8, 8, None, None, None, None]) == 1  # device_status is required
    assert _verify(L, outs=[8, 8, 8, None, None, 8], delta=float("nan")) == 4
    assert _verify(L, outs=[8, 8, 8, None, None, 8], delta=0.0) == 4
    assert _verify(L, ws=None, ws_bytes=big) == 5  # no workspace
    assert _verify(L, ws=256 * 3 + 8, ws_bytes=big) == 5  # misaligned
    assert _verify(L, ws=256 * 4, ws_bytes=16) == 5  # too small


def test_noalloc_argument_errors(L):
    # every host-checkable problem is reported before the fixed scratch is looked up (no GPU
    # here: any HIP call would fail with SV_ERR_HIP instead)
    def call(dtype=0, B=1, k_max=4, V=100, n_d=1, ptrs=None, outs=None, delta=1.0):
        ptrs = ptrs if ptrs is not None else [8] * 5 + [None]
        outs = outs if outs is not None else [8, 8, None, None, None, 8]
        return L.sv_verify_block_noalloc(dtype, B, k_max, V, V, V, n_d, *ptrs, delta, *outs, None)

    assert call(dtype=3) == 3
    assert call(B=0) == 2
    assert call(k_max=65) == 2
    assert call(n_d=5) == 2
    assert call(ptrs=[None, 8, 8, 8, 8, None]) == 1
    assert call(outs=[8, 8, None, None, None, None]) == 1
    assert call(outs=[8, 8, 8, None, None, 8], delta=float("nan")) == 4
    assert L.sv_status_string(7).decode().startswith("the call needs more scratch")


def test_rkl_argument_errors(L):
    def call(dtype=1, n=2, nt=2, V=10, ldt=10, ldd=10, tp=8, dp=8, idx=None, delta=1.0, out=8,
             st=8, ws=None, wsb=0):
        return L.sv_clipped_rkl(dtype, n, nt, V, ldt, ldd, tp, dp, idx, delta, out, st, ws, wsb,
                                None)

    assert call(dtype=9) == 3
    assert call(n=0) == 2
    assert call(nt=1) == 2  # identity pairing needs n_target_rows >= n_rows
    assert call(ldd=9) == 2
    assert call(tp=None) == 1
    assert call(out=None) == 1
    assert call(delta=-1.0) == 4
    assert call(delta=float("inf")) == 4
    assert call(ws=None, wsb=1 << 30) == 5


def test_opd_argument_errors(L):
    def call(dtype=1, B=1, n=2, nt=2, V=10, ldt=10, ldd=10, tp=8, dp=8, idx=None, k=8,
             delta=1.0, alpha=0.8, rkl=8, hard=8, top1=None, opd=8, st=8, ws=None, wsb=0):
        return L.sv_opd_loss(dtype, B, n, nt, V, ldt, ldd, tp, dp, idx, k, delta, alpha, rkl,
                             hard, top1, opd, st, ws, wsb, None)

    assert call(hard=None) == 1
    assert call(k=None) == 1  # the per-request loss needs k
    assert call(B=0) == 2
    assert call(alpha=1.5) == 4
    assert call(alpha=float("nan")) == 4
    assert call(dtype=9) == 3
    assert call(n=0) == 2
    assert call(delta=0.0) == 4
    assert call(rkl=None) == 1
    assert call(ws=None, wsb=1 << 30) == 5
    assert call(k=None, opd=None, ws=None, wsb=1 << 30) == 5  # per-row outputs only: k optional


def test_opd_grad_argument_errors(L):
    def call(dtype=1, B=1, n=2, nt=2, V=10, ldt=10, ldd=10, tp=8, dp=8, idx=None, k=8,
             delta=1.0, alpha=0.8, rkl=8, hard=8, top1=None, opd=None, gdt=1, ldg=10, g=8,
             st=8, ws=None, wsb=0):
        return L.sv_opd_loss_grad(dtype, B, n, nt, V, ldt, ldd, tp, dp, idx, k, delta, alpha, rkl,
                                  hard, top1, opd, gdt, ldg, g, st, ws, wsb, None)

    assert call(g=None) == 1
    assert call(k=None) == 1
    assert call(hard=None) == 1
    assert call(ldg=9) == 2
    assert call(B=0) == 2
    assert call(gdt=7) == 3
    assert call(alpha=-0.1) == 4
    assert call(delta=float("nan")) == 4
    assert call(ws=None, wsb=1 << 30) == 5
    assert L.sv_opd_grad_workspace_size(2, 10, 1) > L.sv_rkl_workspace_size(2, 10, 1)
    assert L.sv_opd_grad_workspace_size(0, 10, 1) == 0


def test_greedy_argument_errors(L):
    def call(dtype=1, B=1, kmax=2, V=10, ldt=10, nd=2, tp=8, k=8, tok=8, al=8, ot=8, st=8,
             ws=None, wsb=0):
        return L.sv_verify_block_greedy(dtype, B, kmax, V, ldt, nd, tp, k, tok, al, ot, st, ws,
                                        wsb, None)

    assert call(dtype=5) == 3
    assert call(B=0) == 2
    assert call(kmax=65) == 2
    assert call(ldt=9) == 2
    assert call(nd=3) == 2  # more draft rows than B * k_max
    assert call(tp=None) == 1
    assert call(tok=None) == 1
    assert call(st=None) == 1
    assert call(ws=None, wsb=1 << 30) == 5


def test_length_head_argument_errors(L):
    def call(B=2, k=4, H=64, Hf=16, h=16, ldh=64, W1=16, ldw=64, b1=None, w2=16, b2=0.0,
             gamma=1.0, ah=16, kh=16, off=None, ws=None, wsb=0):
        return L.sv_length_head(B, k, H, Hf, h, ldh, W1, ldw, b1, w2, b2, gamma, ah, kh, off, ws,
                                wsb, None)

    assert call(H=48) == 2  # not a multiple of 32
    assert call(k=65) == 2
    assert call(Hf=0) == 2
    assert call(ldh=60) == 2
    assert call(ldw=68 + 2) == 2  # not a multiple of 8
    assert call(h=None) == 1
    assert call(w2=None) == 1
    assert call(h=8) == 2  # not 16-byte aligned
    assert call(gamma=0.0) == 4
    assert call(ws=None, wsb=1 << 30) == 5
    assert L.sv_length_head_workspace_size(4, 15, 4096, 256) >= 4 * 16 * 256 * 4
    assert L.sv_length_head_workspace_size(4, 65, 4096, 256) == 0
    assert L.sv_length_head_workspace_size(4, 15, 48, 256) == 0
    assert L.sv_length_loss(0, 8, 8, 8, 8, None, None) == 2
    assert L.sv_length_loss(2, None, 8, 8, 8, None, None) == 1


def test_branch_lookup_argument_errors(L):
    def call(B=2, k_max=15, n_branch=24, n_tokens=32, k=16, al=16, out=16, pos=16, tok=16, hit=16):
        return L.sv_branch_lookup(B, k_max, n_branch, n_tokens, k, al, out, pos, tok, hit, None)

    assert call(B=0) == 2
    assert call(k_max=65) == 2
    assert call(n_branch=0) == 2
    assert call(n_branch=4097) == 2
    assert call(n_tokens=0) == 2
    assert call(k=None) == 1
    assert call(out=None) == 1
    assert call(tok=None) == 1
    assert call(hit=None) == 1


def test_tree_argument_errors(L):
    def call(dtype=0, B=2, mx=60, V=1000, ld=1000, n=10, tgt=16, nn=16, par=16, tok=16, al=16,
             out=16, nodes=None, st=16, ws=None, wsb=0):
        return L.sv_verify_tree_greedy(dtype, B, mx, V, ld, n, tgt, nn, par, tok, al, out, nodes, st,
                                       ws, wsb, None)

    assert call(dtype=7) == 3
    assert call(B=0) == 2
    assert call(mx=1025) == 2
    assert call(n=1) == 2  # fewer nodes than requests
    assert call(n=200) == 2  # more than B * max_nodes
    assert call(ld=999) == 2
    assert call(tgt=None) == 1
    assert call(par=None) == 1
    assert call(st=None) == 1
    assert call(ws=None, wsb=1 << 30) == 5
    assert L.sv_tree_workspace_size(2, 10) >= 12 * 4
    assert L.sv_tree_workspace_size(2, 1) == 0


def test_read_probe_argument_errors(L):
    # fake pointers, never dereferenced: every case fails on the host
    assert L.sv_read_probe(None, 1024, 16, None) == 1
    assert L.sv_read_probe(16, 1024, None, None) == 1
    assert L.sv_read_probe(16, 0, 16, None) == 2
    assert L.sv_read_probe(16, 1000, 16, None) == 2  # not a multiple of 16
    assert L.sv_read_probe(8, 1024, 16, None) == 4  # not 16-byte aligned


def test_split_records_are_optional_in_the_workspace(L):
    # calls of at most 128 rows reserve lane records for split rows; larger calls do not
    small = L.sv_workspace_size(1, 15, 151936, 0)
    big = L.sv_workspace_size(128, 15, 151936, 0)
    assert small > big > 0
    assert L.sv_rkl_workspace_size(15, 151936, 0) > L.sv_rkl_workspace_size(129, 151936, 0) > 0
    # short rows never split
    assert L.sv_rkl_workspace_size(15, 4096, 0) < 64 * 1024
