"""Python binding of libspecverify: argument marshalling only.

Every step of the verification runs in the library's HIP kernels; this module
checks tensor shapes (the C ABI trusts its caller for buffer extents), passes raw
device pointers and the current HIP stream, and allocates outputs.  There is no
fallback: if the library is not built, or a tensor is not on the GPU, calls raise.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspecverify.so")
_lib = None

SV_BF16, SV_F32 = 0, 1
SV_DEV_BAD_LENGTH, SV_DEV_ROWS_MISMATCH, SV_DEV_BAD_TOKEN = 1, 2, 4
SV_DEV_BAD_TEMPERATURE, SV_DEV_BAD_UNIFORM = 8, 16
SV_MAX_K = 64

_c_i32, _c_i64, _c_f32, _c_sz, _c_p = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                       ctypes.c_size_t, ctypes.c_void_p)


class SpecVerifyError(RuntimeError):
    pass


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise SpecVerifyError(f"{_LIB_PATH} is not built: run `python __graft_entry__.py` "
                              "or draft_block_verification_sv_amd.build.build_library()")
    L = ctypes.CDLL(_LIB_PATH)
    L.sv_workspace_size.argtypes = [_c_i32, _c_i32, _c_i64, _c_i32]
    L.sv_workspace_size.restype = _c_sz
    L.sv_rkl_workspace_size.argtypes = [_c_i64, _c_i64, _c_i32]
    L.sv_rkl_workspace_size.restype = _c_sz
    L.sv_verify_block.argtypes = [_c_i32, _c_i32, _c_i32, _c_i64, _c_i64, _c_i64, _c_i64,
                                  _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_f32,
                                  _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]
    L.sv_verify_block.restype = _c_i32
    L.sv_verify_block_noalloc.argtypes = [_c_i32, _c_i32, _c_i32, _c_i64, _c_i64, _c_i64, _c_i64,
                                          _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_f32,
                                          _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p]
    L.sv_verify_block_noalloc.restype = _c_i32
    L.sv_clipped_rkl.argtypes = [_c_i32, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_p,
                                 _c_p, _c_f32, _c_p, _c_p, _c_p, _c_sz, _c_p]
    L.sv_clipped_rkl.restype = _c_i32
    L.sv_opd_loss.argtypes = [_c_i32, _c_i32, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_p,
                              _c_p, _c_p, _c_f32, _c_f32, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                              _c_sz, _c_p]
    L.sv_opd_loss.restype = _c_i32
    L.sv_length_head_workspace_size.argtypes = [_c_i32, _c_i32, _c_i32, _c_i32]
    L.sv_length_head_workspace_size.restype = _c_sz
    L.sv_length_head.argtypes = [_c_i32, _c_i32, _c_i32, _c_i32, _c_p, _c_i64, _c_p, _c_i64, _c_p,
                                 _c_p, _c_f32, _c_f32, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]
    L.sv_length_head.restype = _c_i32
    L.sv_length_loss.argtypes = [_c_i32, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p]
    L.sv_length_loss.restype = _c_i32
    L.sv_verify_block_greedy.argtypes = [_c_i32, _c_i32, _c_i32, _c_i64, _c_i64, _c_i64, _c_p,
                                         _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]
    L.sv_verify_block_greedy.restype = _c_i32
    L.sv_opd_grad_workspace_size.argtypes = [_c_i64, _c_i64, _c_i32]
    L.sv_opd_grad_workspace_size.restype = _c_sz
    L.sv_opd_loss_grad.argtypes = [_c_i32, _c_i32, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_p,
                                   _c_p, _c_p, _c_p, _c_f32, _c_f32, _c_p, _c_p, _c_p, _c_p,
                                   _c_i32, _c_i64, _c_p, _c_p, _c_p, _c_sz, _c_p]
    L.sv_opd_loss_grad.restype = _c_i32
    L.sv_tree_workspace_size.argtypes = [_c_i32, _c_i64]
    L.sv_tree_workspace_size.restype = _c_sz
    L.sv_verify_tree_greedy.argtypes = [_c_i32, _c_i32, _c_i32, _c_i64, _c_i64, _c_i64, _c_p, _c_p,
                                        _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]
    L.sv_verify_tree_greedy.restype = _c_i32
    L.sv_branch_lookup.argtypes = [_c_i32, _c_i32, _c_i32, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p,
                                   _c_p, _c_p]
    L.sv_branch_lookup.restype = _c_i32
    L.sv_status_string.argtypes = [_c_i32]
    L.sv_status_string.restype = ctypes.c_char_p
    L.sv_version.argtypes = []
    L.sv_version.restype = ctypes.c_char_p
    L.sv_read_probe.argtypes = [_c_p, _c_i64, _c_p, _c_p]
    L.sv_read_probe.restype = _c_i32
    L.sv_profile_enable.argtypes = [_c_i32]
    L.sv_profile_enable.restype = _c_i32
    L.sv_profile_reset.argtypes = []
    L.sv_profile_reset.restype = _c_i32
    L.sv_profile_count.argtypes = []
    L.sv_profile_count.restype = _c_i32
    L.sv_profile_get.argtypes = [_c_i32, ctypes.c_char_p, _c_sz, ctypes.POINTER(_c_i64),
                                 ctypes.POINTER(ctypes.c_double)]
    L.sv_profile_get.restype = _c_i32
    _lib = L
    return L


def _check(status: int, what: str):
    if status != 0:
        msg = lib().sv_status_string(status).decode()
        raise SpecVerifyError(f"{what}: status {status} ({msg})")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype, numel: int, device):
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous() or t.numel() != numel:
        raise ValueError(f"{name} must be contiguous with {numel} elements, got {tuple(t.shape)}")


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def version() -> str:
    return lib().sv_version().decode()


def workspace_size(B: int, k_max: int, V: int, dtype: int) -> int:
    return int(lib().sv_workspace_size(B, k_max, V, dtype))


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    """A 256-byte aligned device buffer (torch's caching allocator aligns to >= 512 B)."""
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    assert ws.data_ptr() % 256 == 0
    return ws


def verify_block(target: torch.Tensor, draft: torch.Tensor, k: torch.Tensor,
                 draft_tokens: torch.Tensor, uniforms: torch.Tensor,
                 temperature: Optional[torch.Tensor] = None, delta: float = 1.0, *,
                 k_max: Optional[int] = None, with_rkl: bool = True, with_probs: bool = True,
                 workspace: Optional[torch.Tensor] = None, out: Optional[dict] = None,
                 stream=None) -> dict:
    """Runs sv_verify_block on the current stream and returns its outputs as tensors.

    target [n_draft_rows + B, >= V] and draft [n_draft_rows, >= V] share the dtype
    (bfloat16 or float32); V is their column count and the row strides are their
    leading dimensions.  ``k_max`` defaults to the largest k_b the row count allows
    (no device read is needed for it).
    """
    dev = target.device
    if dev.type != "cuda":
        raise ValueError("target must be a GPU tensor")
    code = _dtype_code(target)
    if draft.dtype != target.dtype:
        raise TypeError("target and draft must share a dtype")
    if target.dim() != 2 or draft.dim() != 2 or target.stride(1) != 1 or draft.stride(1) != 1:
        raise ValueError("logits must be 2-D with unit column stride")
    B = int(k.numel())
    n_d = int(draft.shape[0])
    V = int(target.shape[1])
    if int(draft.shape[1]) != V or int(target.shape[0]) != n_d + B:
        raise ValueError(f"shapes: target {tuple(target.shape)} must be [n_draft_rows + B, V], "
                         f"draft {tuple(draft.shape)} [n_draft_rows, V], B = {B}")
    if k_max is None:
        k_max = max(1, min(SV_MAX_K, n_d - B + 1))
    _need(k, "k", torch.int32, B, dev)
    _need(draft_tokens, "draft_tokens", torch.int32, n_d, dev)
    _need(uniforms, "uniforms", torch.float32, n_d + B, dev)
    if temperature is not None:
        _need(temperature, "temperature", torch.float32, B, dev)
    if workspace is None:
        nbytes = workspace_size(B, k_max, V, code)
        if nbytes == 0:
            raise SpecVerifyError(f"invalid shape B={B} k_max={k_max} V={V}")
        workspace = alloc_workspace(nbytes, dev)
    if out is None:
        out = {
            "accept_len": torch.empty(B, dtype=torch.int32, device=dev),
            "out_tokens": torch.empty(n_d + B, dtype=torch.int32, device=dev),
            "rkl": torch.empty(n_d, dtype=torch.float32, device=dev) if with_rkl else None,
            "p_at_draft": torch.empty(n_d, dtype=torch.float32, device=dev) if with_probs else None,
            "q_at_draft": torch.empty(n_d, dtype=torch.float32, device=dev) if with_probs else None,
            "device_status": torch.empty(1, dtype=torch.int32, device=dev),
        }
    else:  # caller-provided outputs: the C ABI writes them without bounds, so check here
        _need(out["accept_len"], "accept_len", torch.int32, B, dev)
        _need(out["out_tokens"], "out_tokens", torch.int32, n_d + B, dev)
        for name in ("rkl", "p_at_draft", "q_at_draft"):
            if out.get(name) is not None:
                _need(out[name], name, torch.float32, n_d, dev)
        _need(out["device_status"], "device_status", torch.int32, 1, dev)
    st = lib().sv_verify_block(
        code, B, k_max, V, target.stride(0), draft.stride(0), n_d, _ptr(target), _ptr(draft),
        _ptr(k), _ptr(draft_tokens), _ptr(uniforms), _ptr(temperature), float(delta),
        _ptr(out["accept_len"]), _ptr(out["out_tokens"]), _ptr(out.get("rkl")),
        _ptr(out.get("p_at_draft")), _ptr(out.get("q_at_draft")), _ptr(out["device_status"]),
        _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "sv_verify_block")
    return out


def verify_block_greedy(target: torch.Tensor, k: torch.Tensor, draft_tokens: torch.Tensor, *,
                        k_max: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
                        out: Optional[dict] = None, stream=None) -> dict:
    """sv_verify_block_greedy: every request greedy; reads only the target logits
    [n_draft_rows + B, V].  Returns accept_len, out_tokens and device_status."""
    dev = target.device
    if dev.type != "cuda":
        raise ValueError("target must be a GPU tensor")
    code = _dtype_code(target)
    if target.dim() != 2 or target.stride(1) != 1:
        raise ValueError("target must be 2-D with unit column stride")
    B = int(k.numel())
    n_d = int(draft_tokens.numel())
    V = int(target.shape[1])
    if int(target.shape[0]) != n_d + B:
        raise ValueError(f"target {tuple(target.shape)} must have n_draft_rows + B rows")
    if k_max is None:
        k_max = max(1, min(SV_MAX_K, n_d - B + 1))
    _need(k, "k", torch.int32, B, dev)
    _need(draft_tokens, "draft_tokens", torch.int32, n_d, dev)
    if workspace is None:
        nbytes = workspace_size(B, k_max, V, code)
        if nbytes == 0:
            raise SpecVerifyError(f"invalid shape B={B} k_max={k_max} V={V}")
        workspace = alloc_workspace(nbytes, dev)
    if out is None:
        out = {
            "accept_len": torch.empty(B, dtype=torch.int32, device=dev),
            "out_tokens": torch.empty(n_d + B, dtype=torch.int32, device=dev),
            "device_status": torch.empty(1, dtype=torch.int32, device=dev),
        }
    else:
        _need(out["accept_len"], "accept_len", torch.int32, B, dev)
        _need(out["out_tokens"], "out_tokens", torch.int32, n_d + B, dev)
        _need(out["device_status"], "device_status", torch.int32, 1, dev)
    st = lib().sv_verify_block_greedy(code, B, k_max, V, target.stride(0), n_d, _ptr(target),
                                      _ptr(k), _ptr(draft_tokens), _ptr(out["accept_len"]),
                                      _ptr(out["out_tokens"]), _ptr(out["device_status"]),
                                      _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "sv_verify_block_greedy")
    return out


def length_head(h: torch.Tensor, W1: torch.Tensor, w2: torch.Tensor, b1=None, b2: float = 0.0,
                gamma: float = 1.0, *, workspace: Optional[torch.Tensor] = None,
                out: Optional[dict] = None, stream=None) -> dict:
    """sv_length_head: h bfloat16 [B, k, H] (unit stride along H), W1 bfloat16 [H', H], w2 and
    b1 float32 [H'].  Returns a_hat [B], k_hat [B] and the packed target-row offsets off_t."""
    dev = h.device
    if h.dtype != torch.bfloat16 or W1.dtype != torch.bfloat16:
        raise TypeError("h and W1 must be bfloat16")
    if h.dim() != 3 or W1.dim() != 2 or h.stride(2) != 1 or W1.stride(1) != 1:
        raise ValueError("h must be [B, k, H] and W1 [H', H], both with unit stride along H")
    B, k, H = (int(x) for x in h.shape)
    Hf = int(W1.shape[0])
    if int(W1.shape[1]) != H:
        raise ValueError("W1 must have H columns")
    if h.stride(0) != k * h.stride(1):
        raise ValueError("h's positions must be packed request by request (stride(0) = k stride(1))")
    _need(w2, "w2", torch.float32, Hf, dev)
    if b1 is not None:
        _need(b1, "b1", torch.float32, Hf, dev)
    if workspace is None:
        nbytes = int(lib().sv_length_head_workspace_size(B, k, H, Hf))
        if nbytes == 0:
            raise SpecVerifyError(f"invalid shape B={B} H'={Hf}")
        workspace = alloc_workspace(nbytes, dev)
    if out is None:
        out = {"a_hat": torch.empty(B, dtype=torch.float32, device=dev),
               "k_hat": torch.empty(B, dtype=torch.int32, device=dev),
               "off_t": torch.empty(B + 1, dtype=torch.int32, device=dev)}
    else:
        _need(out["a_hat"], "a_hat", torch.float32, B, dev)
        _need(out["k_hat"], "k_hat", torch.int32, B, dev)
        if out.get("off_t") is not None:
            _need(out["off_t"], "off_t", torch.int32, B + 1, dev)
    st = lib().sv_length_head(B, k, H, Hf, _ptr(h), h.stride(1), _ptr(W1), W1.stride(0), _ptr(b1),
                              _ptr(w2), float(b2), float(gamma), _ptr(out["a_hat"]),
                              _ptr(out["k_hat"]), _ptr(out.get("off_t")), _ptr(workspace),
                              workspace.numel(), _stream(stream))
    _check(st, "sv_length_head")
    return out


def length_loss(a_hat: torch.Tensor, accept_len: torch.Tensor, k_hat: torch.Tensor,
                stream=None) -> tuple:
    """sv_length_loss: (loss [B], dloss/da_hat [B])."""
    dev = a_hat.device
    B = int(a_hat.numel())
    _need(a_hat, "a_hat", torch.float32, B, dev)
    _need(accept_len, "accept_len", torch.int32, B, dev)
    _need(k_hat, "k_hat", torch.int32, B, dev)
    loss = torch.empty(B, dtype=torch.float32, device=dev)
    dloss = torch.empty(B, dtype=torch.float32, device=dev)
    _check(lib().sv_length_loss(B, _ptr(a_hat), _ptr(accept_len), _ptr(k_hat), _ptr(loss),
                                _ptr(dloss), _stream(stream)), "sv_length_loss")
    return loss, dloss


def branch_lookup(k: torch.Tensor, accept_len: torch.Tensor, out_tokens: torch.Tensor,
                  branch_pos: torch.Tensor, branch_tok: torch.Tensor, *, k_max: Optional[int] = None,
                  stream=None) -> torch.Tensor:
    """sv_branch_lookup: hit [B], the first prepared branch whose key (branch_pos, branch_tok;
    int32 [B, n_branch], token -1 = any) matches the verification outcome (accept_len, the
    token after the accepted drafts in the packed out_tokens), -1 for a miss."""
    dev = k.device
    B = int(k.numel())
    if branch_pos.dim() != 2 or int(branch_pos.shape[0]) != B:
        raise ValueError("branch_pos must be [B, n_branch]")
    n_branch = int(branch_pos.shape[1])
    _need(k, "k", torch.int32, B, dev)
    _need(accept_len, "accept_len", torch.int32, B, dev)
    _need(branch_pos, "branch_pos", torch.int32, B * n_branch, dev)
    _need(branch_tok, "branch_tok", torch.int32, B * n_branch, dev)
    n_tokens = int(out_tokens.numel())
    _need(out_tokens, "out_tokens", torch.int32, n_tokens, dev)
    if k_max is None:
        k_max = int(k.max().item())
    hit = torch.empty(B, dtype=torch.int32, device=dev)
    _check(lib().sv_branch_lookup(B, int(k_max), n_branch, n_tokens, _ptr(k), _ptr(accept_len),
                                  _ptr(out_tokens), _ptr(branch_pos), _ptr(branch_tok), _ptr(hit),
                                  _stream(stream)), "sv_branch_lookup")
    return hit


def verify_tree_greedy(target: torch.Tensor, n_nodes: torch.Tensor, parent: torch.Tensor,
                       tree_tokens: torch.Tensor, *, max_nodes: Optional[int] = None,
                       workspace: Optional[torch.Tensor] = None, out: Optional[dict] = None,
                       stream=None) -> dict:
    """sv_verify_tree_greedy: target [sum_b (n_b + 1), V] (bf16 or fp32, unit column stride;
    request b's rows are its root then its nodes), n_nodes int32 [B], parent and tree_tokens
    int32 [sum_b n_b].  Returns accept_len [B], out_tokens [sum_b (n_b + 1)], out_nodes
    [sum_b n_b] and device_status [1]."""
    dev = target.device
    code = _dtype_code(target)
    if target.dim() != 2 or target.stride(1) != 1:
        raise ValueError("target must be a 2-D tensor with unit column stride")
    B = int(n_nodes.numel())
    n_tot = int(parent.numel())
    V = int(target.shape[1])
    if int(target.shape[0]) != n_tot + B:
        raise ValueError("target must have sum_b (n_b + 1) rows")
    _need(n_nodes, "n_nodes", torch.int32, B, dev)
    _need(parent, "parent", torch.int32, n_tot, dev)
    _need(tree_tokens, "tree_tokens", torch.int32, n_tot, dev)
    if max_nodes is None:
        max_nodes = int(n_nodes.max().item())
    if workspace is None:
        nbytes = int(lib().sv_tree_workspace_size(B, n_tot))
        if nbytes == 0:
            raise SpecVerifyError(f"invalid shape B={B} nodes={n_tot}")
        workspace = alloc_workspace(nbytes, dev)
    if out is None:
        out = {"accept_len": torch.empty(B, dtype=torch.int32, device=dev),
               "out_tokens": torch.empty(n_tot + B, dtype=torch.int32, device=dev),
               "out_nodes": torch.empty(n_tot, dtype=torch.int32, device=dev),
               "device_status": torch.empty(1, dtype=torch.int32, device=dev)}
    else:
        _need(out["accept_len"], "accept_len", torch.int32, B, dev)
        _need(out["out_tokens"], "out_tokens", torch.int32, n_tot + B, dev)
        if out.get("out_nodes") is not None:
            _need(out["out_nodes"], "out_nodes", torch.int32, n_tot, dev)
        _need(out["device_status"], "device_status", torch.int32, 1, dev)
    st = lib().sv_verify_tree_greedy(code, B, int(max_nodes), V, target.stride(0), n_tot,
                                     _ptr(target), _ptr(n_nodes), _ptr(parent), _ptr(tree_tokens),
                                     _ptr(out["accept_len"]), _ptr(out["out_tokens"]),
                                     _ptr(out.get("out_nodes")), _ptr(out["device_status"]),
                                     _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "sv_verify_tree_greedy")
    return out


def _row_pair_shapes(target: torch.Tensor, draft: torch.Tensor,
                     p_row_index: Optional[torch.Tensor]):
    dev = target.device
    code = _dtype_code(target)
    if draft.dtype != target.dtype or target.dim() != 2 or draft.dim() != 2:
        raise ValueError("target/draft must be 2-D tensors of one dtype")
    if target.stride(1) != 1 or draft.stride(1) != 1:
        raise ValueError("logits must have unit column stride")
    n = int(draft.shape[0])
    V = int(draft.shape[1])
    if int(target.shape[1]) != V:
        raise ValueError("target and draft must have the same column count")
    if p_row_index is None:
        if int(target.shape[0]) < n:
            raise ValueError("without p_row_index target needs at least as many rows as draft")
    else:
        _need(p_row_index, "p_row_index", torch.int32, n, dev)
    return dev, code, n, V


def opd_loss(target: torch.Tensor, draft: torch.Tensor, k: Optional[torch.Tensor] = None,
             delta: float = 1.0, alpha: float = 0.8, p_row_index: Optional[torch.Tensor] = None,
             *, workspace: Optional[torch.Tensor] = None, out: Optional[dict] = None,
             stream=None) -> dict:
    """sv_opd_loss: per draft row the clipped rKL, -ln q(x*) and x*; with k (int32 [B], draft
    rows packed request by request) the per-request OPD loss.  Returns a dict of tensors."""
    dev, code, n, V = _row_pair_shapes(target, draft, p_row_index)
    B = 1
    if k is not None:
        if k.dim() != 1:
            raise ValueError("k must be 1-D")
        B = int(k.numel())
        _need(k, "k", torch.int32, B, dev)
    if workspace is None:
        nbytes = int(lib().sv_rkl_workspace_size(n, V, code))
        if nbytes == 0:
            raise SpecVerifyError(f"invalid shape n_rows={n} V={V}")
        workspace = alloc_workspace(nbytes, dev)
    if out is None:
        out = {
            "rkl": torch.empty(n, dtype=torch.float32, device=dev),
            "hard_ce": torch.empty(n, dtype=torch.float32, device=dev),
            "top1": torch.empty(n, dtype=torch.int32, device=dev),
            "opd": torch.empty(B, dtype=torch.float32, device=dev) if k is not None else None,
            "device_status": torch.empty(1, dtype=torch.int32, device=dev),
        }
    else:
        _need(out["rkl"], "rkl", torch.float32, n, dev)
        _need(out["hard_ce"], "hard_ce", torch.float32, n, dev)
        if out.get("top1") is not None:
            _need(out["top1"], "top1", torch.int32, n, dev)
        if k is not None:
            _need(out["opd"], "opd", torch.float32, B, dev)
        _need(out["device_status"], "device_status", torch.int32, 1, dev)
    st = lib().sv_opd_loss(code, B, n, int(target.shape[0]), V, target.stride(0), draft.stride(0),
                           _ptr(target), _ptr(draft), _ptr(p_row_index), _ptr(k), float(delta),
                           float(alpha), _ptr(out["rkl"]), _ptr(out["hard_ce"]),
                           _ptr(out.get("top1")), _ptr(out.get("opd") if k is not None else None),
                           _ptr(out["device_status"]), _ptr(workspace),
                           workspace.numel(), _stream(stream))
    _check(st, "sv_opd_loss")
    return out


def opd_loss_grad(target: torch.Tensor, draft: torch.Tensor, k: torch.Tensor,
                  delta: float = 1.0, alpha: float = 0.8,
                  p_row_index: Optional[torch.Tensor] = None, *,
                  grad_dtype: Optional[torch.dtype] = None,
                  workspace: Optional[torch.Tensor] = None, out: Optional[dict] = None,
                  stream=None) -> dict:
    """sv_opd_loss_grad: the sv_opd_loss outputs plus "grad", d l_OPD / d draft logits
    ([n_rows, V], bfloat16 or float32; default the logits' dtype)."""
    dev, code, n, V = _row_pair_shapes(target, draft, p_row_index)
    if k.dim() != 1:
        raise ValueError("k must be 1-D")
    B = int(k.numel())
    _need(k, "k", torch.int32, B, dev)
    gdt = target.dtype if grad_dtype is None else grad_dtype
    gcode = _dtype_code(torch.empty(0, dtype=gdt))
    if workspace is None:
        nbytes = int(lib().sv_opd_grad_workspace_size(n, V, code))
        if nbytes == 0:
            raise SpecVerifyError(f"invalid shape n_rows={n} V={V}")
        workspace = alloc_workspace(nbytes, dev)
    if out is None:
        out = {
            "rkl": torch.empty(n, dtype=torch.float32, device=dev),
            "hard_ce": torch.empty(n, dtype=torch.float32, device=dev),
            "top1": torch.empty(n, dtype=torch.int32, device=dev),
            "opd": torch.empty(B, dtype=torch.float32, device=dev),
            "grad": torch.empty(n, V, dtype=gdt, device=dev),
            "device_status": torch.empty(1, dtype=torch.int32, device=dev),
        }
    else:
        _need(out["rkl"], "rkl", torch.float32, n, dev)
        _need(out["hard_ce"], "hard_ce", torch.float32, n, dev)
        if out.get("top1") is not None:
            _need(out["top1"], "top1", torch.int32, n, dev)
        if out.get("opd") is not None:
            _need(out["opd"], "opd", torch.float32, B, dev)
        _need(out["device_status"], "device_status", torch.int32, 1, dev)
    g = out["grad"]
    if (g.device != dev or g.dtype != gdt or g.dim() != 2 or g.shape[0] != n or g.shape[1] != V
            or g.stride(1) != 1):
        raise ValueError(f"grad must be a [{n}, {V}] {gdt} tensor with unit column stride")
    st = lib().sv_opd_loss_grad(code, B, n, int(target.shape[0]), V, target.stride(0),
                                draft.stride(0), _ptr(target), _ptr(draft), _ptr(p_row_index),
                                _ptr(k), float(delta), float(alpha), _ptr(out["rkl"]),
                                _ptr(out["hard_ce"]), _ptr(out.get("top1")), _ptr(out.get("opd")),
                                gcode, g.stride(0), _ptr(g), _ptr(out["device_status"]),
                                _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "sv_opd_loss_grad")
    return out


def clipped_rkl(target: torch.Tensor, draft: torch.Tensor, delta: float = 1.0,
                p_row_index: Optional[torch.Tensor] = None, *,
                workspace: Optional[torch.Tensor] = None, stream=None) -> tuple:
    """sv_clipped_rkl: returns (rkl [n_rows] float32, device_status [1] int32)."""
    dev = target.device
    code = _dtype_code(target)
    if draft.dtype != target.dtype or target.dim() != 2 or draft.dim() != 2:
        raise ValueError("target/draft must be 2-D tensors of one dtype")
    if target.stride(1) != 1 or draft.stride(1) != 1:
        raise ValueError("logits must have unit column stride")
    n = int(draft.shape[0])
    V = int(draft.shape[1])
    if int(target.shape[1]) != V:
        raise ValueError("target and draft must have the same column count")
    if p_row_index is None:
        if int(target.shape[0]) < n:
            raise ValueError("without p_row_index target needs at least as many rows as draft")
    else:
        _need(p_row_index, "p_row_index", torch.int32, n, dev)
    if workspace is None:
        nbytes = int(lib().sv_rkl_workspace_size(n, V, code))
        if nbytes == 0:
            raise SpecVerifyError(f"invalid shape n_rows={n} V={V}")
        workspace = alloc_workspace(nbytes, dev)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    st = lib().sv_clipped_rkl(code, n, int(target.shape[0]), V, target.stride(0), draft.stride(0),
                              _ptr(target), _ptr(draft), _ptr(p_row_index), float(delta),
                              _ptr(out), _ptr(status), _ptr(workspace), workspace.numel(),
                              _stream(stream))
    _check(st, "sv_clipped_rkl")
    return out, status


# ----------------------------------------------------------------------------- profiling
READ_PROBE_WORDS = 1024


def read_probe(data, out=None, stream=None):
    """Plain read of the bytes of a contiguous device tensor (diagnostics: the read ceiling).
    Returns the [READ_PROBE_WORDS] int32 tensor the kernel folds the words into."""
    if not data.is_cuda or not data.is_contiguous():
        raise ValueError("read_probe needs a contiguous device tensor")
    if out is None:
        out = torch.empty(READ_PROBE_WORDS, dtype=torch.int32, device=data.device)
    nbytes = data.numel() * data.element_size()
    _check(lib().sv_read_probe(data.data_ptr(), nbytes, out.data_ptr(), _stream(stream)),
           "sv_read_probe")
    return out


def profile_enable(on: bool = True):
    _check(lib().sv_profile_enable(1 if on else 0), "sv_profile_enable")


def profile_reset():
    _check(lib().sv_profile_reset(), "sv_profile_reset")


def profile_read() -> dict:
    """{kernel name: (launches, total ms)} for every kernel launched while profiling."""
    L = lib()
    res = {}
    buf = ctypes.create_string_buffer(64)
    for i in range(L.sv_profile_count()):
        n = _c_i64(0)
        ms = ctypes.c_double(0.0)
        _check(L.sv_profile_get(i, buf, 64, ctypes.byref(n), ctypes.byref(ms)), "sv_profile_get")
        if n.value:
            res[buf.value.decode()] = (int(n.value), float(ms.value))
    return res


def verify_block_noalloc(target: torch.Tensor, draft: torch.Tensor, k: torch.Tensor,
                         draft_tokens: torch.Tensor, uniforms: torch.Tensor,
                         temperature: Optional[torch.Tensor], delta: float, out: dict, *,
                         k_max: Optional[int] = None, stream=None) -> dict:
    """sv_verify_block_noalloc: sv_verify_block on the library's own fixed scratch buffer.
    Allocates nothing: the caller passes every output in ``out`` (accept_len, out_tokens,
    device_status, and rkl / p_at_draft / q_at_draft or None)."""
    dev = target.device
    if dev.type != "cuda":
        raise ValueError("target must be a GPU tensor")
    code = _dtype_code(target)
    if draft.dtype != target.dtype:
        raise TypeError("target and draft must share a dtype")
    if target.dim() != 2 or draft.dim() != 2 or target.stride(1) != 1 or draft.stride(1) != 1:
        raise ValueError("logits must be 2-D with unit column stride")
    B = int(k.numel())
    n_d = int(draft.shape[0])
    V = int(target.shape[1])
    if int(draft.shape[1]) != V or int(target.shape[0]) != n_d + B:
        raise ValueError(f"shapes: target {tuple(target.shape)} must be [n_draft_rows + B, V], "
                         f"draft {tuple(draft.shape)} [n_draft_rows, V], B = {B}")
    if k_max is None:
        k_max = max(1, min(SV_MAX_K, n_d - B + 1))
    _need(k, "k", torch.int32, B, dev)
    _need(draft_tokens, "draft_tokens", torch.int32, n_d, dev)
    _need(uniforms, "uniforms", torch.float32, n_d + B, dev)
    if temperature is not None:
        _need(temperature, "temperature", torch.float32, B, dev)
    _need(out["accept_len"], "accept_len", torch.int32, B, dev)
    _need(out["out_tokens"], "out_tokens", torch.int32, n_d + B, dev)
    for name in ("rkl", "p_at_draft", "q_at_draft"):
        if out.get(name) is not None:
            _need(out[name], name, torch.float32, n_d, dev)
    _need(out["device_status"], "device_status", torch.int32, 1, dev)
    st = lib().sv_verify_block_noalloc(
        code, B, k_max, V, target.stride(0), draft.stride(0), n_d, _ptr(target), _ptr(draft),
        _ptr(k), _ptr(draft_tokens), _ptr(uniforms), _ptr(temperature), float(delta),
        _ptr(out["accept_len"]), _ptr(out["out_tokens"]), _ptr(out.get("rkl")),
        _ptr(out.get("p_at_draft")), _ptr(out.get("q_at_draft")), _ptr(out["device_status"]),
        _stream(stream))
    _check(st, "sv_verify_block_noalloc")
    return out
