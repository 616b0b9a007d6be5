"""Oracle: looking up a prepared successor block after verification (test infrastructure only).

Source: the review page "D3D: Decoupled Diffusion Drafting for Asynchronous Speculative
Decoding" (Methodology, inference paragraph).  While the target verifies the current block, a packed drafter pass prepares
successor blocks for selected rejection positions and for the full-acceptance case; C
positions are covered with F candidate tokens each, and for block size B the packed budget is
B((C - 1) F + 2) tokens.  A verified prefix that matches a prepared branch is a cache hit and
that branch is reused; otherwise the target waits for a new synchronous draft.

Reading (the page gives no key format): a branch is keyed by the verification outcome that
fixes the next round's prefix -- the accept length a (0..k_b, k_b meaning every draft was
accepted) and the token emitted after the accepted drafts (the residual draw, the greedy
replacement, or the bonus token).  A key token of -1 matches any emitted token (a branch
prepared before that token is known, e.g. for the full-acceptance case).  The hit is the
first branch, in the request's list order, whose key matches; a request whose verification
was invalid (accept length -1) never hits.
"""

from __future__ import annotations

import numpy as np


def branch_lookup(accept_len, final_token, branch_pos, branch_tok) -> np.ndarray:
    """hit[b] = first j with branch_pos[b, j] == accept_len[b] and branch_tok[b, j] in
    {final_token[b], -1}; -1 if none or if accept_len[b] < 0."""
    accept_len = np.asarray(accept_len, dtype=np.int64)
    final_token = np.asarray(final_token, dtype=np.int64)
    branch_pos = np.asarray(branch_pos, dtype=np.int64)
    branch_tok = np.asarray(branch_tok, dtype=np.int64)
    B, n = branch_pos.shape
    hit = np.full(B, -1, dtype=np.int64)
    for b in range(B):
        if accept_len[b] < 0:
            continue
        for j in range(n):
            if branch_pos[b, j] == accept_len[b] and branch_tok[b, j] in (final_token[b], -1):
                hit[b] = j
                break
    return hit


def final_tokens(out_tokens, accept_len, k) -> np.ndarray:
    """The token emitted after the accepted drafts of each request, read from the packed
    output rows (request b owns rows off_t[b] .. off_t[b] + k_b); -1 for invalid requests."""
    k = np.asarray(k, dtype=np.int64)
    off_t = np.concatenate([[0], np.cumsum(k + 1)])
    out = np.full(k.shape[0], -1, dtype=np.int64)
    for b in range(k.shape[0]):
        a = int(accept_len[b])
        if 0 <= a <= k[b]:
            out[b] = int(out_tokens[off_t[b] + a])
    return out
