"""Oracle: greedy verification of a draft tree (test infrastructure only).

Sources: the DFlash notes (zhangshuibai.github.io), Section 5.1 (EAGLE-2/3 propose a dynamic draft
tree of about 60 candidate tokens and verify it in one target pass with tree attention) and
Section 5.2 worked example #4 (greedy verification accepts a draft token iff it equals the
target's argmax at its prefix and replaces the first mismatch by that argmax); the AdaFlash paper,
Appendix B.1 (greedy decoding, temperature 0, is the default) and Section 4.1 (EAGLE-3 with a
tree budget as a baseline).

Reading (the pages give no tree algorithm): node j of a request's tree holds a drafted token and
its parent (-1 for the root, the verified anchor; otherwise an earlier node, so the nodes come in
topological order).  The target scores the root and every node: row 0 is its distribution after
the root, row 1 + j after node j.  Starting from the root, the walk moves to the child (lowest
index among equals) whose token is the argmax of the current node's row; it stops at a node none
of whose children matches, and that node's argmax is emitted after the accepted path.  A chain
(node j's parent is j - 1) is exactly the greedy verification of a linear block.  Stochastic
tree verification is not covered.
"""

from __future__ import annotations

import numpy as np

from .verify import greedy_argmax, widen_logits


def tree_valid(parent, tokens, V: int) -> bool:
    parent = np.asarray(parent, dtype=np.int64)
    tokens = np.asarray(tokens, dtype=np.int64)
    n = parent.shape[0]
    return bool(n >= 1 and np.all((parent >= -1) & (parent < np.arange(n)))
                and np.all((tokens >= 0) & (tokens < V)))


def verify_tree_greedy(target_logits: np.ndarray, parent, tokens) -> dict:
    """One request: target_logits [n + 1, V] (row 0 the root, row 1 + j node j), parent [n],
    tokens [n].  Returns the accepted path (node indices), accept_len, and the emitted tokens
    (the path's tokens, then the argmax at its last node)."""
    parent = np.asarray(parent, dtype=np.int64)
    tokens = np.asarray(tokens, dtype=np.int64)
    n = parent.shape[0]
    V = target_logits.shape[1]
    if not tree_valid(parent, tokens, V):
        return {"valid": False, "accept_len": -1, "path": [], "tokens": [-1] * (n + 1)}
    path = []
    cur = -1
    while True:
        g = greedy_argmax(target_logits[cur + 1])
        nxt = -1
        for j in range(n):  # lowest index among the matching children
            if parent[j] == cur and tokens[j] == g:
                nxt = j
                break
        if nxt < 0:
            break
        path.append(nxt)
        cur = nxt
    emitted = [int(tokens[j]) for j in path] + [int(g)]
    return {"valid": True, "accept_len": len(path), "path": path,
            "tokens": emitted + [-1] * (n + 1 - len(emitted))}


def verify_tree_block(*, target, dtype, V: int, n_nodes, parent, tokens) -> dict:
    """Packed batch: request b owns target rows off_t[b] .. off_t[b] + n_b (off_t[b] =
    sum_{c<b} (n_c + 1)) and nodes off_n[b] .. off_n[b] + n_b - 1 (off_n[b] = sum_{c<b} n_c).
    out_tokens follows the target rows (n_b + 1 slots per request, -1 after the emitted ones);
    out_nodes follows the nodes (the accepted path, then -1)."""
    n_nodes = np.asarray(n_nodes, dtype=np.int64)
    B = n_nodes.shape[0]
    off_t = np.concatenate([[0], np.cumsum(n_nodes + 1)])
    off_n = np.concatenate([[0], np.cumsum(n_nodes)])
    res = {"accept_len": np.full(B, -1, dtype=np.int64),
           "out_tokens": np.full(int(off_t[-1]), -1, dtype=np.int64),
           "out_nodes": np.full(int(off_n[-1]), -1, dtype=np.int64),
           "valid": np.zeros(B, dtype=bool)}
    for b in range(B):
        tl = widen_logits(target[off_t[b]: off_t[b + 1], :V], dtype)
        r = verify_tree_greedy(tl, parent[off_n[b]: off_n[b + 1]], tokens[off_n[b]: off_n[b + 1]])
        res["valid"][b] = r["valid"]
        res["accept_len"][b] = r["accept_len"]
        res["out_tokens"][off_t[b]: off_t[b + 1]] = r["tokens"]
        res["out_nodes"][off_n[b]: off_n[b] + len(r["path"])] = r["path"]
    return res
