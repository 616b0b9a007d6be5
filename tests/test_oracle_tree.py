"""Pins of the greedy tree-verification oracle (DFlash notes, Sections 5.1-5.2; AdaFlash paper,
Appendix B.1): a chain is the greedy verification of a linear block (the oracle's own linear path,
itself pinned by the DFlash greedy trace); a hand-built tree; brute force over every node's
ancestor path on random trees with distinct sibling tokens; the lowest index among equal
siblings; invalid parents."""

import numpy as np

from oracle import greedy_argmax, tree_valid, verify_request, verify_tree_greedy


def _rows(rng, n_rows, V, argmaxes):
    """Random logits with a planted unique maximum per row."""
    L = rng.normal(size=(n_rows, V))
    for r, a in enumerate(argmaxes):
        L[r, a] = L[r].max() + 1.0 + rng.random()
    return L


def test_chain_is_linear_greedy_verification():
    rng = np.random.default_rng(3)
    V, k = 12, 15
    for trial in range(30):
        amax = rng.integers(0, V, size=k + 1)
        L = _rows(rng, k + 1, V, amax)
        x = np.where(rng.random(k) < 0.8, amax[:k], rng.integers(0, V, size=k))
        lin = verify_request(L, L[:k], x, np.zeros(k + 1), 0.0, 1.0, with_rkl=False)
        tr = verify_tree_greedy(L, np.arange(k) - 1, x)
        assert tr["accept_len"] == lin["accept_len"]
        assert tr["tokens"] == lin["tokens"].tolist()
        assert tr["path"] == list(range(lin["accept_len"]))


def test_hand_built_tree():
    # root -> {n0: 5, n1: 7}; n1 -> {n2: 3, n3: 9}; n0 -> {n4: 1}
    parent = [-1, -1, 1, 1, 0]
    tokens = [5, 7, 3, 9, 1]
    V = 16
    amax = [7, 2, 9, 4, 11, 6]  # rows: root, n0 .. n4
    L = _rows(np.random.default_rng(4), 6, V, amax)
    r = verify_tree_greedy(L, parent, tokens)
    assert r["path"] == [1, 3] and r["accept_len"] == 2
    assert r["tokens"][:3] == [7, 9, 11] and r["tokens"][3:] == [-1] * 3


def _brute(L, parent, tokens):
    """Nodes whose every ancestor step matches the argmax of the step's parent row, by depth."""
    n = len(parent)
    arg = [greedy_argmax(L[r]) for r in range(n + 1)]
    good = []
    for j in range(n):
        path, c = [], j
        while c >= 0:
            path.append(c)
            c = parent[c]
        if all(tokens[c] == arg[parent[c] + 1] for c in path):
            good.append(path[::-1])
    best = max(good, key=len) if good else []
    last = best[-1] if best else -1
    return best, [tokens[j] for j in best] + [arg[last + 1]]


def test_random_trees_against_brute_force():
    rng = np.random.default_rng(5)
    V = 20
    for trial in range(200):
        n = int(rng.integers(1, 40))
        parent, tokens = [], []
        for j in range(n):
            p = int(rng.integers(-1, j))
            used = {tokens[i] for i in range(j) if parent[i] == p}
            free = [t for t in range(V) if t not in used]
            parent.append(p)
            tokens.append(int(rng.choice(free)))
        amax = rng.integers(0, V, size=n + 1)
        # steer some rows to a child's token so that paths get long
        for j in range(n):
            if rng.random() < 0.6:
                amax[parent[j] + 1] = tokens[j]
        L = _rows(rng, n + 1, V, amax)
        r = verify_tree_greedy(L, parent, tokens)
        path, emitted = _brute(L, parent, tokens)
        assert r["path"] == path
        assert r["tokens"][: len(emitted)] == emitted


def test_equal_siblings_take_the_lowest_index_and_invalid_parents():
    V = 8
    L = _rows(np.random.default_rng(6), 4, V, [3, 1, 2, 5])
    r = verify_tree_greedy(L, [-1, -1, -1], [3, 3, 3])
    assert r["path"] == [0] and r["tokens"][:2] == [3, 1]
    assert not tree_valid([-1, 2, 0], [1, 1, 1], V)  # a parent after its child
    assert not tree_valid([-1, -2], [1, 1], V)
    assert not tree_valid([-1, 0], [1, V], V)
    assert verify_tree_greedy(L, [-1, 1, 0], [1, 1, 1])["accept_len"] == -1
