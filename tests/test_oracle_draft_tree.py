"""Pins of the draft-tree construction oracle (oracle/draft_tree.py) to what the pages
and the mathematics fix: a brute force over root-to-node paths, the top-k = 1 chain in
closed form, a hand-worked example (tests/golden/draft_tree_k2s2.json) and invariants."""
import json
import math
import os

import numpy as np
import pytest

from oracle.draft_tree import build_draft_tree, candidate_count, expanded_count

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute(rows, root, k, s, D):
    """Every root-to-node path of the full k-ary expansion, enumerated recursively; a
    path's logits row is found from its creation index (parent index * k + rank + 1), its
    normaliser with math.fsum and its top-k by repeated scans; then one full sort."""
    paths = []

    def rec(path, idx, score, depth):
        if depth == s:
            return
        row = [float(x) for x in rows[idx]]
        m = max(row)
        lse = m + math.log(math.fsum(math.exp(x - m) for x in row))
        chosen = []
        for _ in range(k):
            best = None
            for t in range(len(row)):
                if t in chosen:
                    continue
                if best is None or row[t] > row[best]:
                    best = t
            chosen.append(best)
        for r, t in enumerate(chosen):
            child = idx * k + r + 1
            sc = score + (row[t] - lse)
            paths.append((path + (r,), child, t, sc, depth + 1))
            rec(path + (r,), child, sc, depth + 1)

    rec((), 0, 0.0, 0)
    kept = sorted(paths, key=lambda p: (-p[3], p[4], p[1]))[: D - 1]
    slot = {(): 0}
    for i, p in enumerate(kept):
        slot[p[0]] = i + 1
    parents = [-1] + [slot[p[0][:-1]] for p in kept]
    tokens = [root] + [p[2] for p in kept]
    return parents, tokens


@pytest.mark.parametrize("k,s,D,V", [(2, 3, 8, 64), (2, 3, 15, 32), (3, 2, 7, 50), (1, 6, 7, 40), (4, 2, 9, 70),
                                     (2, 4, 12, 33)])
def test_matches_brute_force_over_paths(k, s, D, V):
    rng = np.random.default_rng(100 + 7 * k + s + D)
    B = 12
    E = expanded_count(k, s)
    logits = rng.gumbel(size=(B, E, V))
    root = rng.integers(V, size=B)
    par, tok, _ = build_draft_tree(logits, root, k, s, D)
    for b in range(B):
        bp, bt = _brute(logits[b], int(root[b]), k, s, D)
        assert par[b].tolist() == bp
        assert tok[b].tolist() == bt


def test_top1_is_the_argmax_chain():
    rng = np.random.default_rng(5)
    s, V = 7, 90
    logits = rng.normal(size=(4, s, V))
    root = np.array([1, 2, 3, 4])
    for D in (1, 2, 5, 8):
        par, tok, cum = build_draft_tree(logits, root, 1, s, D)
        assert par[:, :D].tolist() == [list(range(-1, D - 1))] * 4
        for b in range(4):
            assert tok[b, 0] == root[b]
            for i in range(1, D):
                assert tok[b, i] == int(np.argmax(logits[b, i - 1]))
            # closed form of the chain's score: sum of the chosen log-softmax values
            run = 0.0
            for i in range(1, D):
                row = logits[b, i - 1]
                run += row.max() - math.log(np.exp(row).sum())
                assert abs(cum[b, i] - run) < 1e-12


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "draft_tree_k2s2.json")))
    logits = np.array([g["logits"]], dtype=np.float64)
    par, tok, cum = build_draft_tree(logits, np.array([g["root_tok"]]), g["topk"], g["steps"], g["D"])
    assert par[0].tolist() == g["parents"]
    assert tok[0].tolist() == g["draft"]
    assert np.abs(cum[0] - np.array(g["cum"])).max() < 1e-12


def test_invariants_and_budget_limits():
    rng = np.random.default_rng(9)
    k, s, V = 2, 3, 128
    E, N = expanded_count(k, s), candidate_count(k, s)
    assert (E, N) == (7, 14)
    logits = rng.gumbel(size=(20, E, V))
    root = rng.integers(V, size=20)
    par, tok, cum = build_draft_tree(logits, root, k, s, N + 1)  # keep every candidate
    for b in range(20):
        assert par[b, 0] == -1 and all(0 <= par[b, i] < i for i in range(1, N + 1))
        assert all(cum[b, i] >= cum[b, i + 1] for i in range(1, N))  # rank order
        for i in range(1, N + 1):
            p = par[b, i]
            sibs = [j for j in range(1, N + 1) if par[b, j] == p]
            assert len({int(tok[b, j]) for j in sibs}) == len(sibs)
            assert cum[b, i] < cum[b, p] or p == 0 and cum[b, i] <= 0.0
    with pytest.raises(ValueError):
        build_draft_tree(logits, root, k, s, N + 2)
    with pytest.raises(ValueError):
        build_draft_tree(logits[:, :5], root, k, s, 4)


def test_equal_logits_resolve_by_depth_then_creation():
    # every row flat: all candidates of a level tie; the shallower level wins, then the
    # earlier-created candidate, and tokens are the smallest ids
    k, s, V = 2, 3, 5
    logits = np.zeros((1, expanded_count(k, s), V))
    par, tok, _ = build_draft_tree(logits, np.array([4]), k, s, 8)
    assert par[0].tolist() == [-1, 0, 0, 1, 1, 2, 2, 3]
    assert tok[0].tolist() == [4, 0, 1, 0, 1, 0, 1, 0]
