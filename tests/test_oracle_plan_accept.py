"""Pins of the oracle's plan (O1) and acceptance (O4) against brute force, closed
forms, a hand-worked example and generator statistics.  CPU only."""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def all_trees(D):
    """Every parent array with parents[0] = -1 and 0 <= parents[i] < i."""
    for tail in itertools.product(*[range(i) for i in range(1, D)]):
        yield np.array((-1,) + tail, dtype=np.int64)


def walk_ancestors(par, i):
    """Brute force: follow parent pointers from i to the root."""
    out = [i]
    while par[out[-1]] != -1:
        out.append(int(par[out[-1]]))
    return out


@pytest.mark.parametrize("D", [1, 2, 3, 4, 5, 6, 7])
def test_plan_exhaustive_vs_parent_walk(D):
    trees = np.stack(list(all_trees(D)))
    assert len(trees) == math.factorial(D - 1)
    anc, depth, err = oracle.build_plan(trees)
    assert (err == 0).all()
    for b, par in enumerate(trees):
        for i in range(D):
            w = walk_ancestors(par, i)
            assert set(np.nonzero(anc[b, i])[0]) == set(w)
            assert depth[b, i] == len(w) - 1


def test_plan_chain_closed_form():
    D = 9
    par = np.array([[-1] + list(range(D - 1))])
    anc, depth, err = oracle.build_plan(par)
    assert (anc[0] == np.tril(np.ones((D, D), dtype=bool))).all()
    assert (depth[0] == np.arange(D)).all()
    bits = oracle.anc_to_bits(anc)[0]
    assert [int(x) for x in bits] == [(1 << (i + 1)) - 1 for i in range(D)]


def test_plan_rejects_bad_parents():
    bad = np.array([[0, 0, 1], [-1, 1, 0], [-1, 0, 2], [-1, -1, 0], [-1, 0, 5]])
    good = np.array([[-1, 0, 1]])
    anc, depth, err = oracle.build_plan(np.concatenate([bad, good]))
    assert list(err) == [oracle.SEQ_BAD_PARENT] * 4 + [oracle.SEQ_BAD_PARENT, 0]
    assert not anc[:5].any()


def test_golden_accept_tree7():
    g = json.load(open(os.path.join(GOLD, "accept_tree7.json")))
    par = np.array([g["parents"]])
    anc, depth, err = oracle.build_plan(par)
    assert list(depth[0]) == g["depth"]
    assert [sorted(np.nonzero(anc[0, i])[0].tolist()) for i in range(par.shape[1])] == g["anc_sets"]
    m, path, bonus = oracle.accept(par, anc, depth, np.array([g["draft"]]), np.array([g["target"]]))
    assert m[0] == g["m"] and bonus[0] == g["bonus"]
    assert list(path[0]) == g["path"]


def brute_accept(par, draft, target):
    """Enumerate root-to-leaf paths; on each, the longest prefix whose drafts all match."""
    D = len(par)
    kids = {i: [j for j in range(1, D) if par[j] == i] for i in range(D)}
    leaves = [i for i in range(D) if not kids[i]]
    best = (0, 0)  # (depth, -index) maximised
    for leaf in leaves:
        p = list(reversed(walk_ancestors(par, leaf)))
        k = 0
        while k + 1 < len(p) and draft[p[k + 1]] == target[p[k]]:
            k += 1
        cand = (k, -p[k])
        if cand > best:
            best = cand
    node = -best[1]
    return best[0], list(reversed(walk_ancestors(par, node))), node


@pytest.mark.parametrize("D", [2, 3, 4, 5, 6])
def test_accept_exhaustive_small_trees(D):
    rng = np.random.default_rng(7 + D)
    trees = list(all_trees(D))
    for par in trees:
        for _ in range(4):
            # a 2-token vocabulary makes matches, multi-match siblings and ties common
            draft = rng.integers(0, 2, size=D)
            target = rng.integers(0, 2, size=D)
            anc, depth, err = oracle.build_plan(par[None])
            m, path, bonus = oracle.accept(par[None], anc, depth, draft[None], target[None])
            bm, bpath, bnode = brute_accept(par, draft, target)
            assert m[0] == bm
            assert list(path[0, :bm + 1]) == bpath
            assert (path[0, bm + 1:] == -1).all()
            assert bonus[0] == target[bnode]


def test_accept_chain_closed_form():
    rng = np.random.default_rng(3)
    D = 8
    par = np.array([[-1] + list(range(D - 1))])
    anc, depth, _ = oracle.build_plan(par)
    for _ in range(200):
        draft = rng.integers(0, 3, size=(1, D))
        target = rng.integers(0, 3, size=(1, D))
        k = 0
        while k + 1 < D and draft[0, k + 1] == target[0, k]:
            k += 1
        m, path, bonus = oracle.accept(par, anc, depth, draft, target)
        assert m[0] == k
        assert list(path[0, :k + 1]) == list(range(k + 1))
        assert bonus[0] == target[0, k]


def expected_m(par, p):
    """E[m] under the generator's agreement model: each node's acceptance probability is
    the product over its chain of p(1-p)^(sibling rank - 1)."""
    D = len(par)
    rank = np.zeros(D, dtype=int)
    for i in range(1, D):
        rank[i] = sum(1 for j in range(1, i) if par[j] == par[i])
    tot = 0.0
    for i in range(1, D):
        pr = 1.0
        for v in walk_ancestors(par, i)[:-1]:
            pr *= p * (1 - p) ** rank[v]
        tot += pr
    return tot


@pytest.mark.parametrize("k,D,p", [(1, 8, 0.6), (2, 8, 0.6), (2, 6, 0.5), (1, 5, 0.7)])
def test_accept_statistics_match_generator_law(k, D, p):
    """Mean accepted drafts over 4000 seeded trees vs the closed-form expectation (4 sigma)."""
    w = synth.Workload("stat", 1, D, 1, 1, 8, "f32", (4,), 0, k, D - 1 if k == 1 else 3, p, 4242)
    ms, exp = [], []
    for t in range(4000):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(4242, spawn_key=(t,))))
        par, draft = synth.draft_tree(rng, w.topk, w.steps, D)
        tgt = synth.target_tokens(rng, par, draft, p)
        anc, depth, _ = oracle.build_plan(par[None])
        m, _, _ = oracle.accept(par[None], anc, depth, draft[None], tgt[None])
        ms.append(m[0])
        exp.append(expected_m(par, p))
    ms = np.array(ms, dtype=float)
    mu = float(np.mean(exp))
    sigma = ms.std() / math.sqrt(len(ms))
    assert abs(ms.mean() - mu) < 4 * sigma + 1e-9, (ms.mean(), mu, sigma)
    if k == 1:
        assert abs(mu - sum(p ** j for j in range(1, D))) < 1e-12


def test_generator_tree_shape():
    for k, s, D in [(2, 3, 8), (2, 3, 6), (1, 7, 8), (2, 4, 6), (3, 2, 7)]:
        rng = np.random.default_rng(11)
        for _ in range(50):
            par, draft = synth.draft_tree(rng, k, s, D)
            assert par[0] == -1 and all(0 <= par[i] < i for i in range(1, D))
            kids = {}
            for i in range(1, D):
                kids.setdefault(int(par[i]), []).append(int(draft[i]))
            for u, toks in kids.items():
                assert len(toks) <= k and len(set(toks)) == len(toks)
            anc, depth, _ = oracle.build_plan(par[None])
            assert depth.max() <= s
