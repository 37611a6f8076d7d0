"""Pins of the oracle's compression pieces: from-scratch compression (O6) against
closed forms and hand-worked values; chain-wise scratch entries (O3) against
compressing each chain's own token sequence from scratch; multi-step refresh (O5)
against from-scratch compression of the committed history; commit-log invariants;
isolation of rejected branches; pool overflow.  CPU only, float64."""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def arange_hist(P, Hkv=1, d=3):
    x = np.broadcast_to(np.arange(P, dtype=float)[None, :, None], (Hkv, P, d)).copy()
    return x


def test_golden_compress_arange10():
    g = json.load(open(os.path.join(GOLD, "compress_arange10.json")))
    P = g["P"]
    x = arange_hist(P)
    st = oracle.from_scratch([x], [x * 2], g["levels"], [8, 8, 8])
    for l in range(len(g["levels"])):
        n = st.n[l][0]
        assert list(st.pool_k[l][0, 0, :n, 0]) == g["entries"][l]
        assert list(st.pool_v[l][0, 0, :n, 1]) == [2 * e for e in g["entries"][l]]
        assert st.open_k[l][0, 0, 2] == g["open"][l]
    r = P % g["levels"][0]
    assert list(st.tail_k[0, 0, :r, 0]) == g["tail_level0"]


@pytest.mark.parametrize("C,P", [(1, 7), (4, 0), (4, 3), (4, 16), (4, 18), (128, 130), (3, 11)])
def test_from_scratch_closed_forms(C, P):
    x = arange_hist(P)
    st = oracle.from_scratch([x], [x], (C,), [max(P // C, 1)])
    n = P // C
    assert st.n[0][0] == n and st.P[0] == P
    for j in range(n):
        assert st.pool_k[0][0, 0, j, 0] == j * C + (C - 1) / 2  # mean of jC .. jC+C-1
    lo = n * C
    assert st.open_k[0][0, 0, 0] == (lo + P - 1) * (P - lo) / 2  # arithmetic series
    assert list(st.tail_k[0, 0, :P - lo, 0]) == list(range(lo, P))
    if C == 1:
        np.testing.assert_array_equal(st.pool_k[0][0, :, :P], x)


def test_from_scratch_constant_input():
    x = np.full((2, 300, 4), 0.375)
    st = oracle.from_scratch([x], [x], (4, 128), [80, 4])
    assert (st.pool_k[0][0, :, :75] == 0.375).all() and (st.pool_k[1][0, :, :2] == 0.375).all()
    assert np.allclose(st.open_k[1][0], 0.375 * (300 - 256))


def chain_history(hk, hv, kt, vt, par, b, i):
    """Raw history of node i's own chain: committed tokens then the chain's tree tokens."""
    path = []
    u = i
    while u != -1:
        path.append(u)
        u = int(par[b, u])
    path = path[::-1]
    return (np.concatenate([hk[b], kt[b, path].transpose(1, 0, 2)], axis=1),
            np.concatenate([hv[b], vt[b, path].transpose(1, 0, 2)], axis=1))


@pytest.mark.parametrize("P", [0, 1, 2, 3, 4, 125, 126, 127, 128, 253])
def test_scratch_equals_each_chain_compressed_alone(P):
    rng = np.random.default_rng(P)
    B, D, Hkv, d = 2, 10, 2, 4
    levels = (4, 128)
    hk = [rng.standard_normal((Hkv, P, d)) for _ in range(B)]
    hv = [rng.standard_normal((Hkv, P, d)) for _ in range(B)]
    st = oracle.from_scratch(hk, hv, levels, [P // 4 + 8, P // 128 + 2])
    par = np.stack([[-1] + [int(rng.integers(0, i)) for i in range(1, D)] for _ in range(B)])
    kt = rng.standard_normal((B, D, Hkv, d))
    vt = rng.standard_normal((B, D, Hkv, d))
    anc, depth, _ = oracle.build_plan(par)
    sc = oracle.build_scratch(kt, vt, anc, depth, st)
    for b in range(B):
        for i in range(D):
            ck, cv = chain_history(hk, hv, kt, vt, par, b, i)
            ref = oracle.from_scratch([ck], [cv], levels, [ck.shape[1] // 4 + 1, ck.shape[1] // 128 + 1])
            pos = P + depth[b, i]
            for l, C in enumerate(levels):
                closes = (pos + 1) % C == 0
                assert sc.closes[l][b, i] == closes
                if closes:
                    j = pos // C
                    np.testing.assert_allclose(sc.entry_k[l][b, i], ref.pool_k[l][0, :, j], rtol=0, atol=1e-12)
                    np.testing.assert_allclose(sc.entry_v[l][b, i], ref.pool_v[l][0, :, j], rtol=0, atol=1e-12)
                np.testing.assert_allclose(sc.open_k[l][b, i], ref.open_k[l][0], rtol=0, atol=1e-12)
                np.testing.assert_allclose(sc.open_v[l][b, i], ref.open_v[l][0], rtol=0, atol=1e-12)


def test_golden_refresh_chain():
    g = json.load(open(os.path.join(GOLD, "refresh_chain.json")))
    x = arange_hist(6, d=2)
    st = oracle.from_scratch([x], [x], (4,), [4])
    par = np.array([g["parents"]])
    D = par.shape[1]
    vals = 100.0 + np.arange(D)
    kt = np.broadcast_to(vals[None, :, None, None], (1, D, 1, 2)).copy()
    r = oracle.step(st, par, np.array([g["draft"]]), np.array([g["target"]]),
                    np.zeros((1, D, 1, 2)), kt, kt.copy())
    assert r.m[0] == g["m"] and r.bonus[0] == g["bonus"]
    s2 = r.state
    assert s2.P[0] == g["P_after"]
    assert list(s2.pool_k[0][0, 0, :s2.n[0][0], 0]) == g["entries_after"]
    assert s2.open_k[0][0, 0, 0] == g["open_after"]
    assert list(s2.tail_k[0, 0, :s2.P[0] % 4, 0]) == g["tail_after"]
    assert [list(x) for x in r.commit_log[0, 0] if x[0] >= 0] == g["commit_log"]


def check_commit_log(log, st_before, st_after, path, m, depth, levels):
    """Invariants: destinations are exactly the new slots n..n'-1 in order; each source
    is on the accepted path and sits at the last position of the block it fills."""
    B = path.shape[0]
    for b in range(B):
        P = st_before.P[b]
        for l, C in enumerate(levels):
            rows = [tuple(r) for r in log[b, l] if r[0] >= 0]
            assert [r[0] for r in rows] == list(range(st_before.n[l][b], st_after.n[l][b]))
            for j, u in rows:
                assert u in list(path[b, :m[b] + 1])
                assert P + depth[b, u] == j * C + C - 1


@pytest.mark.parametrize("levels,P0,p", [((4, 128), 125, 0.8), ((4, 16), 3, 0.5), ((1, 4), 7, 0.9), ((8,), 0, 0.7)])
def test_multistep_refresh_equals_from_scratch(levels, P0, p):
    rng = np.random.default_rng(sum(levels) + P0)
    w = synth.Workload("ms", 3, 8, 4, 2, 8, "f32", levels, P0, 2, 3, p, 77)
    B, D, Hkv, d = w.B, w.D, w.Hkv, w.d
    hist_k = [rng.standard_normal((Hkv, P0, d)) for _ in range(B)]
    hist_v = [rng.standard_normal((Hkv, P0, d)) for _ in range(B)]
    T = 60
    caps = [(P0 + T * D) // C + 2 for C in levels]
    st = oracle.from_scratch(hist_k, hist_v, levels, caps)
    crossed = set()
    for t in range(T):
        s = synth.step_inputs(w, t)
        kt = oracle.widen(s.k_tree, "f32")
        vt = oracle.widen(s.v_tree, "f32")
        q = oracle.widen(s.q, "f32")
        r = oracle.step(st, s.parents, s.draft, s.target, q, kt, vt)
        assert (r.err == 0).all()
        check_commit_log(r.commit_log, st, r.state, r.path, r.m, r.depth, levels)
        for b in range(B):
            acc = r.path[b, :r.m[b] + 1]
            hist_k[b] = np.concatenate([hist_k[b], kt[b, acc].transpose(1, 0, 2)], axis=1)
            hist_v[b] = np.concatenate([hist_v[b], vt[b, acc].transpose(1, 0, 2)], axis=1)
            for C in levels:
                if r.state.P[b] // C > st.P[b] // C:
                    crossed.add(C)
        st = r.state
        ref = oracle.from_scratch(hist_k, hist_v, levels, caps)
        assert (st.P == ref.P).all()
        for l in range(len(levels)):
            assert (st.n[l] == ref.n[l]).all()
            for b in range(B):
                n = st.n[l][b]
                np.testing.assert_allclose(st.pool_k[l][b, :, :n], ref.pool_k[l][b, :, :n], rtol=0, atol=1e-12)
                np.testing.assert_allclose(st.pool_v[l][b, :, :n], ref.pool_v[l][b, :, :n], rtol=0, atol=1e-12)
            np.testing.assert_allclose(st.open_k[l], ref.open_k[l], rtol=0, atol=1e-12)
            np.testing.assert_allclose(st.open_v[l], ref.open_v[l], rtol=0, atol=1e-12)
        for b in range(B):
            rr = st.P[b] % levels[0]
            np.testing.assert_array_equal(st.tail_k[b, :, :rr], ref.tail_k[b, :, :rr])
    assert crossed == set(levels)  # every level committed at least one block


def test_rejected_branches_never_reach_state():
    """Poisoning every non-path node's tree K/V and scratch leaves the refreshed state
    unchanged (TSD-V4 §3.2 isolation)."""
    rng = np.random.default_rng(31)
    w = synth.Workload("iso", 4, 8, 2, 1, 4, "f32", (4, 8), 13, 2, 3, 0.6, 5)
    hk = [rng.standard_normal((1, 13, 4)) for _ in range(4)]
    st = oracle.from_scratch(hk, hk, (4, 8), [10, 6])
    s = synth.step_inputs(w, 0)
    kt, vt = s.k_tree.astype(float), s.v_tree.astype(float)
    r = oracle.step(st, s.parents, s.draft, s.target, s.q.astype(float), kt, vt)
    kt2, vt2 = kt.copy(), vt.copy()
    sc2 = r.scratch
    for b in range(4):
        on = set(r.path[b, :r.m[b] + 1].tolist())
        for i in range(8):
            if i not in on:
                kt2[b, i] = np.nan
                vt2[b, i] = np.nan
                for l in range(2):
                    sc2.entry_k[l][b, i] = np.nan
                    sc2.open_k[l][b, i] = np.nan
    new2, log2, _ = oracle.refresh(st, sc2, kt2, vt2, r.m, r.path)
    for l in range(2):
        np.testing.assert_array_equal(new2.pool_k[l], r.state.pool_k[l])
        np.testing.assert_array_equal(new2.open_k[l], r.state.open_k[l])
    np.testing.assert_array_equal(new2.tail_k, r.state.tail_k)
    np.testing.assert_array_equal(log2, r.commit_log)


def test_pool_full_leaves_sequence_unchanged():
    x = arange_hist(15)
    st = oracle.from_scratch([x, x], [x, x], (4,), [3])  # 3 entries used, capacity 3
    par = np.array([[-1, 0, 1], [-1, 0, 1]])
    draft = np.array([[0, 1, 2], [0, 5, 6]])
    target = np.array([[1, 2, 3], [9, 9, 9]])  # seq 0 accepts 2 drafts, seq 1 none
    kt = np.ones((2, 3, 1, 3))
    r = oracle.step(st, par, draft, target, np.zeros((2, 3, 1, 3)), kt, kt)
    # seq 0: P 15 -> 18 closes block 3 -> needs slot 3 > capacity -> POOL_FULL
    assert r.err[0] == oracle.SEQ_POOL_FULL and r.state.P[0] == 15 and r.state.n[0][0] == 3
    # seq 1: P 15 -> 16 also closes block 3 ((15 + 1) % 4 == 0) -> POOL_FULL as well
    assert r.err[1] == oracle.SEQ_POOL_FULL
    st2 = oracle.from_scratch([x[:, :13], x[:, :13]], [x[:, :13], x[:, :13]], (4,), [3])
    r2 = oracle.step(st2, par, draft, target, np.zeros((2, 3, 1, 3)), kt, kt)
    # seq 1: P 13 -> 14, no block closes -> fine; seq 0: 13 -> 16 closes block 3 -> full
    assert r2.err[1] == 0 and r2.state.P[1] == 14
    assert r2.err[0] == oracle.SEQ_POOL_FULL
