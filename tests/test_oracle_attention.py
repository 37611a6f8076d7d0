"""Pins of the oracle's branch-aware attention (O2): per-path causal attention computed
alone by torch's SDPA (a library routine), D = 1 and chain reductions, the Q = 0
closed form, node relabelling, a hand-worked example, and a check that the mask
matters on tree-dominant inputs.  CPU only, float64."""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rand_state(rng, B, Hkv, d, levels, P, caps=None):
    hk = [rng.standard_normal((Hkv, P, d)) for _ in range(B)]
    hv = [rng.standard_normal((Hkv, P, d)) for _ in range(B)]
    caps = caps or [P // c + 8 for c in levels]
    return oracle.from_scratch(hk, hv, levels, caps)


def rand_tree(rng, D):
    return np.array([-1] + [int(rng.integers(0, i)) for i in range(1, D)])


def visible_prefix(st, b, g):
    """What the shared prefix holds for (b, g), assembled from the state's arrays."""
    ks, vs = [], []
    for l in range(len(st.levels)):
        ks.append(st.pool_k[l][b, g, :st.n[l][b]])
        vs.append(st.pool_v[l][b, g, :st.n[l][b]])
    r = st.P[b] % st.levels[0]
    ks.append(st.tail_k[b, g, :r])
    vs.append(st.tail_v[b, g, :r])
    return np.concatenate(ks), np.concatenate(vs)


def sdpa_path(q_rows, k_rows, v_rows, n_prefix):
    """Causal attention of the path tokens over prefix + path (library routine).

    q_rows [T][d] are the path tokens' queries for one head; keys are prefix rows
    followed by the T path rows; path row t sees the whole prefix and path rows 0..t.
    """
    T = q_rows.shape[0]
    N = n_prefix + T
    mask = torch.zeros(T, N, dtype=torch.bool)
    mask[:, :n_prefix] = True
    mask[:, n_prefix:] = torch.tril(torch.ones(T, T, dtype=torch.bool))
    q = torch.from_numpy(q_rows)[None, None]
    k = torch.from_numpy(k_rows)[None, None]
    v = torch.from_numpy(v_rows)[None, None]
    return F.scaled_dot_product_attention(q, k, v, attn_mask=mask[None, None])[0, 0].numpy()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tree_equals_each_path_alone(seed):
    rng = np.random.default_rng(seed)
    B, D, Hq, Hkv, d = 2, 9, 4, 2, 16
    levels, P = (4, 16), 41 + seed
    st = rand_state(rng, B, Hkv, d, levels, P)
    par = np.stack([rand_tree(rng, D) for _ in range(B)])
    q = rng.standard_normal((B, D, Hq, d)) * 2
    kt = rng.standard_normal((B, D, Hkv, d))
    vt = rng.standard_normal((B, D, Hkv, d))
    anc, depth, err = oracle.build_plan(par)
    out, lse = oracle.verify_attention(q, kt, vt, anc, st, err)
    G = Hq // Hkv
    for b in range(B):
        for leaf in range(D):
            path = []
            u = leaf
            while u != -1:
                path.append(u)
                u = int(par[b, u])
            path = path[::-1]
            for h in range(Hq):
                g = h // G
                pk, pv = visible_prefix(st, b, g)
                ref = sdpa_path(q[b, path, h], np.concatenate([pk, kt[b, path, g]]),
                                np.concatenate([pv, vt[b, path, g]]), len(pk))
                np.testing.assert_allclose(out[b, path, h], ref, rtol=0, atol=1e-12)


def test_lse_is_logsumexp_of_visible_scores():
    rng = np.random.default_rng(5)
    B, D, Hq, Hkv, d = 1, 6, 2, 1, 8
    st = rand_state(rng, B, Hkv, d, (4,), 23)
    par = rand_tree(rng, D)[None]
    q = rng.standard_normal((B, D, Hq, d))
    kt = rng.standard_normal((B, D, Hkv, d))
    vt = rng.standard_normal((B, D, Hkv, d))
    anc, depth, err = oracle.build_plan(par)
    out, lse = oracle.verify_attention(q, kt, vt, anc, st)
    pk, _ = visible_prefix(st, 0, 0)
    for i in range(D):
        keys = np.concatenate([pk, kt[0, np.nonzero(anc[0, i])[0], 0]])
        for h in range(Hq):
            s = torch.from_numpy(keys @ q[0, i, h] / math.sqrt(d))
            assert abs(lse[0, i, h] - torch.logsumexp(s, 0).item()) < 1e-12


def test_single_node_is_plain_attention():
    rng = np.random.default_rng(9)
    B, Hq, Hkv, d = 3, 8, 2, 32
    st = rand_state(rng, B, Hkv, d, (4, 128), 389)
    q = rng.standard_normal((B, 1, Hq, d))
    kt = rng.standard_normal((B, 1, Hkv, d))
    vt = rng.standard_normal((B, 1, Hkv, d))
    anc, depth, err = oracle.build_plan(np.full((B, 1), -1))
    out, _ = oracle.verify_attention(q, kt, vt, anc, st)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            pk, pv = visible_prefix(st, b, g)
            k = torch.from_numpy(np.concatenate([pk, kt[b, :, g]]))[None, None]
            v = torch.from_numpy(np.concatenate([pv, vt[b, :, g]]))[None, None]
            ref = F.scaled_dot_product_attention(torch.from_numpy(q[b, :, h])[None, None], k, v)
            np.testing.assert_allclose(out[b, 0, h], ref[0, 0, 0].numpy(), rtol=0, atol=1e-12)


def test_chain_is_causal_attention():
    rng = np.random.default_rng(10)
    D, Hq, Hkv, d = 7, 4, 1, 16
    st = rand_state(rng, 1, Hkv, d, (4,), 30)
    par = np.array([[-1] + list(range(D - 1))])
    q = rng.standard_normal((1, D, Hq, d))
    kt = rng.standard_normal((1, D, Hkv, d))
    vt = rng.standard_normal((1, D, Hkv, d))
    anc, _, _ = oracle.build_plan(par)
    out, _ = oracle.verify_attention(q, kt, vt, anc, st)
    pk, pv = visible_prefix(st, 0, 0)
    for h in range(Hq):
        ref = sdpa_path(q[0, :, h], np.concatenate([pk, kt[0, :, 0]]), np.concatenate([pv, vt[0, :, 0]]), len(pk))
        np.testing.assert_allclose(out[0, :, h], ref, rtol=0, atol=1e-12)


def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(12)
    B, D, Hq, Hkv, d = 2, 8, 4, 2, 8
    st = rand_state(rng, B, Hkv, d, (4, 8), 37)
    par = np.stack([rand_tree(rng, D) for _ in range(B)])
    q = np.zeros((B, D, Hq, d))
    kt = rng.standard_normal((B, D, Hkv, d))
    vt = rng.standard_normal((B, D, Hkv, d))
    anc, depth, _ = oracle.build_plan(par)
    out, lse = oracle.verify_attention(q, kt, vt, anc, st)
    for b in range(B):
        for h in range(Hq):
            g = h // 2
            _, pv = visible_prefix(st, b, g)
            for i in range(D):
                vis = np.nonzero(anc[b, i])[0]
                n_vis = len(pv) + len(vis)
                mean = (pv.sum(axis=0) + vt[b, vis, g].sum(axis=0)) / n_vis
                np.testing.assert_allclose(out[b, i, h], mean, rtol=0, atol=1e-12)
                assert abs(lse[b, i, h] - math.log(n_vis)) < 1e-12


def test_relabelling_permutes_outputs():
    """Renumbering nodes by another topological order permutes the outputs."""
    rng = np.random.default_rng(13)
    D, Hq, Hkv, d = 8, 2, 1, 8
    st = rand_state(rng, 1, Hkv, d, (4,), 22)
    par = np.array([-1, 0, 0, 1, 2, 1, 3, 4])
    # new order: 0,2,1,4,3,5,7,6 is topological for this tree
    perm = np.array([0, 2, 1, 4, 3, 5, 7, 6])
    inv = np.argsort(perm)
    par2 = np.array([-1 if par[perm[k]] == -1 else inv[par[perm[k]]] for k in range(D)])
    assert all(0 <= par2[i] < i for i in range(1, D))
    q = rng.standard_normal((1, D, Hq, d))
    kt = rng.standard_normal((1, D, Hkv, d))
    vt = rng.standard_normal((1, D, Hkv, d))
    a1, _, _ = oracle.build_plan(par[None])
    a2, _, _ = oracle.build_plan(par2[None])
    o1, _ = oracle.verify_attention(q, kt, vt, a1, st)
    o2, _ = oracle.verify_attention(q[:, perm], kt[:, perm], vt[:, perm], a2, st)
    np.testing.assert_allclose(o2[0], o1[0, perm], rtol=0, atol=1e-13)


def test_golden_chain2():
    g = json.load(open(os.path.join(GOLD, "attention_chain2.json")))
    d = g["d"]
    q = np.zeros((1, 2, 1, d))
    q[0, :, 0, 0] = 2 * math.log(3)
    st = oracle.from_entries([[(np.array(g["prefix_k"], float)[None], np.array(g["prefix_v"], float)[None])]],
                             [1], [1], [4], d)
    # one C = 1 level holding the single prefix entry: P = 1, n = 1, no tail
    kt = np.array(g["tree_k"], float)[None, :, None]
    vt = np.array(g["tree_v"], float)[None, :, None]
    anc, _, _ = oracle.build_plan(np.array([g["parents"]]))
    out, lse = oracle.verify_attention(q, kt, vt, anc, st)
    np.testing.assert_allclose(out[0, :, 0], np.array(g["out"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, :, 0], np.array(g["lse"]), rtol=0, atol=1e-12)


def test_mask_is_discriminating_on_tree_dominant_inputs():
    """With tree keys aligned to the queries, ignoring the mask changes outputs by far
    more than the bf16 tolerance: a GPU kernel with a mask bug cannot pass."""
    rng = np.random.default_rng(21)
    B, D, Hq, Hkv, d = 1, 8, 8, 1, 128
    st = rand_state(rng, B, Hkv, d, (4,), 64)
    par = np.array([[-1, 0, 0, 1, 1, 2, 2, 3]])
    q = rng.standard_normal((B, D, Hq, d))
    qbar = q.mean(axis=(1, 2))
    kt = 0.25 * qbar[:, None, None, :] + 0.1 * rng.standard_normal((B, D, Hkv, d))
    vt = rng.standard_normal((B, D, Hkv, d))
    anc, _, _ = oracle.build_plan(par)
    out, _ = oracle.verify_attention(q, kt, vt, anc, st)
    everything = np.ones_like(anc)
    out_all, _ = oracle.verify_attention(q, kt, vt, everything, st)
    assert np.abs(out - out_all).max() > 10 * 2e-2
