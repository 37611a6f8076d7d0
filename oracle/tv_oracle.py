"""Plain fp64 CPU oracle of the target-verify path of tree speculation on
compressed-attention KV.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` use it.  It shares no code with the HIP library (no kernels, headers,
helpers, tables or pre/post-processing); both take their inputs from the seeded
generator in ``synth/``.

Source: "Adapting Tree-Structured Speculative Decoding to DeepSeek-V4 for Efficient
Inference" (cited TSD-V4; the page has no numbered headings, the section numbers
below are inferred from its own cross-references "Sec. 5.2"/"Sec. 5.3" and the order
of topics):

  §3.1  a candidate attends to the accepted context and to the ancestors on its own
        branch only; the result of verification is a specific path, not a length.
  §3.2  compressed state built from tentative tokens must not leak; after acceptance
        token history, cache and compressed states must all describe one prefix.
  §4.1  verify preprocess turns the tree into a plan (chains + compression
        boundaries); branches are compressed independently after they diverge.
  §4.2  branch states live in a scratch pad until the path is known; then only the
        accepted path's states refresh the persistent state.
  §2.2  CSA/HCA compress along the sequence axis at several granularities.

The pages do not define the compressor.  The stand-in used throughout is the
unweighted mean over aligned blocks of C consecutive positions (C = 4 and C = 128,
the pages' "C4"/"C128"), separately for K and V and per KV head.

Every function below is the definition written out plainly in float64; loops are
over sequences, heads and nodes, and a library matrix product or sum is the only
vectorisation.  Readings of points the pages leave open are marked "Reading:".

Pins (see tests/test_oracle_*.py): brute-force ancestor walks over every tree with
D <= 7; per-node causal attention over the root-to-node path computed alone and by
torch's scaled_dot_product_attention; Q = 0 closed form; chain reduction to
prefix-match acceptance; from-scratch compression against closed forms; the
refreshed state after many steps equals compressing the committed history from
scratch.  The real CSA/HCA compressor and real-model acceptance are parity unpinned
(no definition, no model).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

SEQ_OK = 0
SEQ_BAD_PARENT = 1
SEQ_POOL_FULL = 2


# ----------------------------------------------------------------------------- inputs

def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of an input array ('bf16' = uint16 bit patterns, 'f32' = float32)."""
    if dtype == "bf16":
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------- O1 plan

def build_plan(parents: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Verification plan of each tree (TSD-V4 §4.1, verify preprocess).

    ``parents``: [B][D] int.  Returns ``anc`` [B][D][D] bool with anc[b,i,j] true iff
    node j is an ancestor of node i or i itself, ``depth`` [B][D] and ``err`` [B].
    A tree is valid iff parents[0] == -1 and 0 <= parents[i] < i for i >= 1
    (nodes in topological order).  Invalid trees get err = SEQ_BAD_PARENT and
    anc/depth all zero.

    The chains of the plan are the rows of ``anc`` read as node sets; a node closes a
    compression block of size C iff (P + depth + 1) is a multiple of C (the
    compression boundary of its chain).
    """
    parents = np.asarray(parents)
    B, D = parents.shape
    anc = np.zeros((B, D, D), dtype=bool)
    depth = np.zeros((B, D), dtype=np.int64)
    err = np.zeros(B, dtype=np.int64)
    for b in range(B):
        ok = parents[b, 0] == -1 and all(0 <= parents[b, i] < i for i in range(1, D))
        if not ok:
            err[b] = SEQ_BAD_PARENT
            continue
        anc[b, 0, 0] = True
        for i in range(1, D):
            p = int(parents[b, i])
            anc[b, i] = anc[b, p]
            anc[b, i, i] = True
            depth[b, i] = depth[b, p] + 1
    return anc, depth, err


def anc_to_bits(anc: np.ndarray) -> np.ndarray:
    """Pack anc [..][D][D] bool into uint64 masks (bit j = node j), for comparison with the ABI."""
    D = anc.shape[-1]
    w = np.array([1 << j for j in range(D)], dtype=np.uint64)
    return (anc.astype(np.uint64) * w).sum(axis=-1, dtype=np.uint64)


# ----------------------------------------------------------------------------- state

@dataclasses.dataclass
class State:
    """Persistent compressed state of B sequences, in float64.

    levels: compression block sizes, finest first.
    pool_k/pool_v[l]: [B][Hkv][cap_l][d] committed compressed entries (first n[l][b] valid).
    open_k/open_v[l]: [B][Hkv][d] sum of the committed tokens of the open block of level l.
    tail_k/tail_v:    [B][Hkv][C0-1][d] raw tokens of the open block of the finest level
                      (positions floor(P/C0)*C0 .. P-1; first P mod C0 valid).
    P: [B] committed length (tokens whose K/V are in the state).
    """

    levels: Tuple[int, ...]
    pool_k: List[np.ndarray]
    pool_v: List[np.ndarray]
    n: List[np.ndarray]
    open_k: List[np.ndarray]
    open_v: List[np.ndarray]
    tail_k: np.ndarray
    tail_v: np.ndarray
    P: np.ndarray

    def copy(self) -> "State":
        return State(self.levels, [a.copy() for a in self.pool_k], [a.copy() for a in self.pool_v],
                     [a.copy() for a in self.n], [a.copy() for a in self.open_k],
                     [a.copy() for a in self.open_v], self.tail_k.copy(), self.tail_v.copy(),
                     self.P.copy())


def from_scratch(hist_k: Sequence[np.ndarray], hist_v: Sequence[np.ndarray],
                 levels: Sequence[int], caps: Sequence[int]) -> State:
    """Compressed state of a committed raw history, computed directly (O6).

    hist_k[b], hist_v[b]: [Hkv][P_b][d] float64 raw K/V of sequence b's committed tokens.
    For level C: entry j = mean of positions jC .. jC+C-1 for every complete block;
    open sum = sum of the positions of the incomplete last block.  The finest level
    also keeps that block's raw tokens as the tail.  (TSD-V4 §2.2: sequence-axis
    compression; mean-pool stand-in.)
    """
    B = len(hist_k)
    Hkv, _, d = hist_k[0].shape
    levels = tuple(int(c) for c in levels)
    C0 = levels[0] if levels else 1
    st = State(levels,
               [np.zeros((B, Hkv, cap, d)) for cap in caps], [np.zeros((B, Hkv, cap, d)) for cap in caps],
               [np.zeros(B, dtype=np.int64) for _ in levels],
               [np.zeros((B, Hkv, d)) for _ in levels], [np.zeros((B, Hkv, d)) for _ in levels],
               np.zeros((B, Hkv, max(C0 - 1, 0), d)), np.zeros((B, Hkv, max(C0 - 1, 0), d)),
               np.zeros(B, dtype=np.int64))
    for b in range(B):
        P = hist_k[b].shape[1]
        st.P[b] = P
        for l, C in enumerate(levels):
            n = P // C
            if n > caps[l]:
                raise ValueError("pool capacity too small for the history")
            st.n[l][b] = n
            for j in range(n):
                st.pool_k[l][b, :, j] = hist_k[b][:, j * C:(j + 1) * C].sum(axis=1) / C
                st.pool_v[l][b, :, j] = hist_v[b][:, j * C:(j + 1) * C].sum(axis=1) / C
            st.open_k[l][b] = hist_k[b][:, n * C:P].sum(axis=1)
            st.open_v[l][b] = hist_v[b][:, n * C:P].sum(axis=1)
        if levels:
            t0 = (P // C0) * C0
            st.tail_k[b, :, :P - t0] = hist_k[b][:, t0:P]
            st.tail_v[b, :, :P - t0] = hist_v[b][:, t0:P]
    return st


def from_entries(entries: Sequence[Sequence[Tuple[np.ndarray, np.ndarray]]], P: Sequence[int],
                 levels: Sequence[int], caps: Sequence[int], d: int) -> State:
    """State whose committed compressed entries are given directly.

    entries[b][l] = (K, V) [Hkv][n_l][d] float64 for sequence b, level l.  Every P[b]
    must be a multiple of every level's C, so open sums are zero and the tail empty.
    """
    B = len(entries)
    levels = tuple(int(c) for c in levels)
    Hkv = entries[0][0][0].shape[0]
    C0 = levels[0]
    st = State(levels,
               [np.zeros((B, Hkv, cap, d)) for cap in caps], [np.zeros((B, Hkv, cap, d)) for cap in caps],
               [np.zeros(B, dtype=np.int64) for _ in levels],
               [np.zeros((B, Hkv, d)) for _ in levels], [np.zeros((B, Hkv, d)) for _ in levels],
               np.zeros((B, Hkv, C0 - 1, d)), np.zeros((B, Hkv, C0 - 1, d)),
               np.asarray(P, dtype=np.int64).copy())
    for b in range(B):
        for l, C in enumerate(levels):
            if P[b] % C != 0:
                raise ValueError("from_entries needs P to be a multiple of every C")
            k, v = entries[b][l]
            n = k.shape[1]
            if n != P[b] // C:
                raise ValueError("entry count does not match P // C")
            st.pool_k[l][b, :, :n] = k
            st.pool_v[l][b, :, :n] = v
            st.n[l][b] = n
    return st


# ----------------------------------------------------------------------------- O2 attention

def prefix_rows(st: State, b: int, g: int) -> Tuple[np.ndarray, np.ndarray]:
    """The shared visible prefix of sequence b for KV head g: (K, V) [N][d].

    Reading: one softmax spans every committed compressed entry of every level plus
    the raw tokens of the finest level's open block (TSD-V4 §2.2 "multi-resolution
    history"; §3.1 "the accepted context").  Compressed entries formed inside the
    tree during this verify are not attended (they only go to the scratch pad).
    """
    ks, vs = [], []
    for l in range(len(st.levels)):
        n = int(st.n[l][b])
        ks.append(st.pool_k[l][b, g, :n])
        vs.append(st.pool_v[l][b, g, :n])
    if st.levels:
        r = int(st.P[b]) % st.levels[0]
        ks.append(st.tail_k[b, g, :r])
        vs.append(st.tail_v[b, g, :r])
    d = st.tail_k.shape[-1]
    if not ks:
        return np.zeros((0, d)), np.zeros((0, d))
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


def verify_attention(q: np.ndarray, k_tree: np.ndarray, v_tree: np.ndarray,
                     anc: np.ndarray, st: State, err: Optional[np.ndarray] = None
                     ) -> Tuple[np.ndarray, np.ndarray]:
    """Branch-aware causal attention of the D tree nodes (TSD-V4 §3.1, §4.1 target verify).

    q: [B][D][Hq][d]; k_tree, v_tree: [B][D][Hkv][d]; anc from build_plan.
    Query head h reads KV head h // (Hq/Hkv).  For node i the visible rows are the
    shared prefix of ``prefix_rows`` and the tree nodes j with anc[i, j] (its
    ancestors and itself).  Non-visible rows are left out of the sum (never read),
    so their values cannot matter.  Scale 1/sqrt(d); no positional term inside the
    path (Q and K arrive position-encoded).

    Returns out [B][D][Hq][d] and lse [B][D][Hq] (natural log of the softmax
    denominator, including the max).  Sequences with err != 0 get zeros / -inf.
    """
    B, D, Hq, d = q.shape
    Hkv = k_tree.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, D, Hq, d))
    lse = np.full((B, D, Hq), -np.inf)
    scale = 1.0 / np.sqrt(d)
    for b in range(B):
        if err is not None and err[b] != 0:
            continue
        for g in range(Hkv):
            pk, pv = prefix_rows(st, b, g)
            for i in range(D):
                vis = np.nonzero(anc[b, i])[0]
                keys = np.concatenate([pk, k_tree[b, vis, g]], axis=0)
                vals = np.concatenate([pv, v_tree[b, vis, g]], axis=0)
                for h in range(g * G, (g + 1) * G):
                    s = keys @ q[b, i, h] * scale
                    M = s.max()
                    e = np.exp(s - M)
                    Z = e.sum()
                    out[b, i, h] = (e @ vals) / Z
                    lse[b, i, h] = M + np.log(Z)
    return out, lse


# ----------------------------------------------------------------------------- O3 scratch

@dataclasses.dataclass
class Scratch:
    """Per-branch compression results (TSD-V4 §4.2 scratch pad), per level l:

    entry_k/entry_v[l]: [B][D][Hkv][d] compressed entry of the block that node i closes
                        (only meaningful where closes[l][b, i]).
    closes[l]:          [B][D] bool: position P + depth(i) is the last of a C-block.
    open_k/open_v[l]:   [B][D][Hkv][d] sum of the open block after node i along its
                        own chain (zero when node i closes a block).
    """

    entry_k: List[np.ndarray]
    entry_v: List[np.ndarray]
    closes: List[np.ndarray]
    open_k: List[np.ndarray]
    open_v: List[np.ndarray]


def build_scratch(k_tree: np.ndarray, v_tree: np.ndarray, anc: np.ndarray, depth: np.ndarray,
                  st: State, err: Optional[np.ndarray] = None) -> Scratch:
    """Chain-wise compression of every node's own branch (TSD-V4 §4.1 compression
    boundaries, §4.2 per-chain temporary compressed states).

    Node i sits at position pos = P + depth(i).  Its block for level C starts at
    b0 = floor(pos / C) * C.  The block's tokens are the committed tokens at
    positions b0 .. P-1 (present only if b0 < P; their sum is the committed open
    sum of that level) followed by the tokens of i's own chain at positions
    max(b0, P) .. pos.  Tokens of other chains never enter (no mixing of chains).
    If pos + 1 is a multiple of C the block is complete: entry = sum / C, open = 0;
    otherwise open = sum.
    """
    B, D, Hkv, d = k_tree.shape
    L = len(st.levels)
    sc = Scratch([np.zeros((B, D, Hkv, d)) for _ in range(L)], [np.zeros((B, D, Hkv, d)) for _ in range(L)],
                 [np.zeros((B, D), dtype=bool) for _ in range(L)],
                 [np.zeros((B, D, Hkv, d)) for _ in range(L)], [np.zeros((B, D, Hkv, d)) for _ in range(L)])
    for b in range(B):
        if err is not None and err[b] != 0:
            continue
        P = int(st.P[b])
        for l, C in enumerate(st.levels):
            for i in range(D):
                pos = P + int(depth[b, i])
                b0 = (pos // C) * C
                sk = st.open_k[l][b].copy() if b0 < P else np.zeros((Hkv, d))
                sv = st.open_v[l][b].copy() if b0 < P else np.zeros((Hkv, d))
                for u in np.nonzero(anc[b, i])[0]:
                    if P + int(depth[b, u]) >= b0:
                        sk += k_tree[b, u]
                        sv += v_tree[b, u]
                if (pos + 1) % C == 0:
                    sc.closes[l][b, i] = True
                    sc.entry_k[l][b, i] = sk / C
                    sc.entry_v[l][b, i] = sv / C
                else:
                    sc.open_k[l][b, i] = sk
                    sc.open_v[l][b, i] = sv
    return sc


# ----------------------------------------------------------------------------- O4 accept

def accept(parents: np.ndarray, anc: np.ndarray, depth: np.ndarray,
           draft: np.ndarray, target: np.ndarray, err: Optional[np.ndarray] = None
           ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Greedy accepted-path selection (TSD-V4 §3.1, §4.1: the verify result is a path).

    Reading: a draft node i >= 1 is correct iff its token equals the target model's
    greedy token after its parent, target[parent(i)].  A node is accepted iff every
    node on its chain below the root is correct (the root is always accepted).  The
    accepted path ends at the deepest accepted node; among equally deep ones the
    smallest index wins.  Returns per sequence:
      m [B]:        depth of that node = number of accepted draft tokens,
      path [B][D]:  the path's nodes root first, -1 after position m,
      bonus [B]:    target token after the path's last node (the next root).
    Sequences with err != 0 get m = -1, path all -1, bonus = -1.
    """
    B, D = parents.shape
    m = np.full(B, -1, dtype=np.int64)
    path = np.full((B, D), -1, dtype=np.int64)
    bonus = np.full(B, -1, dtype=np.int64)
    for b in range(B):
        if err is not None and err[b] != 0:
            continue
        acc = np.zeros(D, dtype=bool)
        acc[0] = True
        for i in range(1, D):
            p = int(parents[b, i])
            acc[i] = acc[p] and int(draft[b, i]) == int(target[b, p])
        best = 0
        for i in range(D):
            if acc[i] and depth[b, i] > depth[b, best]:
                best = i
        m[b] = depth[b, best]
        for u in np.nonzero(anc[b, best])[0]:
            path[b, depth[b, u]] = u
        bonus[b] = target[b, best]
    return m, path, bonus


# ----------------------------------------------------------------------------- O5 refresh

def refresh(st: State, sc: Scratch, k_tree: np.ndarray, v_tree: np.ndarray,
            m: np.ndarray, path: np.ndarray, err: Optional[np.ndarray] = None
            ) -> Tuple[State, np.ndarray, np.ndarray]:
    """Accepted-path state refresh (TSD-V4 §3.2, §4.2 refresh; §4.3 C4/C128 states).

    The root and the m accepted drafts (path[0..m]) become committed tokens at
    positions P .. P+m; P' = P + m + 1.  For level C every block j that completes in
    that range, floor(P/C) <= j < floor(P'/C), takes the scratch entry of the path
    node at its last position (depth jC + C - 1 - P); the open sum becomes the path
    leaf's scratch open sum; the finest level's tail becomes the raw tokens at
    positions floor(P'/C0)*C0 .. P'-1 (old tail below P, path tokens from P on).
    Rejected nodes are never read.  If a level would exceed its pool capacity the
    sequence is left unchanged with err = SEQ_POOL_FULL.

    Returns (new state, commit_log [B][L][D][2] with (dst slot, src node) rows, -1
    padded, err').
    """
    new = st.copy()
    B, D = path.shape
    L = len(st.levels)
    log = np.full((B, L, D, 2), -1, dtype=np.int64)
    err2 = np.zeros(B, dtype=np.int64) if err is None else np.asarray(err, dtype=np.int64).copy()
    for b in range(B):
        if err2[b] != 0 or m[b] < 0:
            continue
        P = int(st.P[b])
        P2 = P + int(m[b]) + 1
        if any(P2 // C > st.pool_k[l].shape[2] for l, C in enumerate(st.levels)):
            err2[b] = SEQ_POOL_FULL
            continue
        leaf = int(path[b, m[b]])
        for l, C in enumerate(st.levels):
            r = 0
            for j in range(P // C, P2 // C):
                u = int(path[b, j * C + C - 1 - P])
                new.pool_k[l][b, :, j] = sc.entry_k[l][b, u]
                new.pool_v[l][b, :, j] = sc.entry_v[l][b, u]
                log[b, l, r] = (j, u)
                r += 1
            new.n[l][b] = P2 // C
            new.open_k[l][b] = sc.open_k[l][b, leaf]
            new.open_v[l][b] = sc.open_v[l][b, leaf]
        if L:
            C0 = st.levels[0]
            t_old, t_new = (P // C0) * C0, (P2 // C0) * C0
            for pos in range(t_new, P2):
                if pos < P:
                    new.tail_k[b, :, pos - t_new] = st.tail_k[b, :, pos - t_old]
                    new.tail_v[b, :, pos - t_new] = st.tail_v[b, :, pos - t_old]
                else:
                    u = int(path[b, pos - P])
                    new.tail_k[b, :, pos - t_new] = k_tree[b, u]
                    new.tail_v[b, :, pos - t_new] = v_tree[b, u]
        new.P[b] = P2
    return new, log, err2


# ----------------------------------------------------------------------------- one step

@dataclasses.dataclass
class StepResult:
    anc: np.ndarray
    depth: np.ndarray
    err: np.ndarray
    out: np.ndarray
    lse: np.ndarray
    scratch: Scratch
    m: np.ndarray
    path: np.ndarray
    bonus: np.ndarray
    commit_log: np.ndarray
    state: State


def step(st: State, parents, draft, target, q, k_tree, v_tree) -> StepResult:
    """One target-verify step: plan, attention + scratch, accept, refresh (TSD-V4 §4.4)."""
    anc, depth, err = build_plan(parents)
    out, lse = verify_attention(q, k_tree, v_tree, anc, st, err)
    sc = build_scratch(k_tree, v_tree, anc, depth, st, err)
    m, path, bonus = accept(parents, anc, depth, draft, target, err)
    new, log, err2 = refresh(st, sc, k_tree, v_tree, m, path, err)
    return StepResult(anc, depth, err2, out, lse, sc, m, path, bonus, log, new)
