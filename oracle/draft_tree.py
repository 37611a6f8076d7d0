"""Plain fp64 CPU oracle of draft-tree construction (expansion and budget pruning).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and bench.py's CPU-baseline leg may use it; it shares no
code with the HIP library.

Source: TSD-V4 §2.1 (the draft expands the accepted prefix into a candidate tree, then
pruning keeps promising candidates so that the verified tokens stay within the
verification budget; Fig. 1: top-k = 2 over three drafting steps), §4.1 (draft extend
organises the candidate topology; the final shape depends on the draft outputs, the
branch parameters and the budget) and §4.3 (such metadata can be prepared on the
device).  The pages give no formula; the readings below are the plainest ones the
text supports.

Reading (expansion): every node created in the first ``steps - 1`` levels, and the
root, is expanded: its children are the ``topk`` tokens with the largest logits of its
own draft distribution (ties: the smaller token id first).  Nodes are created level by
level, a level's nodes in the order of their parents, a parent's children in top-k
order; so node e's children are nodes e*topk + 1 .. e*topk + topk, and the expanded
nodes are 0 .. E-1 with E = 1 + topk + ... + topk^(steps-1).
Reading (score): a child's cumulative draft log-probability is its parent's plus
log_softmax(logits of the parent)[token]; the root's is 0.
Reading (pruning): keep the D - 1 non-root candidates with the highest cumulative
log-probability, ties to the shallower, then the earlier-created one.  A log-softmax
value is <= 0, so a child never outranks its parent and the kept set is connected.
Reading (numbering): root first, then the kept candidates in rank order; so every
parent index is smaller than its child's.

Precision: the ranking is decided in float64 on both sides (an integer result decided
by floating point).  Pins: tests/test_oracle_draft_tree.py (brute force over root-to-
node paths, the topk = 1 chain closed form, a hand-worked example, invariants).
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def expanded_count(topk: int, steps: int) -> int:
    """E: the root and every candidate of depth < steps (each gets one logits row)."""
    return sum(topk ** l for l in range(steps))


def candidate_count(topk: int, steps: int) -> int:
    """N: candidates below the root after `steps` levels of expansion."""
    return sum(topk ** l for l in range(1, steps + 1))


def build_draft_tree(logits: np.ndarray, root_tok: np.ndarray, topk: int, steps: int,
                     D: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Draft trees of D nodes from the expanded nodes' logits.

    logits [B][E][V] (row e = logits of the draft distribution after node e),
    root_tok [B].  Returns parents [B][D] int32 (parents[:, 0] = -1), draft tokens
    [B][D] int32 and cumulative draft log-probabilities [B][D] float64.
    """
    logits = np.asarray(logits, dtype=np.float64)
    B, E, V = logits.shape
    if E != expanded_count(topk, steps):
        raise ValueError("one logits row per expanded node is needed")
    if not 1 <= D <= candidate_count(topk, steps) + 1:
        raise ValueError("budget D outside 1 .. candidates + 1")
    parents = np.full((B, D), -1, dtype=np.int32)
    draft = np.zeros((B, D), dtype=np.int32)
    cum_out = np.zeros((B, D), dtype=np.float64)
    for b in range(B):
        # expansion, level by level
        par = [-1]
        dep = [0]
        tok = [int(root_tok[b])]
        cum = [0.0]
        frontier = [0]
        for _ in range(steps):
            nxt = []
            for u in frontier:
                row = logits[b, u]
                m = row.max()
                lse = m + np.log(np.sum(np.exp(row - m)))
                order = sorted(range(V), key=lambda t: (-row[t], t))[:topk]
                for t in order:
                    par.append(u)
                    dep.append(dep[u] + 1)
                    tok.append(t)
                    cum.append(cum[u] + (row[t] - lse))
                    nxt.append(len(par) - 1)
            frontier = nxt
        # pruning to the budget
        ranked = sorted(range(1, len(par)), key=lambda c: (-cum[c], dep[c], c))[: D - 1]
        keep = [0] + ranked
        slot = {c: i for i, c in enumerate(keep)}
        for i, c in enumerate(keep):
            parents[b, i] = -1 if c == 0 else slot[par[c]]
            draft[b, i] = tok[c]
            cum_out[b, i] = cum[c]
    return parents, draft, cum_out
