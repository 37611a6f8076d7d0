"""Seeded synthetic inputs for the target-verify path.

This module only *draws* inputs: draft trees, draft/target token ids, Q/K/V values
and initial compressed-pool contents.  It computes none of the verify path itself
(no tree plan, no attention, no compression of a prefix, no acceptance, no refresh),
so the fp64 oracle and the HIP path can both take their inputs from here and see
identical bits while sharing no arithmetic.

Source of the workload shapes: "Adapting Tree-Structured Speculative Decoding to
DeepSeek-V4 for Efficient Inference" (cited as TSD-V4).  §2.1 gives the shape of a
draft tree (top-k expansion for a number of drafting steps, then pruning to a
verification budget of D tokens), §5.1 names configurations "sS_kK_dD" (draft steps,
top-k, budget) and sweeps D in 5..8 and batch 1..64.  The pages run a real model on
GSM8K / MBPP / ShareGPT; none of that is available, so a per-node agreement
probability ``p_agree`` stands in for task predictability (high p ~ regular reasoning
chains, low p ~ divergent dialogue).

Conventions shared with the C ABI (layouts, not arithmetic):
  * ``parents[b][i]``: parent of node i, ``parents[b][0] == -1``, ``0 <= parents[i] < i``.
  * D counts the root (node 0 = last committed-but-not-yet-cached token).
  * bf16 values are carried as ``numpy.uint16`` bit patterns; fp32 as ``float32``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

# Independent random streams, keyed by SeedSequence spawn_key.
_STREAM_PREFIX = 0
_STREAM_TREE = 1
_STREAM_QKV = 2
_STREAM_RAWHIST = 3


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, dtype, tree recipe and seed."""

    name: str
    B: int                 # batch (sequences)
    D: int                 # verified tree nodes per sequence, root included
    Hq: int                # query heads
    Hkv: int               # KV heads (grouped-query: Hq % Hkv == 0)
    d: int                 # head dim
    dtype: str             # "f32" or "bf16" (storage and input dtype)
    levels: Tuple[int, ...]  # compression block sizes, finest first (e.g. (4, 128))
    P: int                 # committed prefix length at step 0
    topk: int              # draft top-k
    steps: int             # drafting steps
    p_agree: float         # probability that the target agrees with a draft child
    seed: int
    prefix: str = "pooled"  # "raw": raw prefix tokens are drawn (both sides compress them)
                            # "pooled": compressed pool entries are drawn directly
    vocab: int = 1024

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def n_entries(self) -> Tuple[int, ...]:
        return tuple(self.P // c for c in self.levels)

    @property
    def spec_name(self) -> str:
        """The pages' configuration naming: draft steps / top-k / budget."""
        return f"s{self.steps}_k{self.topk}_d{self.D}"

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _mk(name, B, D, Hq, Hkv, d, dtype, levels, P, topk, steps, p, seed, prefix="pooled"):
    return Workload(name=name, B=B, D=D, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype,
                    levels=tuple(levels), P=P, topk=topk, steps=steps, p_agree=p,
                    seed=seed, prefix=prefix)


#: The named workloads.  Tiny is the small fp32 parity case; High batch is the
#: throughput workload (B=64, D=8, 64/8 heads, d=128, bf16, 32768-token prefix); wide_tree
#: is the same batch with a 16-node tree (top-k 2, 4 steps), 128 query rows per KV head.
WORKLOADS: Dict[str, Workload] = {
    "tiny": _mk("tiny", 1, 6, 4, 1, 64, "f32", (4,), 256, 2, 3, 0.6, 1000, prefix="raw"),
    "linear": _mk("linear", 8, 8, 64, 8, 128, "bf16", (4, 128), 4096, 1, 7, 0.7, 1001),
    "tree": _mk("tree", 4, 6, 64, 8, 128, "bf16", (4, 128), 8192, 2, 3, 0.5, 1002),
    "high_batch": _mk("high_batch", 64, 8, 64, 8, 128, "bf16", (4, 128), 32768, 2, 3, 0.6, 1003),
    "wide_tree": _mk("wide_tree", 64, 16, 64, 8, 128, "bf16", (4, 128), 32768, 2, 4, 0.6, 1004),
}


def sweep_workloads() -> List[Workload]:
    """Budget sweep at long context: D in 5..8 x batch in {1,4,16,64} x top-k {1,2} x p {0.5,0.7}."""
    out = []
    idx = 0
    for D in (5, 6, 7, 8):
        for B in (1, 4, 16, 64):
            for k in (1, 2):
                for p in (0.5, 0.7):
                    steps = D - 1 if k == 1 else 3
                    out.append(_mk(f"sweep_s{steps}_k{k}_d{D}_b{B}_p{p}", B, D, 64, 8, 128, "bf16",
                                   (4, 128), 131072, k, steps, p, 1100 + idx))
                    idx += 1
    return out


# ----------------------------------------------------------------------------- rng

def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


# ----------------------------------------------------------------------------- bf16 bits

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # no wrap-around for any finite value or infinity; NaNs are fixed up below
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _values(rng: np.random.Generator, shape, dtype: str, scale: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


# ----------------------------------------------------------------------------- trees

def draft_tree(rng: np.random.Generator, topk: int, steps: int, D: int,
               vocab: int = 1024) -> Tuple[np.ndarray, np.ndarray]:
    """One draft tree of D nodes (root included), as (parents, draft_tokens).

    Expansion: every node of the last level gets the top-k tokens of its own draft
    distribution, for ``steps`` levels (TSD-V4 §2.1, the expanded candidate tree).
    The draft distribution of each expanded node is log_softmax of iid Gumbel(0,1)
    noise over the vocabulary.  Pruning keeps the D-1 non-root candidates with the
    highest cumulative draft log-probability (TSD-V4 §2.1, budget-aware pruning);
    ties go to the shallower, then the earlier-created candidate.  Because every
    increment is strictly negative an ancestor always outranks its descendants, so
    the kept set is connected.  Nodes are numbered root first, then by rank, which
    makes every parent index smaller than its child's.
    """
    if D < 1:
        raise ValueError("D must be >= 1")
    par = [-1]
    dep = [0]
    tok = [int(rng.integers(vocab))]
    cum = [0.0]
    frontier = [0]
    for _ in range(steps):
        nxt = []
        for u in frontier:
            g = rng.gumbel(size=vocab)
            gmax = g.max()
            lse = gmax + math.log(np.exp(g - gmax).sum())
            top = np.argsort(-g, kind="stable")[:topk]
            for t in top:
                par.append(u)
                dep.append(dep[u] + 1)
                tok.append(int(t))
                cum.append(cum[u] + float(g[t] - lse))
                nxt.append(len(par) - 1)
        frontier = nxt
    if len(par) - 1 < D - 1:
        raise ValueError(f"tree of {len(par)} candidates cannot fill budget D={D}")
    ranked = sorted(range(1, len(par)), key=lambda c: (-cum[c], dep[c], c))[: D - 1]
    keep = [0] + ranked
    pos = {c: i for i, c in enumerate(keep)}
    parents = np.array([-1] + [pos[par[c]] for c in ranked], dtype=np.int32)
    draft = np.array([tok[c] for c in keep], dtype=np.int32)
    return parents, draft


def target_tokens(rng: np.random.Generator, parents: np.ndarray, draft: np.ndarray,
                  p_agree: float, vocab: int = 1024) -> np.ndarray:
    """Target-model token after each node (its greedy next token), drawn synthetically.

    For a node u with kept children c1, c2, ... (in index order), the target agrees
    with c1's draft token with probability p; otherwise with c2's with probability p;
    and so on.  If none is chosen the target token is uniform over the vocabulary
    minus the children's tokens.  Leaves get a uniform token (the bonus token).
    """
    D = len(parents)
    children: List[List[int]] = [[] for _ in range(D)]
    for i in range(1, D):
        children[int(parents[i])].append(i)
    tgt = np.empty(D, dtype=np.int32)
    for u in range(D):
        chosen = None
        for c in children[u]:
            if rng.random() < p_agree:
                chosen = int(draft[c])
                break
        if chosen is None:
            excl = {int(draft[c]) for c in children[u]}
            while True:
                t = int(rng.integers(vocab))
                if t not in excl:
                    break
            chosen = t
        tgt[u] = chosen
    return tgt


# ----------------------------------------------------------------------------- step inputs

@dataclasses.dataclass
class StepInputs:
    parents: np.ndarray    # [B][D] int32
    draft: np.ndarray      # [B][D] int32
    target: np.ndarray     # [B][D] int32
    q: np.ndarray          # [B][D][Hq][d]  (uint16 bf16 bits or float32)
    k_tree: np.ndarray     # [B][D][Hkv][d]
    v_tree: np.ndarray     # [B][D][Hkv][d]


def step_inputs(w: Workload, step: int, q_scale: float = 1.0,
                batch: Optional[range] = None) -> StepInputs:
    """Inputs of decoding step ``step``; sequence b's draws depend only on (seed, step, b)."""
    bs = list(batch) if batch is not None else list(range(w.B))
    par, dr, tg, qs, ks, vs = [], [], [], [], [], []
    for b in bs:
        rt = _rng(w.seed, _STREAM_TREE, step, b)
        p_, d_ = draft_tree(rt, w.topk, w.steps, w.D, w.vocab)
        t_ = target_tokens(rt, p_, d_, w.p_agree, w.vocab)
        par.append(p_); dr.append(d_); tg.append(t_)
        rv = _rng(w.seed, _STREAM_QKV, step, b)
        qs.append(_values(rv, (w.D, w.Hq, w.d), w.dtype, q_scale))
        ks.append(_values(rv, (w.D, w.Hkv, w.d), w.dtype))
        vs.append(_values(rv, (w.D, w.Hkv, w.d), w.dtype))
    return StepInputs(np.stack(par), np.stack(dr), np.stack(tg),
                      np.stack(qs), np.stack(ks), np.stack(vs))


def raw_prefix(w: Workload, b: int, length: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Raw (uncompressed) prefix K, V of sequence b: [Hkv][length][d], N(0,1) values."""
    L = w.P if length is None else length
    r = _rng(w.seed, _STREAM_RAWHIST, b)
    return _values(r, (w.Hkv, L, w.d), w.dtype), _values(r, (w.Hkv, L, w.d), w.dtype)


def pooled_prefix(w: Workload, b: int) -> List[Tuple[np.ndarray, np.ndarray]]:
    """Committed compressed entries of sequence b, drawn directly: per level (K, V) [Hkv][n_C][d].

    A mean over C iid N(0,1) tokens is N(0, 1/C); the entries are drawn from that
    law directly (independently per level), which keeps multi-GB prefixes cheap to
    generate.  Used only where P is a multiple of every level's C, so the open
    block of every level is empty at step 0.
    """
    out = []
    r = _rng(w.seed, _STREAM_PREFIX, b)
    for C, n in zip(w.levels, w.n_entries):
        s = 1.0 / math.sqrt(C)
        out.append((_values(r, (w.Hkv, n, w.d), w.dtype, s), _values(r, (w.Hkv, n, w.d), w.dtype, s)))
    return out

