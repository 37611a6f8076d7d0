"""Device draft-tree construction against the oracle (oracle/draft_tree.py): parents
and draft tokens bit-exact, scores within fp32 rounding, over tree shapes from a chain
to the largest candidate count, flat and -inf logits, ragged vocabularies, D = 1, and
the device tree fed straight into the plan kernel."""
import sys

import numpy as np
import pytest

import oracle
from oracle.draft_tree import build_draft_tree, expanded_count

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_device(logits, root, k, s, D):
    import torch
    import tree_speculative_decoding_amd as tv
    B = logits.shape[0]
    lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).cuda()
    rt = torch.from_numpy(np.ascontiguousarray(root, dtype=np.int32)).cuda()
    par = torch.full((B, D), -7, dtype=torch.int32, device="cuda")
    tok = torch.full((B, D), -7, dtype=torch.int32, device="cuda")
    cum = torch.full((B, D), float("nan"), dtype=torch.float32, device="cuda")
    tv.tv_build_draft_tree(lg, rt, k, s, par, tok, cum)
    torch.cuda.synchronize()
    return par.cpu().numpy(), tok.cpu().numpy(), cum.cpu().numpy()


def check(logits, root, k, s, D):
    par, tok, cum = run_device(logits, root, k, s, D)
    # the oracle sees the same float32 logits, widened exactly
    opar, otok, ocum = build_draft_tree(np.asarray(logits, dtype=np.float32).astype(np.float64), root, k, s, D)
    assert (par == opar).all(), "parents differ"
    assert (tok == otok).all(), "draft tokens differ"
    fin = np.isfinite(ocum)
    assert (np.isfinite(cum) == fin).all()
    assert np.abs(cum[fin] - ocum[fin]).max(initial=0.0) <= 1e-5 * (1.0 + np.abs(ocum[fin]).max(initial=0.0))
    return par, tok


CASES = [  # (topk, steps, D, vocab, B)
    (2, 3, 8, 1024, 256),    # the pages' s3_k2 shape at D = 8
    (2, 3, 6, 1024, 128),    # s3_k2_d6
    (1, 7, 8, 1024, 64),     # linear chain s7_k1_d8
    (2, 4, 8, 1000, 64),     # s4_k2, ragged vocabulary
    (2, 3, 15, 257, 64),     # every candidate kept
    (3, 3, 20, 513, 32),
    (4, 3, 64, 300, 16),     # D = TV_MAX_D
    (16, 2, 64, 100, 8),     # wide: 272 candidates
    (2, 10, 64, 37, 2),      # 2046 candidates, 1023 expanded rows
    (2, 3, 8, 2000, 16),     # vocabulary past the 1024 kept in registers
]


@pytest.mark.parametrize("k,s,D,V,B", CASES)
def test_gumbel_logits(k, s, D, V, B):
    _say(f"draft tree k={k} s={s} D={D} V={V} B={B}")
    rng = np.random.default_rng(500 + k * 31 + s * 7 + D)
    logits = rng.gumbel(size=(B, expanded_count(k, s), V)).astype(np.float32)
    root = rng.integers(V, size=B)
    check(logits, root, k, s, D)


def test_root_only():
    rng = np.random.default_rng(3)
    logits = rng.gumbel(size=(4, 7, 64)).astype(np.float32)
    par, tok = check(logits, np.array([5, 6, 7, 8]), 2, 3, 1)
    assert par[:, 0].tolist() == [-1] * 4 and tok[:, 0].tolist() == [5, 6, 7, 8]


def test_flat_rows_tie_break():
    # every logit equal: ties everywhere, resolved by token id, depth and creation order
    logits = np.zeros((3, expanded_count(2, 3), 50), dtype=np.float32)
    par, tok = check(logits, np.array([1, 2, 3]), 2, 3, 8)
    assert par[0].tolist() == [-1, 0, 0, 1, 1, 2, 2, 3]
    assert tok[0].tolist() == [1, 0, 1, 0, 1, 0, 1, 0]


def test_quantised_logits_and_minus_inf():
    # coarse logits (many exact ties) with some tokens masked to -inf
    rng = np.random.default_rng(11)
    k, s, V, B = 3, 3, 96, 32
    logits = np.round(rng.normal(size=(B, expanded_count(k, s), V)) * 2.0).astype(np.float32) / 2.0
    logits[rng.random(logits.shape) < 0.3] = -np.inf
    check(logits, rng.integers(V, size=B), k, s, 13)


def test_device_tree_feeds_the_plan():
    import torch
    import tree_speculative_decoding_amd as tv
    rng = np.random.default_rng(21)
    k, s, D, V, B = 2, 3, 8, 1024, 64
    logits = rng.gumbel(size=(B, expanded_count(k, s), V)).astype(np.float32)
    root = rng.integers(V, size=B)
    lg = torch.from_numpy(logits).cuda()
    rt = torch.from_numpy(root.astype(np.int32)).cuda()
    par = torch.zeros(B, D, dtype=torch.int32, device="cuda")
    tok = torch.zeros(B, D, dtype=torch.int32, device="cuda")
    anc = torch.zeros(B, D, dtype=torch.int64, device="cuda")
    depth = torch.zeros(B, D, dtype=torch.int32, device="cuda")
    err = torch.full((B,), 9, dtype=torch.int32, device="cuda")
    tv.tv_build_draft_tree(lg, rt, k, s, par, tok)
    tv.tv_build_tree_mask(par, anc, depth, err)
    torch.cuda.synchronize()
    opar, _, _ = build_draft_tree(logits.astype(np.float64), root, k, s, D)
    oanc, odepth, oerr = oracle.build_plan(opar)
    assert (err.cpu().numpy() == 0).all() and (oerr == 0).all()
    assert (anc.cpu().numpy().view(np.uint64) == oracle.anc_to_bits(oanc)).all()
    assert (depth.cpu().numpy() == odepth).all()
