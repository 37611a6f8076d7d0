"""GPU parity of tv_build_tree_mask and tv_accept against the oracle: bit-exact on every
tree with D <= 7, on random trees up to D = 64, on generator trees and on invalid trees."""
import itertools
import sys

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def all_trees(D):
    return np.array([(-1,) + t for t in itertools.product(*[range(i) for i in range(1, D)])], dtype=np.int32)


def random_trees(rng, B, D, mode):
    out = np.empty((B, D), dtype=np.int32)
    out[:, 0] = -1
    for b in range(B):
        for i in range(1, D):
            if mode == "chain":
                out[b, i] = i - 1
            elif mode == "star":
                out[b, i] = 0
            elif mode == "deep":
                out[b, i] = max(0, i - 1 - int(rng.integers(0, 2)))
            else:
                out[b, i] = int(rng.integers(0, i))
    return out


def gpu_plan(parents):
    import torch
    import tree_speculative_decoding_amd as tv
    B, D = parents.shape
    p = torch.from_numpy(parents).cuda()
    anc = torch.full((B, D), -7, dtype=torch.int64, device="cuda")
    depth = torch.full((B, D), -7, dtype=torch.int32, device="cuda")
    err = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    tv.tv_build_tree_mask(p, anc, depth, err)
    torch.cuda.synchronize()
    return anc.cpu().numpy().view(np.uint64), depth.cpu().numpy(), err.cpu().numpy()


def check_plan(parents):
    anc, depth, err = gpu_plan(parents)
    ra, rd, re = oracle.build_plan(parents)
    assert (err == re).all()
    assert (anc == oracle.anc_to_bits(ra)).all()
    assert (depth == rd).all()


@pytest.mark.parametrize("D", [1, 2, 3, 4, 5, 6, 7])
def test_plan_every_tree(D):
    _say(f"plan: every tree D={D}")
    check_plan(all_trees(D))


@pytest.mark.parametrize("D", [8, 13, 32, 63, 64])
@pytest.mark.parametrize("mode", ["random", "chain", "star", "deep"])
def test_plan_random_trees(D, mode):
    _say(f"plan: random trees D={D} {mode}")
    check_plan(random_trees(np.random.default_rng(D), 97, D, mode))


def test_plan_invalid_trees():
    _say("plan: invalid trees")
    good = random_trees(np.random.default_rng(1), 6, 9, "random")
    bad = good.copy()
    bad[0, 0] = 0          # root with a parent
    bad[1, 4] = 4          # self loop
    bad[2, 5] = 7          # forward reference
    bad[3, 8] = -1         # second root
    bad[4, 2] = 100        # out of range
    check_plan(np.concatenate([good, bad]))
    anc, depth, err = gpu_plan(bad)
    assert list(err) == [1, 1, 1, 1, 1, 0]
    assert (anc[:5] == 0).all() and (depth[:5] == 0).all()


def gpu_accept(parents, draft, target, seq_err=None):
    import torch
    import tree_speculative_decoding_amd as tv
    B, D = parents.shape
    i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()
    p = i32(parents)
    anc = torch.zeros((B, D), dtype=torch.int64, device="cuda")
    depth = torch.zeros((B, D), dtype=torch.int32, device="cuda")
    err = torch.zeros((B,), dtype=torch.int32, device="cuda")
    tv.tv_build_tree_mask(p, anc, depth, err)
    if seq_err is not None:
        err = i32(seq_err)
    m = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    path = torch.full((B, D), -7, dtype=torch.int32, device="cuda")
    bonus = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    tv.tv_accept(p, anc, depth, i32(draft), i32(target), err, m, path, bonus)
    torch.cuda.synchronize()
    return m.cpu().numpy(), path.cpu().numpy(), bonus.cpu().numpy()


def check_accept(parents, draft, target, seq_err=None):
    m, path, bonus = gpu_accept(parents, draft, target, seq_err)
    ra, rd, re = oracle.build_plan(parents)
    if seq_err is not None:
        re = np.asarray(seq_err)
    rm, rp, rb = oracle.accept(parents, ra, rd, draft, target, re)
    assert (m == rm).all(), (m, rm)
    assert (path == rp).all()
    assert (bonus == rb).all()


@pytest.mark.parametrize("D", [2, 3, 4, 5, 6, 7])
def test_accept_every_tree_small_vocab(D):
    _say(f"accept: every tree D={D}")
    par = all_trees(D)
    rng = np.random.default_rng(100 + D)
    for rep in range(3):
        draft = rng.integers(0, 2, size=par.shape).astype(np.int32)
        target = rng.integers(0, 2, size=par.shape).astype(np.int32)
        check_accept(par, draft, target)


@pytest.mark.parametrize("D", [8, 40, 64])
def test_accept_random_large_trees(D):
    _say(f"accept: random trees D={D}")
    rng = np.random.default_rng(D)
    for mode in ("random", "chain", "deep"):
        par = random_trees(rng, 200, D, mode)
        draft = rng.integers(0, 3, size=par.shape).astype(np.int32)
        target = rng.integers(0, 3, size=par.shape).astype(np.int32)
        check_accept(par, draft, target)


@pytest.mark.parametrize("k,steps,D,p", [(2, 3, 8, 0.6), (1, 7, 8, 0.7), (2, 3, 6, 0.5), (2, 4, 7, 0.9)])
def test_accept_generator_trees(k, steps, D, p):
    _say(f"accept: generator trees s{steps}_k{k}_d{D}")
    w = synth.Workload("acc", 300, D, 1, 1, 8, "f32", (4,), 0, k, steps, p, 9000 + D)
    s = synth.step_inputs(w, 0)
    check_accept(s.parents, s.draft, s.target)


def test_accept_skips_flagged_sequences():
    _say("accept: flagged sequences")
    w = synth.Workload("acc", 8, 8, 1, 1, 8, "f32", (4,), 0, 2, 3, 0.8, 9100)
    s = synth.step_inputs(w, 0)
    err = np.array([0, 1, 0, 2, 0, 0, 3, 0], dtype=np.int32)
    check_accept(s.parents, s.draft, s.target, err)
    m, path, bonus = gpu_accept(s.parents, s.draft, s.target, err)
    assert (m[err != 0] == -1).all() and (path[err != 0] == -1).all() and (bonus[err != 0] == -1).all()
