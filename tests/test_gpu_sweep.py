"""The long-context budget sweep (64/8 heads, d=128, bf16, 131072-token prefix compressed
to 32768 C4 + 1024 C128 entries; D in 5..8, top-k 1 or 2, batch 1..64) at full size, in
the launch configuration the sweep benchmark times (the library's own split plan): one
whole step per case.  Acceptance is bit-exact for every sequence; attention, the scratch
pad and the refreshed state are compared with the oracle on every sequence at batch 1 and
on sampled sequences at batch 64, counts and finiteness for all."""
import sys

import numpy as np
import pytest

import oracle
import synth
from harness import (Runner, check_attention, compare_state, device_state, host_f64, oracle_state, pooled_caps,
                     upload_step, widen_step)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _point(D, k, B, p):
    for w in synth.sweep_workloads():
        if (w.D, w.topk, w.B, w.p_agree) == (D, k, B, p):
            return w
    raise KeyError((D, k, B, p))


def _full_step(w, sample):
    import torch
    caps = pooled_caps(w, 64)
    _say(f"sweep {w.name}: building state")
    dst = device_state(w, caps, poison=True)
    ost = oracle_state(w, caps, batch=sample)
    s = synth.step_inputs(w, 0)
    r = Runner(dst, w.D, w.Hq)  # the library's split plan, as timed
    n_before = [dst.n[l].clone() for l in range(len(w.levels))]
    P_before = dst.P.clone()
    _say(f"sweep {w.name}: step")
    r.step(upload_step(s, w.dtype))
    torch.cuda.synchronize()

    anc, depth, err = oracle.build_plan(s.parents)
    m, path, bonus = oracle.accept(s.parents, anc, depth, s.draft, s.target, err)
    assert (r.m.cpu().numpy() == m).all() and (r.path.cpu().numpy() == path).all()
    assert (r.bonus.cpu().numpy() == bonus).all()
    assert (r.err.cpu().numpy() == 0).all()
    P2 = P_before.cpu().numpy() + m + 1
    assert (dst.P.cpu().numpy() == P2).all()
    for l, C in enumerate(w.levels):
        assert (dst.n[l].cpu().numpy() == P2 // C).all()
    out = host_f64(r.out, w.dtype)
    assert np.isfinite(out).all() and torch.isfinite(r.lse).all()

    _say(f"sweep {w.name}: oracle on sequences {sample}")
    ss = synth.step_inputs(w, 0, batch=sample)
    h = widen_step(ss, w.dtype)
    ref = oracle.step(ost, ss.parents, ss.draft, ss.target, h.q, h.kt, h.vt)
    check_attention(out[sample], ref.out, w.dtype)
    assert np.abs(r.lse.cpu().numpy()[sample] - ref.lse).max() <= 1e-2
    first = [n_before[l].cpu().numpy()[sample] for l in range(len(w.levels))]
    compare_state(dst, ref.state, w.dtype, w.name, batch=sample, first_entry=first)


@pytest.mark.parametrize("D,k", [(5, 1), (6, 2), (7, 1), (8, 2)])
def test_long_context_batch1(D, k):
    """Batch 1: 8 (sequence, KV head) units split over many workgroups, so every output
    row goes through the split-KV merge."""
    _full_step(_point(D, k, 1, 0.5), [0])


def test_long_context_batch64_sampled():
    """Batch 64, D=5 (40 query rows per KV head, a partial MFMA row block): 8.9 GB of
    compressed pools, one whole (sequence, KV head) prefix per workgroup."""
    _full_step(_point(5, 2, 64, 0.7), [0, 41, 63])


def test_long_context_batch16_split():
    """Batch 16, D=7 chains: 128 (sequence, KV head) prefixes over about 500 workgroups, so
    every prefix is split over several slices and merged; sampled sequences."""
    _full_step(_point(7, 1, 16, 0.7), [0, 7, 15])


def test_long_context_batch64_d8_sampled():
    """Batch 64, D=8 (64 query rows per KV head, whole MFMA row blocks), top-k 2: one
    whole prefix per workgroup, the scratch pad's workgroups behind the stream's."""
    _full_step(_point(8, 2, 64, 0.5), [0, 63])

