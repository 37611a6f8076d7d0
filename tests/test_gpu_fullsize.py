"""The throughput workload at full size (B=64, D=8, 64/8 heads, d=128, bf16, 32768-token
prefix compressed to 8192 C4 + 256 C128 entries), and the same batch with a 16-node tree,
in the launch configuration the benchmark times: acceptance bit-exact for every
sequence; attention, scratch and the refreshed state compared with the oracle on sampled
sequences; counts and finiteness checked for all."""
import sys

import numpy as np
import pytest

import oracle
import synth
from harness import (Runner, check_attention, compare_state, device_state, host_f64, oracle_state, pooled_caps,
                     upload_step, widen_step)

pytestmark = pytest.mark.gpu

SAMPLE = [0, 29, 63]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("name", ["high_batch", "wide_tree"])
def test_full_size(name):
    """high_batch: 64 query rows per KV head (4-wave units); wide_tree: D = 16, 128 rows
    per KV head (8-wave units)."""
    import torch
    w = synth.WORKLOADS[name]
    _say(f"full size {name}: building state")
    caps = pooled_caps(w, 64)
    dst = device_state(w, caps, poison=True)
    ost = oracle_state(w, caps, batch=SAMPLE)
    s = synth.step_inputs(w, 0)
    x = upload_step(s, w.dtype)
    r = Runner(dst, w.D, w.Hq)  # auto split plan, as timed
    _say(f"full size: step ({r.ws.numel() * 4} B workspace)")
    n_before = [dst.n[l].clone() for l in range(len(w.levels))]
    P_before = dst.P.clone()
    r.step(x)
    torch.cuda.synchronize()

    # acceptance for every sequence: bit-exact
    anc, depth, err = oracle.build_plan(s.parents)
    m, path, bonus = oracle.accept(s.parents, anc, depth, s.draft, s.target, err)
    assert (r.m.cpu().numpy() == m).all() and (r.path.cpu().numpy() == path).all()
    assert (r.bonus.cpu().numpy() == bonus).all()
    assert (r.anc.cpu().numpy().view(np.uint64) == oracle.anc_to_bits(anc)).all()

    # counts for every sequence follow P' = P + m + 1, n' = P' // C
    P2 = P_before.cpu().numpy() + m + 1
    assert (dst.P.cpu().numpy() == P2).all()
    for l, C in enumerate(w.levels):
        assert (dst.n[l].cpu().numpy() == P2 // C).all()

    out = host_f64(r.out, w.dtype)
    assert np.isfinite(out).all() and torch.isfinite(r.lse).all()

    # sampled sequences against the oracle
    _say(f"full size {name}: oracle on sampled sequences")
    ss = synth.step_inputs(w, 0, batch=SAMPLE)
    h = widen_step(ss, w.dtype)
    ref = oracle.step(ost, ss.parents, ss.draft, ss.target, h.q, h.kt, h.vt)
    check_attention(out[SAMPLE], ref.out, w.dtype)
    lse = r.lse.cpu().numpy()[SAMPLE]
    assert np.abs(lse - ref.lse).max() <= 1e-2
    first = [n_before[l].cpu().numpy()[SAMPLE] for l in range(len(w.levels))]
    compare_state(dst, ref.state, w.dtype, "full size", batch=SAMPLE, first_entry=first)
