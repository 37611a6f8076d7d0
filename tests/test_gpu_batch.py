"""Per-sequence results do not depend on the batch (TSD-V4 §5.3 reads acceptance as a
property of each sequence, and every call of the step is independent per sequence): the
same sequences in permuted batch slots, and a subset of them run as a batch of its own,
give bit-identical outputs, LSE, plans, acceptance, commit logs and refreshed states over
several steps.  The prefix stream is split at unit boundaries (one workgroup per
(sequence, KV head) prefix), so each unit's summation order is the same in every run."""
import sys

import pytest

import synth
from harness import Runner, device_state, pooled_caps, upload_step

pytestmark = pytest.mark.gpu

W = synth.Workload("perm", 4, 8, 16, 2, 128, "bf16", (4, 128), 700, 2, 3, 0.7, 3400, prefix="raw")
STEPS = 3


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _select(st, seqs):
    """A new state whose slot s holds sequence seqs[s] of st (every byte of the pools,
    poisoned slots included)."""
    import torch
    import tree_speculative_decoding_amd as tv
    out = tv.DeviceState(len(seqs), st.Hkv, st.d, st.dtype, st.levels, st.caps)
    idx = torch.tensor(seqs, dtype=torch.long, device="cuda")
    for l in range(len(st.levels)):
        K, VT = st.logical_k(l), st.logical_vt(l)
        for s, b in enumerate(seqs):
            out.write_seq(l, s, K[b].contiguous(), VT[b].contiguous())
        out.n[l].copy_(st.n[l][idx])
        out.open_k[l].copy_(st.open_k[l][idx])
        out.open_v[l].copy_(st.open_v[l][idx])
    if st.tail_k is not None:
        out.tail_k.copy_(st.tail_k[idx])
        out.tail_v.copy_(st.tail_v[idx])
    out.P.copy_(st.P[idx])
    torch.cuda.synchronize()
    return out


def _results(r, st):
    """Everything a step writes, per sequence (dim 0 is the batch slot)."""
    res = [r.out, r.lse, r.anc, r.depth, r.m, r.path, r.bonus, r.log, r.err, st.P]
    for l in range(len(st.levels)):
        res += [st.logical_k(l), st.logical_vt(l), st.n[l], st.open_k[l], st.open_v[l]]
    if st.tail_k is not None:
        res += [st.tail_k, st.tail_v]
    return res


def _same_bits(a, b):
    import torch
    if a.dtype in (torch.bfloat16, torch.float16):
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


def _run(st, seqs):
    """STEPS steps of the sequences `seqs` (slot s = sequence seqs[s]); the results after
    each step, on the host."""
    import torch
    units = len(seqs) * W.Hkv * ((W.Hq // W.Hkv * W.D + 63) // 64)
    r = Runner(st, W.D, W.Hq, num_parts=units)  # one workgroup per unit
    got = []
    for t in range(STEPS):
        r.step(upload_step(synth.step_inputs(W, t, batch=seqs), W.dtype))
        torch.cuda.synchronize()
        got.append([x.clone() for x in _results(r, st)])
    return got


@pytest.mark.parametrize("seqs", [[2, 0, 3, 1], [3, 1], [2]], ids=["permuted", "subset", "alone"])
def test_results_independent_of_batch_slot(seqs):
    import torch
    _say(f"batch invariance: sequences {seqs}")
    caps = pooled_caps(W, STEPS * W.D + 8)
    base = device_state(W, caps, poison=True)
    other = _select(base, seqs)
    ref = _run(base, list(range(W.B)))
    got = _run(other, seqs)
    idx = torch.tensor(seqs, dtype=torch.long, device="cuda")
    for t in range(STEPS):
        for i, (a, b) in enumerate(zip(got[t], ref[t])):
            assert _same_bits(a, b[idx]), f"step {t}: result {i} differs for sequences {seqs}"
