"""The calls of a step (plan, verify attention with the scratch pad, accept and refresh as
two calls or as tv_accept_refresh) captured once in a HIP graph and replayed: the library
allocates nothing, synchronises nothing and records no memset inside the calls, so a
replay must equal the eager step bit for bit.  Each replay starts from the same restored state, with eager work and a
synchronisation between replays, and every replay is compared with the eager result
(outputs, acceptance, commit log and the refreshed state)."""
import sys

import pytest

import synth
from harness import Runner, device_state, pooled_caps, upload_step

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _snapshot(st):
    return [t.clone() for t in _live(st)]


def _live(st):
    ts = [st.P] + st.n + st.open_k + st.open_v + st.pool_k + st.pool_vt
    return ts + [t for t in (st.tail_k, st.tail_v) if t is not None]


def _restore(st, snap):
    for dst, src in zip(_live(st), snap):
        dst.copy_(src)


def _results(r, st):
    return [r.out, r.lse, r.anc, r.depth, r.m, r.path, r.bonus, r.log, r.err] + _live(st) + \
        r.sc.entry_k + r.sc.entry_v + r.sc.open_k + r.sc.open_v


def _same(a, b):
    import torch
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


CASES = {
    # one workgroup per (sequence, KV head) prefix (32 of them): no finish kernel
    "whole_units": (synth.Workload("g1", 4, 8, 64, 8, 128, "bf16", (4, 128), 4096 - 3, 2, 3, 0.7, 5001,
                                   prefix="raw"), 32),
    # split units: the finish kernel merges partials
    "split_units": (synth.Workload("g2", 2, 6, 64, 8, 128, "bf16", (4, 128), 2048 + 1, 2, 3, 0.6, 5002,
                                   prefix="raw"), 37),
    # the vector path (fp32) with its tail and chain in the finish kernel
    "f32": (synth.Workload("g3", 2, 6, 8, 2, 64, "f32", (4, 16), 611, 2, 3, 0.6, 5003, prefix="raw"), 0),
    # paged pools (random page table), split units
    "paged": (synth.Workload("g4", 3, 8, 64, 8, 128, "bf16", (4, 128), 1500 + 2, 2, 3, 0.7, 5004, prefix="raw"), 29),
}
PAGE_SEEDS = {"paged": 77}


@pytest.mark.parametrize("fused", [False, True], ids=["four_calls", "fused_accept_refresh"])
@pytest.mark.parametrize("name", list(CASES))
def test_graph_replay_equals_eager(name, fused):
    import torch
    w, parts = CASES[name]
    _say(f"graph replay {name} fused={fused}")
    caps = pooled_caps(w, 64)
    st = device_state(w, caps, poison=True, page_seed=PAGE_SEEDS.get(name), spare_pages=3 if name in PAGE_SEEDS else 0)
    r = Runner(st, w.D, w.Hq, parts)
    x = upload_step(synth.step_inputs(w, 0), w.dtype)
    snap = _snapshot(st)

    r.step(x, fused=fused)  # eager reference (also loads every kernel before capture)
    torch.cuda.synchronize()
    ref = [t.clone() for t in _results(r, st)]

    _restore(st, snap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        r.step(x, fused=fused)
    torch.cuda.synchronize()
    for rep in range(3):
        _restore(st, snap)
        for t in _results(r, st)[:9]:
            t.zero_()  # outputs must come from the replay, not from the capture
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _results(r, st)
        for i, (a, b) in enumerate(zip(got, ref)):
            assert _same(a, b), f"replay {rep}: result {i} differs from the eager step"
