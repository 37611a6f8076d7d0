"""GPU parity of tv_verify_attn (attention + scratch pad) and tv_compress_prefix against
the oracle, on the seeded workloads and on edge shapes; split-count invariance,
determinism and isolation (poisoned rows never reach the outputs, bit-exact)."""
import sys

import numpy as np
import pytest

import oracle
import synth
from harness import (ATT_ATOL, LSE_ATOL, Runner, check_attention, compare_state, device_state, entry_tol,
                     host_f64, open_tol, oracle_state, pooled_caps, upload_step, widen_step)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_verify(w, step=0, q_scale=1.0, num_parts=0, poison=True, mutate=None, extra_tokens=64):
    """Run plan + verify on the GPU and in the oracle for workload w (pools sized for
    extra_tokens past the prefix); returns both sides."""
    import torch
    caps = pooled_caps(w, extra_tokens)
    dst = device_state(w, caps, poison=poison)
    ost = oracle_state(w, caps)
    s = synth.step_inputs(w, step, q_scale=q_scale)
    if mutate is not None:
        mutate(s)
    h = widen_step(s, w.dtype)
    x = upload_step(s, w.dtype)
    r = Runner(dst, w.D, w.Hq, num_parts)
    r.plan(x)
    r.attend(x)
    torch.cuda.synchronize()
    anc, depth, err = oracle.build_plan(s.parents)
    out, lse = oracle.verify_attention(h.q, h.kt, h.vt, anc, ost, err)
    sc = oracle.build_scratch(h.kt, h.vt, anc, depth, ost, err)
    return dict(w=w, dst=dst, ost=ost, s=s, h=h, x=x, r=r, anc=anc, depth=depth, err=err, out=out, lse=lse, sc=sc)


def check_outputs(res):
    w, r = res["w"], res["r"]
    got = host_f64(r.out, w.dtype)
    check_attention(got, res["out"], w.dtype, res["err"])
    lse = r.lse.cpu().numpy().astype(np.float64)
    ok = res["err"] == 0
    assert np.abs(lse[ok] - res["lse"][ok]).max() <= LSE_ATOL[w.dtype]


def check_scratch(res):
    w, r, sc = res["w"], res["r"], res["sc"]
    for l in range(len(w.levels)):
        ek = host_f64(r.sc.entry_k[l], w.dtype)
        ev = host_f64(r.sc.entry_v[l], w.dtype)
        ok_ = r.sc.open_k[l].cpu().numpy().astype(np.float64)
        ov_ = r.sc.open_v[l].cpu().numpy().astype(np.float64)
        cl = sc.closes[l]
        assert (np.abs(ek[cl] - sc.entry_k[l][cl]) <= entry_tol(w.dtype, sc.entry_k[l][cl])).all()
        assert (np.abs(ev[cl] - sc.entry_v[l][cl]) <= entry_tol(w.dtype, sc.entry_v[l][cl])).all()
        assert (np.abs(ok_ - sc.open_k[l]) <= open_tol(sc.open_k[l])).all()
        assert (np.abs(ov_ - sc.open_v[l]) <= open_tol(sc.open_v[l])).all()


@pytest.mark.parametrize("name", ["tiny", "linear", "tree"])
def test_verify_parity_workloads(name):
    _say(f"verify parity: {name}")
    res = run_verify(synth.WORKLOADS[name])
    if res["w"].prefix == "raw":
        compare_state(res["dst"], res["ost"], res["w"].dtype, "compressed prefix")
    check_outputs(res)
    check_scratch(res)


@pytest.mark.parametrize("name", ["tiny", "tree"])
def test_verify_sharp_logits(name):
    """Q scaled by 8: concentrated softmax, so errors in individual scores show."""
    _say(f"verify sharp: {name}")
    check_outputs(run_verify(synth.WORKLOADS[name], q_scale=8.0))


def test_verify_tree_dominant():
    """Queries and tree keys share a strong common direction, so every visible tree node
    carries far more weight than the prefix: a mask error (a node seeing another branch,
    or missing an ancestor) moves outputs far beyond tolerance."""
    _say("verify tree-dominant")
    w = synth.Workload("dom", 4, 8, 64, 8, 128, "bf16", (4, 128), 256, 2, 3, 0.6, 1500)
    u = np.random.default_rng(6).standard_normal(w.d)
    u /= np.linalg.norm(u)

    def mutate(s):
        rng = np.random.default_rng(5)
        q = synth.bf16_bits_to_f32(s.q).astype(np.float64) + 9.0 * u
        kt = 12.0 * u + 0.5 * rng.standard_normal(s.k_tree.shape)
        s.q[...] = synth.f32_to_bf16_bits(q.astype(np.float32))
        s.k_tree[...] = synth.f32_to_bf16_bits(kt.astype(np.float32))

    res = run_verify(w, mutate=mutate)
    check_outputs(res)
    check_scratch(res)
    # the oracle with every node visible to every node differs by far more than the tolerance
    allvis = np.ones_like(res["anc"])
    wrong, _ = oracle.verify_attention(res["h"].q, res["h"].kt, res["h"].vt, allvis, res["ost"])
    assert np.abs(wrong - res["out"]).max() > 10 * ATT_ATOL["bf16"]


# 12 nodes x 8 query heads per KV head = 96 rows: 128-row units in 8-wave workgroups
WIDE_SMALL = synth.Workload("wide_small", 3, 12, 64, 8, 128, "bf16", (4, 128), 4099, 2, 4, 0.6, 1501, prefix="raw")


@pytest.mark.parametrize("name,parts", [("linear", p) for p in (1, 2, 3, 7, 33, 1000)] +
                         [("wide_small", p) for p in (1, 3, 33, 1000)])
def test_partition_invariance(name, parts):
    """Any cut of the prefix stream into workgroup slices gives the same result (within
    tolerance): slices that start or end inside a prefix, several prefixes per slice; for
    64-row and 128-row units.  The scratch pad is built where the cut puts it (workgroups
    ahead of or behind the stream's in the same launch, or a kernel of its own) and
    matches the oracle in every case."""
    _say(f"verify {name} parts={parts}")
    w = WIDE_SMALL if name == "wide_small" else synth.WORKLOADS[name]
    res = run_verify(w, num_parts=parts)
    check_outputs(res)
    check_scratch(res)


# one sequence, one KV head, a 32768-token prefix: a single unit of 134 chunk slots
LONG_ONE = synth.Workload("long_one", 1, 8, 8, 1, 128, "bf16", (4, 128), 32768, 2, 3, 0.6, 1503)


@pytest.mark.parametrize("parts", [5, 10, 20, 40, 100, 1000])
def test_merge_shapes(parts):
    """One prefix split over 5 .. 134 slices: the merge of split prefixes spreads a row's
    slices over 2, 4 or 8 thread groups, reads 4, 8 or 16 slices per thread in one round,
    and beyond 128 slices (1000 requested: one chunk each) reads the rest in further
    rounds; slices of 8 chunks or more (5 and 10) store and read their partials with the
    nontemporal hint.  Every case matches the oracle."""
    _say(f"verify long_one parts={parts}")
    res = run_verify(LONG_ONE, num_parts=parts)
    check_outputs(res)
    check_scratch(res)


@pytest.mark.parametrize("name,parts", [("linear", 100), ("tree", 100), ("linear", 0), ("tree", 0)])
def test_pool_headroom(name, parts):
    """The same committed history in pools with about 4x headroom: three quarters of the
    capacity slots the slices are cut over hold no committed entry (whole slices of
    them, for the later workgroups); the rows and the scratch pad still match the oracle."""
    _say(f"headroom {name} parts={parts}")
    w = synth.WORKLOADS[name]
    b = run_verify(w, num_parts=parts, extra_tokens=3 * w.P + 64)
    assert b["dst"].caps[0] >= 3 * (w.P // w.levels[0]), b["dst"].caps
    check_outputs(b)
    check_scratch(b)


def test_scratch_pad_paths_bit_identical():
    """The scratch pad built by workgroups ahead of the stream's in the prefix launch (a
    small cut leaves room for them), behind them (a cut that fills the device) and by the
    scratch kernel of its own (128-row units) is the same bits: the same code adds the same
    values in the same order."""
    _say("scratch pad paths")
    import torch
    w = synth.WORKLOADS["linear"]
    a = run_verify(w, num_parts=64)     # 64 stream + 64 pad workgroups fit: pad ahead of the stream
    b = run_verify(w, num_parts=1000)   # no room: pad workgroups behind the stream's
    for l in range(len(w.levels)):
        for name in ("entry_k", "entry_v", "open_k", "open_v"):
            x, y = getattr(a["r"].sc, name)[l], getattr(b["r"].sc, name)[l]
            assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                               y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32)), (l, name)
    check_scratch(a)


def test_determinism_bit_identical():
    _say("verify determinism")
    import torch
    res = run_verify(synth.WORKLOADS["tree"], num_parts=4)
    r, x = res["r"], res["x"]
    a = r.out.clone()
    l1 = r.lse.clone()
    r.attend(x)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), r.out.view(torch.int16))
    assert torch.equal(l1, r.lse)


def test_poisoned_pool_tail_is_never_read():
    """Slots beyond each pool's committed count hold NaN in one run, zeros in the other:
    outputs and scratch are bit-identical."""
    _say("verify pool poison")
    import torch
    w = synth.WORKLOADS["tree"]
    a = run_verify(w, poison=True)
    b = run_verify(w, poison=False)
    assert torch.equal(a["r"].out.view(torch.int16), b["r"].out.view(torch.int16))
    assert torch.equal(a["r"].lse, b["r"].lse)
    for l in range(len(w.levels)):
        assert torch.equal(a["r"].sc.open_k[l], b["r"].sc.open_k[l])


def test_other_branches_never_read():
    """For a chosen leaf, every tree node off its chain gets NaN K/V: the outputs of the
    chain's nodes are bit-identical to the clean run (TSD-V4 §3.1 branch isolation)."""
    _say("verify branch poison")
    import torch
    import tree_speculative_decoding_amd as tv
    w = synth.WORKLOADS["tree"]
    res = run_verify(w, poison=False)
    r, x, anc = res["r"], res["x"], res["anc"]
    clean = r.out.clone()
    B, D = w.B, w.D
    for leaf in range(D):
        kt = x.kt.clone()
        vt = x.vt.clone()
        onchain = anc[:, leaf, :]  # [B][D]
        for b in range(B):
            off = np.nonzero(~onchain[b])[0]
            if len(off):
                kt[b, off] = float("nan")
                vt[b, off] = float("nan")
        tv.tv_verify_attn(x.q, kt, vt, r.anc, r.depth, r.err, r.st, r.sc, r.out, r.lse, r.ws, 0)
        torch.cuda.synchronize()
        for b in range(B):
            for i in np.nonzero(onchain[b])[0]:
                assert torch.equal(r.out[b, i].view(torch.int16), clean[b, i].view(torch.int16))


EDGE = {
    # bf16, head dim 64 -> vector kernel
    "bf16_d64": synth.Workload("e1", 3, 7, 8, 2, 64, "bf16", (4, 128), 384, 2, 3, 0.6, 2001),
    # 128 query rows per KV head -> one 128-row unit (8-wave workgroups)
    "two_row_blocks": synth.Workload("e2", 2, 8, 32, 2, 128, "bf16", (4, 128), 640, 2, 3, 0.6, 2002),
    # a single node (no drafts)
    "root_only": synth.Workload("e3", 3, 1, 16, 2, 128, "bf16", (4, 128), 256, 1, 0, 0.6, 2003),
    # one level with a long raw tail, ragged count inside the last chunk
    "one_level_c128": synth.Workload("e4", 2, 8, 16, 2, 128, "bf16", (128,), 1000, 1, 7, 0.7, 2004, prefix="raw"),
    # empty committed prefix
    "empty_prefix": synth.Workload("e5", 2, 6, 16, 2, 128, "bf16", (4, 128), 0, 2, 3, 0.6, 2005, prefix="raw"),
    # fp32, head dim 128, 2 levels, prefix not a multiple of 4
    "f32_ragged": synth.Workload("e6", 2, 8, 8, 2, 128, "f32", (4, 16), 203, 2, 3, 0.6, 2006, prefix="raw"),
    # bf16 d128 with entries not a multiple of the 64-entry chunk
    "bf16_ragged": synth.Workload("e7", 3, 5, 40, 8, 128, "bf16", (4, 128), 4733, 2, 3, 0.6, 2007, prefix="raw"),
    # D = 64 chain
    "deep_chain": synth.Workload("e8", 1, 64, 8, 1, 128, "bf16", (4,), 100, 1, 63, 0.9, 2008, prefix="raw"),
    # tail + tree = 2 + 24 entries: two 16-entry tiles in the prefix kernel's tree chunk
    "tree_two_tiles": synth.Workload("e9", 2, 24, 16, 2, 128, "bf16", (4, 128), 1502, 3, 5, 0.6, 2009, prefix="raw"),
    # tail + tree = 3 + 61 = 64 entries: the largest tree chunk, 4 blocks of 128 rows
    "tree_full_chunk": synth.Workload("e10", 1, 61, 8, 1, 128, "bf16", (4, 128), 1203, 4, 5, 0.6, 2010, prefix="raw"),
    # 64 rows per KV head (G = 2, D = 32) with a 35-entry tail + tree chunk: four 16-entry
    # tiles in a 4-wave, 64-row unit
    "tree_four_tiles_64rows": synth.Workload("e11", 2, 32, 4, 2, 128, "bf16", (4, 128), 1501, 2, 5, 0.6, 2011,
                                             prefix="raw"),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_verify_edge_shapes(name):
    _say(f"verify edge: {name}")
    res = run_verify(EDGE[name])
    if res["w"].prefix == "raw":
        compare_state(res["dst"], res["ost"], res["w"].dtype, "compressed prefix")
    check_outputs(res)
    check_scratch(res)


def test_ragged_prefix_lengths():
    """Sequences of one batch with different committed lengths (tails of 0..3 raw tokens)."""
    _say("verify ragged lengths")
    import torch
    import tree_speculative_decoding_amd as tv
    w = synth.Workload("rag", 5, 8, 16, 2, 128, "bf16", (4, 128), 700, 2, 3, 0.6, 2100, prefix="raw")
    lens = [700, 699, 130, 3, 257]
    caps = pooled_caps(w, 64)
    dst = tv.DeviceState(w.B, w.Hkv, w.d, w.dtype, w.levels, caps)
    for t in dst.pool_k + dst.pool_vt:
        t.fill_(float("nan"))
    rk = np.stack([synth.raw_prefix(w, b)[0] for b in range(w.B)])
    rv = np.stack([synth.raw_prefix(w, b)[1] for b in range(w.B)])
    dst.P.copy_(torch.tensor(lens, dtype=torch.int32))
    err = torch.zeros(w.B, dtype=torch.int32, device="cuda")
    tv.tv_compress_prefix(dst, tv.to_device(rk, w.dtype), tv.to_device(rv, w.dtype), err)
    hk = [oracle.widen(rk[b][:, :lens[b]], w.dtype) for b in range(w.B)]
    hv = [oracle.widen(rv[b][:, :lens[b]], w.dtype) for b in range(w.B)]
    ost = oracle.from_scratch(hk, hv, w.levels, caps)
    torch.cuda.synchronize()
    compare_state(dst, ost, w.dtype, "ragged prefix")
    s = synth.step_inputs(w, 0)
    h = widen_step(s, w.dtype)
    x = upload_step(s, w.dtype)
    r = Runner(dst, w.D, w.Hq)
    r.plan(x)
    r.attend(x)
    torch.cuda.synchronize()
    anc, depth, e = oracle.build_plan(s.parents)
    out, lse = oracle.verify_attention(h.q, h.kt, h.vt, anc, ost, e)
    check_attention(host_f64(r.out, w.dtype), out, w.dtype)


def test_compress_prefix_errors():
    _say("compress errors")
    import torch
    import tree_speculative_decoding_amd as tv
    st = tv.DeviceState(3, 1, 64, "f32", (4,), [64])
    st.P.copy_(torch.tensor([10, 300, -1], dtype=torch.int32))  # 300 > max_len, 300/4 > cap too
    raw = torch.zeros(3, 1, 200, 64, device="cuda")
    err = torch.zeros(3, dtype=torch.int32, device="cuda")
    tv.tv_compress_prefix(st, raw, raw, err)
    torch.cuda.synchronize()
    assert list(err.cpu().numpy()) == [0, tv.TV_SEQ_BAD_PREFIX, tv.TV_SEQ_BAD_PREFIX]
    st2 = tv.DeviceState(1, 1, 64, "f32", (4,), [64])
    st2.P.fill_(400)
    raw2 = torch.zeros(1, 1, 400, 64, device="cuda")
    tv.tv_compress_prefix(st2, raw2, raw2, err[:1])
    torch.cuda.synchronize()
    assert err[0].item() == tv.TV_SEQ_POOL_FULL


def test_flagged_sequence_outputs():
    _say("verify flagged sequence")
    import torch
    w = synth.WORKLOADS["tree"]
    res = run_verify(w, mutate=lambda s: s.parents.__setitem__((1, 3), 9))  # tree 1 invalid
    r = res["r"]
    assert r.err.cpu().numpy()[1] == 1
    check_outputs(res)
    assert (r.out[1].float() == 0).all() and torch.isinf(r.lse[1]).all()
