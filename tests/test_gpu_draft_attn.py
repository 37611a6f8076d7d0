"""Draft-decode reuse of the branch-aware attention (tv_draft_attn): the candidate tree
grows level by level in creation order, one plan of the whole expansion is shared by
every level, and each level's call must equal the oracle's attention over the partial
tree.  Also: a node's row is the same whether it is computed at its own draft level or
by the verify call over the whole tree (bit-identical when the launch has the same
work split)."""
import sys

import numpy as np
import pytest

import oracle
import synth
from harness import check_attention, device_state, host_f64, oracle_state, pooled_caps
from oracle.draft_tree import candidate_count, expanded_count

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def expansion(w, k, s, seed):
    """Inputs of the full k-ary expansion of s levels in creation order (node c's parent is
    (c - 1) // k): parents, and Q / tree K / tree V values of the workload's dtype."""
    n = 1 + candidate_count(k, s)
    rng = np.random.default_rng(seed)
    par = np.array([-1] + [(c - 1) // k for c in range(1, n)], dtype=np.int32)
    parents = np.tile(par, (w.B, 1))

    def vals(shape):
        x = rng.standard_normal(size=shape, dtype=np.float32)
        return synth.f32_to_bf16_bits(x) if w.dtype == "bf16" else x

    q = vals((w.B, n, w.Hq, w.d))
    kt = vals((w.B, n, w.Hkv, w.d))
    vt = vals((w.B, n, w.Hkv, w.d))
    return parents, q, kt, vt


def run_levels(w, k, s, seed=0):
    import torch
    import tree_speculative_decoding_amd as tv
    caps = pooled_caps(w, 64)
    dst = device_state(w, caps, poison=True)
    ost = oracle_state(w, caps)
    parents, q, kt, vt = expansion(w, k, s, seed)
    n = parents.shape[1]
    # one plan of the whole expansion, shared by every level
    anc = torch.zeros(w.B, n, dtype=torch.int64, device="cuda")
    depth = torch.zeros(w.B, n, dtype=torch.int32, device="cuda")
    err = torch.zeros(w.B, dtype=torch.int32, device="cuda")
    tv.tv_build_tree_mask(torch.from_numpy(parents).cuda(), anc, depth, err)
    outs = []
    for t in range(1, s + 1):
        D = expanded_count(k, t)  # nodes of depth < t: the ones whose children this level drafts
        qd = tv.to_device(q[:, :D], w.dtype)
        kd = tv.to_device(kt[:, :D], w.dtype)
        vd = tv.to_device(vt[:, :D], w.dtype)
        out = torch.zeros(w.B, D, w.Hq, w.d, dtype=qd.dtype, device="cuda")
        lse = torch.zeros(w.B, D, w.Hq, dtype=torch.float32, device="cuda")
        ws = torch.empty(tv.tv_verify_attn_workspace_bytes(D, w.Hq, dst) // 4 + 64, dtype=torch.float32,
                         device="cuda")
        tv.tv_draft_attn(qd, kd, vd, anc, err, dst, out, lse, ws)
        torch.cuda.synchronize()
        a_p, _, e_p = oracle.build_plan(parents[:, :D])
        ref, ref_lse = oracle.verify_attention(oracle.widen(q[:, :D], w.dtype), oracle.widen(kt[:, :D], w.dtype),
                                               oracle.widen(vt[:, :D], w.dtype), a_p, ost, e_p)
        got = host_f64(out, w.dtype)
        check_attention(got, ref, w.dtype)
        assert np.abs(lse.cpu().numpy() - ref_lse).max() <= (1e-2 if w.dtype == "bf16" else 1e-5)
        outs.append(out)
    return dst, parents, q, kt, vt, anc, err, outs


DRAFT = {
    # bf16 MFMA path, 2 query heads per KV head: every level fits one 64-row block
    "bf16_g2_k2s4": (synth.Workload("da1", 3, 31, 16, 8, 128, "bf16", (4, 128), 1000, 2, 4, 0.6, 3001,
                                    prefix="raw"), 2, 4),
    # bf16, 8 query heads per KV head: later levels span several row blocks
    "bf16_g8_k2s3": (synth.Workload("da2", 2, 15, 64, 8, 128, "bf16", (4, 128), 2048, 2, 3, 0.6, 3002), 2, 3),
    # fp32 head dim 64: the vector kernel and the merge kernel's chain path
    "f32_k3s3": (synth.Workload("da3", 2, 40, 4, 1, 64, "f32", (4, 16), 301, 3, 3, 0.6, 3003, prefix="raw"), 3, 3),
}


@pytest.mark.parametrize("name", list(DRAFT))
def test_draft_levels_match_oracle(name):
    w, k, s = DRAFT[name]
    _say(f"draft attention {name}")
    run_levels(w, k, s)


def test_draft_rows_equal_verify_rows():
    """With every level in one 64-row block and the same split of the prefix, a node's
    row computed at its draft level is bit-identical to its row in the verify call over
    the whole expansion (tree nodes a row does not see contribute exact zeros)."""
    import torch
    import tree_speculative_decoding_amd as tv
    w, k, s = DRAFT["bf16_g2_k2s4"]
    _say("draft rows vs verify rows")
    dst, parents, q, kt, vt, anc, err, outs = run_levels(w, k, s, seed=4)
    n = parents.shape[1]
    out = torch.zeros(w.B, n, w.Hq, w.d, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(w.B, n, w.Hq, dtype=torch.float32, device="cuda")
    ws = torch.empty(tv.tv_verify_attn_workspace_bytes(n, w.Hq, dst) // 4 + 64, dtype=torch.float32, device="cuda")
    depth = torch.zeros(w.B, n, dtype=torch.int32, device="cuda")
    tv.tv_build_tree_mask(torch.from_numpy(parents).cuda(), anc, depth, err)
    tv.tv_verify_attn(tv.to_device(q, w.dtype), tv.to_device(kt, w.dtype), tv.to_device(vt, w.dtype), anc, depth, err,
                      dst, None, out, lse, ws)
    torch.cuda.synchronize()
    for t, o in enumerate(outs, start=1):
        D = expanded_count(k, t)
        assert torch.equal(o.view(torch.int16), out[:, :D].view(torch.int16)), f"level {t}"
