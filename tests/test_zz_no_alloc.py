"""tv_verify_attn_noalloc (the verify call for callers that cannot allocate: the split-prefix
partials live in the library's own device array) against tv_verify_attn with a caller
workspace: bit-identical outputs, LSE and scratch pad, on two calls in a row, the second
with a smaller input (fewer sequences, a shorter prefix), both on shapes that split
prefixes over several slices (so the partials are used); and the oracle within the
attention tolerance.  A shape that needs more partials than the array holds is refused
before any launch."""
import sys

import numpy as np
import pytest

import oracle
import synth
from harness import Runner, check_attention, device_state, host_f64, oracle_state, pooled_caps, upload_step, widen_step

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


CASES = [
    # 4 sequences x 8 heads at an 8192-token prefix: 32 prefixes over ~512 slices
    synth.Workload("na1", 4, 6, 64, 8, 128, "bf16", (4, 128), 8195, 2, 3, 0.5, 5101, prefix="raw"),
    # then fewer sequences and a shorter prefix (the array keeps the first call's contents)
    synth.Workload("na2", 2, 8, 64, 8, 128, "bf16", (4, 128), 2050, 1, 7, 0.7, 5102, prefix="raw"),
]


def test_noalloc_equals_workspace_call_twice():
    import torch
    import tree_speculative_decoding_amd as tv
    for k, w in enumerate(CASES):
        _say(f"noalloc call {k}: {w.name} B={w.B} D={w.D} P={w.P}")
        caps = pooled_caps(w, 64)
        dst = device_state(w, caps, poison=True)
        s = synth.step_inputs(w, 0)
        x = upload_step(s, w.dtype)
        r = Runner(dst, w.D, w.Hq)  # the workspace call
        assert r.ws.numel() * 4 > 4096, "the shape must split prefixes"
        r.plan(x)
        r.attend(x)
        out2 = torch.zeros_like(r.out)
        lse2 = torch.full_like(r.lse, 7.0)
        sc2 = tv.DeviceScratch(w.B, w.D, w.Hkv, w.d, w.dtype, len(w.levels))
        tv.tv_verify_attn_noalloc(x.q, x.kt, x.vt, r.anc, r.depth, r.err, dst, sc2, out2, lse2)
        torch.cuda.synchronize()
        assert torch.equal(_bits(r.out), _bits(out2))
        assert torch.equal(_bits(r.lse), _bits(lse2))
        for l in range(len(w.levels)):
            for name in ("entry_k", "entry_v", "open_k", "open_v"):
                assert torch.equal(_bits(getattr(r.sc, name)[l]), _bits(getattr(sc2, name)[l])), (l, name)
        # and the oracle
        ost = oracle_state(w, caps)
        h = widen_step(s, w.dtype)
        anc, depth, err = oracle.build_plan(s.parents)
        ref, _ = oracle.verify_attention(h.q, h.kt, h.vt, anc, ost, err)
        check_attention(host_f64(out2, w.dtype), ref, w.dtype)


def test_noalloc_refuses_shapes_beyond_its_array():
    import torch
    import tree_speculative_decoding_amd as tv
    _say("noalloc refuses a shape beyond its array")
    # 64 sequences x 8 heads at a 4096-token prefix cut into ~4000 slices of 3 chunks:
    # (3072 + 512 - 1) x 64 rows x 520 bytes of partials, far beyond 24 MiB
    w = synth.Workload("na3", 64, 8, 64, 8, 128, "bf16", (4, 128), 4096, 2, 3, 0.5, 5103)
    caps = [tv.round_cap(w.P // C + 8) for C in w.levels]
    st = tv.DeviceState(w.B, w.Hkv, w.d, w.dtype, w.levels, caps)
    need = tv.tv_verify_attn_workspace_bytes(w.D, w.Hq, st, 4000)
    assert need > (24 << 20)
    assert tv.tv_verify_attn_workspace_bytes(w.D, w.Hq, st, 0) <= (24 << 20)  # the library's own cut fits
    z = lambda *shape, dt=torch.bfloat16: torch.zeros(*shape, dtype=dt, device="cuda")
    q, kt, vt = z(w.B, w.D, w.Hq, w.d), z(w.B, w.D, w.Hkv, w.d), z(w.B, w.D, w.Hkv, w.d)
    anc = z(w.B, w.D, dt=torch.int64)
    depth = z(w.B, w.D, dt=torch.int32)
    out = z(w.B, w.D, w.Hq, w.d)
    with pytest.raises(tv.TvError) as ei:
        tv.tv_verify_attn_noalloc(q, kt, vt, anc, depth, None, st, None, out, None, num_parts=4000)
    assert ei.value.status == tv.TV_EWORKSPACE
