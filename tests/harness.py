"""Test harness: puts the same seeded inputs into the oracle (float64) and into the
HIP path (device tensors), and compares results.  Test infrastructure only."""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

import oracle
import synth

# Tolerances.  Attention: the stated bounds, max-abs 2e-2 (bf16 in, fp32
# accumulate) and 1e-5 (fp32), plus a relative Frobenius bound per sequence that
# bites even when outputs are small (bf16: P is rounded to bf16 for the PV
# product, relative 2^-9 per weight; fp32: accumulation over <= 1e4 terms).
ATT_ATOL = {"bf16": 2e-2, "f32": 1e-5}
ATT_REL = {"bf16": 1e-2, "f32": 1e-5}
LSE_ATOL = {"bf16": 1e-2, "f32": 1e-5}


def entry_tol(dtype: str, ref: np.ndarray) -> np.ndarray:
    """Committed/scratch compressed entries: one rounding to the storage type after an
    fp32 sum of <= C values of magnitude ~1."""
    if dtype == "bf16":
        return 2.0 ** -8 * np.abs(ref) + 1e-5
    return 1e-6 * np.abs(ref) + 1e-5


def open_tol(ref: np.ndarray) -> np.ndarray:
    """fp32 running sums of <= 127 values of magnitude ~1."""
    return 1e-5 * np.abs(ref) + 1e-4


@dataclasses.dataclass
class Host:
    """Host copies of one step's inputs: raw (as generated) and float64 (for the oracle)."""
    s: synth.StepInputs
    q: np.ndarray
    kt: np.ndarray
    vt: np.ndarray


def widen_step(s: synth.StepInputs, dtype: str) -> Host:
    return Host(s, oracle.widen(s.q, dtype), oracle.widen(s.k_tree, dtype), oracle.widen(s.v_tree, dtype))


def pooled_caps(w: synth.Workload, extra_tokens: int) -> List[int]:
    from tree_speculative_decoding_amd import round_cap
    return [round_cap((w.P + extra_tokens) // C + 1) for C in w.levels]


# ----------------------------------------------------------------------------- oracle side

def oracle_state(w: synth.Workload, caps: List[int], batch: Optional[List[int]] = None) -> oracle.State:
    bs = batch if batch is not None else list(range(w.B))
    if w.prefix == "raw":
        hk, hv = [], []
        for b in bs:
            k, v = synth.raw_prefix(w, b)
            hk.append(oracle.widen(k, w.dtype))
            hv.append(oracle.widen(v, w.dtype))
        return oracle.from_scratch(hk, hv, w.levels, caps)
    ents = []
    for b in bs:
        ents.append([(oracle.widen(k, w.dtype), oracle.widen(v, w.dtype)) for k, v in synth.pooled_prefix(w, b)])
    return oracle.from_entries(ents, [w.P] * len(bs), w.levels, caps, w.d)


# ----------------------------------------------------------------------------- device side

def device_state(w: synth.Workload, caps: List[int], poison: bool = False, page_seed: Optional[int] = None,
                 spare_pages: int = 0):
    """Device state of workload w at step 0.  With poison=True every pool slot beyond the
    committed entries holds NaN (they must never be read).  page_seed: a paged pool with a
    random page table (and spare_pages unused pages, poisoned too)."""
    import torch
    import tree_speculative_decoding_amd as tv
    st = tv.DeviceState(w.B, w.Hkv, w.d, w.dtype, w.levels, caps, page_seed=page_seed, spare_pages=spare_pages)
    if poison:
        for t in st.pool_k + st.pool_vt:
            t.fill_(float("nan"))
    if w.prefix == "raw":
        rk = np.stack([synth.raw_prefix(w, b)[0] for b in range(w.B)])
        rv = np.stack([synth.raw_prefix(w, b)[1] for b in range(w.B)])
        st.P.fill_(w.P)
        err = torch.zeros(w.B, dtype=torch.int32, device="cuda")
        tv.tv_compress_prefix(st, tv.to_device(rk, w.dtype), tv.to_device(rv, w.dtype), err)
        torch.cuda.synchronize()
        assert (err.cpu().numpy() == 0).all()
        return st
    import concurrent.futures as cf

    def draw(b):
        return [(k, tv.tv.tile_vt(v, st.caps[l])) for l, (k, v) in enumerate(synth.pooled_prefix(w, b))]

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        for b, lv in enumerate(ex.map(draw, range(w.B))):
            for l, (k, vt) in enumerate(lv):
                st.write_seq(l, b, tv.to_device(k, w.dtype), tv.to_device(vt, w.dtype))
                st.n[l][b] = k.shape[1]
    st.P.fill_(w.P)
    torch.cuda.synchronize()
    return st


@dataclasses.dataclass
class DevStep:
    parents: "torch.Tensor"
    draft: "torch.Tensor"
    target: "torch.Tensor"
    q: "torch.Tensor"
    kt: "torch.Tensor"
    vt: "torch.Tensor"


def upload_step(s: synth.StepInputs, dtype: str) -> DevStep:
    import torch
    import tree_speculative_decoding_amd as tv
    i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()
    return DevStep(i32(s.parents), i32(s.draft), i32(s.target), tv.to_device(s.q, dtype),
                   tv.to_device(s.k_tree, dtype), tv.to_device(s.v_tree, dtype))


class Runner:
    """Owns the per-step device buffers of one (B, D, Hq) shape and runs the four calls."""

    def __init__(self, st, D: int, Hq: int, num_parts: int = 0, in_place: bool = True, deferred: int = 0):
        import torch
        import tree_speculative_decoding_amd as tv
        self.st, self.D, self.Hq = st, D, Hq
        B, Hkv, d = st.B, st.Hkv, st.d
        dev = "cuda"
        self.anc = torch.zeros(B, D, dtype=torch.int64, device=dev)
        self.depth = torch.zeros(B, D, dtype=torch.int32, device=dev)
        self.err = torch.zeros(B, dtype=torch.int32, device=dev)
        self.out = torch.zeros(B, D, Hq, d, dtype=_tdt(st.dtype), device=dev)
        self.lse = torch.zeros(B, D, Hq, dtype=torch.float32, device=dev)
        self.m = torch.zeros(B, dtype=torch.int32, device=dev)
        self.path = torch.zeros(B, D, dtype=torch.int32, device=dev)
        self.bonus = torch.zeros(B, dtype=torch.int32, device=dev)
        self.log = torch.zeros(B, max(len(st.levels), 1), D, 2, dtype=torch.int32, device=dev)
        self.sc = tv.DeviceScratch(B, D, Hkv, d, st.dtype, len(st.levels), in_place=in_place, deferred=deferred)
        self.num_parts = num_parts
        nbytes = tv.tv_verify_attn_workspace_bytes(D, Hq, st, num_parts)
        assert nbytes > 0
        self.ws = torch.empty(nbytes // 4 + 64, dtype=torch.float32, device=dev)

    def plan(self, x: DevStep):
        import tree_speculative_decoding_amd as tv
        tv.tv_build_tree_mask(x.parents, self.anc, self.depth, self.err)

    def attend(self, x: DevStep):
        import tree_speculative_decoding_amd as tv
        tv.tv_verify_attn(x.q, x.kt, x.vt, self.anc, self.depth, self.err, self.st, self.sc, self.out,
                          self.lse, self.ws, self.num_parts)

    def accept(self, x: DevStep):
        import tree_speculative_decoding_amd as tv
        tv.tv_accept(x.parents, self.anc, self.depth, x.draft, x.target, self.err, self.m, self.path, self.bonus)

    def refresh(self, x: DevStep):
        import tree_speculative_decoding_amd as tv
        tv.tv_refresh_state(self.st, self.sc, x.kt, x.vt, self.m, self.path, self.log, self.err)

    def accept_refresh(self, x: DevStep):
        import tree_speculative_decoding_amd as tv
        tv.tv_accept_refresh(self.st, self.sc, x.parents, self.anc, self.depth, x.draft, x.target, x.kt, x.vt,
                             self.m, self.path, self.bonus, self.log, self.err)

    def step(self, x: DevStep, fused: bool = False):
        self.plan(x)
        self.attend(x)
        if fused:
            self.accept_refresh(x)
        else:
            self.accept(x)
            self.refresh(x)


def _tdt(dtype):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]


def host_f64(t, dtype: str) -> np.ndarray:
    import tree_speculative_decoding_amd as tv
    a = tv.to_host(t)
    if dtype == "bf16" and a.dtype == np.uint16:
        return oracle.widen(a, "bf16")
    return a.astype(np.float64)


def anc_bits(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint64)


# ----------------------------------------------------------------------------- comparisons

def check_attention(out_gpu: np.ndarray, out_ref: np.ndarray, dtype: str, err: Optional[np.ndarray] = None):
    """max-abs bound everywhere plus a per-sequence relative Frobenius bound."""
    diff = np.abs(out_gpu - out_ref)
    assert np.isfinite(out_gpu).all(), "non-finite attention output"
    assert diff.max() <= ATT_ATOL[dtype], f"max abs diff {diff.max():.3e} > {ATT_ATOL[dtype]}"
    for b in range(out_ref.shape[0]):
        if err is not None and err[b] != 0:
            continue
        num = np.linalg.norm(out_gpu[b] - out_ref[b])
        den = np.linalg.norm(out_ref[b])
        assert num <= ATT_REL[dtype] * den, f"seq {b}: rel Frobenius {num / den:.3e} > {ATT_REL[dtype]}"
    return float(diff.max())


def compare_state(dst, ost: oracle.State, dtype: str, what: str = "", batch: Optional[List[int]] = None,
                  first_entry: Optional[List[np.ndarray]] = None):
    """Device state vs oracle state: counts and tail bit-exact, entries/open sums within
    tolerance.  ``batch`` maps oracle sequence k to device sequence batch[k];
    ``first_entry[l][k]`` limits the entry comparison to slots from there on."""
    import tree_speculative_decoding_amd as tv
    bs = list(range(dst.B)) if batch is None else list(batch)
    P = dst.P.cpu().numpy()[bs]
    assert (P == ost.P).all(), f"{what} P {P} vs {ost.P}"
    for l in range(len(ost.levels)):
        n = dst.n[l].cpu().numpy()[bs]
        assert (n == ost.n[l]).all(), f"{what} level {l} n {n} vs {ost.n[l]}"
        for k, b in enumerate(bs):
            nb = int(n[k])
            lo = 0 if first_entry is None else int(first_entry[l][k])
            rk = ost.pool_k[l][k, :, lo:nb]
            rv = ost.pool_v[l][k, :, lo:nb]
            gk = host_f64(dst.logical_k(l)[b, :, lo:nb].contiguous(), dtype)
            gv = tv.tv.untile_vt(host_f64(dst.logical_vt(l)[b].contiguous(), dtype))[:, lo:nb]
            assert (np.abs(gk - rk) <= entry_tol(dtype, rk)).all(), f"{what} level {l} seq {b} K entries"
            assert (np.abs(gv - rv) <= entry_tol(dtype, rv)).all(), f"{what} level {l} seq {b} V entries"
        ok_ = dst.open_k[l].cpu().numpy().astype(np.float64)[bs]
        ov_ = dst.open_v[l].cpu().numpy().astype(np.float64)[bs]
        assert (np.abs(ok_ - ost.open_k[l]) <= open_tol(ost.open_k[l])).all(), f"{what} level {l} open K"
        assert (np.abs(ov_ - ost.open_v[l]) <= open_tol(ost.open_v[l])).all(), f"{what} level {l} open V"
    if ost.levels and ost.levels[0] > 1:
        tk = host_f64(dst.tail_k, dtype)[bs]
        tvv = host_f64(dst.tail_v, dtype)[bs]
        for k in range(len(bs)):
            r = int(P[k]) % ost.levels[0]
            assert (tk[k, :, :r] == ost.tail_k[k, :, :r]).all(), f"{what} tail K seq {bs[k]}"
            assert (tvv[k, :, :r] == ost.tail_v[k, :, :r]).all(), f"{what} tail V seq {bs[k]}"
