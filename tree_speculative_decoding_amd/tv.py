"""ctypes binding of libtv (include/tv.h): the same entry points, taking torch tensors.

This module only marshals arguments: it turns tensors into device pointers, fills
the tv_state / tv_scratch structs and raises on a non-OK status.  Every step of
the path runs in the HIP kernels of libtv.so; there is no fallback.  PyTorch is
used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtv.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "tv.h")

TV_OK, TV_EINVAL, TV_EUNSUPPORTED, TV_EWORKSPACE, TV_EHIP = 0, -1, -2, -3, -4
TV_F32, TV_BF16 = 0, 1
TV_SEQ_OK, TV_SEQ_BAD_PARENT, TV_SEQ_POOL_FULL, TV_SEQ_BAD_PREFIX, TV_SEQ_BAD_PATH, TV_SEQ_BAD_PAGE = 0, 1, 2, 3, 4, 5
TV_MAX_LEVELS = 2
TV_MAX_D = 64
TV_POOL_ALIGN = 64
TV_TILE_RUN = 16


class TvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"tv status {status}: {msg}")
        self.status = status


class TvLevel(ctypes.Structure):
    _fields_ = [("C", ctypes.c_int32), ("cap", ctypes.c_int32), ("k", ctypes.c_void_p),
                ("vt", ctypes.c_void_p), ("n", ctypes.c_void_p), ("open_k", ctypes.c_void_p),
                ("open_v", ctypes.c_void_p), ("page_table", ctypes.c_void_p),
                ("pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32)]


class TvState(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("n_levels", ctypes.c_int32),
                ("lvl", TvLevel * TV_MAX_LEVELS), ("tail_k", ctypes.c_void_p),
                ("tail_v", ctypes.c_void_p), ("P", ctypes.c_void_p)]


class TvScratch(ctypes.Structure):
    _fields_ = [("entry_k", ctypes.c_void_p * TV_MAX_LEVELS), ("entry_v", ctypes.c_void_p * TV_MAX_LEVELS),
                ("open_k", ctypes.c_void_p * TV_MAX_LEVELS), ("open_v", ctypes.c_void_p * TV_MAX_LEVELS),
                ("in_place", ctypes.c_void_p), ("deferred", ctypes.c_uint32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libtv.so; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m tree_speculative_decoding_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        sig = {
            "tv_build_tree_mask": ([i32, i32, vp, vp, vp, vp, vp], i32),
            "tv_verify_attn_workspace_bytes": ([i32, i32, ctypes.POINTER(TvState), i32], sz),
            "tv_verify_attn": ([i32, i32, vp, vp, vp, vp, vp, vp, ctypes.POINTER(TvState),
                                ctypes.POINTER(TvScratch), vp, vp, vp, sz, i32, vp], i32),
            "tv_accept": ([i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp], i32),
            "tv_refresh_state": ([i32, ctypes.POINTER(TvState), ctypes.POINTER(TvScratch), vp, vp, vp,
                                  vp, vp, vp, vp], i32),
            "tv_accept_refresh": ([i32, ctypes.POINTER(TvState), ctypes.POINTER(TvScratch), vp, vp, vp, vp, vp,
                                   vp, vp, vp, vp, vp, vp, vp, vp], i32),
            "tv_compress_prefix": ([ctypes.POINTER(TvState), vp, vp, i32, vp, vp], i32),
            "tv_build_draft_tree": ([i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp], i32),
            "tv_verify_attn_noalloc": ([i32, i32, vp, vp, vp, vp, vp, vp, ctypes.POINTER(TvState),
                                        ctypes.POINTER(TvScratch), vp, vp, i32, vp], i32),
            "tv_draft_attn": ([i32, i32, i32, vp, vp, vp, vp, vp, ctypes.POINTER(TvState), vp, vp, vp, sz, i32,
                               vp], i32),
            "tv_status_string": ([i32], ctypes.c_char_p),
            "tv_last_error": ([], ctypes.c_char_p),
            "tv_version": ([], i32),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def header_symbols() -> list:
    """Names of the functions include/tv.h declares."""
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"TV_API\s+[^;(]*?\b(tv_\w+)\s*\(", txt)))


# ----------------------------------------------------------------------------- marshalling

def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libtv must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(status: int):
    if status != TV_OK:
        raise TvError(status, lib().tv_last_error().decode())


def torch_dtype(dtype: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]


def tv_dtype(dtype: str) -> int:
    return {"bf16": TV_BF16, "f32": TV_F32}[dtype]


def to_device(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """numpy input (bf16 as uint16 bit patterns, or float32) -> device tensor of that dtype."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy (bf16 as uint16 bit patterns)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def tile_vt(v: np.ndarray, cap: int) -> np.ndarray:
    """Entry-major V rows [..., n, d] -> the pool's tiled transposed layout [..., cap/64, d, 64]
    (entries n..cap-1 zero).  Layout conversion only."""
    *lead, n, d = v.shape
    full = np.zeros((*lead, cap, d), dtype=v.dtype)
    full[..., :n, :] = v
    t = full.reshape(*lead, cap // TV_POOL_ALIGN, TV_POOL_ALIGN, d)
    return np.ascontiguousarray(np.swapaxes(t, -1, -2))


def untile_vt(vt: np.ndarray) -> np.ndarray:
    """Inverse of tile_vt: [..., cap/64, d, 64] -> [..., cap, d]."""
    *lead, nt, d, w = vt.shape
    return np.swapaxes(vt, -1, -2).reshape(*lead, nt * w, d)


def round_cap(n: int) -> int:
    return max(TV_POOL_ALIGN, -(-n // TV_POOL_ALIGN) * TV_POOL_ALIGN)


def contiguous_tile_index(B: int, Hkv: int, cap: int) -> np.ndarray:
    """[B][Hkv][cap/64] int64: the tile of a contiguous pool that holds tile t of (sequence b,
    KV head g) (runs of TV_TILE_RUN tiles of one (b, g), run ranges of all (b, g) side by
    side, the last T mod R tiles of each (b, g) at the end; include/tv.h).  Layout only."""
    R, T = TV_TILE_RUN, cap // TV_POOL_ALIGN
    full = T // R
    b = np.arange(B)[:, None, None]
    g = np.arange(Hkv)[None, :, None]
    t = np.arange(T)[None, None, :]
    q, w = t // R, t % R
    in_run = ((q * B + b) * Hkv + g) * R + w
    tail = full * B * Hkv * R + (b * Hkv + g) * (T - full * R) + w
    return np.where(q < full, in_run, tail).astype(np.int64)


class DeviceState:
    """Device tensors of a tv_state: pools (K row-major, V transposed), counts, open
    sums, tail and committed lengths.  Allocation and data movement only; no arithmetic.

    Contiguous pools are B*Hkv*cap/64 tiles, [64][d] (K) and [d][64] (V^T), placed as
    contiguous_tile_index says (runs of TV_TILE_RUN tiles per (sequence, head), the
    sequences' runs side by side); logical_k / logical_vt give the per-sequence views.

    With ``page_seed`` set the pools are paged: each level holds B * cap/64 (+ ``spare_pages``)
    physical pages of 64 entries for all KV heads, and a page table maps every
    sequence's 64-entry tiles to a random permutation of them."""

    def __init__(self, B: int, Hkv: int, d: int, dtype: str, levels: Sequence[int],
                 caps: Sequence[int], device="cuda", page_seed: Optional[int] = None, spare_pages: int = 0):
        if len(levels) > TV_MAX_LEVELS:
            raise ValueError("at most two levels")
        self.B, self.Hkv, self.d, self.dtype = B, Hkv, d, dtype
        self.levels = tuple(int(c) for c in levels)
        self.caps = tuple(round_cap(int(c)) for c in caps)
        td = torch_dtype(dtype)
        z = lambda *s, dt=td: torch.zeros(*s, dtype=dt, device=device)
        self.paged = page_seed is not None
        A = TV_POOL_ALIGN
        if self.paged:
            rng = np.random.default_rng(page_seed)
            self.page_table, self.num_pages = [], []
            self.pool_k, self.pool_vt = [], []
            for c in self.caps:
                pps = c // A
                npg = B * pps + spare_pages
                perm = rng.permutation(npg)[: B * pps].reshape(B, pps).astype(np.int32)
                self.page_table.append(torch.from_numpy(perm).to(device))
                self.num_pages.append(npg)
                self.pool_k.append(z(npg, Hkv, A, d))
                self.pool_vt.append(z(npg, Hkv, d, A))
        else:  # tiles placed as contiguous_tile_index says
            self.page_table, self.num_pages = None, None
            self.pool_k = [z(B * Hkv * (c // A), A, d) for c in self.caps]
            self.pool_vt = [z(B * Hkv * (c // A), d, A) for c in self.caps]
            self.tile_index = [torch.from_numpy(contiguous_tile_index(B, Hkv, c)).to(device) for c in self.caps]
        self.n = [z(B, dt=torch.int32) for _ in self.levels]
        self.open_k = [z(B, Hkv, d, dt=torch.float32) for _ in self.levels]
        self.open_v = [z(B, Hkv, d, dt=torch.float32) for _ in self.levels]
        c0 = self.levels[0] if self.levels else 1
        self.tail_k = z(B, Hkv, c0 - 1, d) if c0 > 1 else None
        self.tail_v = z(B, Hkv, c0 - 1, d) if c0 > 1 else None
        self.P = z(B, dt=torch.int32)
        self._struct = None

    def struct(self) -> TvState:
        """The tv_state of these tensors.  They are allocated once and only ever updated
        in place, so the pointers are taken once (a copy is returned: callers may edit it)."""
        if self._struct is None:
            self._struct = self._make_struct()
        return TvState.from_buffer_copy(self._struct)

    def _make_struct(self) -> TvState:
        s = TvState()
        s.B, s.Hkv, s.d, s.dtype, s.n_levels = self.B, self.Hkv, self.d, tv_dtype(self.dtype), len(self.levels)
        for l, C in enumerate(self.levels):
            L = s.lvl[l]
            L.C, L.cap = C, self.caps[l]
            L.k, L.vt = self.pool_k[l].data_ptr(), self.pool_vt[l].data_ptr()
            L.n = self.n[l].data_ptr()
            L.open_k, L.open_v = self.open_k[l].data_ptr(), self.open_v[l].data_ptr()
            if self.paged:
                L.page_table = self.page_table[l].data_ptr()
                L.pages_per_seq = self.caps[l] // TV_POOL_ALIGN
                L.num_pages = self.num_pages[l]
        s.tail_k = self.tail_k.data_ptr() if self.tail_k is not None else None
        s.tail_v = self.tail_v.data_ptr() if self.tail_v is not None else None
        s.P = self.P.data_ptr()
        return s


    def write_seq(self, l: int, b: int, k: torch.Tensor, vt: torch.Tensor) -> None:
        """Level l's entries of sequence b: k [Hkv][n][d] (n <= cap), vt the V tiles
        [Hkv][cap/64][d][64] (tile_vt); both of the state's element type."""
        A = TV_POOL_ALIGN
        n = k.shape[1]
        if not self.paged:  # K: only entries < n are written; V^T: whole tiles
            idx = self.tile_index[l][b]  # [Hkv][cap/64]
            full, r = n // A, n % A
            if full:
                self.pool_k[l][idx[:, :full].reshape(-1)] = k[:, :full * A].reshape(self.Hkv * full, A, self.d)
            if r:
                self.pool_k[l][idx[:, full], :r] = k[:, full * A:n]
            self.pool_vt[l][idx.reshape(-1)] = vt.reshape(-1, self.d, A)
            return
        pps = self.caps[l] // A
        pages = self.page_table[l][b].long()
        kk = torch.zeros(self.Hkv, self.caps[l], self.d, dtype=k.dtype, device=k.device)
        kk[:, :n] = k
        self.pool_k[l][pages] = kk.reshape(self.Hkv, pps, A, self.d).permute(1, 0, 2, 3)
        self.pool_vt[l][pages] = vt.permute(1, 0, 2, 3)

    def logical_k(self, l: int) -> torch.Tensor:
        """Level l's K pool as [B][Hkv][cap][d] (a gather)."""
        if not self.paged:
            return self.pool_k[l][self.tile_index[l].reshape(-1)].reshape(self.B, self.Hkv, self.caps[l], self.d)
        A = TV_POOL_ALIGN
        g = self.pool_k[l][self.page_table[l].long()]  # [B][pps][Hkv][64][d]
        return g.permute(0, 2, 1, 3, 4).reshape(self.B, self.Hkv, self.caps[l], self.d)

    def logical_vt(self, l: int) -> torch.Tensor:
        """Level l's V tiles as [B][Hkv][cap/64][d][64] (a gather)."""
        if not self.paged:
            T = self.caps[l] // TV_POOL_ALIGN
            return self.pool_vt[l][self.tile_index[l].reshape(-1)].reshape(self.B, self.Hkv, T, self.d, TV_POOL_ALIGN)
        g = self.pool_vt[l][self.page_table[l].long()]  # [B][pps][Hkv][d][64]
        return g.permute(0, 2, 1, 3, 4)


class DeviceScratch:
    """Device tensors of a tv_scratch for B sequences of D nodes.  in_place=True gives the
    struct its in_place mask array (the verify writes one chain's entries straight into the
    pools and the refresh skips them); False leaves it NULL (every entry is copied).
    deferred: mask of the levels the refresh brings up to date from the accepted path
    (no scratch tensors are allocated for them; their pointers stay NULL)."""

    def __init__(self, B: int, D: int, Hkv: int, d: int, dtype: str, n_levels: int, device="cuda",
                 in_place: bool = True, deferred: int = 0):
        td = torch_dtype(dtype)
        mk = lambda l, t: None if (deferred >> l) & 1 else torch.zeros(B, D, Hkv, d, dtype=t, device=device)
        self.entry_k = [mk(l, td) for l in range(n_levels)]
        self.entry_v = [mk(l, td) for l in range(n_levels)]
        self.open_k = [mk(l, torch.float32) for l in range(n_levels)]
        self.open_v = [mk(l, torch.float32) for l in range(n_levels)]
        self.in_place = torch.zeros(B, dtype=torch.int64, device=device) if in_place else None
        self.deferred = deferred
        self._struct = None

    def struct(self) -> TvScratch:
        """The tv_scratch of these tensors (pointers taken once, as for DeviceState)."""
        if self._struct is None:
            self._struct = self._make_struct()
        return TvScratch.from_buffer_copy(self._struct)

    def _make_struct(self) -> TvScratch:
        s = TvScratch()
        ptr = lambda t: t.data_ptr() if t is not None else None
        for l in range(len(self.entry_k)):
            s.entry_k[l] = ptr(self.entry_k[l])
            s.entry_v[l] = ptr(self.entry_v[l])
            s.open_k[l] = ptr(self.open_k[l])
            s.open_v[l] = ptr(self.open_v[l])
        s.in_place = ptr(self.in_place)
        s.deferred = self.deferred
        return s


def _state(st) -> TvState:
    if isinstance(st, DeviceState):
        if st._struct is None:
            st._struct = st._make_struct()
        return st._struct
    return st


def _scratch(sc) -> Optional[TvScratch]:
    if isinstance(sc, DeviceScratch):
        if sc._struct is None:
            sc._struct = sc._make_struct()
        return sc._struct
    return sc


# ----------------------------------------------------------------------------- entry points

def tv_build_tree_mask(parents: torch.Tensor, anc: torch.Tensor, depth: torch.Tensor,
                       seq_err: torch.Tensor, stream=None) -> None:
    B, D = parents.shape
    _check(lib().tv_build_tree_mask(B, D, _ptr(parents), _ptr(anc), _ptr(depth), _ptr(seq_err),
                                    _stream(stream)))


def tv_build_draft_tree(logits: torch.Tensor, root_tok: torch.Tensor, topk: int, steps: int,
                        parents: torch.Tensor, draft_tok: torch.Tensor, cum_logp: Optional[torch.Tensor] = None,
                        stream=None) -> None:
    B, E, V = logits.shape
    D = parents.shape[1]
    _check(lib().tv_build_draft_tree(B, topk, steps, D, V, _ptr(logits), _ptr(root_tok), _ptr(parents),
                                     _ptr(draft_tok), _ptr(cum_logp), _stream(stream)))


def tv_verify_attn_workspace_bytes(D: int, Hq: int, st, num_parts: int = 0) -> int:
    s = _state(st)
    return int(lib().tv_verify_attn_workspace_bytes(D, Hq, ctypes.byref(s), num_parts))


def tv_verify_attn(q: torch.Tensor, k_tree: torch.Tensor, v_tree: torch.Tensor, anc: torch.Tensor,
                   depth: torch.Tensor, seq_err: Optional[torch.Tensor], st, scratch,
                   out: torch.Tensor, lse: Optional[torch.Tensor], workspace: torch.Tensor,
                   num_parts: int = 0, stream=None) -> None:
    B, D, Hq, d = q.shape
    s = _state(st)
    sc = _scratch(scratch)
    _check(lib().tv_verify_attn(D, Hq, _ptr(q), _ptr(k_tree), _ptr(v_tree), _ptr(anc), _ptr(depth),
                                _ptr(seq_err), ctypes.byref(s),
                                ctypes.byref(sc) if sc is not None else None, _ptr(out), _ptr(lse),
                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                num_parts, _stream(stream)))


def tv_verify_attn_noalloc(q: torch.Tensor, k_tree: torch.Tensor, v_tree: torch.Tensor, anc: torch.Tensor,
                           depth: torch.Tensor, seq_err: Optional[torch.Tensor], st, scratch,
                           out: torch.Tensor, lse: Optional[torch.Tensor], num_parts: int = 0, stream=None) -> None:
    """tv_verify_attn with the library's own device array for the split-prefix partials."""
    B, D, Hq, d = q.shape
    s = _state(st)
    sc = _scratch(scratch)
    _check(lib().tv_verify_attn_noalloc(D, Hq, _ptr(q), _ptr(k_tree), _ptr(v_tree), _ptr(anc), _ptr(depth),
                                        _ptr(seq_err), ctypes.byref(s),
                                        ctypes.byref(sc) if sc is not None else None, _ptr(out), _ptr(lse),
                                        num_parts, _stream(stream)))


def tv_draft_attn(q: torch.Tensor, k_tree: torch.Tensor, v_tree: torch.Tensor, anc: torch.Tensor,
                  seq_err: Optional[torch.Tensor], st, out: torch.Tensor, lse: Optional[torch.Tensor],
                  workspace: torch.Tensor, num_parts: int = 0, stream=None) -> None:
    """One draft-decode level: q, k_tree, v_tree, out cover the D nodes created so far;
    anc is the [B][anc_ld] plan of the whole expansion."""
    B, D, Hq, d = q.shape
    anc_ld = anc.shape[1]
    s = _state(st)
    _check(lib().tv_draft_attn(D, anc_ld, Hq, _ptr(q), _ptr(k_tree), _ptr(v_tree), _ptr(anc), _ptr(seq_err),
                               ctypes.byref(s), _ptr(out), _ptr(lse), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), num_parts, _stream(stream)))


def tv_accept(parents, anc, depth, draft_tok, target_tok, seq_err, m, path, bonus, stream=None) -> None:
    B, D = parents.shape
    _check(lib().tv_accept(B, D, _ptr(parents), _ptr(anc), _ptr(depth), _ptr(draft_tok), _ptr(target_tok),
                           _ptr(seq_err), _ptr(m), _ptr(path), _ptr(bonus), _stream(stream)))


def tv_refresh_state(st, scratch, k_tree, v_tree, m, path, commit_log, seq_err, stream=None) -> None:
    D = k_tree.shape[1]
    s = _state(st)
    sc = _scratch(scratch)
    _check(lib().tv_refresh_state(D, ctypes.byref(s), ctypes.byref(sc) if sc is not None else None,
                                  _ptr(k_tree), _ptr(v_tree), _ptr(m), _ptr(path), _ptr(commit_log),
                                  _ptr(seq_err), _stream(stream)))


def tv_accept_refresh(st, scratch, parents, anc, depth, draft_tok, target_tok, k_tree, v_tree, m, path, bonus,
                      commit_log, seq_err, stream=None) -> None:
    """tv_accept followed by tv_refresh_state, in one launch."""
    D = k_tree.shape[1]
    s = _state(st)
    sc = _scratch(scratch)
    _check(lib().tv_accept_refresh(D, ctypes.byref(s), ctypes.byref(sc) if sc is not None else None,
                                   _ptr(parents), _ptr(anc), _ptr(depth), _ptr(draft_tok), _ptr(target_tok),
                                   _ptr(k_tree), _ptr(v_tree), _ptr(m), _ptr(path), _ptr(bonus), _ptr(commit_log),
                                   _ptr(seq_err), _stream(stream)))


def tv_compress_prefix(st, raw_k: torch.Tensor, raw_v: torch.Tensor, seq_err: torch.Tensor,
                       stream=None) -> None:
    s = _state(st)
    max_len = raw_k.shape[2]
    _check(lib().tv_compress_prefix(ctypes.byref(s), _ptr(raw_k), _ptr(raw_v), max_len, _ptr(seq_err),
                                    _stream(stream)))


def tv_version() -> int:
    return int(lib().tv_version())
