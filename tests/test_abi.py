"""CPU checks of the C ABI: libtv.so loads, exports every function include/tv.h
declares, and rejects invalid arguments on the host (before any launch, so these
calls touch no GPU)."""
import ctypes

import pytest

import tree_speculative_decoding_amd as tv
from tree_speculative_decoding_amd.tv import TvScratch, TvState


def test_library_exports_every_declared_symbol():
    L = tv.lib()
    names = tv.header_symbols()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert tv.tv_version() == 140


def test_struct_layout_matches_header():
    # tv_level: 2 x int32 + 6 pointers + 2 x int32; tv_state: 5 x int32, 2 levels, 3 pointers
    assert ctypes.sizeof(tv.tv.TvLevel) == 64
    assert tv.tv.TvLevel.page_table.offset == 48 and tv.tv.TvLevel.num_pages.offset == 60
    assert ctypes.sizeof(TvState) == 176
    assert TvState.lvl.offset == 24 and TvState.P.offset == 168
    assert ctypes.sizeof(TvScratch) == 80 and TvScratch.in_place.offset == 64 and TvScratch.deferred.offset == 72


def fake_state(**kw):
    s = TvState()
    s.B, s.Hkv, s.d, s.dtype, s.n_levels = 2, 2, 128, 1, 2
    for l, C in enumerate((4, 128)):
        s.lvl[l].C, s.lvl[l].cap = C, 128
        for f in ("k", "vt", "n", "open_k", "open_v"):
            setattr(s.lvl[l], f, 0x1000)
    s.tail_k = s.tail_v = s.P = 0x1000
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def status(f, *a):
    return f(*a)


P = ctypes.c_void_p(0x1000)


def test_tree_mask_rejects_bad_sizes():
    L = tv.lib()
    assert L.tv_build_tree_mask(2, 0, P, P, P, P, None) == tv.TV_EINVAL
    assert L.tv_build_tree_mask(2, 65, P, P, P, P, None) == tv.TV_EINVAL
    assert L.tv_build_tree_mask(-1, 8, P, P, P, P, None) == tv.TV_EINVAL
    assert L.tv_build_tree_mask(2, 8, None, P, P, P, None) == tv.TV_EINVAL
    assert b"NULL" in L.tv_last_error()
    assert L.tv_build_tree_mask(0, 8, None, None, None, None, None) == tv.TV_OK  # B = 0: nothing to do


def test_accept_rejects_bad_sizes():
    L = tv.lib()
    assert L.tv_accept(4, 70, P, P, P, P, P, None, P, P, P, None) == tv.TV_EINVAL
    assert L.tv_accept(4, 8, P, P, P, P, None, None, P, P, P, None) == tv.TV_EINVAL


@pytest.mark.parametrize("mut,code", [
    (dict(d=96), tv.TV_EUNSUPPORTED),
    (dict(dtype=7), tv.TV_EINVAL),
    (dict(n_levels=3), tv.TV_EINVAL),
    (dict(Hkv=0), tv.TV_EINVAL),
    (dict(P=None), tv.TV_EINVAL),
    (dict(tail_k=None), tv.TV_EINVAL),
])
def test_verify_rejects_bad_state(mut, code):
    L = tv.lib()
    s = fake_state(**mut)
    r = L.tv_verify_attn(8, 16, P, P, P, P, P, None, ctypes.byref(s), None, P, None, P, 1 << 30, 1, None)
    assert r == code, tv.lib().tv_last_error()


def test_verify_rejects_bad_levels_and_workspace():
    L = tv.lib()
    s = fake_state()
    s.lvl[1].C = 4  # not increasing
    assert L.tv_verify_attn(8, 16, P, P, P, P, P, None, ctypes.byref(s), None, P, None, P, 1 << 30, 1, None) == tv.TV_EINVAL
    s = fake_state()
    s.lvl[0].cap = 100  # not a multiple of 64
    assert L.tv_verify_attn(8, 16, P, P, P, P, P, None, ctypes.byref(s), None, P, None, P, 1 << 30, 1, None) == tv.TV_EINVAL
    s = fake_state()
    assert L.tv_verify_attn(8, 15, P, P, P, P, P, None, ctypes.byref(s), None, P, None, P, 1 << 30, 1, None) == tv.TV_EINVAL  # Hq % Hkv
    need = L.tv_verify_attn_workspace_bytes(8, 16, ctypes.byref(s), 3)
    # 4 units (2 seq x 2 heads x 1 row block) of 2 + 2 chunks = 16 chunks in 3 slices (5, 5, 6):
    # (slice, unit) pairs are numbered slice + unit < 3 + 4 - 1 -> 6 partial blocks of 64
    # rows x (128 floats + a (max, sum) pair)
    assert need == 6 * 64 * 128 * 4 + 6 * 64 * 8
    # 4 slices of 4 chunks: every prefix is one slice's, nothing goes to the workspace
    assert L.tv_verify_attn_workspace_bytes(8, 16, ctypes.byref(s), 4) == 256
    # the fp32 vector kernel always writes partials (its merge adds the tail and the chain)
    s.dtype = 0
    assert L.tv_verify_attn_workspace_bytes(8, 16, ctypes.byref(s), 4) == (4 + 4 - 1) * 64 * (128 * 4 + 8)
    s.dtype = 1
    assert L.tv_verify_attn(8, 16, P, P, P, P, P, None, ctypes.byref(s), None, P, None, P, need - 1, 3, None) == tv.TV_EWORKSPACE
    assert L.tv_verify_attn_workspace_bytes(0, 16, ctypes.byref(s), 3) == 0


def test_refresh_and_compress_reject_bad_args():
    L = tv.lib()
    s = fake_state()
    assert L.tv_refresh_state(8, ctypes.byref(s), None, P, P, P, P, None, P, None) == tv.TV_EINVAL  # no scratch
    sc = TvScratch()
    assert L.tv_refresh_state(8, ctypes.byref(s), ctypes.byref(sc), P, P, P, P, None, P, None) == tv.TV_EINVAL
    # every level deferred: no scratch pointers are needed, but a bit past n_levels is refused
    sc.deferred = 0x4
    assert L.tv_refresh_state(8, ctypes.byref(s), ctypes.byref(sc), P, P, P, P, None, P, None) == tv.TV_EINVAL
    assert b"n_levels" in L.tv_last_error()
    assert L.tv_compress_prefix(ctypes.byref(s), P, P, -1, P, None) == tv.TV_EINVAL
    assert L.tv_compress_prefix(ctypes.byref(s), None, P, 10, P, None) == tv.TV_EINVAL


def test_accept_refresh_rejects_bad_args():
    L = tv.lib()
    s = fake_state()
    sc = TvScratch()
    args = [P] * 12 + [None]  # parents .. seq_err, stream
    assert L.tv_accept_refresh(8, ctypes.byref(s), None, *args) == tv.TV_EINVAL  # no scratch
    assert L.tv_accept_refresh(8, ctypes.byref(s), ctypes.byref(sc), *args) == tv.TV_EINVAL  # NULL scratch levels
    assert L.tv_accept_refresh(0, ctypes.byref(s), ctypes.byref(sc), *args) == tv.TV_EINVAL  # D < 1
    assert L.tv_accept_refresh(65, ctypes.byref(s), ctypes.byref(sc), *args) == tv.TV_EINVAL  # D > 64
    nulls = [P] * 12
    nulls[4] = None  # target tokens
    assert L.tv_accept_refresh(8, ctypes.byref(s), ctypes.byref(sc), *nulls, None) == tv.TV_EINVAL


def test_status_strings():
    L = tv.lib()
    for code in (0, -1, -2, -3, -4):
        assert L.tv_status_string(code)


def test_draft_tree_rejects_bad_sizes():
    L = tv.lib()
    f = L.tv_build_draft_tree
    assert f(2, 0, 3, 8, 1024, P, P, P, P, None, None) == tv.TV_EINVAL       # topk 0
    assert f(2, 2, 0, 8, 1024, P, P, P, P, None, None) == tv.TV_EINVAL       # steps 0
    assert f(2, 2, 3, 16, 1024, P, P, P, P, None, None) == tv.TV_EINVAL      # D > N + 1 = 15
    assert f(2, 2, 3, 0, 1024, P, P, P, P, None, None) == tv.TV_EINVAL       # D 0
    assert f(2, 4, 3, 65, 1024, P, P, P, P, None, None) == tv.TV_EINVAL      # D > TV_MAX_D
    assert f(2, 2, 11, 8, 1024, P, P, P, P, None, None) == tv.TV_EINVAL      # N = 4094 > 2048
    assert b"candidates" in L.tv_last_error()
    assert f(2, 8, 3, 8, 4, P, P, P, P, None, None) == tv.TV_EINVAL          # vocab < topk
    assert f(2, 2, 3, 8, 1024, None, P, P, P, None, None) == tv.TV_EINVAL    # NULL logits
    assert f(0, 2, 3, 8, 1024, None, None, None, None, None, None) == tv.TV_OK  # B = 0


@pytest.mark.parametrize("B,Hkv,cap", [(1, 1, 64), (3, 2, 640), (2, 8, 1024), (64, 8, 8384), (5, 3, 2112), (4, 8, 33792)])
def test_contiguous_tile_index_is_a_permutation_with_runs(B, Hkv, cap):
    """The contiguous pool layout (include/tv.h): every (sequence, head, tile) has its own
    tile, all B*Hkv*cap/64 tiles are used, tiles within a run of TV_TILE_RUN are
    consecutive, and tile t of every (b, g) lies in the same window for complete runs."""
    import numpy as np
    from tree_speculative_decoding_amd.tv import TV_TILE_RUN, contiguous_tile_index
    idx = contiguous_tile_index(B, Hkv, cap)
    T = cap // 64
    assert idx.shape == (B, Hkv, T)
    assert np.array_equal(np.sort(idx.reshape(-1)), np.arange(B * Hkv * T))
    R, full = TV_TILE_RUN, T // TV_TILE_RUN
    for t in range(T):
        if t % R and (t // R < full or t >= full * R):
            assert (idx[:, :, t] == idx[:, :, t - 1] + 1).all()  # runs (and the last tiles) are consecutive
    for q in range(full):  # run range q of every (b, g): one window of B*Hkv*R tiles
        w = idx[:, :, q * R:(q + 1) * R]
        assert w.min() == q * B * Hkv * R and w.max() == (q + 1) * B * Hkv * R - 1
