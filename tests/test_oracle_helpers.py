"""Pins of the oracle's input and state helpers, against values fixed by the number
format and by the compression stand-in's definition rather than by the oracle itself:

- widen('bf16'): hand-decoded bfloat16 bit patterns (sign, 8 exponent bits, 7 mantissa
  bits; the IEEE-754 binary32 layout with the low 16 bits dropped), including the
  subnormal, infinite, NaN and signed-zero cases;
- from_entries: a state built from the committed entries of a raw history (several
  entries, several KV heads and levels, every P a multiple of every C) equals the
  state compressed from that history, and each entry lands at its own (sequence,
  head, slot) (sentinel values);
- prefix_rows: the shared visible prefix of a state compressed from a raw history
  equals block means and raw tail tokens computed here directly from that history
  (TSD-V4 §2.2: compression along the sequence axis; the finest level's open block
  stays raw), in the order every level's entries then the tail.

CPU only, float64; the oracle is not modified by these tests."""
import math

import numpy as np
import pytest

import oracle


# ----------------------------------------------------------------------------- widen

BF16_CASES = [
    (0x3F80, 1.0),                          # sign 0, exponent 127, mantissa 0
    (0xBF80, -1.0),
    (0xC040, -3.0),                         # exponent 128, mantissa 0b1000000: -1.5 * 2
    (0x4049, 3.140625),                     # 2 * (1 + 73/128)
    (0x3F81, 1.0 + 2.0 ** -7),              # one mantissa step above 1
    (0x0080, 2.0 ** -126),                  # smallest normal
    (0x0001, 2.0 ** -133),                  # smallest subnormal: 2^-126 * 2^-7
    (0x007F, 127 * 2.0 ** -133),            # largest subnormal
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),  # largest finite
    (0x7F80, math.inf),
    (0xFF80, -math.inf),
    (0x0000, 0.0),
]


@pytest.mark.parametrize("bits,value", BF16_CASES)
def test_widen_bf16_hand_values(bits, value):
    got = oracle.widen(np.array([bits], dtype=np.uint16), "bf16")
    assert got.dtype == np.float64
    assert got[0] == value


@pytest.mark.filterwarnings("ignore:invalid value encountered in cast")
def test_widen_bf16_signed_zero_and_nan():
    z = oracle.widen(np.array([0x8000], dtype=np.uint16), "bf16")[0]
    assert z == 0.0 and math.copysign(1.0, z) == -1.0
    for bits in (0x7FC0, 0xFFC1, 0x7F81):
        assert math.isnan(oracle.widen(np.array([bits], dtype=np.uint16), "bf16")[0])


@pytest.mark.filterwarnings("ignore:invalid value encountered in cast")
def test_widen_bf16_every_pattern_against_a_decoder():
    """All 65536 patterns against a decoder written from the format's fields."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    got = oracle.widen(bits.astype(np.uint16), "bf16")
    for b in range(1 << 16):  # decoded field by field
        s, e, f = b >> 15, (b >> 7) & 0xFF, b & 0x7F
        if e == 0xFF:
            ref = math.nan if f else math.inf
        elif e == 0:
            ref = f * 2.0 ** -133
        else:
            ref = (1.0 + f / 128.0) * 2.0 ** (e - 127)
        ref = -ref if s else ref
        if math.isnan(ref):
            assert math.isnan(got[b])
        else:
            assert got[b] == ref, hex(b)


def test_widen_bf16_shape_and_f32_path():
    x = np.array([[0x3F80, 0x4000], [0x4040, 0x4080]], dtype=np.uint16)
    np.testing.assert_array_equal(oracle.widen(x, "bf16"), [[1.0, 2.0], [3.0, 4.0]])
    f = np.array([0.1, -2.5, 1e-40], dtype=np.float32)  # 1e-40 is an fp32 subnormal
    got = oracle.widen(f, "f32")
    assert got.dtype == np.float64
    assert got[0] == 0.100000001490116119384765625  # the exact binary32 value nearest 0.1
    assert got[1] == -2.5 and got[2] == float(np.float32(1e-40))
    with pytest.raises(ValueError):
        oracle.widen(f, "f16")


# ----------------------------------------------------------------------------- from_entries

def test_from_entries_equals_from_scratch_of_the_same_history():
    rng = np.random.default_rng(31)
    levels, Hkv, d = (2, 8), 3, 5
    P = [16, 40, 0]  # multiples of every C, one empty sequence
    caps = [24, 6]
    hk = [rng.standard_normal((Hkv, p, d)) for p in P]
    hv = [rng.standard_normal((Hkv, p, d)) for p in P]
    ref = oracle.from_scratch(hk, hv, levels, caps)
    ents = [[(ref.pool_k[l][b, :, :ref.n[l][b]].copy(), ref.pool_v[l][b, :, :ref.n[l][b]].copy())
             for l in range(len(levels))] for b in range(len(P))]
    st = oracle.from_entries(ents, P, levels, caps, d)
    assert st.levels == ref.levels
    np.testing.assert_array_equal(st.P, ref.P)
    for l in range(len(levels)):
        np.testing.assert_array_equal(st.n[l], ref.n[l])
        np.testing.assert_array_equal(st.pool_k[l], ref.pool_k[l])
        np.testing.assert_array_equal(st.pool_v[l], ref.pool_v[l])
        np.testing.assert_array_equal(st.open_k[l], ref.open_k[l])  # zero: P closes every block
        np.testing.assert_array_equal(st.open_v[l], ref.open_v[l])
    assert st.tail_k.shape == ref.tail_k.shape == (len(P), Hkv, levels[0] - 1, d)
    np.testing.assert_array_equal(st.tail_k, ref.tail_k)


def test_from_entries_places_each_entry_at_its_slot():
    B, levels, Hkv, d = 2, (4, 16), 2, 3
    P = [32, 16]
    caps = [12, 4]
    ents = []
    for b in range(B):
        lv = []
        for l, C in enumerate(levels):
            n = P[b] // C
            k = np.zeros((Hkv, n, d))
            for g in range(Hkv):
                for j in range(n):
                    k[g, j] = 1000 * b + 100 * l + 10 * g + j + np.arange(d) / 8
            lv.append((k, -k))
        ents.append(lv)
    st = oracle.from_entries(ents, P, levels, caps, d)
    for b in range(B):
        for l, C in enumerate(levels):
            n = P[b] // C
            assert st.n[l][b] == n
            for g in range(Hkv):
                for j in range(caps[l]):
                    want = 1000 * b + 100 * l + 10 * g + j + np.arange(d) / 8 if j < n else np.zeros(d)
                    np.testing.assert_array_equal(st.pool_k[l][b, g, j], want)
                    np.testing.assert_array_equal(st.pool_v[l][b, g, j], -want)


def test_from_entries_rejects_inconsistent_counts():
    k = np.zeros((1, 3, 2))
    with pytest.raises(ValueError):
        oracle.from_entries([[(k, k)]], [8], [4], [4], 2)   # 3 entries for P // 4 = 2
    with pytest.raises(ValueError):
        oracle.from_entries([[(k, k)]], [13], [4], [4], 2)  # P not a multiple of C


# ----------------------------------------------------------------------------- prefix_rows

def direct_prefix(xk, xv, levels):
    """The visible prefix from a raw history [Hkv][P][d], head by head: for every level
    C (finest first) the mean of each complete aligned block, then the raw tokens of the
    finest level's incomplete block."""
    Hkv, P, d = xk.shape
    out = []
    for g in range(Hkv):
        rows_k, rows_v = [], []
        for C in levels:
            j = 0
            while (j + 1) * C <= P:
                bk = np.zeros(d)
                bv = np.zeros(d)
                for t in range(j * C, (j + 1) * C):
                    bk += xk[g, t]
                    bv += xv[g, t]
                rows_k.append(bk / C)
                rows_v.append(bv / C)
                j += 1
        start = (P // levels[0]) * levels[0]
        for t in range(start, P):
            rows_k.append(xk[g, t])
            rows_v.append(xv[g, t])
        out.append((np.array(rows_k).reshape(-1, d), np.array(rows_v).reshape(-1, d)))
    return out


@pytest.mark.parametrize("levels,P", [((4, 16), 45), ((4, 16), 48), ((4,), 3), ((2, 8), 0), ((3, 9), 29),
                                      ((1,), 5)])
def test_prefix_rows_against_the_raw_history(levels, P):
    rng = np.random.default_rng(P * 7 + len(levels))
    Hkv, d = 3, 4
    xk = [rng.standard_normal((Hkv, P, d)) for _ in range(2)]
    xv = [rng.standard_normal((Hkv, P, d)) for _ in range(2)]
    caps = [P // C + 2 for C in levels]
    st = oracle.from_scratch(xk, xv, levels, caps)
    for b in range(2):
        want = direct_prefix(xk[b], xv[b], levels)
        for g in range(Hkv):
            pk, pv = oracle.prefix_rows(st, b, g)
            wk, wv = want[g]
            assert pk.shape == wk.shape == (sum(P // C for C in levels) + P % levels[0], d)
            np.testing.assert_allclose(pk, wk, rtol=0, atol=1e-13)
            np.testing.assert_allclose(pv, wv, rtol=0, atol=1e-13)


def test_prefix_rows_reads_the_counts_not_the_capacity():
    """Slots past the committed count (poisoned here) are not part of the prefix."""
    rng = np.random.default_rng(4)
    xk = [rng.standard_normal((2, 21, 3))]
    st = oracle.from_scratch(xk, xk, (4, 8), [9, 5])
    for l in range(2):
        st.pool_k[l][0, :, st.n[l][0]:] = np.nan
        st.pool_v[l][0, :, st.n[l][0]:] = np.nan
    st.tail_k[0, :, 21 % 4:] = np.nan
    for g in range(2):
        pk, pv = oracle.prefix_rows(st, 0, g)
        assert pk.shape[0] == 5 + 2 + 1 and np.isfinite(pk).all() and np.isfinite(pv).all()
