"""Pins that tie the CPU oracle to facts other than itself.

Each ``pin_*`` function raises AssertionError on failure. ``test_oracle_pins``
runs them; ``test_oracle_mutations`` plants each deliberate mistake in the
oracle and checks that at least one pin fails, which shows that the pins
would catch a dropped term, a wrong sign or index, a wrong rounding or a
wrong bit order.

Sources of truth used here (none of them is the oracle's own formula):
  * numpy's independent IEEE binary16 conversion;
  * brute-force nearest-level search in exact rational arithmetic;
  * groups built on an exactly representable grid (closed form);
  * hand-written bit patterns of LSB-first packing;
  * a hand-worked layout example;
  * exact integer matvec (int64) and exact rational dot products;
  * closed-form bounds of the in-cell residual (CellFill abstract:
    residual strictly inside the cell, bit-identical re-quantisation,
    revocable, bounded drift).
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

import oracle
from oracle import exact


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
# binary16 conversion vs numpy (an independent implementation)
# --------------------------------------------------------------------------
def pin_f16_conversion():
    r = _rng(1)
    mags = 10.0 ** r.uniform(-9, 5.2, 100_000)
    vals = r.choice([-1.0, 1.0], mags.size) * mags
    h = np.arange(0, 0x7C00, dtype=np.uint16)
    f = h.view(np.float16).astype(np.float64)
    mids = (f[:-1] + f[1:]) / 2                       # exact ties
    special = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, 2.0 ** -24, 2.0 ** -25,
                        3 * 2.0 ** -25, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25])
    vals = np.concatenate([vals, mids, -mids, f, -f, special, -special])
    with np.errstate(over="ignore"):
        want = vals.astype(np.float16).view(np.uint16)
    got = oracle.f16_from_f64(vals)
    assert np.array_equal(got, want), "f64->f16 differs from numpy"
    v32 = vals.astype(np.float32)
    with np.errstate(over="ignore"):
        want32 = v32.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f16_from_f32(v32), want32), "f32->f16 differs from numpy"
    allh = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = (allh & 0x7C00) != 0x7C00
    dec = oracle.f64_from_f16(allh[finite])
    assert np.array_equal(dec, allh[finite].view(np.float16).astype(np.float64)), "f16 decode"


# --------------------------------------------------------------------------
# Quantiser: brute-force nearest level, exact grids, scale/offset nearness
# --------------------------------------------------------------------------
def pin_rtn_nearest_level(trials=(60, 40, 20, 6)):
    r = _rng(11)
    checked = 0
    for b, n_trials in zip((1, 2, 4, 8), trials):
        L = (1 << b) - 1
        for _ in range(n_trials):
            w = (r.standard_normal(64) * 0.02).astype(np.float32)
            s16, o16, q = oracle.quantize_group(w, b)
            s, o = exact.f16_value(s16), exact.f16_value(o16)
            assert s > 0
            for j in range(64):
                wj = Fraction(float(w[j]))
                t = (wj - o) / s
                frac = t - math.floor(t)
                if abs(frac - Fraction(1, 2)) < Fraction(1, 10 ** 4):
                    continue                          # binary32 evaluation may round across .5
                near = exact.nearest_levels(wj, s, o, L)
                assert len(near) == 1 and int(q[j]) == near[0], (b, j, int(q[j]), near)
                checked += 1
    assert checked > 5000


def pin_rtn_scale_offset_nearest():
    """offset16 is the binary16 value nearest to min(w); scale16 is within half
    a binary16 ulp (plus binary32 slop) of (max - min) / (2^b - 1)."""
    r = _rng(12)
    for b in (1, 2, 4, 8):
        L = (1 << b) - 1
        for _ in range(200):
            w = (r.standard_normal(64) * 0.02).astype(np.float32)
            s16, o16, _ = oracle.quantize_group(w, b)
            lo, hi = Fraction(float(w.min())), Fraction(float(w.max()))
            o = exact.f16_value(o16)
            for nb in (o16 - 1, o16 + 1):
                if 0 <= nb < 0x7C00 or 0x8000 <= nb < 0xFC00:
                    assert abs(o - lo) <= abs(exact.f16_value(nb) - lo)
            s = exact.f16_value(s16)
            ratio = (hi - lo) / L
            e = math.floor(math.log2(float(s)))
            half_ulp = Fraction(2) ** (max(e, -14) - 11)
            assert abs(s - ratio) <= half_ulp + ratio * Fraction(2) ** -22, (b, float(s), float(ratio))


def pin_rtn_exact_grid():
    """Weights placed exactly on an fp16 grid o + s*q (with both ends present)
    must give back s, o and q exactly."""
    r = _rng(13)
    for b in (1, 2, 4, 8):
        L = (1 << b) - 1
        for _ in range(60):
            s = np.float32(int(r.integers(1, 8)) * 2.0 ** -int(r.integers(6, 12)))
            o = np.float32(-int(r.integers(0, 64)) * 2.0 ** -8)
            qt = r.integers(0, L + 1, 64)
            i0, i1 = r.choice(64, 2, replace=False)
            qt[i0], qt[i1] = 0, L
            w = (np.float64(o) + np.float64(s) * qt).astype(np.float32)
            assert np.array_equal(w.astype(np.float64), np.float64(o) + np.float64(s) * qt)
            s16, o16, q = oracle.quantize_group(w, b)
            assert exact.f16_value(s16) == Fraction(float(s)), (b, s16, float(s))
            assert exact.f16_value(o16) == Fraction(float(o))
            assert np.array_equal(q, qt), b


def pin_rtn_degenerate_group():
    """A constant group has range 0: scale 0, offset = the value, codes 0."""
    w = np.full(64, 0.0123, np.float32)
    for b in (1, 2, 4, 8):
        s16, o16, q = oracle.quantize_group(w, b)
        assert s16 == 0 and (q == 0).all()
        assert o16 == int(np.float32(0.0123).astype(np.float16).view(np.uint16))


# --------------------------------------------------------------------------
# Packing: hand-written LSB-first bit patterns and round trips
# --------------------------------------------------------------------------
def pin_canonical_lsb_first():
    j = np.arange(64)
    # b=1, codes 0,1,0,1,...: every odd bit set
    assert list(oracle.pack_group_canonical(j % 2, 1)) == [0xAAAAAAAA] * 2
    # b=2, codes 0,1,2,3 repeating: each byte is 0b11_10_01_00
    assert list(oracle.pack_group_canonical(j % 4, 2)) == [0xE4E4E4E4] * 4
    # b=4, codes j % 16: nibbles ascending from the low end
    assert list(oracle.pack_group_canonical(j % 16, 4)) == [0x76543210, 0xFEDCBA98] * 4
    # b=8, codes j: bytes ascending from the low end
    assert list(oracle.pack_group_canonical(j, 8)) == [
        (4 * i) | ((4 * i + 1) << 8) | ((4 * i + 2) << 16) | ((4 * i + 3) << 24) for i in range(16)]
    # b=1, a single code at position 33 -> word 1, bit 1
    q = np.zeros(64, np.uint8)
    q[33] = 1
    assert list(oracle.pack_group_canonical(q, 1)) == [0, 2]
    r = _rng(14)
    for b in (1, 2, 4, 8):
        for _ in range(50):
            q = r.integers(0, 1 << b, 64).astype(np.uint8)
            assert np.array_equal(oracle.unpack_group_canonical(oracle.pack_group_canonical(q, b), b), q)


def pin_record_even_odd():
    """Record words: with h = 16/b, pair p = (code 2p, code 2p+1) sits in word
    p // h, code 2p at bit (p % h)*b of the low half, code 2p+1 at the same
    position of the high half."""
    j = np.arange(64)
    # b=8, codes j: word w holds pairs 2w and 2w+1
    assert list(oracle.pack_group_record(j, 8)) == [
        (4 * w) | ((4 * w + 2) << 8) | ((4 * w + 1) << 16) | ((4 * w + 3) << 24) for w in range(16)]
    # b=1: odd codes set, even clear -> high halves full
    q = (j % 2).astype(np.uint8)
    assert list(oracle.pack_group_record(q, 1)) == [0xFFFF0000, 0xFFFF0000]
    # b=1: only code 17 set -> pair 8 (odd member), word 0, bit 16 + 8
    q = np.zeros(64, np.uint8)
    q[17] = 1
    assert list(oracle.pack_group_record(q, 1)) == [1 << 24, 0]
    # b=1: only code 34 set -> pair 17 (even member), word 1, bit 1
    q = np.zeros(64, np.uint8)
    q[34] = 1
    assert list(oracle.pack_group_record(q, 1)) == [0, 2]
    # b=4, codes j % 16: word w low half = codes 8w, 8w+2, 8w+4, 8w+6; high = the odd ones
    words = oracle.pack_group_record(j % 16, 4)
    for w in range(8):
        lo = sum(((8 * w + 2 * f) % 16) << (4 * f) for f in range(4))
        hi = sum(((8 * w + 2 * f + 1) % 16) << (4 * f) for f in range(4))
        assert int(words[w]) == lo | (hi << 16)
    r = _rng(15)
    for b in (1, 2, 4, 8):
        for _ in range(50):
            q = r.integers(0, 1 << b, 64).astype(np.uint8)
            assert np.array_equal(oracle.unpack_group_record(oracle.pack_group_record(q, b), b), q)


# --------------------------------------------------------------------------
# Layout: hand-worked example and structural invariants
# --------------------------------------------------------------------------
def _u32_at(stream, byte):
    assert byte % 4 == 0
    return int(stream[byte // 4])


def _u16_at(stream, byte):
    w = _u32_at(stream, byte & ~3)
    return (w >> 16) if (byte & 2) else (w & 0xFFFF)


def _record(W, row, kg, b):
    """(so word, record words) of group (row, kg) quantised at width b."""
    s16, o16, q = oracle.quantize_group(W[row, 64 * kg:64 * kg + 64], b)
    return s16 | (o16 << 16), [int(v) for v in oracle.pack_group_record(q, b)]


def pin_layout_worked_example():
    """N=2, K=128, widths [[1,8],[2,1]] (hand-worked). One tile, R=2 rows,
    2 columns. Classes (r,l): (0,0)=0, (0,1)=3, (1,0)=1, (1,1)=0.
    Map: column 0 plane0 = 0b10, plane1 = 0; column 1 plane0 = 0b01,
    plane1 = 0b01 -> words [2, 0, 1, 1] (16 B).
    Class 0 list (by column, then row): (0,0), (1,1) -> N_0 = 2, one block:
    codes 16 B at 16, so 8 -> 16 B at 32. Class 1: (1,0): 16 + 16 B at 48.
    Class 3: (0,1): codes 64 B at 80, so 16 B at 144.
    Total 160 B = 10 units; count words 2 | 1<<16 and 0 | 1<<16."""
    widths = np.array([[1, 8], [2, 1]], np.uint8)
    W = (_rng(16).standard_normal((2, 128)) * 0.02).astype(np.float32)
    lay = oracle.pack(W, widths)
    assert oracle.layout_sizes(widths) == (1, 4, 10)
    assert list(lay["tiles"]) == [0, 10, 2 | (1 << 16), 1 << 16, 10, 0, 0, 0]
    so00, w00 = _record(W, 0, 0, 1)
    so11, w11 = _record(W, 1, 1, 1)
    so10, w10 = _record(W, 1, 0, 2)
    so01, w01 = _record(W, 0, 1, 8)
    st = [int(v) for v in lay["stream"]]
    expect = ([2, 0, 1, 1] + w00 + w11 + [so00, so11, 0, 0] + w10 + [so10, 0, 0, 0]
              + w01 + [so01, 0, 0, 0])
    assert st == expect
    # the reader rejects a nonzero padding byte (class 0 so padding, word 10)
    bad = dict(lay, stream=lay["stream"].copy())
    bad["stream"][10] = 1
    try:
        oracle.unpack(bad)
        raise AssertionError("nonzero padding accepted")
    except ValueError:
        pass


def pin_layout_column_major():
    """Record order and a partial block (hand-worked): N=32, K=192, width 1
    everywhere except (r5, l0) = 8 and (r1, l2) = (r3, l2) = 2.
    Class 0 list: column 0 rows 0-4, 6-31 (e = 0..30), column 1 rows 0-31
    (e = 31..62), column 2 rows 0, 2, 4-31 (e = 63..92): N_0 = 93.
    Map 24 -> 32 B. Block (0,0), 64 records, at 32: codes 512 B, so 256 B
    at 544. Block (0,1), 29 records, at 800: codes 232 -> 240 B, so 116 ->
    128 B at 1040. Class 1 list (1,2), (3,2): block at 1168, so at 1200.
    Class 3 (5,0): codes at 1216, so at 1280. Total 1296 B = 81 units.
    A row-major list would put (1,1) at e = 4 instead of (4,0)."""
    N, G = 32, 3
    widths = np.ones((N, G), np.uint8)
    widths[5, 0] = 8
    widths[1, 2] = widths[3, 2] = 2
    W = (_rng(21).standard_normal((N, 64 * G)) * 0.02).astype(np.float32)
    lay = oracle.pack(W, widths)
    assert oracle.layout_sizes(widths) == (1, 96, 81)
    assert list(lay["tiles"]) == [0, 81, 93 | (2 << 16), 1 << 16, 81, 0, 0, 0]
    st = lay["stream"]
    words = lambda at, n: [int(v) for v in st[at // 4:at // 4 + n]]
    # map: column 0 plane0/1 = bit 5 (class 3); column 2 plane0 = bits 1, 3
    assert words(0, 8) == [1 << 5, 1 << 5, 0, 0, (1 << 1) | (1 << 3), 0, 0, 0]
    # (e, row, column, codes byte, so byte) of class 0
    for e, r, l, cat, sat in ((0, 0, 0, 32, 544), (4, 4, 0, 64, 560), (5, 6, 0, 72, 564), (30, 31, 0, 272, 664),
                              (31, 0, 1, 280, 668), (62, 31, 1, 528, 792), (63, 0, 2, 536, 796),
                              (64, 2, 2, 800, 1040), (65, 4, 2, 808, 1044), (92, 31, 2, 1024, 1152)):
        so, w = _record(W, r, l, 1)
        assert words(cat, 2) == w and words(sat, 1) == [so], e
    assert words(1032, 2) == [0, 0] and words(1156, 3) == [0, 0, 0]
    for cat, sat, (r, l) in ((1168, 1200, (1, 2)), (1184, 1204, (3, 2))):
        so, w = _record(W, r, l, 2)
        assert words(cat, 4) == w and words(sat, 1) == [so]
    so, w = _record(W, 5, 0, 8)
    assert words(1216, 16) == w and words(1280, 4) == [so, 0, 0, 0]


def pin_layout_k_tiles():
    """Tile order and ragged tiles (hand-worked): N=40, K=64*65, all widths 1.
    2 row-tiles x 2 k-tiles, t = kt*2 + rt. Tile 0 (32 rows, 64 columns):
    map 512 B + 32 full blocks (codes 512 + so 256 = 768 B) = 25088 B
    (1568 units). Tile 1 (8 rows, 64 columns): 512 + 8*768 = 6656 B (416).
    Tile 2 (32 rows, 1 column): map 8 -> 16 + one block of 32 records
    (codes 256, so 128) = 400 B (25). Tile 3 (8 rows, 1 column): 16 + 64 +
    32 = 112 B (7). Counts N_0 = 2048, 512, 32, 8."""
    N, G = 40, 65
    widths = np.ones((N, G), np.uint8)
    W = (_rng(22).standard_normal((N, 64 * G)) * 0.02).astype(np.float32)
    lay = oracle.pack(W, widths)
    assert oracle.layout_sizes(widths) == (4, N * G, 2016)
    tiles = lay["tiles"].reshape(-1, 4)
    assert [list(map(int, t)) for t in tiles] == [[0, 1568, 2048, 0], [1568, 416, 512, 0], [1984, 25, 32, 0],
                                                  [2009, 7, 8, 0], [2016, 0, 0, 0]]
    st = lay["stream"]
    # tile 1 (rows 32..39): record e = 8 l + r, block e // 64, entry e % 64
    base = 1568 * 16 + 512
    for l, r in ((0, 0), (5, 0), (5, 2), (7, 7), (63, 7)):
        e = 8 * l + r
        so, w = _record(W, 32 + r, l, 1)
        at = base + 768 * (e // 64)
        j = e % 64
        assert [int(v) for v in st[(at + 8 * j) // 4:(at + 8 * j) // 4 + 2]] == w
        assert int(st[(at + 512 + 4 * j) // 4]) == so
    # tile 3 (rows 32..39, column 64): one block of 8, rows in order
    base = 2009 * 16 + 16
    for r in (0, 7):
        so, w = _record(W, 32 + r, 64, 1)
        assert [int(v) for v in st[(base + 8 * r) // 4:(base + 8 * r) // 4 + 2]] == w
        assert int(st[(base + 64 + 4 * r) // 4]) == so


def _walk_layout(widths, N, K):
    """Independent reading of the layout rules (written from the header text,
    not from the oracle's C): yields, per tile, (base byte, size, the two
    count words, map words, [(byte of codes, byte of so, row, kg, b)])."""
    G = K // 64
    RT, KT = -(-N // 32), -(-G // 64)
    up = lambda v: -(-v // 16) * 16
    cls = {1: 0, 2: 1, 4: 2, 8: 3}
    base = 0
    for t in range(RT * KT):
        kt, rt = divmod(t, RT)
        rows = range(32 * rt, min(N, 32 * rt + 32))
        ks = range(64 * kt, min(G, 64 * kt + 64))
        mp = []
        for kg in ks:
            p0 = sum((cls[int(widths[r, kg])] & 1) << (r - 32 * rt) for r in rows)
            p1 = sum((cls[int(widths[r, kg])] >> 1) << (r - 32 * rt) for r in rows)
            mp += [p0, p1]
        lists = [[(r, kg) for kg in ks for r in rows if cls[int(widths[r, kg])] == c] for c in range(4)]
        pos = up(8 * len(ks))
        recs = []
        for c in range(4):
            b = 1 << c
            for k0 in range(0, len(lists[c]), 64):
                blk = lists[c][k0:k0 + 64]
                m = len(blk)
                for j, (r, kg) in enumerate(blk):
                    recs.append((base + pos + 8 * b * j, base + pos + up(8 * b * m) + 4 * j, r, kg, b))
                pos += up(8 * b * m) + up(4 * m)
        n = [len(x) for x in lists]
        yield base, pos, (n[0] | (n[1] << 16), n[2] | (n[3] << 16)), mp, recs
        base += pos


def pin_layout_invariants():
    r = _rng(18)
    cases = [(1, 64), (5, 128), (32, 256), (33, 192), (40, 640), (33, 64 * 70), (18, 64 * 130), (64, 512)]
    for (N, K) in cases:
        G = K // 64
        widths = r.choice(np.array([1, 2, 4, 8], np.uint8), size=(N, G), p=[0.55, 0.2, 0.15, 0.1])
        W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
        lay = oracle.pack(W, widths)
        T, R, B16 = oracle.layout_sizes(widths)
        RT, KT = oracle.tile_grid(N, K)
        assert T == RT * KT and R == N * G
        tiles = lay["tiles"].reshape(-1, 4)
        st = lay["stream"]
        q2, s2, o2 = oracle.quantize_matrix(W, widths)
        seen = np.zeros((N, G), np.int32)
        end = 0
        for t, (base, size, iw, mp, recs) in enumerate(_walk_layout(widths, N, K)):
            assert list(tiles[t]) == [base // 16, size // 16, iw[0], iw[1]]
            assert [int(v) for v in st[base // 4:base // 4 + len(mp)]] == mp
            for (cat, sat, row, kg, b) in recs:
                words = [int(v) for v in oracle.pack_group_record(q2[row, 64 * kg:64 * kg + 64], b)]
                assert [int(v) for v in st[cat // 4:cat // 4 + 2 * b]] == words
                assert int(st[sat // 4]) == int(s2[row, kg]) | (int(o2[row, kg]) << 16)
                seen[row, kg] += 1
            end = base + size
        assert (seen == 1).all()
        assert list(tiles[T]) == [end // 16, 0, 0, 0] and end == 16 * B16
        # reading back gives the quantiser's output in natural order
        q, s, o, w = oracle.unpack(lay)
        assert np.array_equal(q, q2) and np.array_equal(s, s2) and np.array_equal(o, o2)
        assert np.array_equal(w, widths)
        rows = r.choice(N, min(N, 5), replace=False)
        qr, sr, orr, wr = oracle.unpack(lay, rows)
        assert np.array_equal(qr, q2[rows]) and np.array_equal(wr, widths[rows])


# --------------------------------------------------------------------------
# GEMV: exact integer case, exact rationals on tiny matrices
# --------------------------------------------------------------------------
def pin_exact_integer_matvec():
    """All groups 8-bit with integer weights in [0,255] and both 0 and 255 in
    every group: the quantiser must give scale 1, offset 0, codes = weights,
    so y equals the int64 product exactly."""
    r = _rng(19)
    N, K = 96, 768
    Wi = r.integers(0, 256, (N, K))
    Wi[:, 0::64] = 0
    Wi[:, 1::64] = 255
    widths = np.full((N, K // 64), 8, np.uint8)
    lay = oracle.pack(Wi.astype(np.float32), widths)
    q, s, o, _ = oracle.unpack(lay)
    assert (s == 0x3C00).all() and (o == 0).all()
    xi = r.integers(-2, 3, (3, K))
    y = oracle.gemv(q, s, o, xi.astype(np.float16).view(np.uint16))
    assert np.array_equal(y, (xi @ Wi.T).astype(np.float64))


def _tiny_case(seed, N, K, with_resid):
    r = _rng(seed)
    G = K // 64
    widths = r.choice(np.array([1, 2, 4, 8], np.uint8), size=(N, G))
    widths.flat[:4] = [1, 2, 4, 8][:widths.size] if widths.size >= 4 else widths.flat[:4]
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    q, s, o = oracle.quantize_matrix(W, widths)
    x = r.standard_normal((2, K)).astype(np.float16).view(np.uint16)
    resid = None
    if with_resid:
        resid = oracle.make_cell_residual(r.uniform(-0.49, 0.49, (N, K)), np.repeat(s, 64, axis=1)[:, ::64])
    return q, s, o, x, resid


def pin_gemv_exact_rationals():
    for seed, (N, K) in enumerate([(4, 64), (4, 128), (3, 192)]):
        for with_resid in (False, True):
            q, s, o, x, resid = _tiny_case(100 + seed, N, K, with_resid)
            y = oracle.gemv(q, s, o, x, resid)
            ye = exact.gemv_exact(q.tolist(), s.tolist(), o.tolist(), x.tolist(),
                                  None if resid is None else resid.tolist())
            for b in range(2):
                for n in range(N):
                    e = ye[b][n]
                    assert abs(Fraction(float(y[b, n])) - e) <= abs(e) * Fraction(1, 10 ** 14) + Fraction(1, 10 ** 300), \
                        (seed, with_resid, b, n, float(y[b, n]), float(e))


def pin_gemm_bf16_exact():
    r = _rng(21)
    N, K = 3, 128
    widths = np.array([[1, 8], [2, 4], [8, 1]], np.uint8)
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    q, s, o = oracle.quantize_matrix(W, widths)
    import synth
    xb = synth.x_bf16(0, (99,), 3, K)
    y = oracle.gemv(q, s, o, xb, bf16=True)
    ye = exact.gemv_exact(q.tolist(), s.tolist(), o.tolist(), xb.tolist(), bf16=True)
    for m in range(3):
        for n in range(N):
            assert abs(Fraction(float(y[m, n])) - ye[m][n]) <= abs(ye[m][n]) * Fraction(1, 10 ** 14)


def pin_bf16_weights():
    """bfloat16 rounding (8 significant bits, ties to even) on hand-worked
    values, and the bf16 weights of the batched product."""
    f = oracle.f32_to_bf16
    assert f(1.0) == 0x3F80
    assert f(1.0 + 2.0 ** -8) == 0x3F80            # half an ulp above 1: tie, 1 is even
    assert f(1.0 + 3 * 2.0 ** -8) == 0x3F82        # tie between 0x3F81 (odd) and 0x3F82
    assert f(1.0 + 2.0 ** -8 + 2.0 ** -20) == 0x3F81
    assert f(-(1.0 + 2.0 ** -8)) == 0xBF80
    assert f(255.5) == 0x4380 and f(253.5) == 0x437E and f(255.25) == 0x437F
    one, half, quarter = 0x3C00, 0x3800, 0x3400     # fp16 1.0, 0.5, 0.25
    q = np.array([[255, 253, 255, 7] + [0] * 60], np.uint8)
    s16 = np.array([[one]], np.uint16)
    assert list(oracle.dequant_bf16(q, s16, np.array([[half]], np.uint16))[0, :4]) == [0x4380, 0x437E, 0x4380, 0x40F0]
    assert oracle.dequant_bf16(q, s16, np.array([[quarter]], np.uint16))[0, 0] == 0x437F
    # exact grids stay exact; random weights move by at most half a bf16 ulp
    r = _rng(31)
    qi = r.integers(0, 256, (8, 128)).astype(np.uint8)
    s1 = np.full((8, 2), one, np.uint16)
    o0 = np.zeros((8, 2), np.uint16)
    assert np.array_equal(oracle.bf16_to_f64(oracle.dequant_bf16(qi, s1, o0)), qi.astype(np.float64))
    W = (r.standard_normal((16, 256)) * 0.02).astype(np.float32)
    widths = r.choice(np.array([1, 2, 4, 8], np.uint8), size=(16, 4))
    q, s, o = oracle.quantize_matrix(W, widths)
    Wd = oracle.bf16_to_f64(oracle.dequant_bf16(q, s, o))
    Wref = np.repeat(oracle.f64_from_f16(s), 64, 1) * q + np.repeat(oracle.f64_from_f16(o), 64, 1)
    assert np.all(np.abs(Wd - Wref) <= np.abs(Wref) * 2.0 ** -8 + 1e-30)
    assert np.any(Wd != Wref)


# --------------------------------------------------------------------------
# In-cell residual: drift bound, revocation, re-quantisation check
# --------------------------------------------------------------------------
def _cell_case(seed, N=24, K=256, b=4):
    r = _rng(seed)
    widths = np.full((N, K // 64), b, np.uint8)
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    q, s, o = oracle.quantize_matrix(W, widths)
    s_full = np.repeat(s, 64, axis=1)
    u = r.uniform(-0.49, 0.49, (N, K))
    resid = oracle.make_cell_residual(u, s)
    return r, widths, q, s, o, s_full, resid


def pin_drift_bound_and_revocation():
    r, widths, q, s, o, s_full, resid = _cell_case(30)
    K = q.shape[1]
    x = r.standard_normal((2, K)).astype(np.float16).view(np.uint16)
    y0 = oracle.gemv(q, s, o, x)
    yr = oracle.gemv(q, s, o, x, resid)
    xd = oracle.f64_from_f16(x)
    rd = oracle.f64_from_f16(resid)
    sd = oracle.f64_from_f16(s_full)
    drift = np.abs(yr - y0)
    bound = np.abs(xd) @ np.abs(rd).T                 # sum_k |x_k| |r_nk|
    cell = np.abs(xd) @ (sd / 2).T                    # sum_k |x_k| s_g(k) / 2
    assert np.all(drift <= bound * (1 + 1e-12) + 1e-15)
    assert np.all(bound < cell)
    # the residual changes the output, and the change is linear in it
    assert np.max(drift) > 0
    lin = xd @ rd.T
    assert np.allclose(yr - y0, lin, rtol=1e-9, atol=1e-12)
    # revocation: dropping the residual gives back the base output bit-for-bit
    assert np.array_equal(oracle.gemv(q, s, o, x, None), y0)


def pin_drift_bound_attained():
    """The closed-form drift bound is attained by the extremal residual
    r = sign(x) s/2 (the supremum over residuals inside their cells): its
    drift, computed through the GEMV, which shares no arithmetic with the
    closed form, equals the bound for every width; in-cell residuals stay
    below it."""
    for b, std in ((1, 0.02), (2, 0.02), (4, 0.02), (8, 0.5)):
        r = _rng(40 + b)
        N, K = 12, 192
        widths = np.full((N, K // 64), b, np.uint8)
        W = (r.standard_normal((N, K)) * std).astype(np.float32)
        q, s, o = oracle.quantize_matrix(W, widths)
        s_full = oracle.f64_from_f16(np.repeat(s, 64, axis=1))
        x = r.standard_normal((3, K)).astype(np.float16).view(np.uint16)
        xd = oracle.f64_from_f16(x)
        bound = oracle.drift_bound(s, x)
        assert bound.shape == (3, N)
        y0 = oracle.gemv(q, s, o, x)
        for bi in range(3):
            half = s_full / 2 * np.sign(xd[bi])[None, :]
            r16 = oracle.f16_from_f64(half)
            assert np.array_equal(oracle.f64_from_f16(r16), half)     # s/2 is exact in fp16 here
            drift = oracle.gemv(q, s, o, x[bi:bi + 1], r16)[0] - y0[bi]
            assert np.allclose(drift, bound[bi], rtol=1e-12, atol=1e-12)
        resid = oracle.make_cell_residual(r.uniform(-0.49, 0.49, (N, K)), s)
        assert np.all(np.abs(oracle.gemv(q, s, o, x, resid) - y0) <= bound)


def pin_rrq_levels():
    """Recurrent residual levels: every level leaves at most half its scale
    of error (RTN on the fp16 grid, up to the fp16 rounding of the scale and
    offset); a group already on a 4-level fp16 grid is exact after the base
    (the next level is the degenerate group: scale 0, codes 0); the error
    and the GEMV error shrink level by level."""
    r = _rng(50)
    N, K = 16, 256
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[3, 64:128] = np.float32(0.0078125) + np.float32(0.001953125) * r.integers(0, 4, 64).astype(np.float32)
    W[3, 64] = np.float32(0.0078125)
    W[3, 65] = np.float32(0.0078125 + 3 * 0.001953125)
    levels, E = oracle.rrq_levels(W, 4)
    prev = np.abs(W).max()
    Ei = W.astype(np.float64)
    for i, (q, s16, o16) in enumerate(levels):
        s = oracle.f64_from_f16(np.repeat(s16, 64, axis=1))
        o = oracle.f64_from_f16(np.repeat(o16, 64, axis=1))
        assert q.max() <= 3
        Ei = Ei - (s * q + o)                          # fp64 accumulation of the same levels
        err = np.abs(Ei)
        assert np.all(err <= 0.5 * s * (1 + 2.0 ** -6) + 4.0 ** -12), i
        assert err.max() < prev, i
        prev = err.max()
    _, s1, _ = levels[1]
    assert s1[3, 1] == 0 and np.all(levels[1][0][3, 64:128] == 0)
    assert np.allclose(E, Ei, rtol=0, atol=1e-9)       # binary32 recursion vs fp64 bookkeeping
    x = r.standard_normal((2, K)).astype(np.float16).view(np.uint16)
    exact = oracle.f64_from_f16(x) @ W.astype(np.float64).T
    errs = [np.abs(oracle.rrq_gemv(levels[:k + 1], x) - exact).max() for k in range(4)]
    assert all(errs[k + 1] < errs[k] for k in range(3)), errs


def pin_requant_verify():
    r, widths, q, s, o, s_full, resid = _cell_case(31)
    N, K = q.shape
    mism, ooc, first, qp = oracle.requant_verify(q, s, o, widths, resid, want_codes=True)
    assert (mism, ooc, first) == (0, 0, 2 ** 64 - 1)
    assert np.array_equal(qp, q)
    # zero residual: trivially in every cell
    zero = np.zeros_like(resid)
    assert oracle.requant_verify(q, s, o, widths, zero)[:3] == (0, 0, 2 ** 64 - 1)
    # |r| exactly half a cell is outside the (open) cell
    planted = [(3, 5), (7, 130), (20, 255)]
    bad = resid.copy()
    for (n, k) in planted:
        bad[n, k] = oracle.f16_from_f64(np.array([0.5]) * oracle.f64_from_f16(s_full[n, k:k + 1]))[0]
    mism, ooc, first, _ = oracle.requant_verify(q, s, o, widths, bad)
    assert ooc == len(planted) and first == min(n * K + k for n, k in planted)
    # 0.6 of a cell at an interior code moves the code
    interior = np.argwhere((q > 0) & (q < 15))
    sel = interior[r.choice(len(interior), 5, replace=False)]
    bad = resid.copy()
    for n, k in sel:
        bad[n, k] = oracle.f16_from_f64(np.array([0.6]) * oracle.f64_from_f16(s_full[n, k:k + 1]))[0]
    mism, ooc, first, qp = oracle.requant_verify(q, s, o, widths, bad, want_codes=True)
    assert mism == 5 and ooc == 5
    for n, k in sel:
        assert qp[n, k] == q[n, k] + 1
    # A flipped bit in a served artifact: the check re-quantises against the
    # artifact it is given, so it passes; the emitted codes then differ from the
    # released ones in exactly that position (the bit-for-bit comparison).
    q2 = q.copy()
    q2[11, 77] ^= 1
    mism, ooc, first, qp2 = oracle.requant_verify(q2, s, o, widths, resid, want_codes=True)
    assert (mism, ooc) == (0, 0)
    diff = np.argwhere(qp2 != q)
    assert diff.tolist() == [[11, 77]]


def pin_requant_verify_edge_cells():
    """Edge codes clamp (CellFill abstract: re-quantisation returns the released
    codes; the grid of a b-bit group is q in [0, 2^b - 1]). Hand-worked, one
    64-weight group per width b = 1, 2, 4, 8 with s = 0.25, o = -1 (both exact
    in binary16). Weight 0 has q = 0 and r = -0.15625 (= -0.625 s); weight 1
    has q = L = 2^b - 1 and r = +0.15625. Then (v - o) / s = -0.625 and
    L + 0.625 exactly, which round to -1 and L + 1 and clamp back to 0 and L:
    no code changes, but both residuals leave their cells (|r| >= s/2).
    A third residual, +0.625 s at an interior code q = 1 (b >= 2), moves the
    code to 2. Only a clamp to the group's own [0, L] gives these counts."""
    widths = np.array([[1], [2], [4], [8]], np.uint8)
    N, K = 4, 64
    s16 = np.full((N, 1), 0x3400, np.uint16)            # 0.25
    o16 = np.full((N, 1), 0xBC00, np.uint16)            # -1.0
    assert oracle.f64_from_f16(s16[0])[0] == 0.25 and oracle.f64_from_f16(o16[0])[0] == -1.0
    q = np.zeros((N, K), np.uint8)
    r16 = np.zeros((N, K), np.uint16)
    minus, plus = 0xB100, 0x3100                        # -0.15625, +0.15625
    assert list(oracle.f64_from_f16(np.array([minus, plus], np.uint16))) == [-0.15625, 0.15625]
    for i in range(N):
        L = (1 << int(widths[i, 0])) - 1
        q[i, 0], r16[i, 0] = 0, minus
        q[i, 1], r16[i, 1] = L, plus
        q[i, 2:] = np.arange(K - 2) % (L + 1)
    mism, ooc, first, qp = oracle.requant_verify(q, s16, o16, widths, r16, want_codes=True)
    assert (mism, ooc, first) == (0, 8, 0)
    assert np.array_equal(qp, q)
    # the same residuals inside their cells at interior codes (b >= 2): q = 1
    # with +0.625 s moves to 2 (a real mismatch the clamp must not hide)
    q2, r2 = q.copy(), r16.copy()
    for i in range(1, N):
        q2[i, 3], r2[i, 3] = 1, plus
    mism, ooc, first, qp = oracle.requant_verify(q2, s16, o16, widths, r2, want_codes=True)
    assert (mism, ooc, first) == (3, 11, 0)
    assert [int(qp[i, 3]) for i in range(1, N)] == [2, 2, 2]
    # only the edge weights of the 1-bit row: first bad index is its weight 0
    r3 = np.zeros_like(r16)
    r3[0, 1] = plus
    assert oracle.requant_verify(q, s16, o16, widths, r3)[:3] == (0, 1, 1)


def pin_residual_inside_cell():
    """The generated residual satisfies |r| < s/2 and so stays in the cell."""
    _, _, q, s, o, s_full, resid = _cell_case(32)
    rd = np.abs(oracle.f64_from_f16(resid))
    sd = oracle.f64_from_f16(s_full)
    assert np.all(rd <= 0.49 * sd * (1 + 2.0 ** -11)) and np.all(rd < 0.5 * sd)


# --------------------------------------------------------------------------
# Accounting (VBQ abstract: 69% of groups at 1 bit, LM head ~1.09 mean bits,
# 131M model at 1.82 mean bits)
# --------------------------------------------------------------------------
def _golden(name):
    vals = {}
    for line in open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", name)):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            vals[k] = float(v)
    return vals


def pin_cell8_encode_values():
    """Compact in-cell residual, hand-worked (scale s = 0.25 = 0x3400):
    r = fp16(0.1) = 0.0999755859375 -> r/s*256 = 102.375 -> f = 102;
    r = 0.125 -> 128 -> clamped to 127; r = -0.125 -> -127;
    r = -2^-10 -> -1; r = 1.75*2^-9 (0x1B00) -> 3.5 -> 4 (tie to even);
    r = 1.375*2^-9 (0x1980) -> 2.75 -> 3; r = 1.25*2^-9 (0x1900) -> 2.5 -> 2;
    a zero scale gives 0 whatever r."""
    vals = [(0x2E66, 102), (0x3000, 127), (0xB000, -127), (0x9400, -1), (0x1B00, 4), (0x1980, 3), (0x1900, 2)]
    r16 = np.zeros((2, 64), np.uint16)
    for i, (r, _) in enumerate(vals):
        r16[0, i] = r
        r16[1, i] = r
    s16 = np.array([[0x3400], [0x0000]], np.uint16)
    f = oracle.cell8_encode(r16, s16)
    assert [int(v) for v in f[0, :len(vals)]] == [e for _, e in vals]
    assert (f[1] == 0).all()


def pin_cell8_gemv_equals_fp16_residual():
    """With power-of-two scales every s*f/256 is an exact fp16 value, so the
    GEMV with the compact residual must equal, bit for bit, the GEMV with the
    fp16 residual r = fp16(s*f/256) (the two oracle paths share no code for
    the residual term)."""
    r = _rng(31)
    N, K = 5, 256
    G = K // 64
    widths = r.choice(np.array([1, 2, 4, 8], np.uint8), size=(N, G))
    q = np.zeros((N, K), np.uint8)
    for n in range(N):
        for g in range(G):
            q[n, 64 * g:64 * g + 64] = r.integers(0, 1 << int(widths[n, g]), 64)
    s = oracle.f16_from_f64(2.0 ** r.integers(-8, -2, (N, G)).astype(np.float64))
    o = oracle.f16_from_f64(r.standard_normal((N, G)) * 0.05)
    f = r.integers(-127, 128, (N, K)).astype(np.int8)
    sd = np.repeat(oracle.f64_from_f16(s), 64, axis=1)
    r16 = oracle.f16_from_f64(sd * f.astype(np.float64) / 256.0)
    assert np.array_equal(oracle.f64_from_f16(r16), sd * f.astype(np.float64) / 256.0)
    x = oracle.f16_from_f64(r.standard_normal((2, K)))
    y8 = oracle.gemv_cell8(q, s, o, x, f)
    y16 = oracle.gemv(q, s, o, x, resid=r16)
    assert np.array_equal(y8, y16)


def pin_cell8_inside_cell():
    """Whatever residual is encoded, the decoded s*f/256 is inside the cell
    (|.| <= 127/256 s < s/2); a residual already inside the representable
    range comes back within s/512 (half a step of the fraction) plus the
    binary32 rounding of r/s."""
    r = _rng(32)
    N, K = 6, 128
    G = K // 64
    s = oracle.f16_from_f64(np.abs(r.standard_normal((N, G))) * 0.01 + 1e-3)
    sd = np.repeat(oracle.f64_from_f16(s), 64, axis=1)
    wide = oracle.f16_from_f64(r.uniform(-2, 2, (N, K)) * sd)
    f = oracle.cell8_encode(wide, s)
    dec = sd * f.astype(np.float64) / 256.0
    assert (np.abs(dec) <= 127.0 / 256.0 * sd).all() and (np.abs(dec) < 0.5 * sd).all()
    inside = oracle.f16_from_f64(r.uniform(-127 / 256, 127 / 256, (N, K)) * sd)
    f2 = oracle.cell8_encode(inside, s)
    err = np.abs(sd * f2.astype(np.float64) / 256.0 - oracle.f64_from_f16(inside))
    assert (err <= sd / 512.0 * (1 + 1e-6)).all()


def pin_cell8_decode_values():
    """fp16(s f / 256), hand-worked: s = 0.5, f = 1 -> 2^-9 (0x1800);
    s = 1, f = -127 -> -0.49609375 (0xB7F0, exact); s = 2047/2048 (0x3BFF),
    f = 3 -> 6141 * 2^-19, 13 significant bits, rounded to 6140 * 2^-19
    (0x21FF); s = 1027/1024 (0x3C03), f = 3 -> 3081 * 2^-18, a tie between
    1540 and 1541 units of 2^-17, to even 1540 (0x2204); s = 2^-14 (0x0400),
    f = 1 -> 2^-22, subnormal 4 * 2^-24 (0x0004); s = 0x0401, f = 5 ->
    20.02 units of 2^-24, to 20 (0x0014); a zero scale gives +0 for f >= 0
    and, as IEEE multiplication does, -0 (0x8000) for f < 0."""
    cases = [(0x3800, 1, 0x1800), (0x3C00, -127, 0xB7F0), (0x3BFF, 3, 0x21FF), (0x3C03, 3, 0x2204),
             (0x0400, 1, 0x0004), (0x0401, 5, 0x0014), (0x0000, 77, 0x0000), (0x0000, -5, 0x8000)]
    f = np.zeros((len(cases), 64), np.int8)
    s16 = np.zeros((len(cases), 1), np.uint16)
    for i, (s, v, _) in enumerate(cases):
        s16[i, 0] = s
        f[i, :] = v
    r16 = oracle.cell8_decode(f, s16)
    for i, (_, _, want) in enumerate(cases):
        assert (r16[i] == want).all(), (i, hex(int(r16[i, 0])), hex(want))


def pin_cell8_decode_in_cell():
    """Every fraction decodes to a residual the re-quantisation check passes
    (inside its cell, codes come back unchanged), and encoding the decoded
    residual gives the fraction back (r / s * 256 is within binary32 and fp16
    rounding of f, far below half a step)."""
    r = _rng(33)
    N, K = 9, 192
    G = K // 64
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    widths = r.choice(np.array([1, 2, 4, 8], np.uint8), size=(N, G))
    q, s, o = oracle.quantize_matrix(W, widths)
    f = r.integers(-127, 128, (N, K)).astype(np.int8)
    f[0, :] = 127
    f[1, :] = -127
    r16 = oracle.cell8_decode(f, s)
    mism, ooc, first, _ = oracle.requant_verify(q, s, o, widths, r16)
    assert (mism, ooc, first) == (0, 0, 2 ** 64 - 1)
    live = np.repeat(oracle.f64_from_f16(s), 64, axis=1) > 2.0 ** -14    # normal fp16 scales
    back = oracle.cell8_encode(r16, s)
    assert np.array_equal(back[live], f[live])


def pin_abstract_storage_ratios():
    """The VBQ abstract's storage ratios follow from its mean bits when only
    code bits are counted (16 / mean bits per parameter), and do not when the
    fp16 scale and offset per group (+0.5 bit) are counted: so "mean bits" is
    code bits per weight, the quantity the oracle's accounting reports."""
    g = _golden("vbq_abstract_figures.txt")
    codes_only = g["fp16_control_55m_params"] * 16 / (g["model_131m_params"] * g["model_131m_mean_bits"])
    with_meta = g["fp16_control_55m_params"] * 16 / (g["model_131m_params"] * (g["model_131m_mean_bits"] + 0.5))
    assert abs(codes_only - g["storage_ratio_131m_vs_55m"]) / g["storage_ratio_131m_vs_55m"] < 0.05
    assert abs(with_meta - g["storage_ratio_131m_vs_55m"]) / g["storage_ratio_131m_vs_55m"] > 0.2
    # the 1.46B case implies about 1.76 mean code bits at the printed ratio
    implied = g["fp16_control_593m_params"] * 16 / (g["model_1p46b_params"] * g["storage_ratio_1p46b_vs_593m"])
    assert 1.6 < implied < 1.9
    # the oracle's own accounting: a layout's code bits per weight is the mean width
    widths = np.array([[1, 1, 2, 8], [4, 1, 1, 2]], np.uint8)
    lay = oracle.layout_sizes(widths)
    assert lay[1] == widths.size
    assert abs(float(widths.mean()) - 2.5) < 1e-12


def pin_mean_bits_accounting():
    import synth
    g = _golden("vbq_abstract_figures.txt")
    assert abs(synth.mean_bits(synth.MIX_LM_HEAD) - g["lm_head_mean_bits"]) < 0.015
    assert synth.MIX_DEFAULT[1] == g["share_groups_1bit"]
    assert abs(synth.mean_bits(synth.MIX_DEFAULT) - 1.79) < 1e-12
    assert abs(synth.mean_bits(synth.MIX_LM_HEAD) - 1.10) < 1e-12
    w = synth.widths(0, (0, 0, 0), 768, 12, synth.MIX_DEFAULT)
    mean = float(w.mean())
    var = sum(p * (b - 1.79) ** 2 for b, p in synth.MIX_DEFAULT.items())
    se = math.sqrt(var / w.size)
    assert abs(mean - 1.79) < 4 * se and abs(mean - 1.82) < 4 * se + 0.03
    assert abs(float((w == 1).mean()) - 0.69) < 0.03
    # bytes of a layout: codes 8*sum(b) per group, 4 (scale+offset) per group,
    # 2 bits of width per group (8 bytes per column of a tile); padding at most
    # 8 bytes per map and 8 + 12 per block, a tile having at most 4 * 32 blocks
    lay_w = w[:64]
    T, R, B16 = oracle.layout_sizes(lay_w)
    RT, KT = oracle.tile_grid(64, 64 * 12)
    lo = 8 * int(lay_w.astype(np.int64).sum()) + 4 * R + 8 * RT * 12
    assert lo == 8 * int(lay_w.astype(np.int64).sum()) + 4.25 * R
    assert lo <= 16 * B16 <= lo + 8 * T + 20 * 128 * T


ALL_PINS = [
    pin_cell8_encode_values, pin_cell8_gemv_equals_fp16_residual, pin_cell8_inside_cell,
    pin_cell8_decode_values, pin_cell8_decode_in_cell,
    pin_f16_conversion, pin_rtn_nearest_level, pin_rtn_scale_offset_nearest, pin_rtn_exact_grid,
    pin_rtn_degenerate_group, pin_canonical_lsb_first, pin_record_even_odd, pin_layout_k_tiles,
    pin_layout_worked_example, pin_layout_column_major, pin_layout_invariants,
    pin_exact_integer_matvec, pin_gemv_exact_rationals, pin_gemm_bf16_exact,
    pin_drift_bound_and_revocation, pin_drift_bound_attained, pin_rrq_levels, pin_requant_verify,
    pin_requant_verify_edge_cells,
    pin_residual_inside_cell,
    pin_mean_bits_accounting,
    pin_abstract_storage_ratios, pin_bf16_weights,
]
