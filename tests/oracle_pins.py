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


def pin_layout_worked_example():
    """N=2, K=128, widths [[1,8],[2,1]] (hand-worked). One tile. Class 0
    (1-bit) in (row, k-group) order: (row0,kg0), (row1,kg1); class 1: (row1,kg0);
    class 3: (row0,kg1). Blocks: class 0, m=2: codes 16 B, so 8 -> 16 B,
    meta 4 -> 16 B = 48 B at byte 0; class 1, m=1: 16 + 16 + 16 = 48 B at 48;
    class 3, m=1: 64 + 16 + 16 = 96 B at 96; total 192 B = 12 units.
    meta = row | kg<<4 -> 0, 17 (class 0), 1 (class 1), 16 (class 3)."""
    widths = np.array([[1, 8], [2, 1]], np.uint8)
    r = _rng(16)
    W = (r.standard_normal((2, 128)) * 0.02).astype(np.float32)
    lay = oracle.pack(W, widths)
    assert oracle.layout_sizes(widths) == (1, 4, 12)
    assert list(lay["tiles"]) == [0, 0, 2 | (1 << 16), 0 | (1 << 16), 4, 12, 0, 0]
    qs = {}
    for (row, kg, b) in ((0, 0, 1), (1, 1, 1), (1, 0, 2), (0, 1, 8)):
        s16, o16, q = oracle.quantize_group(W[row, 64 * kg:64 * kg + 64], b)
        qs[(row, kg)] = (s16 | (o16 << 16), list(oracle.pack_group_record(q, b)))
    st = [int(v) for v in lay["stream"]]
    assert len(st) == 48
    expect = ([*qs[(0, 0)][1], *qs[(1, 1)][1], qs[(0, 0)][0], qs[(1, 1)][0], 0, 0, 0 | (17 << 16), 0, 0, 0]
              + [*qs[(1, 0)][1], qs[(1, 0)][0], 0, 0, 0, 1, 0, 0, 0]
              + [*qs[(0, 1)][1], qs[(0, 1)][0], 0, 0, 0, 16, 0, 0, 0])
    assert st == expect
    # the reader rejects a nonzero padding byte (class 0 so padding, word 6)
    bad = dict(lay, stream=lay["stream"].copy())
    bad["stream"][6] = 1
    try:
        oracle.unpack(bad)
        raise AssertionError("nonzero padding accepted")
    except ValueError:
        pass


def pin_layout_block_chunks():
    """Records are contiguous inside a block: 16-byte chunk q of record l
    (b >= 2) sits at (l*b/2 + q)*16 bytes. One tile with 3 four-bit records
    (m=3): codes 96 B, then so (12 -> 16 B), then meta (6 -> 16 B)."""
    widths = np.array([[4, 4, 4]], np.uint8)
    W = (_rng(17).standard_normal((1, 192)) * 0.02).astype(np.float32)
    lay = oracle.pack(W, widths)
    assert oracle.layout_sizes(widths) == (1, 3, 8)
    chunks = lay["stream"].reshape(-1, 4)               # 16-byte chunks
    for kg in range(3):
        s16, o16, q = oracle.quantize_group(W[0, 64 * kg:64 * kg + 64], 4)
        words = oracle.pack_group_record(q, 4)
        assert list(chunks[2 * kg + 0]) == list(words[0:4])
        assert list(chunks[2 * kg + 1]) == list(words[4:8])
        assert _u32_at(lay["stream"], 96 + 4 * kg) == s16 | (o16 << 16)
        assert _u16_at(lay["stream"], 112 + 2 * kg) == kg << 4


def pin_layout_block_split():
    """A class segment longer than one block (hand-worked): N=16, K=192, widths
    8 in k-group 0 and at (row 0, kg 1), 1 elsewhere. In (row, kg) order the
    17 eight-bit records are (0,0), (0,1), (1,0), (2,0), ..., (15,0) and the 31
    one-bit records (0,2), (1,1), (1,2), ..., (15,1), (15,2).
    Class 0: one block m=31: codes 248 -> 256, so 124 -> 128, meta 62 -> 64:
    448 B. Class 3 (capacity 16): a full block at 448 (codes 1024: record l at
    448 + 64 l; so at 1472; meta at 1536; 1120 B), then a block of m=1 at 1568
    holding (15,0): codes at 1568, so at 1632, meta at 1648. Total 1664 B."""
    widths = np.ones((16, 3), np.uint8)
    widths[:, 0] = 8
    widths[0, 1] = 8
    W = (_rng(20).standard_normal((16, 192)) * 0.02).astype(np.float32)
    lay = oracle.pack(W, widths)
    assert oracle.layout_sizes(widths) == (1, 48, 104)
    assert list(lay["tiles"]) == [0, 0, 31, 17 << 16, 48, 104, 0, 0]
    st = lay["stream"]
    full = [(0, 0), (0, 1)] + [(r, 0) for r in range(1, 15)]
    for l in (0, 1, 2, 9, 15):
        row, kg = full[l]
        s16, o16, q = oracle.quantize_group(W[row, 64 * kg:64 * kg + 64], 8)
        at = 448 + 64 * l
        assert [int(v) for v in st[at // 4:at // 4 + 16]] == list(oracle.pack_group_record(q, 8))
        assert _u32_at(st, 1472 + 4 * l) == s16 | (o16 << 16)
        assert _u16_at(st, 1536 + 2 * l) == row | (kg << 4)
    s16, o16, q = oracle.quantize_group(W[15, 0:64], 8)
    assert [int(v) for v in st[1568 // 4:1568 // 4 + 16]] == list(oracle.pack_group_record(q, 8))
    assert _u32_at(st, 1632) == s16 | (o16 << 16)
    assert _u16_at(st, 1648) == 15
    # class 0 block: record l at 8l, so at 256 + 4l, meta at 384 + 2l
    s16, o16, q = oracle.quantize_group(W[0, 128:192], 1)
    assert [int(v) for v in st[0:2]] == list(oracle.pack_group_record(q, 1))
    assert _u32_at(st, 256) == s16 | (o16 << 16) and _u16_at(st, 384) == 0 | (2 << 4)
    assert _u16_at(st, 386) == 1 | (1 << 4) and _u16_at(st, 384 + 2 * 30) == 15 | (2 << 4)
    assert _u16_at(st, 384 + 2 * 31) == 0 and _u32_at(st, 256 + 4 * 31) == 0   # padding


def pin_layout_big_blocks():
    """Block capacities (hand-worked): N=16, K=64*20, widths 4 at (row 0,
    kg 0..3) and 1 elsewhere: 316 one-bit records, 4 four-bit records, one
    tile. In (row, kg) order the one-bit records are (0,4..19) then
    (r, 0..19) for r = 1..15, so record i >= 16 is (1 + (i-16)//20, (i-16)%20).
    Class 0, capacity 256: block 0 full (codes 2048, so 1024, meta 512 =
    3584 B: record l at 8l, so at 2048+4l, meta at 3072+2l); block 1 holds
    m=60 at 3584 (codes 480, so 240, meta 120 -> 128: record l at 3584+8l,
    so at 4064+4l, meta at 4304+2l). Class 2 at 4432: codes 4*32 = 128, so
    16, meta 16 (record l at 4432+32l, so at 4560+4l, meta at 4576+2l).
    Total 4592 B = 287 units."""
    N, K = 16, 64 * 20
    widths = np.ones((N, 20), np.uint8)
    widths[0, 0:4] = 4
    W = (_rng(23).standard_normal((N, K)) * 0.02).astype(np.float32)
    lay = oracle.pack(W, widths)
    assert oracle.layout_sizes(widths) == (1, 320, 287)
    assert list(lay["tiles"]) == [0, 0, 316, 4, 320, 287, 0, 0]
    st = lay["stream"]

    def one_bit(i):
        return (0, 4 + i) if i < 16 else (1 + (i - 16) // 20, (i - 16) % 20)

    for i, (code_at, so_at, meta_at) in ((0, (0, 2048, 3072)), (15, (120, 2108, 3102)),
                                         (16, (128, 2112, 3104)), (255, (2040, 3068, 3582)),
                                         (256, (3584, 4064, 4304)), (315, (4056, 4300, 4422))):
        row, kg = one_bit(i)
        s16, o16, q = oracle.quantize_group(W[row, 64 * kg:64 * kg + 64], 1)
        assert [int(v) for v in st[code_at // 4:code_at // 4 + 2]] == list(oracle.pack_group_record(q, 1))
        assert _u32_at(st, so_at) == s16 | (o16 << 16)
        assert _u16_at(st, meta_at) == row | (kg << 4)
    assert one_bit(255) == (12, 19) and one_bit(256) == (13, 0) and one_bit(315) == (15, 19)
    assert _u16_at(st, 4424) == 0 and _u32_at(st, 4428) == 0          # meta padding of block 1
    for kg in range(4):
        s16, o16, q = oracle.quantize_group(W[0, 64 * kg:64 * kg + 64], 4)
        at = 4432 + 32 * kg
        assert [int(v) for v in st[at // 4:at // 4 + 8]] == list(oracle.pack_group_record(q, 4))
        assert _u32_at(st, 4560 + 4 * kg) == s16 | (o16 << 16)
        assert _u16_at(st, 4576 + 2 * kg) == kg << 4


CAP = (256, 64, 64, 16)       # records per block of each width class


def _areas(c, m):
    """(codes, so, meta) area bytes of a block of class c with m records."""
    up = lambda v: -(-v // 16) * 16
    return (up(8 * m) if c == 0 else 8 * (1 << c) * m), up(4 * m), up(2 * m)


def _walk_tile(base, n):
    """Independent reading of one tile from the block rules: yields
    (class, m, l, block byte offset, codes area) per record; returns the tile's
    end byte via StopIteration.value."""
    seg = base
    for c in range(4):
        full = sum(_areas(c, CAP[c]))
        for i in range(n[c]):
            k, l = divmod(i, CAP[c])
            m = min(CAP[c], n[c] - k * CAP[c])
            yield c, m, l, seg + k * full, _areas(c, m)
        k, rem = divmod(n[c], CAP[c])
        seg += k * full + (sum(_areas(c, rem)) if rem else 0)
    return seg


def pin_layout_invariants():
    r = _rng(18)
    cases = [(1, 64), (5, 128), (16, 256), (17, 192), (40, 640), (33, 64 * 70), (18, 64 * 130), (64, 512)]
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
        rec = byte = 0
        for t in range(T):
            kt, rt = divmod(t, RT)                 # k-tile major storage
            blkw = widths[16 * rt:16 * rt + 16, 64 * kt:64 * kt + 64]
            n = [int((blkw == b).sum()) for b in (1, 2, 4, 8)]
            assert list(tiles[t]) == [rec, byte // 16, n[0] | (n[1] << 16), n[2] | (n[3] << 16)]
            seen, keys = set(), {0: [], 1: [], 2: [], 3: []}
            walker = _walk_tile(byte, n)
            while True:
                try:
                    c, m, l, blk, (ca, sa, ma) = next(walker)
                except StopIteration as e:
                    end = e.value
                    break
                mt = _u16_at(st, blk + ca + sa + 2 * l)
                row, kg = 16 * rt + (mt & 15), 64 * kt + (mt >> 4)
                assert (mt >> 10) == 0 and widths[row, kg] == (1 << c)
                keys[c].append(row * 64 + (kg - 64 * kt))
                seen.add((row, kg))
            for c in range(4):
                assert all(a < b for a, b in zip(keys[c], keys[c][1:]))     # (row, kg) order
            assert len(seen) == blkw.size
            rec += sum(n)
            byte = end
        assert list(tiles[T]) == [rec, byte // 16, 0, 0] and byte == 16 * B16
        # reading back gives the quantiser's output in natural order
        q, s, o, w = oracle.unpack(lay)
        q2, s2, o2 = oracle.quantize_matrix(W, widths)
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
    # bytes of a layout: codes 8*sum(b) per group plus 4 (scale+offset) + 2 (meta),
    # plus at most 8 + 12 + 14 bytes of padding per class segment of a tile
    lay_w = w[:64]
    T, R, B16 = oracle.layout_sizes(lay_w)
    code_bytes = 8 * int(lay_w.astype(np.int64).sum())
    assert code_bytes + 6 * R <= 16 * B16 <= code_bytes + 6 * R + 4 * 34 * T


def pin_layout_k_tiles():
    """Tiles are 16 rows x 64 k-groups, stored k-tile major. N=17, K=64*65
    (hand-worked): 2 row-tiles x 2 k-tiles, t = kt*2 + rt. Tile 0 (rt0, kt0):
    1024 one-bit records = 4 full blocks of 2048+1024+512 = 3584 B (896
    units); tile 1 (rt1, kt0): row 16 x 64 groups = one block of m=64,
    512+256+128 = 896 B; tile 2 (rt0, kt1):
    15 one-bit records (codes 120 -> 128, so 60 -> 64, meta 30 -> 32 = 224 B)
    and the 2-bit record of row 3 (16+16+16 = 48 B); tile 3 (rt1, kt1): the
    8-bit record of row 16 (64+16+16 = 96 B)."""
    N, K = 17, 64 * 65
    assert oracle.tile_grid(N, K) == (2, 2)
    widths = np.ones((N, 65), np.uint8)
    widths[16, 64] = 8
    widths[3, 64] = 2
    W = (_rng(19).standard_normal((N, K)) * 0.02).astype(np.float32)
    lay = oracle.pack(W, widths)
    tiles = lay["tiles"].reshape(-1, 4)
    assert oracle.layout_sizes(widths) == (4, N * 65, 975)
    assert [int(t[0]) for t in tiles[:4]] == [0, 1024, 1088, 1104]
    assert [int(t[1]) for t in tiles[:4]] == [0, 896, 952, 969]
    assert [int(t[2]) for t in tiles[:4]] == [1024, 64, 15 | (1 << 16), 0]
    assert [int(t[3]) for t in tiles[:4]] == [0, 0, 0, 1 << 16]
    assert list(tiles[4]) == [1105, 975, 0, 0]
    st = lay["stream"]
    # meta holds the row in the tile and the k-group in the tile
    assert _u16_at(st, 896 * 16 + 512 + 256) == 0                 # tile 1, (row 16, kg 0)
    assert _u16_at(st, 896 * 16 + 512 + 256 + 10) == 5 << 4       # tile 1, (row 16, kg 5)
    assert _u16_at(st, 952 * 16 + 128 + 64) == 0                  # tile 2, (row 0, kg 64)
    assert _u16_at(st, 952 * 16 + 128 + 64 + 28) == 15            # tile 2, (row 15, kg 64)
    assert _u16_at(st, 952 * 16 + 224 + 32) == 3                  # tile 2, 2-bit record of row 3
    assert _u16_at(st, 969 * 16 + 64 + 16) == 0                   # tile 3, (row 16, kg 64)
    s16, o16, q = oracle.quantize_group(W[16, 64 * 64:], 8)
    assert [int(v) for v in st[969 * 4:969 * 4 + 16]] == list(oracle.pack_group_record(q, 8))
    assert _u32_at(st, 969 * 16 + 64) == s16 | (o16 << 16)



ALL_PINS = [
    pin_f16_conversion, pin_rtn_nearest_level, pin_rtn_scale_offset_nearest, pin_rtn_exact_grid,
    pin_rtn_degenerate_group, pin_canonical_lsb_first, pin_record_even_odd, pin_layout_k_tiles,
    pin_layout_worked_example, pin_layout_block_chunks, pin_layout_block_split, pin_layout_invariants,
    pin_exact_integer_matvec, pin_gemv_exact_rationals, pin_gemm_bf16_exact,
    pin_drift_bound_and_revocation, pin_drift_bound_attained, pin_rrq_levels, pin_requant_verify,
    pin_residual_inside_cell,
    pin_mean_bits_accounting,
    pin_abstract_storage_ratios, pin_bf16_weights, pin_layout_big_blocks,
]
