"""Soundness of the record-level bound the requant-verify kernels use to skip
the per-weight quotient (CPU, brute force in numpy binary32).

For a group with fp16 scale s > 0, fp16 offset o and L = 2^b - 1, the kernels
treat every weight whose fp16 residual has |r| < T as keeping its code and
staying in its cell, where T is the largest fp16 value at or below
  thr = 0.5 s - 2^-19 (s (L + 2) + |o|)        (evaluated in binary32).
The re-quantisation itself is the binary32 sequence of the CellFill check:
  deq = f32(s q) + o;  v = deq + r;  q' = clamp(rint((v - o) / s), 0, L).
This test recomputes T here and checks, for every code q of the group and
residuals at and inside +-T (the largest allowed magnitude first), that q'
equals q and |r| < s / 2, over scales from fp16 subnormals to 1e4 and offsets
up to 65504 in magnitude, including the adversarial case of a tiny scale
beside a huge offset (there T is 0 and nothing may skip). A slack too small
or a missing |o| term fails the brute-force checks; the hand-worked value
pins the rounding down to fp16.
"""
import numpy as np
import pytest

F32 = np.float32


def keep_bound(s16: np.ndarray, o16: np.ndarray, L: int) -> np.ndarray:
    """T per group as fp16 bit patterns (0: nothing may skip)."""
    s = s16.astype(F32)
    o = o16.astype(F32)
    with np.errstate(invalid="ignore", over="ignore"):
        thr = F32(0.5) * s - F32(2.0 ** -19) * (s * F32(L + 2) + np.abs(o))
    ok = (s > 0) & np.isfinite(s) & (thr > 0)
    h = thr.astype(np.float16)                          # round to nearest
    hb = h.view(np.uint16).astype(np.int32)
    hb = np.where(h.astype(F32) > thr, hb - 1, hb)      # then down
    return np.where(ok, hb, 0).astype(np.uint16)


def requant(q: np.ndarray, s16, o16, r16, L: int) -> np.ndarray:
    s = s16.astype(F32)
    o = o16.astype(F32)
    r = r16.astype(F32)
    deq = (s * q.astype(F32)) + o
    a = (deq + r) - o
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.rint(a / s)
    return np.clip(t, 0, L)


def _groups(rng, n):
    s_exp = rng.uniform(-24, 13.3, n)                   # fp16 subnormals .. ~1e4
    s = np.float16(2.0) ** s_exp.astype(np.float16)
    s = np.where(s > 0, s, np.float16(2.0 ** -24)).astype(np.float16)
    o_kind = rng.integers(0, 4, n)
    o = np.where(o_kind == 0, rng.normal(0, 1, n) * s.astype(np.float64) * 8,
                 np.where(o_kind == 1, rng.normal(0, 1, n),
                          np.where(o_kind == 2, rng.uniform(-65504, 65504, n), -s.astype(np.float64) * 7)))
    return s, np.clip(o, -65504, 65504).astype(np.float16)


@pytest.mark.parametrize("bits", [1, 2, 4, 8])
def test_keep_bound_is_sound(bits):
    L = (1 << bits) - 1
    rng = np.random.default_rng(900 + bits)
    n = 20000
    s16, o16 = _groups(rng, n)
    T = keep_bound(s16, o16, L)
    live = T > 0
    assert live.mean() > 0.5                             # the bound is not vacuous
    # residual magnitudes: T itself is excluded (|r| < T), so the largest
    # allowed is the fp16 just below T, then a random one inside
    top = np.maximum(T.astype(np.int32) - 1, 0).astype(np.uint16).view(np.float16)
    inner = (rng.random(n) * top.astype(np.float64)).astype(np.float16)
    q = np.arange(L + 1)[None, :]
    for mag in (top, inner):
        for sign in (1, -1):
            r16 = (sign * mag.astype(np.float64)).astype(np.float16)[:, None]
            qp = requant(q, s16[:, None], o16[:, None], r16, L)
            bad = live[:, None] & (qp != q)
            assert not bad.any(), f"{bits}-bit: code changed at s={s16[bad.any(1)][:3]}, o={o16[bad.any(1)][:3]}"
            half = F32(0.5) * s16.astype(F32)
            assert not (live & ~(np.abs(r16[:, 0].astype(F32)) < half)).any()


def test_keep_bound_tiny_scale_huge_offset_skips_nothing():
    # binary32 spacing at |o| = 65504 is 2^-8, far above half of a 2^-20 scale
    s16 = np.array([2.0 ** -20, 2.0 ** -14, 1e-3], np.float16)
    o16 = np.array([65504.0, -65504.0, 65504.0], np.float16)
    assert not keep_bound(s16, o16, 15).any()


def test_keep_bound_hand_worked():
    # s = 1, o = 0, L = 15: thr = 0.5 - 17 * 2^-19 = 0.49996758...; the fp16
    # at or below it is 0.49975586 (0x37FF is 0.49975586, 0x3800 is 0.5)
    T = keep_bound(np.array([1.0], np.float16), np.array([0.0], np.float16), 15)
    assert T[0] == 0x37FF
    # s = 0 or negative or infinite: nothing may skip
    for s in (0.0, -1.0, np.inf):
        assert keep_bound(np.array([s], np.float16), np.array([0.0], np.float16), 15)[0] == 0
