"""Property tests of the oracle over random shapes and width mixes (CPU,
hypothesis). They restate what the layout and the quantiser promise for any
input, not any particular value:
  - the execution layout reads back as the quantiser's natural-order output,
    for any shape (ragged row tiles, one or several k-tiles) and width mix;
  - its size is what the sizing call says, and the tile table is consistent;
  - the dequantised GEMV does not depend on the layout (it is computed from
    the read-back arrays) and is linear in x;
  - a zero residual re-quantises to the same codes; one inside every cell
    (|u| <= 0.49 of the scale) passes the check.
"""
import os
import sys

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle  # noqa: E402

SETTINGS = dict(max_examples=25, deadline=None, suppress_health_check=[HealthCheck.too_slow])


@st.composite
def cases(draw):
    N = draw(st.integers(1, 70))
    G = draw(st.sampled_from([1, 2, 3, 63, 64, 65, 130]))
    p = np.array(draw(st.lists(st.floats(0.0, 1.0), min_size=4, max_size=4)), np.float64) + 1e-3
    seed = draw(st.integers(0, 2 ** 31 - 1))
    r = np.random.default_rng(seed)
    widths = r.choice(np.array([1, 2, 4, 8], np.uint8), size=(N, G), p=p / p.sum())
    W = (r.standard_normal((N, G * 64)) * 0.02).astype(np.float32)
    if N > 1 and draw(st.booleans()):
        W[N // 2, :64] = 0.015          # a constant group (scale 0)
    return W, widths, r


@given(cases())
@settings(**SETTINGS)
def test_layout_round_trip(case):
    W, widths, _ = case
    N, K = W.shape
    lay = oracle.pack(W, widths)
    T, R, B16 = oracle.layout_sizes(widths)
    assert lay["stream"].size * 4 == B16 * 16 and R == N * (K // 64)
    tiles = lay["tiles"].reshape(-1, 4)
    assert tiles.shape[0] == T + 1 and int(tiles[T][0]) == B16
    # tiles are back to back: each starts where the one before it ends
    assert all(int(tiles[t][0]) + int(tiles[t][1]) == int(tiles[t + 1][0]) for t in range(T))
    # the class counts of a tile add up to its groups (32 rows x 64 columns at most)
    RT, KT = oracle.tile_grid(N, K)
    for t in range(T):
        kt, rt = divmod(t, RT)
        rows, cols = min(32, N - 32 * rt), min(64, K // 64 - 64 * kt)
        counts = [int(tiles[t][2]) & 0xFFFF, int(tiles[t][2]) >> 16, int(tiles[t][3]) & 0xFFFF, int(tiles[t][3]) >> 16]
        assert sum(counts) == rows * cols
    q, s, o, w = oracle.unpack(lay)
    q2, s2, o2 = oracle.quantize_matrix(W, widths)
    assert np.array_equal(q, q2) and np.array_equal(s, s2) and np.array_equal(o, o2)
    assert np.array_equal(w, widths)


@given(cases())
@settings(**SETTINGS)
def test_gemv_linear_in_x(case):
    W, widths, r = case
    N, K = W.shape
    q, s, o = oracle.quantize_matrix(W, widths)
    # x with few significant bits, so that a + b and 2a are exact in fp16
    a = (r.integers(-64, 65, (1, K)) / 64.0).astype(np.float16).view(np.uint16)
    b = (r.integers(-64, 65, (1, K)) / 64.0).astype(np.float16).view(np.uint16)
    ab = (a.view(np.float16).astype(np.float64) + b.view(np.float16).astype(np.float64)).astype(np.float16)
    ya, yb = oracle.gemv(q, s, o, a), oracle.gemv(q, s, o, b)
    yab = oracle.gemv(q, s, o, ab.view(np.uint16))
    scale = np.abs(ya).max() + np.abs(yb).max() + 1e-30
    assert np.max(np.abs(yab - (ya + yb))) <= 1e-12 * scale * K


@given(cases())
@settings(**SETTINGS)
def test_in_cell_residuals_pass(case):
    W, widths, r = case
    N, K = W.shape
    q, s, o = oracle.quantize_matrix(W, widths)
    zero = np.zeros((N, K), np.uint16)
    mism, ooc, first, qp = oracle.requant_verify(q, s, o, widths, zero, want_codes=True)
    assert (mism, ooc, first) == (0, 0, 2 ** 64 - 1) and np.array_equal(qp, q)
    u = r.uniform(-0.49, 0.49, (N, K))
    resid = oracle.make_cell_residual(u, s)
    mism, ooc, first, qp = oracle.requant_verify(q, s, o, widths, resid, want_codes=True)
    assert (mism, ooc) == (0, 0) and np.array_equal(qp, q)
