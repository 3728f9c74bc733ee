"""Parity of the HIP library against the CPU oracle (needs an MI355X).

Bars: the packed layout (tile table and byte stream) and the
re-quantisation check are bit-exact; GEMV/GEMM outputs are within 2e-3
relative L2 of the fp64 oracle over each call's whole output, and every GEMV
output is within its own rounding bound of the fp64 oracle (gemv_bound).
"""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
import synth  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def vbq():
    import torch
    assert torch.cuda.is_available()
    import packed_decode_gemv_amd as m
    return m


def _t(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


U = 2.0 ** -24


def _field_bias(b):
    """For code j of a b-bit group: the power of two the kernel's decode adds
    to the code (it ORs the code's field into the mantissa of an fp16 whose
    exponent makes the field's unit 1). Pair P = j // 2 is field F = P % (16/b)
    of its word; the field sits at mantissa bit p = F*b below bit 10 (b = 1,
    2), else after a shift right by 6 (b = 1, 2) or 8 (b = 4, 8); the added
    value is 2^(10 - p)."""
    F = (np.arange(64) // 2) % (16 // b)
    if b == 1:
        p = np.where(F < 10, F, F - 6)
    elif b == 2:
        p = np.where(F < 5, 2 * F, 2 * F - 6)
    elif b == 4:
        p = np.where(F % 2 == 1, 4, 0)
    else:
        p = np.zeros(64, np.int64)
    return 2.0 ** (10 - p)


def gemv_bound(q, s16, o16, widths, x, resid=None, cell=None):
    """Worst-case rounding bound |y - y_exact| per output [B][N] of the
    library's fp32 GEMV, y = sum_g s_g (D_g - beta_g) + o_g X_g (+ residual):
      - D_g = sum (bias_k + q_k) x_k runs on the matrix cores: two chains of
        eight 4x4x4 MFMA steps, each adding four exact fp16 products to an
        fp32 accumulator (at most four roundings a step), and one add of the
        chains: within 33u of its sum of magnitudes. beta_g = sum bias_k x_k
        is four chains of eight v_dot2 steps (at most two roundings a step)
        and three adds: within 19u. With the add of the two and the final
        fma, 56 u A with A = sum_g s_g sum_k (bias_k + q_k)|x_k|;
      - X_g = sum x_k likewise: 20 u B with B = sum_g |o_g| sum_k |x_k|;
      - the record's fma and its add into the row: the row is a sum of at
        most G + 8 terms (a record per group, four wavefront slices), so
        (G + 10) u C with C = sum_k |w_k||x_k|;
      - residual rows: four chains of eight dot2 and a 64-lane sum, 26 u R with
        R = sum_k |r_k||x_k|.
      - compact in-cell residual f (int8): per group the dot D8 of the values
        1152 + f_k with x, started from -1152 X_g (X_g itself within 20 u of
        sum |x|), two chains of sixteen dot2, then times s/256 and added to
        the record's slot: within u (s/256) (40 sum (2304 + f_k)|x_k| +
        23040 sum |x_k|) per group; C then takes the full weight
        s q + o + s f / 256.
    u = 2^-24."""
    N, K = q.shape
    G = K // 64
    xd = np.abs(oracle.f64_from_f16(np.atleast_2d(x)))
    s = oracle.f64_from_f16(s16)
    o = oracle.f64_from_f16(o16)
    bias = np.stack([_field_bias(b) for b in (1, 2, 4, 8)])
    cls = {1: 0, 2: 1, 4: 2, 8: 3}
    bias_full = bias[np.vectorize(cls.get)(widths)].reshape(N, K)
    s_full = np.repeat(s, 64, axis=1)
    o_full = np.repeat(o, 64, axis=1)
    A = xd @ (s_full * (bias_full + q)).T
    Bo = xd @ np.abs(o_full).T
    w_full = s_full * q + o_full
    if cell is not None:
        fd = cell.astype(np.float64)
        s256 = s_full / 256.0
        w_full = w_full + s256 * fd
    C = xd @ np.abs(w_full).T
    b = U * (56 * A + 20 * Bo + (G + 10) * C)
    if cell is not None:
        b = b + U * (40 * (xd @ (s256 * (2304.0 + fd)).T) + 23040 * (xd @ s256.T))
    if resid is not None:
        b = b + U * 26 * (xd @ np.abs(oracle.f64_from_f16(resid)).T)
    return b


def check_gemv(y, q, s, o, widths, x, resid=None, tol=None, cell=None):
    """rel-L2 of the whole output and every output within its bound."""
    ref = oracle.gemv(q, s, o, x, resid) if cell is None else oracle.gemv_cell8(q, s, o, x, cell)
    y = np.asarray(y, np.float64)
    assert y.shape == ref.shape
    assert rel_l2(y, ref) <= (TOL if tol is None else tol)
    err = np.abs(y - ref)
    bound = gemv_bound(q, s, o, widths, x, resid, cell)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), f"output {worst}: error {err[worst]:.3e} above its bound {bound[worst]:.3e}"
    return ref


def rand_case(N, K, seed, p=(0.55, 0.2, 0.15, 0.1), B=1):
    r = np.random.default_rng(seed)
    widths = r.choice(np.array([1, 2, 4, 8], np.uint8), size=(N, K // 64), p=list(p))
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    x = r.standard_normal((B, K)).astype(np.float16).view(np.uint16)
    return W, widths, x


def layout_equal(pm, lay):
    got = pm.host_layout()
    for k in ("tiles", "stream"):
        assert got[k].shape == lay[k].shape, k
        if not np.array_equal(got[k], lay[k]):
            bad = np.flatnonzero(got[k] != lay[k])
            raise AssertionError(f"{k}: {bad.size} differences, first at {bad[:5]}")


SHAPES = [(1, 64), (15, 128), (16, 192), (17, 320), (100, 448), (768, 768), (300, 64 * 70), (40, 14336)]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{n}x{k}" for n, k in SHAPES])
def test_pack_bit_exact(vbq, shape):
    N, K = shape
    W, widths, _ = rand_case(N, K, seed=N * 7 + K)
    print(f"case pack {N}x{K}", flush=True)
    pm = vbq.vbq_pack(_t(W), widths)
    layout_equal(pm, oracle.pack(W, widths))


GEMV_CASES = [(1, 64, 1), (15, 128, 1), (17, 320, 2), (100, 448, 3), (768, 768, 1), (300, 64 * 70, 4),
              (40, 14336, 1), (64, 4096, 8), (33, 2048, 5), (48, 1024, 6), (20, 512, 7),
              (40, 8192, 8), (130, 4160, 8)]   # the largest batch with split K (the last: a 1-group k-tile)


@pytest.mark.parametrize("case", GEMV_CASES, ids=[f"{n}x{k}b{b}" for n, k, b in GEMV_CASES])
def test_gemv_parity(vbq, case):
    import torch
    N, K, B = case
    W, widths, x = rand_case(N, K, seed=N + 3 * K + B, B=B)
    print(f"case gemv {N}x{K} B={B}", flush=True)
    pm = vbq.vbq_pack(_t(W), widths)
    y = vbq.vbq_gemv(pm, _t(x, torch.float16)).cpu().numpy()
    q, s, o = oracle.quantize_matrix(W, widths)
    ref = check_gemv(y, q, s, o, widths, x)
    # also per batch row
    for b in range(B):
        assert rel_l2(y[b], ref[b]) <= TOL


@pytest.mark.parametrize("width", [1, 2, 4, 8])
def test_single_width_with_constant_groups(vbq, width):
    """Every group of one width, so that class's full and partial blocks make
    up the whole stream, and rows past a tile (N = 37); three constant groups
    have scale 0, so every weight there equals the offset (one is all zero).
    Layout bit-exact; GEMV (batch 2, and 5: a four-row pass and a one-row
    pass, each row equal to its single-row call) and GEMM within tolerance
    of the oracle."""
    import torch
    from test_gpu_gemm import check_gemm
    N, K, B = 37, 64 * 9, 2
    r = np.random.default_rng(100 + width)
    widths = np.full((N, K // 64), width, np.uint8)
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    for n, g, v in [(0, 0, 0.01), (17, 4, -0.03), (36, 8, 0.0)]:
        W[n, 64 * g:64 * (g + 1)] = v
    print(f"case single width {width}: {N}x{K} B={B}", flush=True)
    pm = vbq.vbq_pack(_t(W), widths)
    layout_equal(pm, oracle.pack(W, widths))
    q, s, o = oracle.quantize_matrix(W, widths)
    assert all(s[n, g] == 0 for n, g in [(0, 0), (17, 4), (36, 8)])
    x = r.standard_normal((B, K)).astype(np.float16).view(np.uint16)
    y = vbq.vbq_gemv(pm, _t(x, torch.float16)).cpu().numpy()
    ref = check_gemv(y, q, s, o, widths, x)
    for b in range(B):
        assert rel_l2(y[b], ref[b]) <= TOL
    # a pass of four rows (records of the one class taken per column in
    # quads) and one of a single row: within the bound, and every batch row
    # the same bits as a single-row call
    x5 = r.standard_normal((5, K)).astype(np.float16).view(np.uint16)
    y5 = vbq.vbq_gemv(pm, _t(x5, torch.float16))
    check_gemv(y5.cpu().numpy(), q, s, o, widths, x5)
    for b in range(5):
        yb = vbq.vbq_gemv(pm, _t(x5[b:b + 1], torch.float16))
        assert torch.equal(y5[b:b + 1], yb), f"width {width}: batch row {b} differs from its single-row call"
    xb = synth.x_bf16(7, (width,), 70, K)
    yg = vbq.vbq_gemm(pm, _t(xb, torch.bfloat16)).cpu().numpy()
    check_gemm(yg, q, s, o, xb)


def test_gemv_exact_integer(vbq):
    """All groups 8-bit with integer weights (0 and 255 in every group) and small
    integer x: scale 1, offset 0, every partial sum an exact integer in fp32,
    so the GPU result must equal the int64 product exactly."""
    import torch
    r = np.random.default_rng(5)
    N, K = 768, 768
    Wi = r.integers(0, 256, (N, K))
    Wi[:, 0::64] = 0
    Wi[:, 1::64] = 255
    widths = np.full((N, K // 64), 8, np.uint8)
    xi = r.integers(-2, 3, (4, K))
    pm = vbq.vbq_pack(_t(Wi.astype(np.float32)), widths)
    y = vbq.vbq_gemv(pm, _t(xi.astype(np.float16).view(np.uint16), torch.float16)).cpu().numpy()
    assert np.array_equal(y.astype(np.int64), xi @ Wi.T)
    assert np.array_equal(y, (xi @ Wi.T).astype(np.float32))


def test_gemv_deterministic_and_batched(vbq):
    import torch
    mats = []
    for i, (N, K) in enumerate([(1024, 4096), (96, 2048), (4096, 1024)]):
        W, widths, x = rand_case(N, K, seed=40 + i, B=2)
        mats.append((vbq.vbq_pack(_t(W), widths), _t(x, torch.float16)))
    singles = [vbq.vbq_gemv(pm, x) for pm, x in mats]
    again = [vbq.vbq_gemv(pm, x) for pm, x in mats]
    batched = vbq.vbq_gemv_batched([pm for pm, _ in mats], [x for _, x in mats])
    batched2 = vbq.vbq_gemv_batched([pm for pm, _ in mats], [x for _, x in mats])
    torch.cuda.synchronize()
    # Each output row is summed inside one workgroup in an order fixed by the
    # matrix alone (tile blocks in stream order, wavefront slices in order),
    # so single and batched launches agree bit for bit, and so do repeats.
    for a, b, c, d in zip(singles, again, batched, batched2):
        assert torch.equal(a, b), "GEMV not deterministic"
        assert torch.equal(c, d), "batched GEMV not deterministic"
        assert torch.equal(a, c), "batched launch differs from the single launch"


def test_split_k_calls_in_sequence(vbq):
    """Matrices with K > 4096 are summed over k-tiles by the wavefronts of
    one workgroup; calls of different shapes on one stream (different numbers
    of row-tiles and k-tiles, ragged last k-tiles) must each be right."""
    import torch
    for (N, K, B) in [(300, 4480, 4), (2048, 8192, 1), (40, 14336, 1), (700, 64 * 70, 2), (2048, 8192, 1)]:
        W, widths, x = rand_case(N, K, seed=N + K + B, B=B)
        print(f"case split-k {N}x{K} B={B}", flush=True)
        pm = vbq.vbq_pack(_t(W), widths)
        q, s, o = oracle.quantize_matrix(W, widths)
        y = vbq.vbq_gemv(pm, _t(x, torch.float16)).cpu().numpy()
        check_gemv(y, q, s, o, widths, x)


def test_split_k_repeatable_across_streams(vbq):
    """Split-K sums stay inside a workgroup, so calls on several streams at
    once share nothing and repeat bit for bit."""
    import torch
    cases = []
    for (N, K, B) in [(4096, 14336, 1), (1000, 8192, 2)]:
        W, widths, x = rand_case(N, K, seed=5 * N + K, B=B)
        pm = vbq.vbq_pack(_t(W), widths)
        q, s, o = oracle.quantize_matrix(W, widths)
        cases.append((pm, _t(x, torch.float16), oracle.gemv(q, s, o, x)))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = {0: [], 1: []}
    for rep in range(6):
        for ci, (pm, xt, _) in enumerate(cases):
            st = s1 if (rep + ci) % 2 else s2
            with torch.cuda.stream(st):
                outs[ci].append(vbq.vbq_gemv(pm, xt, stream=st))
    torch.cuda.synchronize()
    for ci, (_, _, ref) in enumerate(cases):
        first = outs[ci][0]
        assert rel_l2(first.cpu().numpy(), ref) <= TOL
        for o in outs[ci][1:]:
            assert torch.equal(o, first), "split-K GEMV differs between calls"


@pytest.mark.parametrize("B", [1, 4])
def test_split_k_batched_mix(vbq, B):
    """A batched launch mixing split (K > 4096) and unsplit matrices."""
    import torch
    mats, refs = [], []
    for i, (N, K) in enumerate([(4096, 14336), (512, 4096), (1024, 8192), (64, 4160)]):
        W, widths, x = rand_case(N, K, seed=90 + i, B=B)
        q, s, o = oracle.quantize_matrix(W, widths)
        mats.append((vbq.vbq_pack(_t(W), widths), _t(x, torch.float16)))
        refs.append(oracle.gemv(q, s, o, x))
    for _ in range(2):
        ys = vbq.vbq_gemv_batched([pm for pm, _ in mats], [x for _, x in mats])
        for y, ref in zip(ys, refs):
            assert rel_l2(y.cpu().numpy(), ref) <= TOL
    for (pm, x), y in zip(mats, ys):
        assert torch.equal(y, vbq.vbq_gemv(pm, x))


def test_batched_full_launch_of_mixed_shapes(vbq):
    """32 matrices in one call (the most a launch takes) of mixed shapes,
    some with K > 4096 and ragged k-tiles: every output matches the oracle;
    a 33rd matrix is refused before anything is launched."""
    import torch
    r = np.random.default_rng(77)
    mats, refs = [], []
    for i in range(32):
        N = int(r.choice([16, 40, 96, 256, 513]))
        K = int(r.choice([64, 1024, 4096, 4160, 8192]))
        W, widths, x = rand_case(N, K, seed=300 + i, B=1)
        q, s, o = oracle.quantize_matrix(W, widths)
        mats.append((vbq.vbq_pack(_t(W), widths), _t(x, torch.float16)))
        refs.append((q, s, o, widths, x))
    print("case batched 32 matrices", flush=True)
    ys = vbq.vbq_gemv_batched([pm for pm, _ in mats], [x for _, x in mats])
    for y, (q, s, o, widths, x) in zip(ys, refs):
        check_gemv(y.cpu().numpy(), q, s, o, widths, x)
    with pytest.raises(ValueError):
        vbq.vbq_gemv_batched([pm for pm, _ in mats] + [mats[0][0]], [x for _, x in mats] + [mats[0][1]])


# 32800 rows of one k-group: 1025 row-tiles, more workgroups than an MI355X
# holds at once (four per CU).
FILLER = (32800, 64)


@pytest.mark.parametrize("B", [1, 2])
def test_large_launch_with_small_matrices(vbq, B):
    """A launch with more workgroups than the device holds at once, carrying
    small matrices (ragged row-tiles, shared and split k-tiles) beside a
    filler of 1025 row-tiles: each small matrix's output is the same bits as
    in a launch of its own, in the batched and the allocation-free launches;
    every output is within its bound of the oracle; two levels of the
    filler's shape summed in one launch equal the sum of their GEMVs."""
    import torch
    cases = [(200, 4160), (33, 64), (100, 448), (300, 8192 + 192), (64, 4096), (95, 12288)]
    mats, refs = [], []
    for i, (N, K) in enumerate(cases):
        W, widths, x = rand_case(N, K, seed=500 + i, B=B)
        q, s, o = oracle.quantize_matrix(W, widths)
        mats.append((vbq.vbq_pack(_t(W), widths), _t(x, torch.float16)))
        refs.append((q, s, o, widths, x))
    Wf, wf, xf = rand_case(*FILLER, seed=599, B=B)
    qf, sf, of = oracle.quantize_matrix(Wf, wf)
    fill = (vbq.vbq_pack(_t(Wf), wf), _t(xf, torch.float16))
    pms, xs = [pm for pm, _ in mats], [x for _, x in mats]
    print(f"case large launch B={B}", flush=True)
    alone = [vbq.vbq_gemv(pm, x) for pm, x in mats]
    alone_static = vbq.vbq_gemv_batched(pms, xs, static=True)
    big = vbq.vbq_gemv_batched([fill[0]] + pms, [fill[1]] + xs)
    big_static = vbq.vbq_gemv_batched([fill[0]] + pms, [fill[1]] + xs, static=True)
    torch.cuda.synchronize()
    for i, (N, K) in enumerate(cases):
        assert torch.equal(alone[i], big[i + 1]), f"{N}x{K}: differs beside the filler"
        assert torch.equal(alone[i], alone_static[i]), f"{N}x{K}: split launch differs"
        assert torch.equal(alone[i], big_static[i + 1]), f"{N}x{K}: split launch beside the filler differs"
        check_gemv(big[i + 1].cpu().numpy(), *refs[i])
    check_gemv(big[0].cpu().numpy(), qf, sf, of, wf, xf)
    assert torch.equal(big[0], big_static[0])
    # two levels of the filler's shape, summed in one launch
    W2, w2, _ = rand_case(*FILLER, seed=598, B=B)
    lv2 = vbq.vbq_pack(_t(W2), w2)
    y_lv = vbq.vbq_gemv_levels([fill[0], lv2], fill[1])
    y_sum = vbq.vbq_gemv(fill[0], fill[1]) + vbq.vbq_gemv(lv2, fill[1])
    assert torch.equal(y_lv, y_sum), "levels in one launch differ from the sum of their GEMVs"


def test_graph_replays_match_eager(vbq):
    """Launches captured in a HIP graph (as the benchmark replays a decode
    step) give the eager results on every replay, with other eager work and
    synchronisations in between; the library allocates nothing, so the
    capture needs no eager call before it."""
    import torch
    mats = []
    for i, (N, K) in enumerate([(4096, 14336), (1024, 4096), (2048, 8192)]):
        W, widths, x = rand_case(N, K, seed=200 + i, B=1)
        mats.append((vbq.vbq_pack(_t(W), widths), _t(x, torch.float16)))
    pms, xs = [pm for pm, _ in mats], [x for _, x in mats]
    ys = [torch.empty(1, pm.N, dtype=torch.float32, device="cuda") for pm in pms]
    plan = vbq.GemvPlan(pms, xs, ys)
    plan.launch(vbq._stream())
    torch.cuda.synchronize()
    ref = [y.clone() for y in ys]
    other_W, other_w, other_x = rand_case(300, 4480, seed=210, B=2)
    other = vbq.vbq_pack(_t(other_W), other_w)
    ox = _t(other_x, torch.float16)
    side = torch.cuda.Stream()   # captured with no eager call on it before: nothing to set up
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        plan.launch(vbq._stream())
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for y, r in zip(ys, ref):
            assert torch.equal(y, r), f"replay {rep} differs from the eager launch"
        vbq.vbq_gemv(other, ox)   # eager work with split-K between replays
        torch.cuda.synchronize()


def test_gemv_batch_rows_match_single_rows(vbq):
    import torch
    W, widths, x = rand_case(512, 4096, seed=77, B=4)
    pm = vbq.vbq_pack(_t(W), widths)
    xt = _t(x, torch.float16)
    y4 = vbq.vbq_gemv(pm, xt)
    for b in range(4):
        # every batch row is decoded and summed exactly as a batch-1 call does
        y1 = vbq.vbq_gemv(pm, xt[b:b + 1].contiguous())
        assert torch.equal(y1[0], y4[b]), f"batch row {b} differs from its batch-1 call"


def _cell_inputs(N, K, seed, u_scale=1.0):
    r = np.random.default_rng(seed)
    widths = np.full((N, K // 64), 4, np.uint8)
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    q, s, o = oracle.quantize_matrix(W, widths)
    u = r.uniform(-0.49, 0.49, (N, K)) * u_scale
    resid = oracle.make_cell_residual(u, s)
    x = r.standard_normal((1, K)).astype(np.float16).view(np.uint16)
    return W, widths, q, s, o, resid, x


@pytest.mark.parametrize("shape", [(16, 256), (50, 1024), (33, 4096), (20, 8192), (37, 8192 + 192)])
def test_residual_gemv_and_revocation(vbq, shape):
    import torch
    N, K = shape
    W, widths, q, s, o, resid, x = _cell_inputs(N, K, seed=N + K)
    pm = vbq.vbq_pack(_t(W), widths)
    xt = _t(x, torch.float16)
    rt = _t(resid, torch.float16)
    y = vbq.vbq_gemv(pm, xt, residual=rt).cpu().numpy()
    check_gemv(y, q, s, o, widths, x, resid)
    y0 = vbq.vbq_gemv(pm, xt).cpu().numpy()
    check_gemv(y0, q, s, o, widths, x)
    # a zero residual serves the base weights
    yz = vbq.vbq_gemv(pm, xt, residual=torch.zeros_like(rt)).cpu().numpy()
    assert np.allclose(yz, y0, rtol=1e-6, atol=1e-6)


CELL_SHAPES = [(1, 64), (17, 320), (33, 4096), (70, 64 * 70), (20, 8192 + 192)]


@pytest.mark.parametrize("shape", CELL_SHAPES, ids=[f"{n}x{k}" for n, k in CELL_SHAPES])
def test_cell8_encode_decode_bit_exact(vbq, shape):
    """Compact in-cell residual: the device encoder and decoder against the
    oracle's, bit for bit, with the scales the packed matrix holds (mixed
    widths, a zero-scale group, residuals inside, at the edge of and beyond
    the representable range, ties of the rounding)."""
    import torch
    N, K = shape
    W, widths, _ = rand_case(N, K, seed=3 * N + K)
    if N > 2:
        W[N // 2, :64] = 0.015                  # constant group: scale 0
    if N > 1:
        # row 1: every group spans (2^b - 1) / 16, so its scale is 1/16
        for g in range(K // 64):
            L = (1 << int(widths[1, g])) - 1
            W[1, 64 * g:64 * g + 64] = np.where(np.arange(64) % 2 == 0, 0.0, L / 16.0)
    print(f"case cell8 encode/decode {N}x{K}", flush=True)
    pm = vbq.vbq_pack(_t(W), widths)
    q, s, o = oracle.quantize_matrix(W, widths)
    r = np.random.default_rng(N + 5 * K)
    sd = np.repeat(oracle.f64_from_f16(s), 64, axis=1)
    r16 = oracle.f16_from_f64(r.uniform(-0.8, 0.8, (N, K)) * sd)
    r16[::2] = oracle.f16_from_f64(r.standard_normal((N, K)) * 0.01)[::2]
    if N > 1:
        # half steps of the fraction at an exact scale: r / s * 256 is a tie
        assert (s[1] == 0x2C00).all()
        t = r.integers(-100, 100, K) + 0.5
        r16[1] = oracle.f16_from_f64(t / 256.0 / 16.0)
        assert np.array_equal(oracle.f64_from_f16(r16[1]), t / 4096.0)
    f_gpu = vbq.cell8_encode(pm, _t(r16, torch.float16)).cpu().numpy()
    f_ref = oracle.cell8_encode(r16, s)
    if not np.array_equal(f_gpu, f_ref):
        bad = np.argwhere(f_gpu != f_ref)
        raise AssertionError(f"{len(bad)} fractions differ, first at {bad[:3].tolist()}")
    fr = r.integers(-127, 128, (N, K)).astype(np.int8)
    fr[0, :64] = -127
    d_gpu = vbq.cell8_decode(pm, _t(fr)).cpu().numpy().view(np.uint16)
    assert np.array_equal(d_gpu, oracle.cell8_decode(fr, s))


def test_cell_update_revoke_and_reapply(vbq):
    """CellUpdate: applied, the GEMV is vbq_gemv_cell8's; revoked, it is the
    release's vbq_gemv bit for bit; applied again, the first result bit for
    bit. The packed matrix is byte-identical throughout, and the update's
    decoded residual passes the re-quantisation check."""
    import torch
    N, K = 70, 64 * 70
    W, widths, x = rand_case(N, K, seed=17, B=2)
    pm = vbq.vbq_pack(_t(W), widths)
    stream0 = pm.stream.clone()
    q, s, o = oracle.quantize_matrix(W, widths)
    resid = oracle.make_cell_residual(np.random.default_rng(18).uniform(-0.45, 0.45, (N, K)), s)
    upd = vbq.CellUpdate.from_residual(pm, _t(resid, torch.float16))
    assert np.array_equal(upd.cell.cpu().numpy(), oracle.cell8_encode(resid, s))
    xt = _t(x, torch.float16)
    y_on = upd.gemv(xt)
    assert torch.equal(y_on, vbq.vbq_gemv_cell8(pm, xt, upd.cell))
    upd.revoke()
    y_off = upd.gemv(xt)
    assert torch.equal(y_off, vbq.vbq_gemv(pm, xt))
    upd.apply()
    assert torch.equal(upd.gemv(xt), y_on)
    assert torch.equal(pm.stream, stream0)
    mism, ooc, first, _ = upd.verify()
    assert (mism, ooc, first) == (0, 0, 2 ** 64 - 1)
    check_gemv(y_on.cpu().numpy(), q, s, o, widths, x, cell=upd.cell.cpu().numpy())


CELL_GEMV = [(1, 64, 1), (17, 320, 2), (33, 4096, 1), (100, 448, 3), (70, 64 * 70, 1), (20, 8192 + 192, 4),
             (64, 256, 8)]


@pytest.mark.parametrize("case", CELL_GEMV, ids=[f"{n}x{k}b{b}" for n, k, b in CELL_GEMV])
def test_cell8_gemv_parity(vbq, case):
    """GEMV with the compact in-cell residual against the oracle (every
    output within its bound), repeatable bit for bit, each batch row equal to
    its batch-1 call; the update moves no output further than the drift
    bound, and the base GEMV (the update revoked) is untouched."""
    import torch
    N, K, B = case
    W, widths, x = rand_case(N, K, seed=11 * N + K + B, B=B)
    if N > 2:
        W[N // 2, 64:128 if K > 64 else 64] = -0.01
    print(f"case cell8 gemv {N}x{K} B={B}", flush=True)
    pm = vbq.vbq_pack(_t(W), widths)
    q, s, o = oracle.quantize_matrix(W, widths)
    r = np.random.default_rng(N * K + B)
    f = r.integers(-127, 128, (N, K)).astype(np.int8)
    f[0] = 127
    if N > 1:
        f[1] = -127
    xt = _t(x, torch.float16)
    ft = _t(f)
    y0 = vbq.vbq_gemv(pm, xt)
    yt = vbq.vbq_gemv_cell8(pm, xt, ft)
    y = yt.cpu().numpy()
    check_gemv(y, q, s, o, widths, x, cell=f)
    assert torch.equal(vbq.vbq_gemv_cell8(pm, xt, ft), yt)
    for b in range(B):
        assert torch.equal(vbq.vbq_gemv_cell8(pm, xt[b:b + 1].contiguous(), ft)[0], yt[b])
    bound = vbq.cell_drift_bound(pm, xt).cpu().numpy()
    s_full = oracle.f64_from_f16(np.repeat(s, 64, axis=1))
    xd = oracle.f64_from_f16(x)
    wdq = s_full * q + oracle.f64_from_f16(np.repeat(o, 64, axis=1))
    slack = 1e-5 * (np.abs(xd) @ (np.abs(wdq) + s_full).T)
    base = y0.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(y - base) <= bound + slack)
    assert torch.equal(vbq.vbq_gemv(pm, xt), y0)


def _verify_both(vbq, pm, resid_t):
    """cell_requant_verify with and without the re-quantised stream: the
    counts and first index must agree; returns the first call's result."""
    got = vbq.cell_requant_verify(pm, resid_t, requant_codes=True)
    bare = vbq.cell_requant_verify(pm, resid_t)
    assert bare[:3] == got[:3] and bare[3] is None
    return got


DRIFT_CASES = [(37, 576, 1), (64, 8192 + 128, 3), (20, 4096, 8), (1, 64, 2)]


@pytest.mark.parametrize("case", DRIFT_CASES, ids=[f"{n}x{k}b{b}" for n, k, b in DRIFT_CASES])
def test_drift_bound(vbq, case):
    """cell_drift_bound against the oracle's closed form, repeatable bit for
    bit, and a true bound on the library's own residual GEMV: in-cell
    residuals stay inside it and the extremal residual sign(x) s/2 reaches it
    (up to the rounding of two binary32 GEMVs)."""
    import torch
    N, K, B = case
    W, widths, x = rand_case(N, K, seed=7 * N + K + B, B=B)
    print(f"case drift bound {N}x{K} B={B}", flush=True)
    pm = vbq.vbq_pack(_t(W), widths)
    q, s, o = oracle.quantize_matrix(W, widths)
    xt = _t(x, torch.float16)
    got = vbq.cell_drift_bound(pm, xt).cpu().numpy()
    ref = oracle.drift_bound(s, x)
    assert got.shape == ref.shape == (B, N)
    assert np.all(np.abs(got - ref) <= 5e-5 * ref)
    assert np.array_equal(vbq.cell_drift_bound(pm, xt).cpu().numpy(), got)
    s_full = oracle.f64_from_f16(np.repeat(s, 64, axis=1))
    xd = oracle.f64_from_f16(x)
    wdq = s_full * q + oracle.f64_from_f16(np.repeat(o, 64, axis=1))
    slack = 1e-5 * (np.abs(xd) @ (np.abs(wdq) + s_full).T)      # rounding of the two GEMVs
    y0 = vbq.vbq_gemv(pm, xt).cpu().numpy()
    resid = oracle.make_cell_residual(np.random.default_rng(N + B).uniform(-0.49, 0.49, (N, K)), s)
    yr = vbq.vbq_gemv(pm, xt, residual=_t(resid, torch.float16)).cpu().numpy()
    assert np.all(np.abs(yr.astype(np.float64) - y0) <= got + slack)
    for b in range(B):
        half = s_full / 2 * np.sign(xd[b])[None, :]
        r16 = oracle.f16_from_f64(half)
        assert np.array_equal(oracle.f64_from_f16(r16), half)
        xb = xt[b:b + 1].contiguous()
        ye = vbq.vbq_gemv(pm, xb, residual=_t(r16, torch.float16)).cpu().numpy()[0]
        yb = vbq.vbq_gemv(pm, xb).cpu().numpy()[0]
        assert np.all(np.abs((ye.astype(np.float64) - yb) - got[b]) <= 1e-5 * got[b] + slack[b])


@pytest.mark.parametrize("shape", [(37, 576), (64, 8192 + 128)], ids=["37x576", "64x8320"])
def test_rrq_levels_bit_exact_and_gemv(vbq, shape):
    """Recurrent residual levels: each level's layout is bit-exact against the
    oracle's pack of the error the levels before it leave, and that error is
    bit-exact against the oracle's binary32 recursion; rrq_pack gives the same
    levels; the GEMV over the first 1..4 levels (2 to 8 effective bits)
    matches the oracle at batch 1 and 4."""
    import torch
    N, K = shape
    r = np.random.default_rng(N + K)
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    w2 = np.full((N, K // 64), 2, np.uint8)
    print(f"case rrq {N}x{K}", flush=True)
    E = _t(W)
    pms = []
    for i in range(4):
        E_ref_in = oracle.rrq_levels(W, i)[1]
        pm = vbq.vbq_pack(E, w2)
        layout_equal(pm, oracle.pack(E_ref_in, w2))
        E = vbq.vbq_residual_error(pm, E)
        assert np.array_equal(E.cpu().numpy(), oracle.rrq_levels(W, i + 1)[1]), f"level {i}"
        pms.append(pm)
    for a, b in zip(vbq.rrq_pack(_t(W), 4), pms):
        layout_equal(a, b.host_layout())
    levels, _ = oracle.rrq_levels(W, 4)
    for B in (1, 4):
        x = r.standard_normal((B, K)).astype(np.float16).view(np.uint16)
        for k in range(4):
            y = vbq.vbq_gemv_levels(pms[:k + 1], _t(x, torch.float16)).cpu().numpy()
            ref = oracle.rrq_gemv(levels[:k + 1], x)
            assert rel_l2(y, ref) <= TOL, (B, k)
            bound = sum(gemv_bound(lq, ls, lo, w2, x) for lq, ls, lo in levels[:k + 1])
            assert np.all(np.abs(y - ref) <= bound), (B, k)


@pytest.mark.parametrize("n_levels", [2, 3])
def test_levels_one_row_equals_batch_rows(vbq, n_levels):
    """At one batch row the GEMV over levels takes a row-tile's tiles two at a
    time; with more rows it walks them one at a time. Both add the tiles' row
    sums in the same order, so every batch row of a multi-row call equals the
    one-row call on that row bit for bit (odd and even tile counts, three
    k-tiles per level, ragged rows)."""
    import torch
    N, K = 70, 8192 + 192
    r = np.random.default_rng(71 + n_levels)
    pms = []
    for i in range(n_levels):
        W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
        widths = r.choice(np.array([1, 2, 4, 8], np.uint8), size=(N, K // 64))
        pms.append(vbq.vbq_pack(_t(W), widths))
    x = _t(r.standard_normal((3, K)).astype(np.float16).view(np.uint16), torch.float16)
    print(f"case levels one row vs batch, {n_levels} levels", flush=True)
    yb = vbq.vbq_gemv_levels(pms, x)
    for b in range(3):
        y1 = vbq.vbq_gemv_levels(pms, x[b:b + 1].contiguous())
        assert torch.equal(y1[0], yb[b]), f"batch row {b}"
    y_sum = sum(vbq.vbq_gemv(pm, x[0:1].contiguous()) for pm in pms)
    assert torch.allclose(vbq.vbq_gemv_levels(pms, x[0:1].contiguous()), y_sum, rtol=1e-5, atol=1e-5)


def test_residual_error_any_width(vbq):
    """vbq_residual_error on a mixed-width matrix is E - (f32(s q) + o) bit
    for bit, in place too."""
    N, K = 40, 640
    W, widths, _ = rand_case(N, K, seed=5)
    pm = vbq.vbq_pack(_t(W), widths)
    q, s, o = oracle.quantize_matrix(W, widths)
    sf = oracle.f64_from_f16(np.repeat(s, 64, axis=1)).astype(np.float32)
    of = oracle.f64_from_f16(np.repeat(o, 64, axis=1)).astype(np.float32)
    ref = (W - ((sf * q.astype(np.float32)) + of)).astype(np.float32)
    E = _t(W)
    assert np.array_equal(vbq.vbq_residual_error(pm, E).cpu().numpy(), ref)
    vbq.vbq_residual_error(pm, E, out=E)
    assert np.array_equal(E.cpu().numpy(), ref)


def test_requant_verify_small(vbq):
    import torch
    N, K = 40, 1024
    W, widths, q, s, o, resid, _ = _cell_inputs(N, K, seed=9)
    pm = vbq.vbq_pack(_t(W), widths)
    mism, ooc, first, rq = _verify_both(vbq, pm, _t(resid, torch.float16))
    assert (mism, ooc, first) == (0, 0, 2 ** 64 - 1)
    assert torch.equal(rq, pm.stream), "re-quantised artifact differs from the release"
    # planted: exactly half a cell at three places, 0.6 of a cell at two interior codes
    bad = resid.copy()
    sf = oracle.f64_from_f16(np.repeat(s, 64, axis=1))
    for (n, k) in [(3, 5), (17, 600), (39, 1023)]:
        bad[n, k] = oracle.f16_from_f64(np.array([0.5 * sf[n, k]]))[0]
    interior = np.argwhere((q > 0) & (q < 15))
    for n, k in interior[[10, 2000]]:
        bad[n, k] = oracle.f16_from_f64(np.array([0.6 * sf[n, k]]))[0]
    ref = oracle.requant_verify(q, s, o, widths, bad, want_codes=True)
    mism, ooc, first, rq = _verify_both(vbq, pm, _t(bad, torch.float16))
    assert (mism, ooc, first) == ref[:3]
    # half a cell can round the code across (ties to even), so >= 2 mismatches
    assert ref[0] >= 2 and ref[1] == 5
    # the emitted codes are the oracle's re-quantised codes, packed in the same layout
    lay_rq = pm.host_layout()
    lay_rq["stream"] = rq.cpu().numpy().view(np.uint32)
    q_rq, _, _, _ = oracle.unpack(lay_rq)
    assert np.array_equal(q_rq, ref[3])


def test_requant_verify_near_half_cells(vbq):
    """Residuals within a hair of half a cell on every weight, all widths: the
    re-quantised code is decided right at a half-integer quotient, where the
    binary32 rounding of the division matters; counts, first index and the
    re-quantised codes must still equal the oracle's."""
    import torch
    r = np.random.default_rng(44)
    N, K = 48, 1024
    widths = r.choice(np.array([1, 2, 4, 8], np.uint8), size=(N, K // 64))
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    q, s, o = oracle.quantize_matrix(W, widths)
    hair = r.choice(np.array([0.0, 2.0 ** -14, 2.0 ** -12, 2.0 ** -10, 2.0 ** -8]), size=(N, K))
    u = np.where(r.random((N, K)) < 0.5, -1.0, 1.0) * (0.5 + np.where(r.random((N, K)) < 0.5, -hair, hair))
    resid = oracle.make_cell_residual(u, s)
    pm = vbq.vbq_pack(_t(W), widths)
    ref = oracle.requant_verify(q, s, o, widths, resid, want_codes=True)
    mism, ooc, first, rq = _verify_both(vbq, pm, _t(resid, torch.float16))
    assert (mism, ooc, first) == ref[:3]
    assert ref[0] > 0 and ref[1] > 0
    lay_rq = pm.host_layout()
    lay_rq["stream"] = rq.cpu().numpy().view(np.uint32)
    q_rq, _, _, _ = oracle.unpack(lay_rq)
    assert np.array_equal(q_rq, ref[3])


def test_requant_verify_calls_independent(vbq):
    """Each call reports only its own counts: a failing check, then a clean
    one, then the failing one again on the same stream, in both modes."""
    import torch
    N, K = 48, 2048
    W, widths, q, s, o, resid, _ = _cell_inputs(N, K, seed=21)
    pm = vbq.vbq_pack(_t(W), widths)
    bad = resid.copy()
    sf = oracle.f64_from_f16(np.repeat(s, 64, axis=1))
    for (n, k) in [(0, 0), (20, 1500), (47, 2047)]:
        bad[n, k] = oracle.f16_from_f64(np.array([0.7 * sf[n, k]]))[0]
    ref_bad = oracle.requant_verify(q, s, o, widths, bad)[:3]
    assert ref_bad[1] == 3
    for _ in range(2):
        assert _verify_both(vbq, pm, _t(bad, torch.float16))[:3] == ref_bad
        assert _verify_both(vbq, pm, _t(resid, torch.float16))[:3] == (0, 0, 2 ** 64 - 1)
    torch.cuda.synchronize()


def test_requant_verify_flipped_bit(vbq):
    """A served artifact with one code bit flipped: the check re-quantises
    against the artifact it is given, so it passes, and the re-quantised
    stream it emits is that artifact bit for bit, so comparing it with the
    release finds exactly the flipped word."""
    import torch
    N, K = 40, 1024
    W, widths, q, s, o, resid, _ = _cell_inputs(N, K, seed=13)
    release = vbq.vbq_pack(_t(W), widths)
    served = release.clone()
    w0 = 8 * (K // 64) // 4                   # the first tile's map takes 8 bytes per column
    served.stream[w0:w0 + 1].bitwise_xor_(1)  # lowest code bit of the first record of the stream
    mism, ooc, first, rq = _verify_both(vbq, served, _t(resid, torch.float16))
    assert (mism, ooc, first) == (0, 0, 2 ** 64 - 1)
    assert torch.equal(rq, served.stream)
    diff = torch.nonzero(rq != release.stream).flatten().tolist()
    assert diff == [w0]


def test_requant_verify_in_cell_near_half(vbq):
    """Residuals inside their cells but within 2^-11 .. 2^-8 of half a cell
    most quarters keep every code and take the kernel's estimated-quotient
    path, whose rounding decisions sit right next to the half-integers; the
    counts, first index and re-quantised codes must equal the oracle's."""
    import torch
    r = np.random.default_rng(45)
    N, K = 64, 2048
    widths = r.choice(np.array([1, 2, 4, 8], np.uint8), size=(N, K // 64))
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[5, 64:128] = 0.01          # constant groups: scale 0, residual must be 0 (exact path)
    W[40, 1024:1088] = -0.02
    q, s, o = oracle.quantize_matrix(W, widths)
    assert s[5, 1] == 0 and s[40, 16] == 0
    hair = r.choice(np.array([2.0 ** -11, 2.0 ** -10, 2.0 ** -9, 2.0 ** -8]), size=(N, K))
    u = np.where(r.random((N, K)) < 0.5, -1.0, 1.0) * (0.5 - hair)
    resid = oracle.make_cell_residual(u, s)
    pm = vbq.vbq_pack(_t(W), widths)
    ref = oracle.requant_verify(q, s, o, widths, resid, want_codes=True)
    mism, ooc, first, rq = _verify_both(vbq, pm, _t(resid, torch.float16))
    assert (mism, ooc, first) == ref[:3]
    lay_rq = pm.host_layout()
    lay_rq["stream"] = rq.cpu().numpy().view(np.uint32)
    q_rq, _, _, _ = oracle.unpack(lay_rq)
    assert np.array_equal(q_rq, ref[3])


def test_requant_verify_large_offsets(vbq):
    """Groups whose offset is large against their scale (rows centred at 0,
    1, 30 and 1000), so the binary32 roundings of f32(s q) + o + r - o are a
    sizeable fraction of a cell and the kernel's record-level bound on |r|
    (under which every code provably comes back) is far below s / 2: residuals
    spread over the whole cell, at every width, must still give the oracle's
    counts, first index and re-quantised codes."""
    import torch
    r = np.random.default_rng(46)
    N, K = 64, 2048
    widths = r.choice(np.array([1, 2, 4, 8], np.uint8), size=(N, K // 64))
    centre = np.array([0.0, 1.0, 30.0, 1000.0], np.float32)[np.arange(N) % 4][:, None]
    W = (centre + r.standard_normal((N, K)) * 0.02).astype(np.float32)
    q, s, o = oracle.quantize_matrix(W, widths)
    u = r.uniform(-0.5, 0.5, (N, K))
    near = r.random((N, K)) < 0.25
    u[near] = np.sign(u[near]) * (0.5 - r.choice(np.array([2.0 ** -16, 2.0 ** -12, 2.0 ** -8, 2.0 ** -4]),
                                                 size=int(near.sum())))
    resid = oracle.make_cell_residual(u, s)
    pm = vbq.vbq_pack(_t(W), widths)
    got = _verify_both(vbq, pm, _t(resid, torch.float16))
    ref = oracle.requant_verify(q, s, o, widths, resid, want_codes=True)
    assert got[:3] == ref[:3]
    assert ref[0] > 0
    lay = pm.host_layout()
    lay["stream"] = got[3].cpu().numpy().view(np.uint32)
    assert np.array_equal(oracle.unpack(lay)[0], ref[3])


def test_requant_verify_several_k_tiles(vbq):
    """Three k-tiles with a ragged last one (3 of 64 groups) and a ragged last
    row-tile, mixed widths, residuals spread over the whole cell with some
    outside it: counts, first index and re-quantised codes equal the
    oracle's in both modes (the row-order kernel and the one that writes the
    stream)."""
    import torch
    r = np.random.default_rng(47)
    N, K = 45, 8192 + 192
    widths = r.choice(np.array([1, 2, 4, 8], np.uint8), size=(N, K // 64))
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    q, s, o = oracle.quantize_matrix(W, widths)
    u = r.uniform(-0.5, 0.5, (N, K))
    out = r.random((N, K)) < 0.001
    u[out] = 0.8 * np.sign(u[out])
    resid = oracle.make_cell_residual(u, s)
    pm = vbq.vbq_pack(_t(W), widths)
    got = _verify_both(vbq, pm, _t(resid, torch.float16))
    ref = oracle.requant_verify(q, s, o, widths, resid, want_codes=True)
    assert got[:3] == ref[:3]
    assert ref[1] > 0
    lay = pm.host_layout()
    lay["stream"] = got[3].cpu().numpy().view(np.uint32)
    assert np.array_equal(oracle.unpack(lay)[0], ref[3])


def test_requant_verify_mixed_widths(vbq):
    import torch
    N, K = 48, 2048
    r = np.random.default_rng(21)
    widths = r.choice(np.array([1, 2, 4, 8], np.uint8), size=(N, K // 64))
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    q, s, o = oracle.quantize_matrix(W, widths)
    u = r.uniform(-0.7, 0.7, (N, K))              # some residuals leave their cells
    resid = oracle.make_cell_residual(u, s)
    pm = vbq.vbq_pack(_t(W), widths)
    got = _verify_both(vbq, pm, _t(resid, torch.float16))
    ref = oracle.requant_verify(q, s, o, widths, resid, want_codes=True)
    assert got[:3] == ref[:3]
    assert ref[0] > 0 and ref[1] > 0
    lay = pm.host_layout()
    lay["stream"] = got[3].cpu().numpy().view(np.uint32)
    assert np.array_equal(oracle.unpack(lay)[0], ref[3])


def test_invalid_widths_on_device_are_reported(vbq):
    import ctypes as C

    import torch
    N, K = 32, 256
    W, widths, _ = rand_case(N, K, seed=3)
    sizes = vbq.pack_query(widths)
    pm = vbq.PackedMatrix(N, K, sizes)
    bad = widths.copy()
    bad[5, 2] = 3
    st = vbq.lib.vbq_pack(C.c_void_p(_t(W).data_ptr()), C.c_void_p(_t(bad).data_ptr()), C.byref(pm.desc),
                          vbq._stream())
    assert st == 0
    torch.cuda.synchronize()
    assert vbq.lib.vbq_matrix_check(C.byref(pm.desc), vbq._stream()) == 3


# ---------------------------------------------------------------------------
# Full-size workloads (sampled rows where the oracle would be slow)
# ---------------------------------------------------------------------------
def _sample_rows(N, r, n=96):
    rows = set(r.choice(N, min(N, n), replace=False).tolist())
    rows.update([0, N - 1, (N // 32) * 32 - 1 if N >= 32 else 0, min(N - 1, 32)])
    return np.array(sorted(rows), np.int64)


def _check_proj(vbq, cid, layer, pi, proj, B, full=False, recipe=False):
    import torch
    key = synth.proj_key(cid, layer, pi)
    G = proj.k // 64
    if recipe:
        widths = synth.recipe_widths(layer, pi, proj, synth.C3.layers)
    else:
        widths = synth.widths(synth.SEED, key, proj.n, G, proj.mix)
    W = synth.weights(synth.SEED, key, proj.n, proj.k)
    x = synth.x_f16(synth.SEED, key, B, proj.k)
    print(f"case workload {cid} layer {layer} {proj.name} {proj.n}x{proj.k} B={B}", flush=True)
    pm = vbq.vbq_pack(_t(W), widths)
    y = vbq.vbq_gemv(pm, _t(x, torch.float16)).cpu().numpy()
    rows = np.arange(proj.n) if full else _sample_rows(proj.n, np.random.default_rng(pi + 100 * (layer + 1)))
    q, s, o = oracle.quantize_matrix(W[rows], widths[rows])
    check_gemv(y[:, rows], q, s, o, widths[rows], x)
    # the GPU layout of those rows reads back to the oracle's codes and scales
    qg, sg, og, wg = oracle.unpack(pm.host_layout(), rows)
    assert np.array_equal(qg, q) and np.array_equal(sg, s) and np.array_equal(og, o)
    assert np.array_equal(wg, widths[rows])
    return pm


@pytest.mark.parametrize("B", [1, 4])
def test_workload_1b_layer_full(vbq, B):
    for pi, proj in enumerate(synth.C1.projs):
        _check_proj(vbq, 1, 0, pi, proj, B, full=True)


def test_workload_131m_projection_full(vbq):
    _check_proj(vbq, 0, 0, 0, synth.C0.projs[0], 1, full=True)


@pytest.mark.parametrize("pi", range(7))
def test_workload_9b_layer_sampled(vbq, pi):
    _check_proj(vbq, 3, 0, pi, synth.C3.projs[pi], 1)


def test_workload_9b_lm_head_sampled(vbq):
    _check_proj(vbq, 3, -1, 0, synth.C3.head, 1)


def test_workload_9b_layer_batch4_sampled(vbq):
    for pi in (0, 4, 6):
        _check_proj(vbq, 3, 5, pi, synth.C3.projs[pi], 4)


RECIPE_CASES = [(0, 0), (0, 4), (0, 6), (1, 2), (15, 5), (31, 6), (-1, 0)]


@pytest.mark.parametrize("case", RECIPE_CASES, ids=[f"L{l}p{p}" for l, p in RECIPE_CASES])
def test_workload_9b_recipe_sampled(vbq, case):
    """Matrices of the 9B-class stack under the structured recipe (first MLP
    block at 2.5 bits, SLQ-style per-layer mixes, LM head at 1.1 bits, wide
    groups gathered on hot rows and input channels): sampled rows against
    the oracle and the layout read back, at full shape."""
    layer, pi = case
    proj = synth.C3.head if layer < 0 else synth.C3.projs[pi]
    _check_proj(vbq, 3, layer, pi, proj, 1, recipe=True)


def test_workload_9b_recipe_layer_one_launch(vbq):
    """Layer 0 of the structured recipe (its MLP at 2.5 bits) as one launch of
    both batched entry points: the outputs equal single calls bit for bit,
    and sampled rows match the oracle."""
    import torch
    pms, xs, cases = [], [], []
    for pi, proj in enumerate(synth.C3.projs):
        key = synth.proj_key(3, 0, pi)
        widths = synth.recipe_widths(0, pi, proj, synth.C3.layers)
        W = synth.weights(synth.SEED, key, proj.n, proj.k)
        x = synth.x_f16(synth.SEED, key, 1, proj.k)
        print(f"case 9b recipe layer 0 launch: {proj.name} {proj.n}x{proj.k}", flush=True)
        pms.append(vbq.vbq_pack(_t(W), widths))
        xs.append(_t(x, torch.float16))
        rows = _sample_rows(proj.n, np.random.default_rng(900 + pi), n=48)
        cases.append((rows, W[rows], widths[rows], x))
    ys = vbq.vbq_gemv_batched(pms, xs)
    ys_static = vbq.vbq_gemv_batched(pms, xs, static=True)
    torch.cuda.synchronize()
    for pm, x_t, y, ys_, (rows, Wr, wr, x) in zip(pms, xs, ys, ys_static, cases):
        q, s, o = oracle.quantize_matrix(Wr, wr)
        check_gemv(y.cpu().numpy()[:, rows], q, s, o, wr, x)
        assert torch.equal(y, vbq.vbq_gemv(pm, x_t))
        assert torch.equal(ys_, y)


def test_workload_in_cell_full_size(vbq):
    """4-bit release 14336 x 4096 with an in-cell residual: residual GEMV on
    sampled rows, and the re-quantisation check over the whole matrix."""
    import torch
    proj = synth.C2.projs[0]
    key = synth.proj_key(2, 0, 0)
    N, K = proj.n, proj.k
    widths = synth.widths(synth.SEED, key, N, K // 64, proj.mix)
    W = synth.weights(synth.SEED, key, N, K)
    x = synth.x_f16(synth.SEED, key, 1, K)
    q, s, o = oracle.quantize_matrix(W, widths)
    u = synth.cell_u(synth.SEED, key, N, K)
    resid = oracle.make_cell_residual(u, s)
    print("case workload 2 in-cell 14336x4096", flush=True)
    pm = vbq.vbq_pack(_t(W), widths)
    rt = _t(resid, torch.float16)
    y = vbq.vbq_gemv(pm, _t(x, torch.float16), residual=rt).cpu().numpy()
    rows = _sample_rows(N, np.random.default_rng(2))
    check_gemv(y[:, rows], q[rows], s[rows], o[rows], widths[rows], x, resid[rows])
    mism, ooc, first, rq = _verify_both(vbq, pm, rt)
    assert (mism, ooc, first) == (0, 0, 2 ** 64 - 1)
    assert torch.equal(rq, pm.stream)
    ref_v = oracle.requant_verify(q[rows], s[rows], o[rows], widths[rows], resid[rows])
    assert ref_v[:2] == (0, 0)


def test_workload_in_cell_compact_full_size(vbq):
    """The same 4-bit 14336 x 4096 release with the compact in-cell residual:
    the in-cell fp16 residual encoded on the device equals the oracle's
    encoding over the whole matrix, the fractions decode bit-exactly, and the
    GEMV with random fractions matches the oracle on sampled rows."""
    import torch
    proj = synth.C2.projs[0]
    key = synth.proj_key(2, 0, 0)
    N, K = proj.n, proj.k
    widths = synth.widths(synth.SEED, key, N, K // 64, proj.mix)
    W = synth.weights(synth.SEED, key, N, K)
    x = synth.x_f16(synth.SEED, key, 1, K)
    q, s, o = oracle.quantize_matrix(W, widths)
    resid = oracle.make_cell_residual(synth.cell_u(synth.SEED, key, N, K), s)
    print("case workload 2 compact in-cell 14336x4096", flush=True)
    pm = vbq.vbq_pack(_t(W), widths)
    f_gpu = vbq.cell8_encode(pm, _t(resid, torch.float16)).cpu().numpy()
    assert np.array_equal(f_gpu, oracle.cell8_encode(resid, s))
    f = synth.cell_f(synth.SEED, key, N, K)
    ft = _t(f)
    r16 = vbq.cell8_decode(pm, ft).cpu().numpy().view(np.uint16)
    assert np.array_equal(r16, oracle.cell8_decode(f, s))
    y = vbq.vbq_gemv_cell8(pm, _t(x, torch.float16), ft).cpu().numpy()
    rows = _sample_rows(N, np.random.default_rng(3))
    check_gemv(y[:, rows], q[rows], s[rows], o[rows], widths[rows], x, cell=f[rows])


def test_workload_9b_layer_one_launch_sampled(vbq):
    """The benchmark's launch: the seven projections of a 9B-class layer in
    one vbq_gemv_batched call at full shape (q, k, v, o, gate, up 4096 wide;
    down 14336 wide, four k-tiles shared by one workgroup's wavefronts).
    Sampled rows of every output against the oracle, within tolerance and
    each output within its bound; the batched outputs equal single calls."""
    import torch
    pms, xs, cases = [], [], []
    for pi, proj in enumerate(synth.C3.projs):
        key = synth.proj_key(3, 7, pi)
        widths = synth.widths(synth.SEED, key, proj.n, proj.k // 64, proj.mix)
        W = synth.weights(synth.SEED, key, proj.n, proj.k)
        x = synth.x_f16(synth.SEED, key, 1, proj.k)
        print(f"case 9b layer launch: {proj.name} {proj.n}x{proj.k}", flush=True)
        pms.append(vbq.vbq_pack(_t(W), widths))
        xs.append(_t(x, torch.float16))
        rows = _sample_rows(proj.n, np.random.default_rng(700 + pi), n=64)
        cases.append((rows, W[rows], widths[rows], x))
    ys = vbq.vbq_gemv_batched(pms, xs)
    torch.cuda.synchronize()
    for pm, x_t, y, (rows, Wr, wr, x) in zip(pms, xs, ys, cases):
        q, s, o = oracle.quantize_matrix(Wr, wr)
        check_gemv(y.cpu().numpy()[:, rows], q, s, o, wr, x)
        assert torch.equal(y, vbq.vbq_gemv(pm, x_t))
