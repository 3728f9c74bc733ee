"""Parity of the HIP library against the CPU oracle (needs an MI355X).

Bars: the packed layout (tile table and byte stream) and the
re-quantisation check are bit-exact; GEMV/GEMM outputs are within 2e-3
relative L2 of the fp64 oracle over each call's whole output.
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
    ref = oracle.gemv(q, s, o, x)
    assert y.shape == ref.shape
    assert rel_l2(y, ref) <= TOL
    # also per batch row
    for b in range(B):
        assert rel_l2(y[b], ref[b]) <= TOL


@pytest.mark.parametrize("width", [1, 2, 4, 8])
def test_single_width_with_constant_groups(vbq, width):
    """Every group of one width, so that class's full and partial blocks make
    up the whole stream, and rows past a tile (N = 37); three constant groups
    have scale 0, so every weight there equals the offset (one is all zero).
    Layout bit-exact; GEMV and GEMM within tolerance of the oracle."""
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
    ref = oracle.gemv(q, s, o, x)
    for b in range(B):
        assert rel_l2(y[b], ref[b]) <= TOL
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
    # A launch's work split depends on all its matrices, so a batched launch
    # may add in another order than single launches: each launch shape is
    # bit-for-bit repeatable, and the two agree to rounding.
    for a, b, c, d in zip(singles, again, batched, batched2):
        assert torch.equal(a, b), "GEMV not deterministic"
        assert torch.equal(c, d), "batched GEMV not deterministic"
        assert rel_l2(c.cpu().numpy(), a.cpu().numpy().astype(np.float64)) <= 1e-5


def test_split_k_calls_in_sequence(vbq):
    """Matrices with K > 4096 are summed over k-tiles through the library's
    per-stream workspace; calls of different shapes on one stream (different
    numbers of row ranges and k-tiles) must each be right, in any order."""
    import torch
    for (N, K, B) in [(300, 4480, 4), (2048, 8192, 1), (40, 14336, 1), (700, 64 * 70, 2), (2048, 8192, 1)]:
        W, widths, x = rand_case(N, K, seed=N + K + B, B=B)
        print(f"case split-k {N}x{K} B={B}", flush=True)
        pm = vbq.vbq_pack(_t(W), widths)
        q, s, o = oracle.quantize_matrix(W, widths)
        y = vbq.vbq_gemv(pm, _t(x, torch.float16)).cpu().numpy()
        assert rel_l2(y, oracle.gemv(q, s, o, x)) <= TOL


def test_split_k_repeatable_across_streams(vbq):
    """The k-tile partial rows are added by the last workgroup of each row
    range to arrive; its counters must be rearmed after every call, on every
    stream, and the sum order must not depend on which workgroup came last."""
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


def test_batched_more_matrices_than_one_launch(vbq):
    """40 matrices in one call (more than a launch takes, so the library
    splits them), of mixed shapes, some with K > 4096: every output matches
    the oracle."""
    import torch
    r = np.random.default_rng(77)
    mats, refs = [], []
    for i in range(40):
        N = int(r.choice([16, 40, 96, 256, 513]))
        K = int(r.choice([64, 1024, 4096, 4160, 8192]))
        W, widths, x = rand_case(N, K, seed=300 + i, B=1)
        q, s, o = oracle.quantize_matrix(W, widths)
        mats.append((vbq.vbq_pack(_t(W), widths), _t(x, torch.float16)))
        refs.append(oracle.gemv(q, s, o, x))
    print("case batched 40 matrices", flush=True)
    ys = vbq.vbq_gemv_batched([pm for pm, _ in mats], [x for _, x in mats])
    for y, ref in zip(ys, refs):
        assert rel_l2(y.cpu().numpy(), ref) <= TOL


def test_graph_replays_match_eager(vbq):
    """Launches captured in a HIP graph (as the benchmark replays a decode
    step) give the eager results on every replay, with other eager work and
    synchronisations in between; split-K counters are rearmed by the kernel
    itself, so no replay depends on the previous one."""
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
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):   # the workspace is per stream: warm up the capturing one
        plan.launch(vbq._stream())
    side.synchronize()
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
        # batch 1 and batch 4 split the work differently (fp32 sums in another
        # order): rows must agree to rounding, a wrong row mapping gives O(1)
        y1 = vbq.vbq_gemv(pm, xt[b:b + 1].contiguous())
        assert rel_l2(y1[0].cpu().numpy(), y4[b].cpu().numpy().astype(np.float64)) <= 5e-5


def _cell_inputs(N, K, seed, u_scale=1.0):
    r = np.random.default_rng(seed)
    widths = np.full((N, K // 64), 4, np.uint8)
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    q, s, o = oracle.quantize_matrix(W, widths)
    u = r.uniform(-0.49, 0.49, (N, K)) * u_scale
    resid = oracle.make_cell_residual(u, s)
    x = r.standard_normal((1, K)).astype(np.float16).view(np.uint16)
    return W, widths, q, s, o, resid, x


@pytest.mark.parametrize("shape", [(16, 256), (50, 1024), (33, 4096), (20, 8192)])
def test_residual_gemv_and_revocation(vbq, shape):
    import torch
    N, K = shape
    W, widths, q, s, o, resid, x = _cell_inputs(N, K, seed=N + K)
    pm = vbq.vbq_pack(_t(W), widths)
    xt = _t(x, torch.float16)
    rt = _t(resid, torch.float16)
    y = vbq.vbq_gemv(pm, xt, residual=rt).cpu().numpy()
    ref = oracle.gemv(q, s, o, x, resid)
    assert rel_l2(y, ref) <= TOL
    y0 = vbq.vbq_gemv(pm, xt).cpu().numpy()
    assert rel_l2(y0, oracle.gemv(q, s, o, x)) <= TOL
    # a zero residual serves the base weights
    yz = vbq.vbq_gemv(pm, xt, residual=torch.zeros_like(rt)).cpu().numpy()
    assert np.allclose(yz, y0, rtol=1e-6, atol=1e-6)


def _verify_both(vbq, pm, resid_t):
    """cell_requant_verify with the re-quantised stream (one workgroup per
    tile) and without it (a tile's records split over several workgroups):
    the counts and first index must agree; returns the first call's result."""
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
            assert rel_l2(y, oracle.rrq_gemv(levels[:k + 1], x)) <= TOL, (B, k)


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
    served.stream[0:1].bitwise_xor_(1)        # lowest code bit of the first record of the stream
    mism, ooc, first, rq = _verify_both(vbq, served, _t(resid, torch.float16))
    assert (mism, ooc, first) == (0, 0, 2 ** 64 - 1)
    assert torch.equal(rq, served.stream)
    diff = torch.nonzero(rq != release.stream).flatten().tolist()
    assert diff == [0]


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
    rows.update([0, N - 1, (N // 16) * 16 - 1 if N >= 16 else 0])
    return np.array(sorted(rows), np.int64)


def _check_proj(vbq, cid, layer, pi, proj, B, full=False):
    import torch
    key = synth.proj_key(cid, layer, pi)
    G = proj.k // 64
    widths = synth.widths(synth.SEED, key, proj.n, G, proj.mix)
    W = synth.weights(synth.SEED, key, proj.n, proj.k)
    x = synth.x_f16(synth.SEED, key, B, proj.k)
    print(f"case workload {cid} layer {layer} {proj.name} {proj.n}x{proj.k} B={B}", flush=True)
    pm = vbq.vbq_pack(_t(W), widths)
    y = vbq.vbq_gemv(pm, _t(x, torch.float16)).cpu().numpy()
    rows = np.arange(proj.n) if full else _sample_rows(proj.n, np.random.default_rng(pi + 100 * (layer + 1)))
    q, s, o = oracle.quantize_matrix(W[rows], widths[rows])
    ref = oracle.gemv(q, s, o, x)
    assert rel_l2(y[:, rows], ref) <= TOL
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
    ref = oracle.gemv(q[rows], s[rows], o[rows], x, resid[rows])
    assert rel_l2(y[:, rows], ref) <= TOL
    mism, ooc, first, rq = _verify_both(vbq, pm, rt)
    assert (mism, ooc, first) == (0, 0, 2 ** 64 - 1)
    assert torch.equal(rq, pm.stream)
    ref_v = oracle.requant_verify(q[rows], s[rows], o[rows], widths[rows], resid[rows])
    assert ref_v[:2] == (0, 0)
