"""vbq_gemv_batched_static (the entry point that allocates nothing) against
vbq_gemv_batched, through the C ABI: two calls in a row, the second with
smaller matrices and a smaller batch, each output compared element by
element. The static call sums a row-tile's k-tile partial sums in the order
vbq_gemv_batched uses, so the two agree bit for bit."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vbq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import packed_decode_gemv_amd as vbq
    return vbq


def _layer(vbq, cid, projs, B, rows_cap=None):
    import torch
    import synth
    dev = torch.device("cuda")
    pms, xs = [], []
    for pi, proj in enumerate(projs):
        key = synth.proj_key(cid, 0, pi)
        n = proj.n if rows_cap is None else min(proj.n, rows_cap)
        w = synth.widths(synth.SEED, key, n, proj.k // 64, proj.mix)
        W = torch.from_numpy(synth.weights(synth.SEED, key, n, proj.k)).to(dev)
        pms.append(vbq.vbq_pack(W, w))
        xs.append(torch.from_numpy(synth.x_f16(synth.SEED, key, B, proj.k).view(np.float16)).to(dev))
    return pms, xs


def _compare(vbq, pms, xs):
    import torch
    ref = vbq.vbq_gemv_batched(pms, xs)
    got = vbq.vbq_gemv_batched(pms, xs, static=True)
    torch.cuda.synchronize()
    for r, g in zip(ref, got):
        assert r.shape == g.shape
        assert torch.equal(r, g), float((r - g).abs().max())


def test_static_matches_batched_two_calls(vbq):
    import synth
    # first call: a 9B-class layer (its down projection has 3.5 k-tiles per
    # row-tile), batch 1
    pms, xs = _layer(vbq, 3, synth.C3.projs, 1)
    print("call 1: 9B-class layer, 7 projections, batch 1", flush=True)
    _compare(vbq, pms, xs)
    # second call: smaller, a 1B-class layer (down has 2 k-tiles) cut to 1000
    # rows per projection, batch 3 (a pass of two rows and one of one)
    pms2, xs2 = _layer(vbq, 1, synth.C1.projs, 3, rows_cap=1000)
    print("call 2: 1B-class layer cut to 1000 rows, batch 3", flush=True)
    _compare(vbq, pms2, xs2)
    # and once more the first, after the second left its scratch behind
    _compare(vbq, pms, xs)


def test_static_rejects_oversized_launch(vbq):
    import ctypes as C
    import torch
    # three matrices of 65536 rows x 4095 groups (64 k-tiles) need more
    # partial-sum slots than the scratch holds; the call is refused before
    # anything is enqueued (the descriptors point nowhere: nothing reads them)
    n = 3
    descs = (vbq.vbq_matrix * n)()
    for i in range(n):
        d = descs[i]
        d.n_rows, d.n_cols = 65536, 64 * 4095
        d.n_tiles = (65536 // 32) * 64
        d.n_bytes16 = 16
        d.tiles = 256
        d.stream = 256
    xp = (C.c_void_p * n)(*([256] * n))
    yp = (C.c_void_p * n)(*([256] * n))
    st = vbq.lib.vbq_gemv_batched_static(n, descs, xp, yp, 1, C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 5, st
