"""Host-side checks of the C ABI library (no GPU needed): it loads, exports
every function that include/vbq.h declares, sizes layouts like the oracle,
and rejects bad arguments before touching the GPU."""
import ctypes as C
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "vbq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_entry_points():
    names = header_functions()
    for n in ("vbq_pack", "vbq_gemv", "vbq_gemm", "cell_requant_verify", "cell_drift_bound", "vbq_pack_query",
              "vbq_residual_error", "vbq_gemv_levels", "vbq_gemv_batched_static", "vbq_gemv_cell8",
              "cell8_encode", "cell8_decode",
              "vbq_gemv_batched", "vbq_matrix_check", "vbq_abi_version", "vbq_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import packed_decode_gemv_amd as vbq
    lib = C.CDLL(vbq.LIB_PATH)
    for n in header_functions():
        assert hasattr(lib, n), f"{n} declared in vbq.h but not exported"
    assert vbq.abi_version() == 4
    assert vbq.lib.vbq_status_string(3) == b"width not in {1,2,4,8}"


@pytest.mark.parametrize("shape", [(1, 64), (16, 128), (17, 192), (33, 640), (100, 64 * 37), (20, 64 * 200)])
def test_pack_query_matches_oracle(shape):
    import oracle
    import packed_decode_gemv_amd as vbq
    N, K = shape
    r = np.random.default_rng(N + K)
    w = r.choice(np.array([1, 2, 4, 8], np.uint8), size=(N, K // 64), p=[0.6, 0.2, 0.15, 0.05])
    s = vbq.pack_query(w)
    assert (s.n_tiles, s.n_records, s.n_bytes16) == oracle.layout_sizes(w)
    lay = oracle.pack((np.random.default_rng(1).standard_normal((N, K)) * 0.02).astype(np.float32), w)
    tiles = lay["tiles"].reshape(-1, 4).astype(np.int64)
    assert s.max_tile_bytes16 == int(tiles[:-1, 1].max())
    assert s.code_bits == 64 * int(w.astype(np.int64).sum())
    assert list(s.groups_by_width) == [int((w == b).sum()) for b in (1, 2, 4, 8)]


def test_pack_query_rejects_bad_input():
    import packed_decode_gemv_amd as vbq
    w = np.ones((4, 2), np.uint8)
    out = vbq.vbq_layout_sizes()
    p = w.ctypes.data_as(C.c_void_p)
    assert vbq.lib.vbq_pack_query(p, 4, 100, C.byref(out)) == 2          # K % 64
    assert vbq.lib.vbq_pack_query(p, 0, 128, C.byref(out)) == 2          # N < 1
    assert vbq.lib.vbq_pack_query(None, 4, 128, C.byref(out)) == 1       # null
    w[1, 1] = 3
    assert vbq.lib.vbq_pack_query(p, 4, 128, C.byref(out)) == 3          # width 3


def _fake_matrix(vbq, N=32, K=128, align=256):
    # Descriptor with plausible (never dereferenced) device addresses.
    T = ((N + 31) // 32) * ((K // 64 + 63) // 64)
    base = 0x7F0000000000
    return vbq.vbq_matrix(N, K, T, 10, base, base + align * 64)


def test_compute_calls_reject_bad_arguments_without_a_gpu():
    import packed_decode_gemv_amd as vbq
    L = vbq.lib
    m = _fake_matrix(vbq)
    x = C.c_void_p(0x7F0000100000)
    y = C.c_void_p(0x7F0000200000)
    assert L.vbq_gemv(None, x, 1, None, y, None) == 1
    assert L.vbq_gemv(C.byref(m), None, 1, None, y, None) == 1
    assert L.vbq_gemv(C.byref(m), x, 0, None, y, None) == 5
    assert L.vbq_gemv(C.byref(m), x, 9, None, y, None) == 5
    assert L.vbq_gemv(C.byref(m), C.c_void_p(0x7F0000100008), 1, None, y, None) == 4
    assert L.vbq_gemv(C.byref(m), x, 1, C.c_void_p(0x7F0000300008), y, None) == 4
    bad = _fake_matrix(vbq, K=100)
    assert L.vbq_gemv(C.byref(bad), x, 1, None, y, None) == 2
    bad = _fake_matrix(vbq)
    bad.n_tiles = 5
    assert L.vbq_gemv(C.byref(bad), x, 1, None, y, None) == 6
    bad = _fake_matrix(vbq, align=8)
    bad.stream = 0x7F0000000008
    assert L.vbq_gemv(C.byref(bad), x, 1, None, y, None) == 4
    big = _fake_matrix(vbq, K=64 * 4000)
    assert L.vbq_gemv(C.byref(big), x, 9, None, y, None) == 5      # batch above the maximum
    assert L.vbq_gemm(C.byref(m), x, 0, y, None) == 2
    assert L.vbq_gemm(C.byref(m), C.c_void_p(0x7F0000100004), 64, y, None) == 4
    assert L.cell_requant_verify(C.byref(m), None, y, None, None) == 1
    assert L.cell_requant_verify(C.byref(m), x, C.c_void_p(0x7F0000200004), None, None) == 4
    assert L.cell_drift_bound(C.byref(m), None, 1, y, None) == 1
    assert L.cell_drift_bound(C.byref(m), x, 1, None, None) == 1
    assert L.cell_drift_bound(C.byref(m), x, 0, y, None) == 5
    assert L.cell_drift_bound(C.byref(m), x, 9, y, None) == 5
    assert L.cell_drift_bound(C.byref(m), C.c_void_p(0x7F0000100001), 1, y, None) == 4
    assert L.cell_drift_bound(C.byref(m), x, 1, C.c_void_p(0x7F0000200002), None) == 4
    assert L.cell_drift_bound(C.byref(_fake_matrix(vbq, K=100)), x, 1, y, None) == 2
    assert L.vbq_gemv_cell8(C.byref(m), x, 1, None, y, None) == 1           # the fractions are required
    assert L.vbq_gemv_cell8(C.byref(m), x, 1, C.c_void_p(0x7F0000300008), y, None) == 4
    assert L.vbq_gemv_cell8(C.byref(m), x, 9, C.c_void_p(0x7F0000300000), y, None) == 5
    assert L.vbq_gemv_cell8(C.byref(_fake_matrix(vbq, K=100)), x, 1, C.c_void_p(0x7F0000300000), y, None) == 2
    assert L.cell8_encode(C.byref(m), None, C.c_void_p(0x7F0000300000), None) == 1
    assert L.cell8_encode(C.byref(m), x, None, None) == 1
    assert L.cell8_encode(C.byref(m), x, C.c_void_p(0x7F0000300004), None) == 4
    assert L.cell8_decode(C.byref(m), C.c_void_p(0x7F0000300000), C.c_void_p(0x7F0000100002), None) == 4
    assert L.cell8_decode(None, C.c_void_p(0x7F0000300000), x, None) == 1
    assert L.vbq_residual_error(C.byref(m), None, y, None) == 1
    assert L.vbq_residual_error(C.byref(m), x, C.c_void_p(0x7F0000200004), None) == 4
    two = (vbq.vbq_matrix * 2)(m, _fake_matrix(vbq, N=48))
    assert L.vbq_gemv_levels(2, two, x, 1, y, None) == 2             # levels of different shapes
    assert L.vbq_gemv_levels(0, two, x, 1, y, None) == 1
    assert L.vbq_gemv_levels(33, two, x, 1, y, None) == 1           # more than one launch takes
    same = (vbq.vbq_matrix * 2)(m, m)
    assert L.vbq_gemv_levels(2, same, x, 9, y, None) == 5
    assert L.vbq_gemv_levels(2, same, x, 1, None, None) == 1
    assert L.vbq_pack(None, x, C.byref(m), None) == 1
    assert L.vbq_pack(C.c_void_p(0x7F0000100004), x, C.byref(m), None) == 4
    ms = (vbq.vbq_matrix * 2)(m, m)
    xs = (C.c_void_p * 2)(x.value, x.value)
    ys = (C.c_void_p * 2)(y.value, None)
    assert L.vbq_gemv_batched(2, ms, xs, ys, 1, None) == 1
    assert L.vbq_gemv_batched(0, ms, xs, ys, 1, None) == 1
    many = (vbq.vbq_matrix * 33)(*([m] * 33))
    xs33 = (C.c_void_p * 33)(*([x.value] * 33))
    ys33 = (C.c_void_p * 33)(*([y.value] * 33))
    assert L.vbq_gemv_batched(33, many, xs33, ys33, 1, None) == 1     # more than one launch takes


def test_binding_rejects_bad_tensors_before_any_launch():
    """The C ABI cannot see tensor sizes, so the binding checks dtype, shape,
    contiguity and device first; every case here raises ValueError without
    reaching the library (no GPU is needed)."""
    import torch

    import packed_decode_gemv_amd as vbq
    W = torch.zeros(32, 128)
    widths = np.ones((32, 2), np.uint8)
    with pytest.raises(ValueError, match="GPU"):
        vbq.vbq_pack(W, widths)                                   # host tensor
    with pytest.raises(ValueError, match="dtype"):
        vbq.vbq_pack(W.half(), widths)
    with pytest.raises(ValueError, match="contiguous"):
        vbq.vbq_pack(torch.zeros(128, 32).t(), widths)
    pm = vbq.PackedMatrix(32, 128, vbq.pack_query(widths), device="cpu")   # descriptor only, never launched
    with pytest.raises(ValueError, match="dtype"):
        vbq.vbq_gemv(pm, torch.zeros(1, 128, dtype=torch.float32))
    with pytest.raises(ValueError, match="shape"):
        vbq.vbq_gemv(pm, torch.zeros(1, 64, dtype=torch.float16))
    with pytest.raises(ValueError, match="contiguous"):
        vbq.vbq_gemv(pm, torch.zeros(256, dtype=torch.float16)[::2].view(1, 128))
    with pytest.raises(ValueError, match="batch"):
        vbq.vbq_gemv(pm, torch.zeros(9, 128, dtype=torch.float16))
    with pytest.raises(ValueError, match="residual: dtype"):
        vbq.vbq_gemv(pm, torch.zeros(1, 128, dtype=torch.float16), residual=torch.zeros(32, 128))
    with pytest.raises(ValueError, match="out: shape"):
        vbq.vbq_gemv(pm, torch.zeros(2, 128, dtype=torch.float16), out=torch.zeros(1, 32))
    with pytest.raises(ValueError, match="cell: dtype"):
        vbq.vbq_gemv_cell8(pm, torch.zeros(1, 128, dtype=torch.float16), torch.zeros(32, 128, dtype=torch.uint8))
    with pytest.raises(ValueError, match="cell: shape"):
        vbq.cell8_decode(pm, torch.zeros(32, 64, dtype=torch.int8))
    with pytest.raises(ValueError, match="cell: dtype"):
        vbq.CellUpdate(pm, torch.zeros(32, 128, dtype=torch.int16))
    with pytest.raises(ValueError, match="residual: dtype"):
        vbq.cell8_encode(pm, torch.zeros(32, 128))
    with pytest.raises(ValueError, match="E: dtype"):
        vbq.vbq_residual_error(pm, torch.zeros(32, 128, dtype=torch.float16))
    with pytest.raises(ValueError, match="residual: shape"):
        vbq.cell_requant_verify(pm, torch.zeros(16, 128, dtype=torch.float16))
    with pytest.raises(ValueError, match="x: dtype"):
        vbq.vbq_gemm(pm, torch.zeros(64, 128, dtype=torch.float16))
    with pytest.raises(ValueError, match="x: shape"):
        vbq.cell_drift_bound(pm, torch.zeros(1, 256, dtype=torch.float16))
    with pytest.raises(ValueError, match="different shapes"):
        vbq.vbq_gemv_levels([pm, vbq.PackedMatrix(64, 128, vbq.pack_query(np.ones((64, 2), np.uint8)),
                                                  device="cpu")], torch.zeros(1, 128, dtype=torch.float16))
    with pytest.raises(ValueError, match="widths"):
        vbq.pack_query(np.ones(4, np.uint8))
