"""CPU oracle for packed mixed-bit GEMV -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's cpu_baseline leg may use
this package. The product library never imports it, and it imports nothing
from the product. It wraps ``vbq_oracle.c`` (plain scalar C, fp64 dequantise
and dot, binary32 quantiser decisions) through ctypes, and ``exact.py`` holds a
pure-Python rational-arithmetic mini-oracle for tiny cases.

Citations are in ``vbq_oracle.c``; every function here is a thin wrapper.
Parity status: every function is pinned by tests under ``tests/`` (see the
tests named ``test_oracle_*``); nothing here is "parity unpinned".
"""
from __future__ import annotations

import contextlib
import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vbq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
             "-fexcess-precision=standard"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = C.CDLL(build())
        _declare(_lib)
    return _lib


P = C.c_void_p
I64 = C.c_int64


def _declare(L):
    L.orc_f64_to_f16.restype = C.c_uint16
    L.orc_f64_to_f16.argtypes = [C.c_double]
    L.orc_f16_to_f64.restype = C.c_double
    L.orc_f16_to_f64.argtypes = [C.c_uint16]
    for name in ("orc_f64_to_f16_array", "orc_f32_to_f16_array", "orc_f16_to_f64_array"):
        getattr(L, name).restype = None
        getattr(L, name).argtypes = [P, I64, P]
    L.orc_quantize_group.restype = None
    L.orc_quantize_group.argtypes = [P, C.c_int, P, P, P]
    L.orc_quantize_matrix.restype = C.c_int
    L.orc_quantize_matrix.argtypes = [P, P, C.c_int, C.c_int, P, P, P]
    for name in ("orc_pack_group_canonical", "orc_unpack_group_canonical",
                 "orc_pack_group_record", "orc_unpack_group_record"):
        getattr(L, name).restype = None
        getattr(L, name).argtypes = [P, C.c_int, P]
    L.orc_layout_sizes.restype = C.c_int
    L.orc_layout_sizes.argtypes = [P, C.c_int, C.c_int, P, P, P]
    L.orc_pack.restype = C.c_int
    L.orc_pack.argtypes = [P, P, C.c_int, C.c_int, P, P]
    L.orc_unpack.restype = C.c_int
    L.orc_unpack.argtypes = [P, P, C.c_int, C.c_int, P, I64, P, P, P, P]
    L.orc_gemv.restype = None
    L.orc_gemv.argtypes = [P, P, P, C.c_int, C.c_int, P, C.c_int, C.c_int, P, P]
    L.orc_make_cell_residual.restype = None
    L.orc_f32_to_bf16.restype = C.c_uint16
    L.orc_f32_to_bf16.argtypes = [C.c_float]
    L.orc_dequant_bf16.restype = None
    L.orc_dequant_bf16.argtypes = [P, P, P, C.c_int, C.c_int, P]
    L.orc_make_cell_residual.argtypes = [P, P, C.c_int, C.c_int, P]
    L.orc_requant_verify.restype = None
    L.orc_requant_verify.argtypes = [P, P, P, P, P, C.c_int, C.c_int, P, P]
    L.orc_set_mutation.restype = None
    L.orc_set_mutation.argtypes = [C.c_int]
    L.orc_cell8_encode.restype = None
    L.orc_cell8_encode.argtypes = [P, P, C.c_int, C.c_int, P]
    L.orc_cell8_decode.restype = None
    L.orc_cell8_decode.argtypes = [P, P, C.c_int, C.c_int, P]
    L.orc_gemv_cell8.restype = None
    L.orc_gemv_cell8.argtypes = [P, P, P, C.c_int, C.c_int, P, C.c_int, P, P]


def _p(a):
    return None if a is None else a.ctypes.data_as(P)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


@contextlib.contextmanager
def mutation(m: int):
    """Plant deliberate mistake number ``m`` in the oracle (tests of the pins)."""
    lib().orc_set_mutation(int(m))
    try:
        yield
    finally:
        lib().orc_set_mutation(0)


# ---- conversions -----------------------------------------------------------
def f16_from_f64(v) -> np.ndarray:
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().orc_f64_to_f16_array(_p(v), v.size, _p(out))
    return out


def f16_from_f32(v) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint16)
    lib().orc_f32_to_f16_array(_p(v), v.size, _p(out))
    return out


def f64_from_f16(h) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float64)
    lib().orc_f16_to_f64_array(_p(h), h.size, _p(out))
    return out


# ---- quantiser and packing ----------------------------------------------------
def quantize_group(w, b: int):
    w = _c(w, np.float32)
    assert w.shape == (64,)
    s = np.zeros(1, np.uint16)
    o = np.zeros(1, np.uint16)
    q = np.zeros(64, np.uint8)
    lib().orc_quantize_group(_p(w), int(b), _p(s), _p(o), _p(q))
    return int(s[0]), int(o[0]), q


def quantize_matrix(W, widths):
    W = _c(W, np.float32)
    widths = _c(widths, np.uint8)
    N, K = W.shape
    q = np.zeros((N, K), np.uint8)
    s = np.zeros((N, K // 64), np.uint16)
    o = np.zeros((N, K // 64), np.uint16)
    if lib().orc_quantize_matrix(_p(W), _p(widths), N, K, _p(q), _p(s), _p(o)) != 0:
        raise ValueError("bad shape or width")
    return q, s, o


def _group_words(fn, q, b):
    q = _c(q, np.uint8)
    w = np.zeros(2 * b, np.uint32)
    getattr(lib(), fn)(_p(q), int(b), _p(w))
    return w


def _group_codes(fn, words, b):
    words = _c(words, np.uint32)
    assert words.shape == (2 * b,)
    q = np.zeros(64, np.uint8)
    getattr(lib(), fn)(_p(words), int(b), _p(q))
    return q


def pack_group_canonical(q, b):
    return _group_words("orc_pack_group_canonical", q, b)


def unpack_group_canonical(words, b):
    return _group_codes("orc_unpack_group_canonical", words, b)


def pack_group_record(q, b):
    return _group_words("orc_pack_group_record", q, b)


def unpack_group_record(words, b):
    return _group_codes("orc_unpack_group_record", words, b)


TILE_ROWS = 32
TILE_GROUPS = 64


def tile_grid(N: int, K: int):
    """(row-tiles, k-tiles) of the layout."""
    return (N + TILE_ROWS - 1) // TILE_ROWS, (K // 64 + TILE_GROUPS - 1) // TILE_GROUPS


def layout_sizes(widths):
    widths = _c(widths, np.uint8)
    N, G = widths.shape
    t = np.zeros(3, np.int64)
    if lib().orc_layout_sizes(_p(widths), N, 64 * G, _p(t[0:1]), _p(t[1:2]), _p(t[2:3])) != 0:
        raise ValueError("bad shape or width")
    return int(t[0]), int(t[1]), int(t[2])


def pack(W, widths) -> dict:
    """Quantise and write the execution layout: the tile table and the byte
    stream (as u32 words). Returns numpy arrays."""
    W = _c(W, np.float32)
    widths = _c(widths, np.uint8)
    N, K = W.shape
    T, R, B16 = layout_sizes(widths)
    out = dict(tiles=np.zeros(4 * (T + 1), np.uint32), stream=np.zeros(4 * B16, np.uint32), N=N, K=K)
    rc = lib().orc_pack(_p(W), _p(widths), N, K, _p(out["tiles"]), _p(out["stream"]))
    if rc != 0:
        raise ValueError("bad shape or width")
    return out


def unpack(layout: dict, rows=None):
    """Read a layout (numpy arrays) back to natural order.
    Returns (codes [R][K] u8, scale16 [R][G], offset16 [R][G], widths [R][G])."""
    N, K = int(layout["N"]), int(layout["K"])
    G = K // 64
    r = None if rows is None else _c(rows, np.int64)
    nr = N if r is None else len(r)
    q = np.zeros((nr, K), np.uint8)
    s = np.zeros((nr, G), np.uint16)
    o = np.zeros((nr, G), np.uint16)
    w = np.zeros((nr, G), np.uint8)
    arrs = [_c(layout[k], np.uint32) for k in ("tiles", "stream")]
    rc = lib().orc_unpack(*[_p(a) for a in arrs], N, K, _p(r), nr, _p(q), _p(s), _p(o), _p(w))
    if rc != 0:
        raise ValueError("inconsistent layout")
    return q, s, o, w


# ---- GEMV / GEMM / in-cell ------------------------------------------------------
def gemv(q, s16, o16, x, resid=None, bf16: bool = False) -> np.ndarray:
    """y [B][N] fp64 = x . Wdq^T with Wdq = s*q + o (+ resid), natural k order."""
    q = _c(q, np.uint8)
    s16 = _c(s16, np.uint16)
    o16 = _c(o16, np.uint16)
    x = _c(np.atleast_2d(x), np.uint16)
    N, K = q.shape
    B = x.shape[0]
    assert x.shape[1] == K
    r = None if resid is None else _c(resid, np.uint16)
    if r is not None:
        assert r.shape == (N, K)
    y = np.zeros((B, N), np.float64)
    lib().orc_gemv(_p(q), _p(s16), _p(o16), N, K, _p(x), B, int(bf16), _p(r), _p(y))
    return y


def drift_bound(s16, x) -> np.ndarray:
    """Bound on how far an in-cell residual can move each output (page
    "Nothing Changed but the Model: CellFill -- Bounded In-Cell Learning for
    Bit-Identical, Revocable Updates to Quantized LLMs", section Abstract:
    bounded drift). With every |r[n][k]| below half its group's scale,
    |sum_k x[b][k] r[n][k]| <= sum_k |x[b][k]| s[n][g(k)] / 2; the supremum
    over such residuals. Returns [B][N] fp64 = 0.5 * sum_g s[n][g] * sum_{k in g} |x[b][k]|."""
    s = f64_from_f16(_c(s16, np.uint16))                       # [N][G]
    xa = np.abs(f64_from_f16(_c(np.atleast_2d(x), np.uint16)))  # [B][K]
    B, K = xa.shape
    assert K == s.shape[1] * 64
    return 0.5 * (xa.reshape(B, K // 64, 64).sum(axis=2) @ s.T)


def rrq_levels(W, n_levels: int):
    """Recurrent residual levels (RRQ abstract on page
    thelatestinai.com/papers/2512.18934): a 2-bit RTN base, then 2-bit RTN of what remains. In
    binary32: E_0 = W; level i = RTN(E_i) with every group 2-bit;
    E_{i+1} = E_i - (f32(s_i q_i) + o_i) (s q is exact in binary32, so this
    rounds once per operation). Returns ([(q, s16, o16) per level], E_n)."""
    E = np.ascontiguousarray(W, np.float32)
    N, K = E.shape
    widths = np.full((N, K // 64), 2, np.uint8)
    levels = []
    for _ in range(n_levels):
        q, s16, o16 = quantize_matrix(E, widths)
        s = f64_from_f16(np.repeat(s16, 64, axis=1)).astype(np.float32)
        o = f64_from_f16(np.repeat(o16, 64, axis=1)).astype(np.float32)
        deq = (s * q.astype(np.float32)) + o
        E = (E - deq).astype(np.float32)
        levels.append((q, s16, o16))
    return levels, E


def rrq_gemv(levels, x) -> np.ndarray:
    """y [B][N] fp64 = x . (sum of the levels' dequantised weights)^T."""
    x = f64_from_f16(_c(np.atleast_2d(x), np.uint16))
    Wsum = 0.0
    for q, s16, o16 in levels:
        Wsum = Wsum + f64_from_f16(np.repeat(s16, 64, axis=1)) * q + f64_from_f16(np.repeat(o16, 64, axis=1))
    return x @ np.asarray(Wsum).T


def f32_to_bf16(v: float) -> int:
    return int(lib().orc_f32_to_bf16(float(np.float32(v))))


def bf16_to_f64(u16) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns."""
    u = np.ascontiguousarray(u16, np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def dequant_bf16(q, s16, o16) -> np.ndarray:
    """bfloat16 bit patterns [N][K] of bf16(f32(s*q) + o)."""
    q = _c(q, np.uint8)
    s16 = _c(s16, np.uint16)
    o16 = _c(o16, np.uint16)
    N, K = q.shape
    out = np.zeros((N, K), np.uint16)
    lib().orc_dequant_bf16(_p(q), _p(s16), _p(o16), N, K, _p(out))
    return out


def gemm_bf16_weights(q, s16, o16, x_bf16) -> np.ndarray:
    """y [M][N] fp64 = x . Wbf^T with the weights first rounded to bfloat16
    (dequant_bf16); x bfloat16 bit patterns [M][K]. A library matmul in fp64."""
    W = bf16_to_f64(dequant_bf16(q, s16, o16))
    return bf16_to_f64(x_bf16) @ W.T


def make_cell_residual(u, s16) -> np.ndarray:
    u = _c(u, np.float64)
    s16 = _c(s16, np.uint16)
    N, K = u.shape
    r = np.zeros((N, K), np.uint16)
    lib().orc_make_cell_residual(_p(u), _p(s16), N, K, _p(r))
    return r


def requant_verify(q, s16, o16, widths, r16, want_codes: bool = False):
    """Returns (mismatches, out_of_cell, first_bad_index, q_prime or None)."""
    q = _c(q, np.uint8)
    N, K = q.shape
    counts = np.zeros(3, np.uint64)
    qp = np.zeros((N, K), np.uint8) if want_codes else None
    lib().orc_requant_verify(_p(q), _p(_c(s16, np.uint16)), _p(_c(o16, np.uint16)),
                             _p(_c(widths, np.uint8)), _p(_c(r16, np.uint16)), N, K, _p(counts), _p(qp))
    return int(counts[0]), int(counts[1]), int(counts[2]), qp


def cell8_encode(r16, s16) -> np.ndarray:
    """Compact in-cell residual (this library's own encoding: the CellFill
    page keeps the residual inside its rounding cell but fixes no storage):
    a signed byte f per weight stands for r = s * f / 256, |f| <= 127, so
    every encoded residual is inside its cell. Encodes an fp16 residual in
    binary32: f = clamp(rint(f32(r / s) * 256), -127, 127), 0 where s = 0.
    Returns int8 [N][K]."""
    r16 = _c(r16, np.uint16)
    s16 = _c(s16, np.uint16)
    N, K = r16.shape
    assert s16.shape == (N, K // 64)
    f = np.zeros((N, K), np.int8)
    lib().orc_cell8_encode(_p(r16), _p(s16), N, K, _p(f))
    return f


def cell8_decode(f, s16) -> np.ndarray:
    """The fp16 residual each fraction byte stands for: fp16(s * f / 256)
    (exact before the one rounding). Returns uint16 fp16 bits [N][K]."""
    f = _c(f, np.int8)
    s16 = _c(s16, np.uint16)
    N, K = f.shape
    assert s16.shape == (N, K // 64)
    r16 = np.zeros((N, K), np.uint16)
    lib().orc_cell8_decode(_p(f), _p(s16), N, K, _p(r16))
    return r16


def gemv_cell8(q, s16, o16, x, f) -> np.ndarray:
    """y [B][N] fp64 = x . (s*q + o + s*f/256)^T, natural k order."""
    q = _c(q, np.uint8)
    s16 = _c(s16, np.uint16)
    o16 = _c(o16, np.uint16)
    x = _c(np.atleast_2d(x), np.uint16)
    f = _c(f, np.int8)
    N, K = q.shape
    assert f.shape == (N, K) and x.shape[1] == K
    y = np.zeros((x.shape[0], N), np.float64)
    lib().orc_gemv_cell8(_p(q), _p(s16), _p(o16), N, K, _p(x), x.shape[0], _p(f), _p(y))
    return y
