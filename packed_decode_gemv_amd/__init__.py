"""Thin Python binding of libvbq (packed mixed-bit GEMV for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libvbq.so`` behind the C ABI declared in ``include/vbq.h``.
PyTorch provides device memory and streams. There is no fallback: if the
library is not built, importing this package raises.

Function names follow the C ABI: ``vbq_pack``, ``vbq_gemv``,
``vbq_gemv_batched``, ``vbq_gemm``, ``cell_requant_verify``, ``cell_drift_bound``.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libvbq.so")

GROUP = 64
TILE_ROWS = 16
TILE_GROUPS = 64
MAX_BATCH = 8

STATUS = {0: "ok", 1: "invalid argument", 2: "bad shape", 3: "width not in {1,2,4,8}", 4: "misaligned buffer",
          5: "unsupported size", 6: "layout does not match its buffers", 7: "HIP runtime error"}


class VbqError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)} (status {status})")
        self.status = status


class vbq_matrix(C.Structure):
    _fields_ = [("n_rows", C.c_int32), ("n_cols", C.c_int32), ("n_tiles", C.c_int64), ("n_records", C.c_int64),
                ("n_bytes16", C.c_int64), ("max_tile_bytes16", C.c_int64),
                ("tiles", C.c_void_p), ("stream", C.c_void_p)]


class vbq_layout_sizes(C.Structure):
    _fields_ = [("n_tiles", C.c_int64), ("n_records", C.c_int64), ("n_bytes16", C.c_int64),
                ("max_tile_bytes16", C.c_int64), ("max_tile_records", C.c_int64),
                ("code_bits", C.c_int64), ("groups_by_width", C.c_int64 * 4)]


EXPORTS = ("vbq_abi_version", "vbq_status_string", "vbq_pack_query", "vbq_pack", "vbq_matrix_check",
           "vbq_gemv", "vbq_gemv_batched", "vbq_gemm", "cell_requant_verify", "cell_drift_bound",
           "vbq_residual_error", "vbq_gemv_levels")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libvbq.so is not built ({LIB_PATH}); run __graft_entry__.build() or "
                          "python packed_decode_gemv_amd/build.py")
    lib = C.CDLL(LIB_PATH)
    P, I32 = C.c_void_p, C.c_int32
    lib.vbq_abi_version.restype = C.c_int
    lib.vbq_abi_version.argtypes = []
    lib.vbq_status_string.restype = C.c_char_p
    lib.vbq_status_string.argtypes = [C.c_int]
    lib.vbq_pack_query.restype = C.c_int
    lib.vbq_pack_query.argtypes = [P, I32, I32, C.POINTER(vbq_layout_sizes)]
    lib.vbq_pack.restype = C.c_int
    lib.vbq_pack.argtypes = [P, P, C.POINTER(vbq_matrix), P]
    lib.vbq_matrix_check.restype = C.c_int
    lib.vbq_matrix_check.argtypes = [C.POINTER(vbq_matrix), P]
    lib.vbq_gemv.restype = C.c_int
    lib.vbq_gemv.argtypes = [C.POINTER(vbq_matrix), P, I32, P, P, P]
    lib.vbq_gemv_batched.restype = C.c_int
    lib.vbq_gemv_batched.argtypes = [I32, C.POINTER(vbq_matrix), C.POINTER(C.c_void_p), C.POINTER(C.c_void_p), I32, P]
    lib.vbq_gemm.restype = C.c_int
    lib.vbq_gemm.argtypes = [C.POINTER(vbq_matrix), P, I32, P, P]
    lib.cell_requant_verify.restype = C.c_int
    lib.cell_requant_verify.argtypes = [C.POINTER(vbq_matrix), P, P, P, P]
    lib.cell_drift_bound.restype = C.c_int
    lib.cell_drift_bound.argtypes = [C.POINTER(vbq_matrix), P, I32, P, P]
    lib.vbq_residual_error.restype = C.c_int
    lib.vbq_residual_error.argtypes = [C.POINTER(vbq_matrix), P, P, P]
    lib.vbq_gemv_levels.restype = C.c_int
    lib.vbq_gemv_levels.argtypes = [I32, C.POINTER(vbq_matrix), P, I32, P, P, P]
    return lib


lib = _load()


def _check(st: int, what: str):
    if st != 0:
        raise VbqError(st, what)


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def abi_version() -> int:
    return lib.vbq_abi_version()


def pack_query(widths) -> vbq_layout_sizes:
    """Host-only sizing of the layout for uint8 widths [N][K/64] (numpy)."""
    w = np.ascontiguousarray(widths, dtype=np.uint8)
    N, G = w.shape
    out = vbq_layout_sizes()
    _check(lib.vbq_pack_query(w.ctypes.data_as(C.c_void_p), N, G * GROUP, C.byref(out)), "vbq_pack_query")
    return out


class PackedMatrix:
    """Device buffers of one packed matrix (owned by torch) and their descriptor."""

    def __init__(self, N: int, K: int, sizes: vbq_layout_sizes, device="cuda"):
        import torch
        self.N, self.K = int(N), int(K)
        self.sizes = sizes
        self.tiles = torch.empty(4 * (sizes.n_tiles + 1), dtype=torch.int32, device=device)
        self.stream = torch.empty(4 * sizes.n_bytes16, dtype=torch.int32, device=device)
        self.desc = vbq_matrix(self.N, self.K, sizes.n_tiles, sizes.n_records, sizes.n_bytes16,
                               sizes.max_tile_bytes16, self.tiles.data_ptr(), self.stream.data_ptr())

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.tiles, self.stream))

    def clone(self) -> "PackedMatrix":
        """A copy in new device buffers (same layout)."""
        pm = PackedMatrix(self.N, self.K, self.sizes, device=self.tiles.device)
        pm.tiles.copy_(self.tiles)
        pm.stream.copy_(self.stream)
        return pm

    def host_layout(self) -> dict:
        """The layout as numpy arrays (device-to-host copy), in the oracle's format."""
        return dict(tiles=self.tiles.cpu().numpy().view(np.uint32), stream=self.stream.cpu().numpy().view(np.uint32),
                    N=self.N, K=self.K)


def vbq_pack(W, widths, stream=None, check: bool = True) -> PackedMatrix:
    """Quantise W (torch float32 [N][K] on the GPU) with per-group widths
    (numpy or torch uint8 [N][K/64]) into a PackedMatrix."""
    import torch
    widths_np = widths.cpu().numpy() if isinstance(widths, torch.Tensor) else np.asarray(widths)
    widths_np = np.ascontiguousarray(widths_np, dtype=np.uint8)
    N, K = W.shape
    sizes = pack_query(widths_np)
    pm = PackedMatrix(N, K, sizes, device=W.device)
    wd = torch.from_numpy(widths_np).to(W.device)
    Wc = W.contiguous()
    st = lib.vbq_pack(_ptr(Wc), _ptr(wd), C.byref(pm.desc), _stream(stream))
    _check(st, "vbq_pack")
    if check:
        _check(lib.vbq_matrix_check(C.byref(pm.desc), _stream(stream)), "vbq_matrix_check")
    pm._keep = (Wc, wd)
    return pm


def vbq_gemv(pm: PackedMatrix, x, residual=None, out=None, stream=None):
    """y [B][N] float32 = x [B][K] (fp16) . (dequant(W) + residual)^T."""
    import torch
    x2 = x if x.dim() == 2 else x.view(1, -1)
    B = x2.shape[0]
    if out is None:
        out = torch.empty(B, pm.N, dtype=torch.float32, device=x.device)
    st = lib.vbq_gemv(C.byref(pm.desc), _ptr(x2), B, _ptr(residual), _ptr(out), _stream(stream))
    _check(st, "vbq_gemv")
    return out


def vbq_gemv_batched(pms, xs, ys=None, stream=None):
    """One launch for several independent GEMVs (same batch size)."""
    import torch
    n = len(pms)
    B = xs[0].shape[0] if xs[0].dim() == 2 else 1
    if ys is None:
        ys = [torch.empty(B, pm.N, dtype=torch.float32, device=xs[0].device) for pm in pms]
    descs = (vbq_matrix * n)(*[pm.desc for pm in pms])
    xp = (C.c_void_p * n)(*[x.data_ptr() for x in xs])
    yp = (C.c_void_p * n)(*[y.data_ptr() for y in ys])
    _check(lib.vbq_gemv_batched(n, descs, xp, yp, B, _stream(stream)), "vbq_gemv_batched")
    return ys


class GemvPlan:
    """Pre-marshalled argument block of vbq_gemv_batched, for timing loops."""

    def __init__(self, pms, xs, ys):
        n = len(pms)
        self.n = n
        self.B = xs[0].shape[0]
        self.descs = (vbq_matrix * n)(*[pm.desc for pm in pms])
        self.xp = (C.c_void_p * n)(*[x.data_ptr() for x in xs])
        self.yp = (C.c_void_p * n)(*[y.data_ptr() for y in ys])
        self._keep = (pms, xs, ys)

    def launch(self, stream_handle):
        st = lib.vbq_gemv_batched(self.n, self.descs, self.xp, self.yp, self.B, stream_handle)
        if st != 0:
            raise VbqError(st, "vbq_gemv_batched")


def vbq_gemm(pm: PackedMatrix, x_bf16, out=None, stream=None):
    """y [M][N] float32 = x [M][K] (bf16) . bf16(dequant(W))^T on MFMA."""
    import torch
    M = x_bf16.shape[0]
    if out is None:
        out = torch.empty(M, pm.N, dtype=torch.float32, device=x_bf16.device)
    _check(lib.vbq_gemm(C.byref(pm.desc), _ptr(x_bf16), M, _ptr(out), _stream(stream)), "vbq_gemm")
    return out


def cell_requant_verify(pm: PackedMatrix, residual, requant_codes: bool = False, stream=None):
    """Returns (mismatches, out_of_cell, first_bad_index, re-quantised stream tensor or None)."""
    import torch
    res = torch.empty(3, dtype=torch.int64, device=residual.device)
    rq = torch.empty_like(pm.stream) if requant_codes else None
    _check(lib.cell_requant_verify(C.byref(pm.desc), _ptr(residual), _ptr(res), _ptr(rq), _stream(stream)),
           "cell_requant_verify")
    r = res.cpu().numpy().view(np.uint64)
    return int(r[0]), int(r[1]), int(r[2]), rq


def cell_drift_bound(pm: PackedMatrix, x, out=None, stream=None):
    """bound [B][N] float32 = 0.5 * sum_g s[n][g] * sum_{k in g} |x[b][k]|: no
    residual inside its cells moves y[b][n] further."""
    import torch
    x2 = x if x.dim() == 2 else x.view(1, -1)
    B = x2.shape[0]
    if out is None:
        out = torch.empty(B, pm.N, dtype=torch.float32, device=x.device)
    _check(lib.cell_drift_bound(C.byref(pm.desc), _ptr(x2), B, _ptr(out), _stream(stream)), "cell_drift_bound")
    return out


def vbq_residual_error(pm: PackedMatrix, E, out=None, stream=None):
    """E - dequant(W) in binary32 (N x K float32): what the next residual level quantises."""
    import torch
    if out is None:
        out = torch.empty_like(E)
    _check(lib.vbq_residual_error(C.byref(pm.desc), _ptr(E), _ptr(out), _stream(stream)), "vbq_residual_error")
    return out


def rrq_pack(W, n_levels: int, stream=None):
    """Recurrent residual levels of W: a 2-bit base and n_levels - 1 2-bit
    levels, each packed from the error the levels before it leave."""
    import torch
    widths = np.full((W.shape[0], W.shape[1] // GROUP), 2, np.uint8)
    E = W.contiguous().float()
    levels = []
    for i in range(n_levels):
        pm = vbq_pack(E, widths, stream=stream)
        levels.append(pm)
        if i + 1 < n_levels:
            E = vbq_residual_error(pm, E, stream=stream)
    return levels


def vbq_gemv_levels(pms, x, out=None, stream=None):
    """y [B][N] float32 = sum over levels of x . dequant(W_i)^T."""
    import torch
    x2 = x if x.dim() == 2 else x.view(1, -1)
    B, n = x2.shape[0], len(pms)
    descs = (vbq_matrix * n)(*[pm.desc for pm in pms])
    scratch = torch.empty(n, B, pms[0].N, dtype=torch.float32, device=x.device)
    if out is None:
        out = torch.empty(B, pms[0].N, dtype=torch.float32, device=x.device)
    _check(lib.vbq_gemv_levels(n, descs, _ptr(x2), B, _ptr(scratch), _ptr(out), _stream(stream)), "vbq_gemv_levels")
    return out
