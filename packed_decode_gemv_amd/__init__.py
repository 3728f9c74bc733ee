"""Thin Python binding of libvbq (packed mixed-bit GEMV for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libvbq.so`` behind the C ABI declared in ``include/vbq.h``.
PyTorch provides device memory and streams. There is no fallback: if the
library is not built, importing this package raises.

The C ABI takes plain pointers, so the sizes, dtypes and layouts of the
tensors are checked here, before anything is launched (a wrong tensor raises
``ValueError``).

Function names follow the C ABI: ``vbq_pack``, ``vbq_gemv``,
``vbq_gemv_batched``, ``vbq_gemv_batched_static``, ``vbq_gemv_levels``,
``vbq_gemv_cell8``, ``vbq_gemm``, ``cell_requant_verify``, ``cell_drift_bound``,
``cell8_encode``, ``cell8_decode``, ``vbq_residual_error``.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libvbq.so")

GROUP = 64
TILE_ROWS = 32
TILE_GROUPS = 64
MAX_BATCH = 8
MAX_LAUNCH_MATS = 32

STATUS = {0: "ok", 1: "invalid argument", 2: "bad shape", 3: "width not in {1,2,4,8}", 4: "misaligned buffer",
          5: "unsupported size", 6: "layout does not match its buffers", 7: "HIP runtime error"}


class VbqError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)} (status {status})")
        self.status = status


class vbq_matrix(C.Structure):
    _fields_ = [("n_rows", C.c_int32), ("n_cols", C.c_int32), ("n_tiles", C.c_int64), ("n_bytes16", C.c_int64),
                ("tiles", C.c_void_p), ("stream", C.c_void_p)]


class vbq_layout_sizes(C.Structure):
    _fields_ = [("n_tiles", C.c_int64), ("n_records", C.c_int64), ("n_bytes16", C.c_int64),
                ("max_tile_bytes16", C.c_int64), ("code_bits", C.c_int64), ("groups_by_width", C.c_int64 * 4)]


EXPORTS = ("vbq_abi_version", "vbq_status_string", "vbq_pack_query", "vbq_pack", "vbq_matrix_check",
           "vbq_gemv", "vbq_gemv_batched", "vbq_gemv_batched_static", "vbq_gemv_levels", "vbq_gemm",
           "cell_requant_verify", "cell_drift_bound", "vbq_residual_error", "vbq_gemv_cell8", "cell8_encode",
           "cell8_decode")


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
    lib.vbq_gemv_batched_static.restype = C.c_int
    lib.vbq_gemv_batched_static.argtypes = [I32, C.POINTER(vbq_matrix), C.POINTER(C.c_void_p),
                                            C.POINTER(C.c_void_p), I32, P]
    lib.vbq_gemv_levels.restype = C.c_int
    lib.vbq_gemv_levels.argtypes = [I32, C.POINTER(vbq_matrix), P, I32, P, P]
    lib.vbq_gemm.restype = C.c_int
    lib.vbq_gemm.argtypes = [C.POINTER(vbq_matrix), P, I32, P, P]
    lib.cell_requant_verify.restype = C.c_int
    lib.cell_requant_verify.argtypes = [C.POINTER(vbq_matrix), P, P, P, P]
    lib.cell_drift_bound.restype = C.c_int
    lib.cell_drift_bound.argtypes = [C.POINTER(vbq_matrix), P, I32, P, P]
    lib.vbq_residual_error.restype = C.c_int
    lib.vbq_residual_error.argtypes = [C.POINTER(vbq_matrix), P, P, P]
    lib.vbq_gemv_cell8.restype = C.c_int
    lib.vbq_gemv_cell8.argtypes = [C.POINTER(vbq_matrix), P, I32, P, P, P]
    lib.cell8_encode.restype = C.c_int
    lib.cell8_encode.argtypes = [C.POINTER(vbq_matrix), P, P, P]
    lib.cell8_decode.restype = C.c_int
    lib.cell8_decode.argtypes = [C.POINTER(vbq_matrix), P, P, P]
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


def _need(t, what: str, dtype, shape, device=None):
    """Raises ValueError unless t is a contiguous tensor of this dtype and
    shape (on `device` when given, else on a GPU)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{what}: expected a torch tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{what}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: not contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{what}: on {t.device}, expected {device}")
    if device is None and t.device.type != "cuda":
        raise ValueError(f"{what}: on {t.device}, expected a GPU tensor")


def _rows2(x):
    return x if x.dim() == 2 else x.view(1, -1)


def abi_version() -> int:
    return lib.vbq_abi_version()


def pack_query(widths) -> vbq_layout_sizes:
    """Host-only sizing of the layout for uint8 widths [N][K/64] (numpy)."""
    w = np.ascontiguousarray(widths, dtype=np.uint8)
    if w.ndim != 2:
        raise ValueError(f"widths: expected [N][K/64], got shape {w.shape}")
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
        self.desc = vbq_matrix(self.N, self.K, sizes.n_tiles, sizes.n_bytes16,
                               self.tiles.data_ptr(), self.stream.data_ptr())

    @property
    def device(self):
        return self.stream.device

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
    if not isinstance(W, torch.Tensor) or W.dim() != 2:
        raise ValueError("W: expected a 2-D torch tensor")
    N, K = W.shape
    _need(W, "W", torch.float32, (N, K))
    widths_np = widths.cpu().numpy() if isinstance(widths, torch.Tensor) else np.asarray(widths)
    widths_np = np.ascontiguousarray(widths_np, dtype=np.uint8)
    if K % GROUP or widths_np.shape != (N, K // GROUP):
        raise ValueError(f"widths: shape {widths_np.shape}, expected {(N, K // GROUP)} for W {tuple(W.shape)}")
    sizes = pack_query(widths_np)
    pm = PackedMatrix(N, K, sizes, device=W.device)
    wd = torch.from_numpy(widths_np).to(W.device)
    st = lib.vbq_pack(_ptr(W), _ptr(wd), C.byref(pm.desc), _stream(stream))
    _check(st, "vbq_pack")
    if check:
        _check(lib.vbq_matrix_check(C.byref(pm.desc), _stream(stream)), "vbq_matrix_check")
    pm._keep = (W, wd)
    return pm


def vbq_gemv(pm: PackedMatrix, x, residual=None, out=None, stream=None):
    """y [B][N] float32 = x [B][K] (fp16) . (dequant(W) + residual)^T."""
    import torch
    x2 = _rows2(x)
    B = x2.shape[0]
    _need(x2, "x", torch.float16, (B, pm.K), pm.device)
    if not 1 <= B <= MAX_BATCH:
        raise ValueError(f"x: batch {B} outside 1..{MAX_BATCH}")
    if residual is not None:
        _need(residual, "residual", torch.float16, (pm.N, pm.K), pm.device)
    if out is None:
        out = torch.empty(B, pm.N, dtype=torch.float32, device=x.device)
    _need(out, "out", torch.float32, (B, pm.N), pm.device)
    st = lib.vbq_gemv(C.byref(pm.desc), _ptr(x2), B, _ptr(residual), _ptr(out), _stream(stream))
    _check(st, "vbq_gemv")
    return out


def vbq_gemv_cell8(pm: PackedMatrix, x, cell, out=None, stream=None):
    """y [B][N] float32 = x [B][K] (fp16) . (dequant(W) + s * cell / 256)^T,
    cell int8 [N][K] (the compact in-cell residual)."""
    import torch
    x2 = _rows2(x)
    B = x2.shape[0]
    _need(x2, "x", torch.float16, (B, pm.K), pm.device)
    if not 1 <= B <= MAX_BATCH:
        raise ValueError(f"x: batch {B} outside 1..{MAX_BATCH}")
    _need(cell, "cell", torch.int8, (pm.N, pm.K), pm.device)
    if out is None:
        out = torch.empty(B, pm.N, dtype=torch.float32, device=x.device)
    _need(out, "out", torch.float32, (B, pm.N), pm.device)
    _check(lib.vbq_gemv_cell8(C.byref(pm.desc), _ptr(x2), B, _ptr(cell), _ptr(out), _stream(stream)),
           "vbq_gemv_cell8")
    return out


def cell8_encode(pm: PackedMatrix, residual, out=None, stream=None):
    """int8 [N][K] fractions f = clamp(rint(r / s * 256), -127, 127) of an fp16
    residual, with the scales of the packed matrix."""
    import torch
    _need(residual, "residual", torch.float16, (pm.N, pm.K), pm.device)
    if out is None:
        out = torch.empty(pm.N, pm.K, dtype=torch.int8, device=residual.device)
    _need(out, "out", torch.int8, (pm.N, pm.K), pm.device)
    _check(lib.cell8_encode(C.byref(pm.desc), _ptr(residual), _ptr(out), _stream(stream)), "cell8_encode")
    return out


def cell8_decode(pm: PackedMatrix, cell, out=None, stream=None):
    """fp16 [N][K] residual fp16(s * f / 256) of int8 fractions f."""
    import torch
    _need(cell, "cell", torch.int8, (pm.N, pm.K), pm.device)
    if out is None:
        out = torch.empty(pm.N, pm.K, dtype=torch.float16, device=cell.device)
    _need(out, "out", torch.float16, (pm.N, pm.K), pm.device)
    _check(lib.cell8_decode(C.byref(pm.desc), _ptr(cell), _ptr(out), _stream(stream)), "cell8_decode")
    return out


class CellUpdate:
    """An in-cell update served beside a frozen packed matrix (CellFill
    abstract: the release's codes and scales stay untouched, and dropping the
    residual revokes the update). Holds the matrix and the update's fraction
    bytes; gemv() calls vbq_gemv_cell8 while the update is applied and
    vbq_gemv (the release) once it is revoked. Nothing in the matrix changes
    either way, so revoke() and apply() can alternate freely."""

    def __init__(self, pm: PackedMatrix, cell):
        import torch
        _need(cell, "cell", torch.int8, (pm.N, pm.K), pm.device)
        self.pm, self.cell, self.applied = pm, cell, True

    @classmethod
    def from_residual(cls, pm: PackedMatrix, residual, stream=None) -> "CellUpdate":
        """Encodes an fp16 residual with the matrix's scales (cell8_encode)."""
        return cls(pm, cell8_encode(pm, residual, stream=stream))

    def revoke(self):
        self.applied = False

    def apply(self):
        self.applied = True

    def gemv(self, x, out=None, stream=None):
        if self.applied:
            return vbq_gemv_cell8(self.pm, x, self.cell, out=out, stream=stream)
        return vbq_gemv(self.pm, x, out=out, stream=stream)

    def residual(self, stream=None):
        """The fp16 residual the fraction bytes stand for (cell8_decode)."""
        return cell8_decode(self.pm, self.cell, stream=stream)

    def verify(self, stream=None):
        """cell_requant_verify of the decoded residual: (mismatches,
        out_of_cell, first_bad_index, None)."""
        return cell_requant_verify(self.pm, self.residual(stream=stream), stream=stream)


def vbq_gemv_batched(pms, xs, ys=None, stream=None, static=False):
    """One launch for several independent GEMVs (same batch size). With
    static=True it calls vbq_gemv_batched_static, which allocates nothing and
    gives every k-tile of a long matrix a workgroup of its own."""
    import torch
    name = "vbq_gemv_batched_static" if static else "vbq_gemv_batched"
    n = len(pms)
    if not 1 <= n <= MAX_LAUNCH_MATS or len(xs) != n or (ys is not None and len(ys) != n):
        raise ValueError(f"{name}: {n} matrices, {len(xs)} inputs (1..{MAX_LAUNCH_MATS} each)")
    x2s = [_rows2(x) for x in xs]
    B = x2s[0].shape[0]
    for pm, x in zip(pms, x2s):
        _need(x, "x", torch.float16, (B, pm.K), pm.device)
    if ys is None:
        ys = [torch.empty(B, pm.N, dtype=torch.float32, device=x.device) for pm, x in zip(pms, x2s)]
    for pm, y in zip(pms, ys):
        _need(y, "y", torch.float32, (B, pm.N), pm.device)
    descs = (vbq_matrix * n)(*[pm.desc for pm in pms])
    xp = (C.c_void_p * n)(*[x.data_ptr() for x in x2s])
    yp = (C.c_void_p * n)(*[y.data_ptr() for y in ys])
    _check(getattr(lib, name)(n, descs, xp, yp, B, _stream(stream)), name)
    return ys


class GemvPlan:
    """Pre-marshalled argument block of vbq_gemv_batched (or, with
    static=True, vbq_gemv_batched_static), for timing loops (the tensors are
    checked once, here)."""

    def __init__(self, pms, xs, ys, static=False):
        import torch
        n = len(pms)
        if not 1 <= n <= MAX_LAUNCH_MATS:
            raise ValueError(f"GemvPlan: {n} matrices (1..{MAX_LAUNCH_MATS})")
        self.n = n
        self.B = xs[0].shape[0]
        for pm, x, y in zip(pms, xs, ys):
            _need(x, "x", torch.float16, (self.B, pm.K), pm.device)
            _need(y, "y", torch.float32, (self.B, pm.N), pm.device)
        self.descs = (vbq_matrix * n)(*[pm.desc for pm in pms])
        self.xp = (C.c_void_p * n)(*[x.data_ptr() for x in xs])
        self.yp = (C.c_void_p * n)(*[y.data_ptr() for y in ys])
        self._keep = (pms, xs, ys)
        self.name = "vbq_gemv_batched_static" if static else "vbq_gemv_batched"
        self._fn = getattr(lib, self.name)

    def launch(self, stream_handle):
        st = self._fn(self.n, self.descs, self.xp, self.yp, self.B, stream_handle)
        if st != 0:
            raise VbqError(st, self.name)


def vbq_gemm(pm: PackedMatrix, x_bf16, out=None, stream=None):
    """y [M][N] float32 = x [M][K] (bf16) . bf16(dequant(W))^T on MFMA."""
    import torch
    if not isinstance(x_bf16, torch.Tensor) or x_bf16.dim() != 2:
        raise ValueError("x: expected a 2-D torch tensor")
    M = x_bf16.shape[0]
    _need(x_bf16, "x", torch.bfloat16, (M, pm.K), pm.device)
    if out is None:
        out = torch.empty(M, pm.N, dtype=torch.float32, device=x_bf16.device)
    _need(out, "out", torch.float32, (M, pm.N), pm.device)
    _check(lib.vbq_gemm(C.byref(pm.desc), _ptr(x_bf16), M, _ptr(out), _stream(stream)), "vbq_gemm")
    return out


def cell_requant_verify(pm: PackedMatrix, residual, requant_codes: bool = False, stream=None):
    """Returns (mismatches, out_of_cell, first_bad_index, re-quantised stream tensor or None)."""
    import torch
    _need(residual, "residual", torch.float16, (pm.N, pm.K), pm.device)
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
    x2 = _rows2(x)
    B = x2.shape[0]
    _need(x2, "x", torch.float16, (B, pm.K), pm.device)
    if not 1 <= B <= MAX_BATCH:
        raise ValueError(f"x: batch {B} outside 1..{MAX_BATCH}")
    if out is None:
        out = torch.empty(B, pm.N, dtype=torch.float32, device=x.device)
    _need(out, "out", torch.float32, (B, pm.N), pm.device)
    _check(lib.cell_drift_bound(C.byref(pm.desc), _ptr(x2), B, _ptr(out), _stream(stream)), "cell_drift_bound")
    return out


def vbq_residual_error(pm: PackedMatrix, E, out=None, stream=None):
    """E - dequant(W) in binary32 (N x K float32): what the next residual level quantises."""
    import torch
    _need(E, "E", torch.float32, (pm.N, pm.K), pm.device)
    if out is None:
        out = torch.empty_like(E)
    _need(out, "out", torch.float32, (pm.N, pm.K), pm.device)
    _check(lib.vbq_residual_error(C.byref(pm.desc), _ptr(E), _ptr(out), _stream(stream)), "vbq_residual_error")
    return out


def rrq_pack(W, n_levels: int, stream=None):
    """Recurrent residual levels of W: a 2-bit base and n_levels - 1 2-bit
    levels, each packed from the error the levels before it leave."""
    import torch
    _need(W, "W", torch.float32, tuple(W.shape))
    widths = np.full((W.shape[0], W.shape[1] // GROUP), 2, np.uint8)
    E = W
    levels = []
    for i in range(n_levels):
        pm = vbq_pack(E, widths, stream=stream)
        levels.append(pm)
        if i + 1 < n_levels:
            E = vbq_residual_error(pm, E, stream=stream)
    return levels


def vbq_gemv_levels(pms, x, out=None, stream=None):
    """y [B][N] float32 = sum over levels of x . dequant(W_i)^T, one launch."""
    import torch
    n = len(pms)
    if not 1 <= n <= MAX_LAUNCH_MATS:
        raise ValueError(f"vbq_gemv_levels: {n} levels (1..{MAX_LAUNCH_MATS})")
    x2 = _rows2(x)
    B = x2.shape[0]
    _need(x2, "x", torch.float16, (B, pms[0].K), pms[0].device)
    if any((pm.N, pm.K) != (pms[0].N, pms[0].K) for pm in pms):
        raise ValueError("vbq_gemv_levels: levels of different shapes")
    descs = (vbq_matrix * n)(*[pm.desc for pm in pms])
    if out is None:
        out = torch.empty(B, pms[0].N, dtype=torch.float32, device=x.device)
    _need(out, "out", torch.float32, (B, pms[0].N), pms[0].device)
    _check(lib.vbq_gemv_levels(n, descs, _ptr(x2), B, _ptr(out), _stream(stream)), "vbq_gemv_levels")
    return out
