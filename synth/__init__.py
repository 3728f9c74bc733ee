"""Seeded synthetic inputs for the packed mixed-bit GEMV workloads.

This module only draws random numbers and describes workload shapes. It holds
none of the method's arithmetic (no quantisation, packing, dequantisation or
dot products), so that the oracle and the GPU path can both consume its
outputs without sharing any code of the method.

Workload shapes and bit-width mixes follow the variable bit-width quantisation
(VBQ) abstract (page "In-Cell Learning: Language Models That Update Their Own
Weights in Sequence Without Changing the File They Ship"): 64-weight groups
along K, widths from {1,2,4,8}, 69% of groups at 1 bit, an LM head near 1.09
mean bits, and model scales of 131M / 1.0B / 9B parameters. The in-cell
residual draw follows the CellFill abstract (page "Nothing Changed but the
Model: CellFill -- Bounded In-Cell Learning ...", section Abstract).

Every array is generated in row blocks of ``ROW_BLOCK`` rows, each block from
its own ``numpy.random.SeedSequence`` child, so any row range can be
regenerated on its own (sampled parity checks at full size) and blocks can be
generated in parallel threads.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

GROUP = 64
ROW_BLOCK = 1024

# Stream ids inside a seed key.
S_WIDTHS, S_WEIGHTS, S_X, S_RESID, S_CELL, S_SALIENCE = 0, 1, 2, 3, 4, 5

# Bit-width mixes.
MIX_DEFAULT = {1: 0.69, 2: 0.15, 4: 0.12, 8: 0.04}   # mean 1.79 bits
MIX_LM_HEAD = {1: 0.92, 2: 0.07, 4: 0.01}            # mean 1.10 bits
MIX_UNIFORM4 = {4: 1.0}
# First MLP block of a structured recipe: mean 2.52 bits.
MIX_FIRST_MLP = {1: 0.40, 2: 0.30, 4: 0.22, 8: 0.08}


def _ss(seed: int, key: tuple) -> np.random.SeedSequence:
    return np.random.SeedSequence(entropy=seed, spawn_key=tuple(int(k) for k in key))


def _blocks(n_rows: int):
    for b0 in range(0, n_rows, ROW_BLOCK):
        yield b0 // ROW_BLOCK, b0, min(n_rows, b0 + ROW_BLOCK)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill_rows(n_rows: int, row_shape: tuple, dtype, fill_block, rows=None):
    """Fill an array of ``n_rows`` rows block by block (threads over blocks)."""
    if rows is None:
        out = np.empty((n_rows,) + row_shape, dtype=dtype)
        jobs = list(_blocks(n_rows))
        if len(jobs) == 1:
            blk, r0, r1 = jobs[0]
            out[r0:r1] = fill_block(blk, r1 - r0)
        else:
            def work(j):
                blk, r0, r1 = j
                out[r0:r1] = fill_block(blk, r1 - r0)
            with ThreadPoolExecutor(_threads()) as ex:
                list(ex.map(work, jobs))
        return out
    # Only the requested rows: regenerate their blocks.
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows),) + row_shape, dtype=dtype)
    cache = {}
    for i, r in enumerate(rows):
        blk = int(r) // ROW_BLOCK
        if blk not in cache:
            r0 = blk * ROW_BLOCK
            cache[blk] = fill_block(blk, min(n_rows, r0 + ROW_BLOCK) - r0)
        out[i] = cache[blk][int(r) - blk * ROW_BLOCK]
    return out


def widths(seed: int, key: tuple, n_rows: int, n_groups: int, mix: dict, rows=None) -> np.ndarray:
    """Per-group bit-widths, iid categorical with probabilities ``mix``,
    row-major over (row, group). Returns uint8 [n_rows][n_groups]."""
    vals = np.array(sorted(mix), dtype=np.uint8)
    cum = np.cumsum([mix[v] for v in sorted(mix)])
    cum[-1] = 1.0

    def fill(blk, n):
        rng = np.random.default_rng(_ss(seed, key + (S_WIDTHS, blk)))
        u = rng.random((n, n_groups))
        return vals[np.searchsorted(cum, u, side="right").clip(0, len(vals) - 1)]
    return _fill_rows(n_rows, (n_groups,), np.uint8, fill, rows)


def structured_widths(seed: int, key: tuple, n_rows: int, n_groups: int, mix: dict, rows=None,
                      row_scale: float = 1.0, col_scale: float = 0.7) -> np.ndarray:
    """Per-group bit-widths with the fractions of ``mix`` but placed by a
    salience score, so that wide groups gather on hot rows and hot input
    channels as a learned allocation's do (the VBQ abstract reports the
    allocation as strongly heterogeneous within projection types). Each group
    (n, g) scores z = a_n + c_g + e_ng with a_n ~ row_scale * t_3 per row,
    c_g ~ col_scale * t_3 per k-group (shared by all rows) and e ~ N(0, 1);
    the groups are ranked by z over the whole matrix and the lowest share
    mix[1] of the ranks get the narrowest width, the next share the next
    width, and so on (each width's count is its share of the groups, up to
    rounding). Returns uint8 [n_rows][n_groups] (only ``rows`` if given;
    the ranking always spans the whole matrix)."""
    vals = np.array(sorted(mix), dtype=np.uint8)
    shares = np.array([mix[v] for v in sorted(mix)], np.float64)
    cg = np.random.default_rng(_ss(seed, key + (S_SALIENCE, 1 << 30))).standard_t(3, n_groups) * col_scale

    def fill(blk, n):
        rng = np.random.default_rng(_ss(seed, key + (S_SALIENCE, blk)))
        a = rng.standard_t(3, (n, 1)) * row_scale
        return (a + cg[None, :] + rng.standard_normal((n, n_groups))).astype(np.float32)
    z = _fill_rows(n_rows, (n_groups,), np.float32, fill)
    order = np.argsort(z, axis=None, kind="stable")
    counts = np.floor(np.cumsum(shares) / shares.sum() * z.size + 0.5).astype(np.int64)
    flat = np.empty(z.size, np.uint8)
    start = 0
    for v, end in zip(vals, counts):
        flat[order[start:end]] = v
        start = end
    w = flat.reshape(n_rows, n_groups)
    return w if rows is None else w[np.asarray(rows, dtype=np.int64)]


def layer_mix(layer: int, n_layers: int) -> dict:
    """Per-layer width mix of a structured recipe, in the spirit of the SLQ
    abstract's layer-wise non-uniform widths: the share of 1-bit groups is
    0.72 - 0.25 * 2^-d with d the layer's distance to the nearer end of the
    stack (so the first and last layers are the widest), and the rest is
    split 15 : 12 : 4 over 2, 4 and 8 bits as in MIX_DEFAULT. Over 32 layers
    about 69% of the groups are 1-bit."""
    d = min(layer, n_layers - 1 - layer)
    p1 = 0.72 - 0.25 * 2.0 ** (-d)
    rest = 1.0 - p1
    return {1: p1, 2: rest * 15 / 31, 4: rest * 12 / 31, 8: rest * 4 / 31}


def recipe_mix(layer: int, proj_name: str, n_layers: int) -> dict:
    """Mix of one matrix of the structured 9B-class recipe: the LM head
    (layer -1) at MIX_LM_HEAD, the first MLP block (layer 0 gate, up, down)
    at MIX_FIRST_MLP, everything else at its layer's layer_mix."""
    if layer < 0:
        return MIX_LM_HEAD
    if layer == 0 and proj_name in ("gate", "up", "down"):
        return MIX_FIRST_MLP
    return layer_mix(layer, n_layers)


def recipe_widths(layer: int, pi: int, proj, n_layers: int, rows=None) -> np.ndarray:
    """Widths of matrix (layer, pi) of the structured 9B-class recipe; the
    weights and activations of that matrix are those of workload 3."""
    return structured_widths(SEED, proj_key(5, layer, pi), proj.n, proj.k // GROUP,
                             recipe_mix(layer, proj.name, n_layers), rows=rows)


def weights(seed: int, key: tuple, n_rows: int, n_cols: int, std: float = 0.02, rows=None) -> np.ndarray:
    """Dense fp32 weights W ~ N(0, std^2), float32 [n_rows][n_cols]."""
    def fill(blk, n):
        rng = np.random.default_rng(_ss(seed, key + (S_WEIGHTS, blk)))
        a = rng.standard_normal((n, n_cols), dtype=np.float32)
        a *= np.float32(std)
        return a
    return _fill_rows(n_rows, (n_cols,), np.float32, fill, rows)


def x_f16(seed: int, key: tuple, batch: int, n_cols: int) -> np.ndarray:
    """Activations x ~ N(0,1) rounded to fp16; returned as uint16 bit patterns [batch][n_cols]."""
    rng = np.random.default_rng(_ss(seed, key + (S_X, 0)))
    a = rng.standard_normal((batch, n_cols), dtype=np.float32)
    return a.astype(np.float16).view(np.uint16)


def x_bf16(seed: int, key: tuple, batch: int, n_cols: int) -> np.ndarray:
    """Activations x ~ N(0,1) rounded to bfloat16 (round to nearest even on the
    fp32 bit pattern); returned as uint16 bit patterns [batch][n_cols]."""
    rng = np.random.default_rng(_ss(seed, key + (S_X, 0)))
    a = rng.standard_normal((batch, n_cols), dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def cell_u(seed: int, key: tuple, n_rows: int, n_cols: int, half_width: float = 0.49, rows=None) -> np.ndarray:
    """Uniform draws u ~ U(-half_width, half_width), float64 [n_rows][n_cols].
    The in-cell residual is u times the group's scale; forming it needs the
    scale, which is method arithmetic and therefore not done here."""
    def fill(blk, n):
        rng = np.random.default_rng(_ss(seed, key + (S_RESID, blk)))
        return rng.uniform(-half_width, half_width, size=(n, n_cols))
    return _fill_rows(n_rows, (n_cols,), np.float64, fill, rows)


def cell_f(seed: int, key: tuple, n_rows: int, n_cols: int, rows=None) -> np.ndarray:
    """Uniform integer draws in [-127, 127], int8 [n_rows][n_cols]: the
    fraction bytes of a compact in-cell residual, drawn directly (any byte in
    that range stands for a residual inside its cell, whatever the scale)."""
    def fill(blk, n):
        rng = np.random.default_rng(_ss(seed, key + (S_CELL, blk)))
        return rng.integers(-127, 128, size=(n, n_cols), dtype=np.int8)
    return _fill_rows(n_rows, (n_cols,), np.int8, fill, rows)


# ---------------------------------------------------------------------------
# Workload descriptions
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Proj:
    name: str
    n: int          # output features (rows of W)
    k: int          # input features (columns of W)
    mix: dict = field(default_factory=lambda: MIX_DEFAULT, hash=False, compare=False)


@dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    projs: tuple            # Proj per matrix of one layer (or the single matrix)
    layers: int = 1
    batches: tuple = (1,)
    head: Proj | None = None
    residual: bool = False
    gemm_m: int = 0         # > 0: batched dequant-GEMM with this many tokens (bf16 x)


C0 = Workload(0, "mixed-bit GEMV 768x768 (131M-class projection)",
              (Proj("proj", 768, 768),))
C1 = Workload(1, "1.0B-class decoder layer (hidden 2048, MLP 8192)",
              (Proj("qkv", 6144, 2048), Proj("o", 2048, 2048), Proj("up", 8192, 2048),
               Proj("gate", 8192, 2048), Proj("down", 2048, 8192)), batches=(1, 4))
C2 = Workload(2, "in-cell update on a uniform 4-bit release, K=4096 N=14336",
              (Proj("w", 14336, 4096, MIX_UNIFORM4),), residual=True)
C3 = Workload(3, "9B-class stack, 32 layers + LM head (hidden 4096, MLP 14336)",
              (Proj("q", 4096, 4096), Proj("k", 1024, 4096), Proj("v", 1024, 4096),
               Proj("o", 4096, 4096), Proj("gate", 14336, 4096), Proj("up", 14336, 4096),
               Proj("down", 4096, 14336)),
              layers=32, batches=(1, 4), head=Proj("lm_head", 128256, 4096, MIX_LM_HEAD))
C4 = Workload(4, "batched mixed-bit GEMM M=256 K=4096 N=14336",
              (Proj("w", 14336, 4096),), gemm_m=256)

WORKLOADS = (C0, C1, C2, C3, C4)

SEED = 0


def proj_key(cid: int, layer: int, proj_index: int) -> tuple:
    """Seed key of one matrix: (workload id, layer, projection index).
    The LM head of workload 3 uses layer index -1 mapped to 1_000_000."""
    return (cid, layer if layer >= 0 else 1_000_000, proj_index)


def mean_bits(mix: dict) -> float:
    return float(sum(b * p for b, p in mix.items()))
