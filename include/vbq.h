/*
 * vbq.h -- C ABI of the packed mixed-bit weight library for MI355X (gfx950).
 *
 * The library computes y = x . W^T for a frozen weight matrix W (N x K) that
 * is stored group-quantised: every contiguous group of 64 weights along K has
 * its own bit-width b in {1, 2, 4, 8}, an fp16 scale s and an fp16 offset o,
 * and dequantises as w = s*q + o with integer code q in [0, 2^b - 1].
 *   - Per-group widths from {1,2,4,8} on 64-weight groups, packed low-bit
 *     storage and a fused dequantise-and-multiply for bandwidth-bound decode:
 *     VBQ abstract, page "In-Cell Learning: Language Models That Update Their
 *     Own Weights in Sequence Without Changing the File They Ship".
 *   - Asymmetric (scale + offset) quantisation: SLQ abstract, page
 *     thelatestinai.com/papers/2512.18934.
 *   - Per-weight residual inside each quantisation cell, bit-identical
 *     re-quantisation, revocation by dropping the residual: page "Nothing
 *     Changed but the Model: CellFill -- Bounded In-Cell Learning for
 *     Bit-Identical, Revocable Updates to Quantized LLMs", section Abstract.
 *
 * Conventions for every call:
 *   - Ownership: the caller allocates and frees every buffer it passes.
 *     Buffers marked "device" live in GPU memory of the current HIP device;
 *     "host" buffers are ordinary CPU memory. The library itself keeps, per
 *     (device, stream), one device workspace for the partial row sums and
 *     arrival counters of matrices with K > 4096 (allocated on first need,
 *     grown when a larger one is needed, kept until the process ends);
 *     nothing else. Growing it waits for the stream. Calls captured into a
 *     HIP graph must not need a new or larger workspace: make the same calls
 *     once on the capturing stream before capture.
 *   - Asynchrony: compute calls enqueue work on `stream` and return without
 *     waiting. Argument errors are found before anything is enqueued: the
 *     call returns a non-zero vbq_status and enqueues nothing. A failed kernel
 *     launch returns VBQ_ERR_HIP. No C++ exception crosses this boundary.
 *   - fp16 and bf16 values are passed as their 16-bit patterns (uint16_t).
 *   - Calls that share output buffers must not overlap in time.
 *
 * Execution layout of a packed matrix (see vbq_matrix):
 *   The matrix is cut into tiles of VBQ_TILE_ROWS = 16 rows by
 *   VBQ_TILE_GROUPS = 64 k-groups (4096 columns), stored k-tile major: tile
 *   t = kt * RT + rt covers rows 16rt.. and k-groups 64kt.., with
 *   RT = ceil(N / 16), KT = ceil(K / 4096). Inside a tile the groups are
 *   split by width class c (b = 1,2,4,8 -> c = 0..3) and, inside a class,
 *   ordered by (row ascending, k-group ascending), so that a wavefront decodes
 *   groups of a single width and neighbouring lanes share rows. Each group is
 *   a "record" with
 *     codes : 2b u32 words; with h = 16/b, the pair p = (code 2p, code 2p+1),
 *             p < 32, sits in word p/h: code 2p at bit (p%h)*b (LSB first)
 *             and code 2p+1 at bit 16 + (p%h)*b;
 *     so    : u32, fp16 scale bits 0-15, fp16 offset bits 16-31;
 *     meta  : u16, row within the tile bits 0-3, k-group within the tile
 *             bits 4-9 (bits 10-15 zero).
 *   A class segment keeps its records in blocks of 256, 64, 64, 16 records
 *   (b = 1, 2, 4, 8; a full block carries 2048, 1024, 2048, 1024 code bytes);
 *   the last block may hold fewer (m records). A block of m records is, in
 *   order:
 *     codes area: record l's 2b words at byte 8b*l, in order (for b = 1
 *                 the area is rounded up to 16 bytes);
 *     so area   : record l at byte 4l, rounded up to 16 bytes;
 *     meta area : record l at byte 2l, rounded up to 16 bytes;
 *   padding is zero. A tile is its class segments 0..3 in order, and the tiles
 *   follow each other in storage order in one byte stream, so any range of
 *   consecutive tiles is one contiguous range of bytes.
 *   tiles[4t..4t+3] = { first record of tile t, first 16-byte unit of its
 *   bytes, n0 | n1 << 16, n2 | n3 << 16 } where n_c counts its class-c
 *   records. Entry t = n_tiles holds { total records, total 16-byte units,
 *   invalid-width count, error flags }.
 */
#ifndef VBQ_H
#define VBQ_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VBQ_ABI_VERSION 2
#define VBQ_GROUP 64          /* weights per quantisation group (along K) */
#define VBQ_TILE_ROWS 16      /* rows per layout tile */
#define VBQ_TILE_GROUPS 64    /* k-groups (of 64 weights) per layout tile */
#define VBQ_MAX_GROUPS 4095   /* K / 64 must not exceed this */
#define VBQ_MAX_BATCH 8       /* largest batch of vbq_gemv */

typedef enum vbq_status {
  VBQ_OK = 0,
  VBQ_ERR_INVALID_ARG = 1,   /* null pointer or bad count */
  VBQ_ERR_SHAPE = 2,         /* N < 1, K < 64, K % 64 != 0, K/64 > VBQ_MAX_GROUPS, M < 1 */
  VBQ_ERR_BITWIDTH = 3,      /* a width not in {1,2,4,8} */
  VBQ_ERR_ALIGNMENT = 4,     /* a buffer not aligned as documented */
  VBQ_ERR_UNSUPPORTED = 5,   /* batch out of range, or the batch does not fit on-chip */
  VBQ_ERR_CAPACITY = 6,      /* the layout does not match the buffers it was given */
  VBQ_ERR_HIP = 7            /* a HIP runtime call or kernel launch failed */
} vbq_status;

/* Descriptor of caller-owned device buffers holding one packed matrix.
 * Sizes come from vbq_pack_query; vbq_pack fills the buffers. */
typedef struct vbq_matrix {
  int32_t n_rows;      /* N, output features */
  int32_t n_cols;      /* K, input features, multiple of 64 */
  int64_t n_tiles;     /* ceil(N / 16) * ceil(K / 4096) */
  int64_t n_records;   /* N * K / 64 (one record per group) */
  int64_t n_bytes16;   /* size of `stream` in 16-byte units */
  int64_t max_tile_bytes16;  /* largest tile, 16-byte units */
  uint32_t* tiles;     /* device, (n_tiles + 1) * 4 words, 16-byte aligned */
  uint32_t* stream;    /* device, n_bytes16 * 4 words, 16-byte aligned */
} vbq_matrix;

/* Sizes of the buffers of a packed matrix, plus accounting figures. */
typedef struct vbq_layout_sizes {
  int64_t n_tiles;
  int64_t n_records;
  int64_t n_bytes16;
  int64_t max_tile_bytes16;
  int64_t max_tile_records;
  int64_t code_bits;   /* sum of widths * 64: bits of codes proper */
  int64_t groups_by_width[4]; /* number of groups of width 1, 2, 4, 8 */
} vbq_layout_sizes;

/* ABI version (VBQ_ABI_VERSION of the built library). */
int vbq_abi_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char* vbq_status_string(int status);

/* Host-only sizing of the execution layout.
 * widths_host: host, N x K/64 uint8 in natural (row, k-group) order.
 * out: host. Returns VBQ_ERR_SHAPE or VBQ_ERR_BITWIDTH on bad input.
 * Touches no GPU. */
vbq_status vbq_pack_query(const uint8_t* widths_host, int32_t N, int32_t K, vbq_layout_sizes* out);

/* Quantise W and write the execution layout (offline step).
 * Quantiser, per group of 64 (VBQ abstract for the groups and widths; SLQ
 * abstract for scale + offset), in binary32 without contraction:
 *   lo = min, hi = max; scale16 = fp16(f32(hi - lo) / (2^b - 1));
 *   offset16 = fp16(lo); s, o = those fp16 values;
 *   q = s == 0 ? 0 : clamp(rint(f32(w - o) / s), 0, 2^b - 1)   (ties to even).
 * W: device, N x K float32, row-major, 16-byte aligned.
 * widths: device, N x K/64 uint8 in natural order (the same values given to
 *   vbq_pack_query for the sizes in m).
 * m: host descriptor; every field must be set from vbq_pack_query and the
 *   two device pointers. Invalid widths, or a layout that does not match the
 *   descriptor, are detected on the device: nothing is then written beyond the
 *   tile table, and vbq_matrix_check reports the error. */
vbq_status vbq_pack(const float* W, const uint8_t* widths, const vbq_matrix* m, hipStream_t stream);

/* Waits for `stream` and reads the totals entry written by vbq_pack.
 * Returns VBQ_OK, VBQ_ERR_BITWIDTH (invalid widths on the device) or
 * VBQ_ERR_CAPACITY (layout larger than the descriptor's sizes). */
vbq_status vbq_matrix_check(const vbq_matrix* m, hipStream_t stream);

/* Fused dequantise-and-multiply (VBQ abstract, "custom fused
 * dequantize-and-multiply kernels" for bandwidth-bound decode):
 *   y[b][n] = sum_k x[b][k] * (s*q + o + r[n][k])     (r only if residual != NULL)
 * accumulated in fp32; codes are never expanded in memory.
 * x: device, B x K fp16, 16-byte aligned. B in [1, VBQ_MAX_BATCH]. Each
 *   workgroup stages the 4096 columns of x of one k-tile on-chip; for
 *   matrices with K > 4096 the last workgroup of a row range to finish adds
 *   the k-tiles' partial rows (kept in the library's workspace) in k-tile
 *   order, so results are identical from run to run. Two calls that use the
 *   same stream's workspace must not run concurrently (calls on one stream
 *   never do).
 * residual: device, N x K fp16 row-major (natural order), 16-byte aligned, or
 *   NULL. NULL serves the released artifact; the in-cell update (CellFill
 *   abstract) is revoked simply by passing NULL.
 * y: device, B x N float32, 4-byte aligned; fully overwritten. */
vbq_status vbq_gemv(const vbq_matrix* m, const uint16_t* x, int32_t B, const uint16_t* residual, float* y,
                    hipStream_t stream);

/* Several independent GEMVs in one launch (same batch B, no residual):
 * y_i = x_i . W_i^T for i < count. ms, xs, ys: host arrays of `count` entries
 * (descriptors and device pointers as for vbq_gemv). Used to run all
 * projections of a decoder layer, or a whole stack, as one launch. */
vbq_status vbq_gemv_batched(int32_t count, const vbq_matrix* ms, const uint16_t* const* xs, float* const* ys,
                            int32_t B, hipStream_t stream);

/* Batched dequantise-and-multiply for M >= 64 tokens: tiles of W are decoded
 * to bf16 in LDS and contracted on MFMA with fp32 accumulation.
 *   y[m][n] = sum_k x[m][k] * bf16(fma(s, q, o))
 * where fma is the binary32 fused multiply-add (one rounding of s*q + o) and
 * bf16 rounds to nearest even. Any M >= 1 is accepted; the path pays off from
 * about 64 tokens. x_bf16: device, M x K bfloat16, 16-byte aligned, with
 * M * K * 2 < 2^32 (else VBQ_ERR_UNSUPPORTED). y: device, M x N float32,
 * 16-byte aligned, fully overwritten. */
vbq_status vbq_gemm(const vbq_matrix* m, const uint16_t* x_bf16, int32_t M, float* y, hipStream_t stream);

/* Re-quantisation check of an in-cell update (CellFill abstract: codes and
 * scales of the release frozen, residual strictly inside each cell,
 * re-quantisation returns the released artifact bit-for-bit). For every weight,
 * in binary32 without contraction, with s, o, r the fp16 values:
 *   deq = f32(s*q) + o;  v = deq + r;
 *   q'  = s == 0 ? 0 : clamp(rint((v - o) / s), 0, 2^b - 1)
 *   mismatch    when q' != q
 *   out of cell when s > 0 ? |r| >= 0.5*s : r != 0
 * Scales and offsets are frozen (carried through unchanged).
 * residual: device, N x K fp16 natural order, 16-byte aligned.
 * result: device, 3 x uint64, 8-byte aligned: { mismatches, out-of-cell
 *   count, smallest linear index n*K + k with either, or UINT64_MAX }.
 * requant_codes: device, same size as m->stream (16-byte aligned), receives a
 *   copy of the stream with every code replaced by its re-quantised value
 *   (scales, offsets, meta and padding copied), so the artifact can be
 *   compared bit-for-bit; may be NULL. */
vbq_status cell_requant_verify(const vbq_matrix* m, const uint16_t* residual, uint64_t* result,
                               uint32_t* requant_codes, hipStream_t stream);

/* Recurrent residual levels (page "Recurrent Residual Quantization",
 * section Abstract: a 2-bit base, then 2-bit RTN residual corrections that
 * give 4-, 6- and 8-bit representations from one checkpoint). A level is an
 * ordinary packed matrix (every width 2, from vbq_pack). The error it leaves:
 *   E_out[n][k] = E_in[n][k] - (f32(s*q) + o)
 * in binary32, one rounding per operation; the next level is vbq_pack of
 * E_out. E_in, E_out: device, N x K float32 natural order, 4-byte aligned;
 * E_out may be E_in. Every width is accepted. */
vbq_status vbq_residual_error(const vbq_matrix* m, const float* E_in, float* E_out, hipStream_t stream);

/* GEMV over several levels of one weight matrix (same N and K):
 *   y[b][n] = sum_i x[b] . dequant(W_i)[n]  (levels added in order, binary32)
 * x: device, B x K fp16 (B = 1..8), 16-byte aligned. scratch: device,
 * count x B x N float32 (caller-owned; the per-level outputs), 4-byte
 * aligned. y: device, B x N float32, fully overwritten. Shares the GEMV's
 * workspace rules (vbq_gemv_batched). */
vbq_status vbq_gemv_levels(int32_t count, const vbq_matrix* ms, const uint16_t* x, int32_t B, float* scratch,
                           float* y, hipStream_t stream);

/* Drift bound of an in-cell update (page "Nothing Changed but the Model:
 * CellFill -- Bounded In-Cell Learning for Bit-Identical, Revocable Updates
 * to Quantized LLMs", section Abstract: bounded drift). For every residual
 * with each |r[n][k]| below half its group's scale,
 *   |y_r[b][n] - y[b][n]| = |sum_k x[b][k] r[n][k]| <= bound[b][n], where
 *   bound[b][n] = 0.5 * sum_g s[n][g] * sum_{k in g} |x[b][k]|
 * with s the stored fp16 scales. It is computed in binary32: the group sums
 * in k order, then the groups in order, so repeated calls agree bit for bit.
 * It is the supremum: r = sign(x) s/2 attains it.
 * x: device, B x K fp16 (B = 1..8, else VBQ_ERR_UNSUPPORTED), 2-byte aligned.
 * bound: device, B x N float32, 4-byte aligned, fully overwritten. */
vbq_status cell_drift_bound(const vbq_matrix* m, const uint16_t* x, int32_t B, float* bound, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* VBQ_H */
