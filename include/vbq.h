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
 *     re-quantisation, revocation by dropping the residual, bounded drift:
 *     page "Nothing Changed but the Model: CellFill -- Bounded In-Cell
 *     Learning for Bit-Identical, Revocable Updates to Quantized LLMs",
 *     section Abstract.
 *
 * Conventions for every call:
 *   - Ownership: the caller allocates and frees every buffer it passes. The
 *     library allocates nothing, keeps no state between calls (apart from
 *     cached device attributes) and needs no workspace: partial sums stay
 *     on-chip inside a workgroup. The calls can therefore be captured into a
 *     HIP graph as they are. Buffers marked "device" live in GPU memory of
 *     the current HIP device; "host" buffers are ordinary CPU memory.
 *   - Asynchrony: compute calls enqueue work on `stream` and return without
 *     waiting. Argument errors are found before anything is enqueued: the
 *     call returns a non-zero vbq_status and enqueues nothing. A failed kernel
 *     launch returns VBQ_ERR_HIP. No C++ exception crosses this boundary.
 *   - fp16 and bf16 values are passed as their 16-bit patterns (uint16_t).
 *   - Calls that share output buffers must not overlap in time.
 *   - Results of the GEMV calls are identical from run to run for the same
 *     inputs and shapes (fixed summation order; nothing depends on timing).
 *
 * Execution layout of a packed matrix (see vbq_matrix). The pages give no
 * layout; this one fills every block of 64 records of one width and makes
 * the byte position of every record a closed form of its tile's header, so
 * a kernel can issue all of a tile's loads at once and give each lane one
 * record of any column.
 *   Tiles. The matrix is cut into tiles of VBQ_TILE_ROWS = 32 rows by
 *   VBQ_TILE_GROUPS = 64 k-groups (4096 columns), stored k-tile major: tile
 *   t = kt * RT + rt covers rows 32 rt .. 32 rt + R - 1 and k-groups
 *   64 kt .. 64 kt + G_t - 1, with RT = ceil(N / 32), KT = ceil(K / 4096),
 *   R = min(32, N - 32 rt), G_t = min(64, K/64 - 64 kt). Column l < G_t of a
 *   tile is its k-group 64 kt + l; r < R is its row 32 rt + r.
 *   Width class c = 0, 1, 2, 3 for b = 1, 2, 4, 8.
 *   Records. The groups of class c of a tile are numbered e = 0 .. N_c - 1
 *   in column-major order: column l ascending and, within a column, its
 *   rows of class c ascending. Record e of class c is entry e % 64 of block
 *   e / 64 of the class; block k holds m_k = min(64, N_c - 64 k) records.
 *   A tile's bytes are, in order (every area starts 16-byte aligned and is
 *   zero-padded to a multiple of 16 bytes):
 *     map   : for l < G_t, 8 bytes at 8 l: u32 plane0 then u32 plane1, where
 *             bit r of plane0 is (class of group (r, l)) & 1 and bit r of
 *             plane1 is (class of group (r, l)) >> 1, for r < R (higher bits
 *             zero). These are the 2 bits of width per group.
 *     blocks: for c = 0, 1, 2, 3 and k = 0 .. ceil(N_c / 64) - 1, block
 *             (c, k):
 *               codes area: entry j's 2b u32 words at byte 8 b j;
 *               so area   : entry j's u32 at byte 4 j, fp16 scale in bits
 *                           0-15 and fp16 offset in bits 16-31.
 *   A full block takes 512 b + 256 bytes, so with C_c the byte (from the
 *   tile's start) where class c's first block begins, record e of class c
 *   has its codes at C_c + (e / 64)(512 b + 256) + 8 b (e % 64) and its
 *   scale/offset word at C_c + (e / 64)(512 b + 256) + up16(8 b m) +
 *   4 (e % 64), m being its block's record count; C_0 is the map's size and
 *   C_(c+1) = C_c + (bytes of class c's blocks).
 *   Record words: with h = 16/b, the pair p = (code 2p, code 2p+1), p < 32,
 *   sits in word p/h: code 2p at bit (p%h)*b (LSB first) and code 2p+1 at
 *   bit 16 + (p%h)*b.
 *   The tiles follow each other in storage order in one byte stream.
 *   tiles[4t..4t+3] = { first 16-byte unit of tile t, its size in 16-byte
 *   units, N_0 | N_1 << 16, N_2 | N_3 << 16 }. Entry t = n_tiles holds
 *   { total 16-byte units, invalid-width count, error flags, 0 }.
 */
#ifndef VBQ_H
#define VBQ_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VBQ_ABI_VERSION 4
#define VBQ_GROUP 64          /* weights per quantisation group (along K) */
#define VBQ_TILE_ROWS 32      /* rows per layout tile */
#define VBQ_TILE_GROUPS 64    /* k-groups (of 64 weights) per layout tile */
#define VBQ_MAX_GROUPS 4095   /* K / 64 must not exceed this */
#define VBQ_MAX_BATCH 8       /* largest batch of the GEMV calls */
#define VBQ_MAX_LAUNCH_MATS 32 /* matrices per batched call */

typedef enum vbq_status {
  VBQ_OK = 0,
  VBQ_ERR_INVALID_ARG = 1,   /* null pointer or bad count */
  VBQ_ERR_SHAPE = 2,         /* N < 1, K < 64, K % 64 != 0, K/64 > VBQ_MAX_GROUPS, M < 1, mismatched shapes */
  VBQ_ERR_BITWIDTH = 3,      /* a width not in {1,2,4,8} */
  VBQ_ERR_ALIGNMENT = 4,     /* a buffer not aligned as documented */
  VBQ_ERR_UNSUPPORTED = 5,   /* batch out of range, or a size the kernels do not take */
  VBQ_ERR_CAPACITY = 6,      /* the layout does not match the buffers it was given */
  VBQ_ERR_HIP = 7            /* a HIP runtime call or kernel launch failed */
} vbq_status;

/* Descriptor of caller-owned device buffers holding one packed matrix.
 * Sizes come from vbq_pack_query; vbq_pack fills the buffers. */
typedef struct vbq_matrix {
  int32_t n_rows;      /* N, output features */
  int32_t n_cols;      /* K, input features, multiple of 64 */
  int64_t n_tiles;     /* ceil(N / 32) * ceil(K / 4096) */
  int64_t n_bytes16;   /* size of `stream` in 16-byte units, at most 2^27 - 1 (2 GiB - 16 bytes) */
  uint32_t* tiles;     /* device, (n_tiles + 1) * 4 words, 16-byte aligned */
  uint32_t* stream;    /* device, n_bytes16 * 4 words, 16-byte aligned */
} vbq_matrix;

/* Sizes of the buffers of a packed matrix, plus accounting figures. */
typedef struct vbq_layout_sizes {
  int64_t n_tiles;
  int64_t n_records;         /* N * K / 64 (one record per group) */
  int64_t n_bytes16;
  int64_t max_tile_bytes16;
  int64_t code_bits;         /* sum over groups of 64 * width: bits of codes proper */
  int64_t groups_by_width[4]; /* number of groups of width 1, 2, 4, 8 */
} vbq_layout_sizes;

/* ABI version (VBQ_ABI_VERSION of the built library). */
int vbq_abi_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char* vbq_status_string(int status);

/* Host-only sizing of the execution layout (VBQ abstract: one width per
 * 64-weight group). widths_host: host, N x K/64 uint8 in natural (row,
 * k-group) order. out: host. Returns VBQ_ERR_SHAPE or VBQ_ERR_BITWIDTH on bad
 * input, VBQ_ERR_UNSUPPORTED for a stream above 2 GiB - 16 bytes. Touches no
 * GPU. */
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

/* Fused dequantise-and-multiply (VBQ abstract: a kernel that dequantises and
 * multiplies in one pass, for memory-bandwidth-bound decode):
 *   y[b][n] = sum_k x[b][k] * (s*q + o + r[n][k])     (r only if residual != NULL)
 * accumulated in fp32; codes are never expanded in memory. The sum over a
 * tile's 4096 columns is formed first; several k-tiles (and the residual's
 * part) are then added in a fixed order inside one workgroup.
 * x: device, B x K fp16, 16-byte aligned. B in [1, VBQ_MAX_BATCH].
 * residual: device, N x K fp16 row-major (natural order), 16-byte aligned, or
 *   NULL. NULL serves the released artifact; the in-cell update (CellFill
 *   abstract) is revoked simply by passing NULL.
 * y: device, B x N float32, 4-byte aligned; fully overwritten.
 * Batches run as passes of at most 4 rows (2 with a residual); each code is
 * decoded once per pass and multiplied with every row of the pass. */
vbq_status vbq_gemv(const vbq_matrix* m, const uint16_t* x, int32_t B, const uint16_t* residual, float* y,
                    hipStream_t stream);

/* Compact in-cell residual (CellFill abstract, page "Nothing Changed but the
 * Model: CellFill -- Bounded In-Cell Learning for Bit-Identical, Revocable
 * Updates to Quantized LLMs": the update is a residual inside each weight's
 * rounding cell, served beside the frozen artifact and revoked by dropping
 * it). The page fixes no storage for the residual; this library's compact
 * form is one signed byte f per weight in [-127, 127], standing for
 *   r[n][k] = s[n][g] * f[n][k] / 256        (g = k / 64, s the fp16 scale)
 * so |r| <= 127/256 s < s/2: every encodable residual is inside its cell.
 *
 * vbq_gemv_cell8: y[b][n] = sum_k x[b][k] * (s*q + o + s*f/256), fp32
 *   accumulation, the residual term of each (row, group) added to the
 *   group's record term before the tile's row sums. Arguments as vbq_gemv;
 *   cell: device, N x K int8 row-major (natural order), 16-byte aligned,
 *   not NULL (the base weights are vbq_gemv with residual NULL).
 * cell8_encode: f = clamp(rint(f32(r / s) * 256), -127, 127) per weight in
 *   binary32 (IEEE division, ties to even), f = 0 where s = 0; residuals
 *   beyond the cell clamp to its edge. residual: device, N x K fp16 (finite
 *   values), 16-byte aligned; cell: device, N x K int8, 16-byte aligned,
 *   fully overwritten.
 * cell8_decode: r = fp16(s * f / 256) (exact before the one rounding), the
 *   fp16 residual that vbq_gemv and cell_requant_verify take. cell and
 *   residual as above; residual fully overwritten.
 * Scales come from the packed matrix m, so the residual follows the scales
 * that are served. */
vbq_status vbq_gemv_cell8(const vbq_matrix* m, const uint16_t* x, int32_t B, const int8_t* cell, float* y,
                          hipStream_t stream);
vbq_status cell8_encode(const vbq_matrix* m, const uint16_t* residual, int8_t* cell, hipStream_t stream);
vbq_status cell8_decode(const vbq_matrix* m, const int8_t* cell, uint16_t* residual, hipStream_t stream);

/* Several independent GEMVs in one launch (same batch B, no residual; VBQ
 * abstract, fused dequantise-and-multiply): y_i = x_i . dequant(W_i)^T for
 * i < count <= VBQ_MAX_LAUNCH_MATS. ms, xs, ys: host arrays of `count`
 * entries (descriptors and device pointers as for vbq_gemv). Used to run all
 * projections of a decoder layer as one launch. */
vbq_status vbq_gemv_batched(int32_t count, const vbq_matrix* ms, const uint16_t* const* xs, float* const* ys,
                            int32_t B, hipStream_t stream);

/* vbq_gemv_batched for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation), spread
 * over more workgroups: every k-tile of a matrix with K > 4096 gets a
 * workgroup of its own, and the row sums of a row-tile's k-tiles meet in a
 * scratch area the library keeps in static device memory (one copy per
 * device, 1 MiB of partial sums and 16384 row-tile counters, held until the
 * process ends; nothing is allocated per call). The workgroup that finishes
 * a row-tile's last k-tile adds the partial sums in k-tile order, the order
 * vbq_gemv_batched uses, so both calls give the same bits, and sets the
 * row-tile's counter back to zero. Arguments and results as for
 * vbq_gemv_batched. A launch needing more than the scratch holds (more than
 * 8192 tiles of such matrices at one batch row, 8192 / min(B, 4) at B rows) returns
 * VBQ_ERR_UNSUPPORTED before anything is enqueued. Calls that overlap in
 * time on one device race on the scratch and must not be made; a call whose
 * kernels do not complete can leave counters behind for the next call. */
vbq_status vbq_gemv_batched_static(int32_t count, const vbq_matrix* ms, const uint16_t* const* xs,
                                   float* const* ys, int32_t B, hipStream_t stream);

/* GEMV over several levels of one weight matrix (RRQ abstract on page
 * thelatestinai.com/papers/2512.18934: a 2-bit base plus 2-bit residual
 * levels served from one checkpoint), in one launch:
 *   y[b][n] = sum over levels i of x[b] . dequant(W_i)[n]
 * (the levels' k-tiles are summed in a fixed order, fp32)
 * ms: host array of `count` <= VBQ_MAX_LAUNCH_MATS descriptors of equal N
 * and K (else VBQ_ERR_SHAPE). x: device, B x K fp16 (B = 1..8), 16-byte
 * aligned. y: device, B x N float32, 4-byte aligned, fully overwritten. */
vbq_status vbq_gemv_levels(int32_t count, const vbq_matrix* ms, const uint16_t* x, int32_t B, float* y,
                           hipStream_t stream);

/* Batched dequantise-and-multiply for M >= 64 tokens (VBQ abstract: the fused
 * dequantise-and-multiply, here for many tokens at once): tiles of W are
 * decoded to bf16 in LDS and contracted on MFMA with fp32 accumulation.
 *   y[m][n] = sum_k x[m][k] * bf16(fma(s, q, o))
 * where fma is the binary32 fused multiply-add (one rounding of s*q + o) and
 * bf16 rounds to nearest even. Any M >= 1 is accepted; the path pays off from
 * about 64 tokens. x_bf16: device, M x K bfloat16, 16-byte aligned, with
 * M * K * 2 < 2^32 (else VBQ_ERR_UNSUPPORTED). y: device, M x N float32,
 * 16-byte aligned, fully overwritten. */
vbq_status vbq_gemm(const vbq_matrix* m, const uint16_t* x_bf16, int32_t M, float* y, hipStream_t stream);

/* Re-quantisation check of an in-cell update (CellFill abstract: the
 * release's codes and scales stay frozen, the residual stays inside each
 * weight's cell, and re-quantising gives back the released codes exactly).
 * For every weight, in binary32 without contraction, with s, o, r the fp16
 * values and L = 2^b - 1 of the weight's group:
 *   deq = f32(s*q) + o;  v = deq + r;
 *   q'  = s == 0 ? 0 : clamp(rint((v - o) / s), 0, L)
 *   mismatch    when q' != q
 *   out of cell when s > 0 ? |r| >= 0.5*s : r != 0
 * Scales and offsets are frozen (carried through unchanged).
 * residual: device, N x K fp16 natural order, 16-byte aligned.
 * result: device, 3 x uint64, 8-byte aligned: { mismatches, out-of-cell
 *   count, smallest linear index n*K + k with either, or UINT64_MAX }.
 * requant_codes: device, same size as m->stream (16-byte aligned), receives a
 *   copy of the stream with every code replaced by its re-quantised value
 *   (map, scales, offsets and padding copied), so the artifact can be
 *   compared bit-for-bit; may be NULL. */
vbq_status cell_requant_verify(const vbq_matrix* m, const uint16_t* residual, uint64_t* result,
                               uint32_t* requant_codes, hipStream_t stream);

/* The error a packed level leaves (RRQ abstract on page
 * thelatestinai.com/papers/2512.18934: each residual level quantises what the
 * levels before it leave):
 *   E_out[n][k] = E_in[n][k] - (f32(s*q) + o)
 * in binary32, one rounding per operation; the next level is vbq_pack of
 * E_out. E_in, E_out: device, N x K float32 natural order, 8-byte aligned;
 * E_out may be E_in. Every width is accepted. */
vbq_status vbq_residual_error(const vbq_matrix* m, const float* E_in, float* E_out, hipStream_t stream);

/* Drift bound of an in-cell update (CellFill abstract: bounded drift). For
 * every residual with each |r[n][k]| below half its group's scale,
 *   |y_r[b][n] - y[b][n]| = |sum_k x[b][k] r[n][k]| <= bound[b][n], where
 *   bound[b][n] = 0.5 * sum_g s[n][g] * sum_{k in g} |x[b][k]|
 * with s the stored fp16 scales. It is computed in binary32 (each group's
 * |x| sum in k order; groups added in a fixed order), so repeated calls agree
 * bit for bit. It is the supremum: r = sign(x) s/2 attains it.
 * x: device, B x K fp16 (B = 1..8, else VBQ_ERR_UNSUPPORTED), 16-byte aligned.
 * bound: device, B x N float32, 4-byte aligned, fully overwritten. */
vbq_status cell_drift_bound(const vbq_matrix* m, const uint16_t* x, int32_t B, float* bound, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* VBQ_H */
