// Internal definitions shared by the HIP sources of the library (not public).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vbq.h"

namespace vbq {

constexpr int kGroup = VBQ_GROUP;
constexpr int kTileRows = VBQ_TILE_ROWS;
constexpr int kTileGroups = VBQ_TILE_GROUPS;
constexpr int kWave = 64;

// Error flags in the totals entry of the tile table.
constexpr uint32_t kFlagInvalidWidth = 1u;
constexpr uint32_t kFlagCapacity = 2u;

__host__ __device__ inline int row_tiles(int N) { return (N + kTileRows - 1) / kTileRows; }
__host__ __device__ inline int k_tiles(int G) { return (G + kTileGroups - 1) / kTileGroups; }

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__host__ __device__ inline int class_of_width(int b) {
  return b == 1 ? 0 : b == 2 ? 1 : b == 4 ? 2 : b == 8 ? 3 : -1;
}

// ---- Tile geometry ---------------------------------------------------------------
// A tile's map takes 8 bytes per column; a block of m records of class c
// holds m records of 8 * 2^c code bytes, then m scale/offset words, each
// area rounded up to 16 bytes. The records of class c are listed column by
// column (rows ascending) and cut into blocks of 64.
__host__ __device__ constexpr uint32_t up16(uint32_t v) { return (v + 15u) & ~15u; }
__host__ __device__ constexpr uint32_t map_bytes(uint32_t cols) { return up16(8u * cols); }
__host__ __device__ constexpr uint32_t codes_area(int c, uint32_t m) { return up16((8u << c) * m); }
__host__ __device__ constexpr uint32_t block_bytes(int c, uint32_t m) { return codes_area(c, m) + up16(4u * m); }
__host__ __device__ constexpr uint32_t full_block_bytes(int c) { return (512u << c) + 256u; }

// Bytes of the blocks of a class with n records.
__host__ __device__ inline uint32_t class_bytes(int c, uint32_t n) {
  return (n >> 6) * full_block_bytes(c) + ((n & 63u) ? block_bytes(c, n & 63u) : 0u);
}

// Records of class c in a tile, from the header's count words.
__host__ __device__ inline uint32_t class_count(uint32_t w2, uint32_t w3, int c) {
  return ((c < 2 ? w2 : w3) >> (16 * (c & 1))) & 0xFFFFu;
}

// Byte offsets (from the tile's start) of record e of a class with n records
// whose first block starts at cbase.
struct RecPos {
  uint32_t codes, so;
};
__host__ __device__ inline RecPos record_pos(int c, uint32_t n, uint32_t cbase, uint32_t e) {
  const uint32_t k = e >> 6, j = e & 63u;
  const uint32_t m = n - 64u * k < 64u ? n - 64u * k : 64u;
  const uint32_t bb = cbase + k * full_block_bytes(c);
  RecPos p;
  p.codes = bb + (8u << c) * j;
  p.so = bb + codes_area(c, m) + 4u * j;
  return p;
}

// Rows of one column per width class from the column's map planes (bit r of
// plane0 / plane1 = low / high bit of row r's class); rows >= R are empty.
struct ClassMasks {
  uint32_t m[4];
};
__host__ __device__ inline ClassMasks class_masks(uint32_t p0, uint32_t p1, int R) {
  const uint32_t valid = R >= 32 ? 0xFFFFFFFFu : ((1u << R) - 1u);
  ClassMasks k;
  k.m[0] = ~p0 & ~p1 & valid;
  k.m[1] = p0 & ~p1 & valid;
  k.m[2] = ~p0 & p1 & valid;
  k.m[3] = p0 & p1 & valid;
  return k;
}

// ---- Device helpers shared by the kernels -----------------------------------
// Sum of v over the lanes below this one (lanes of a 64-wide wavefront).
__device__ inline uint32_t wave_excl_scan(uint32_t v, uint32_t lane) {
  uint32_t s = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t u = (uint32_t)__shfl_up((int)s, d, 64);
    if (lane >= (uint32_t)d) s += u;
  }
  return s - v;
}

// Sum of v over the wavefront (every lane gets it).
__device__ inline uint32_t wave_total(uint32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += (uint32_t)__shfl_xor((int)v, d, 64);
  return v;
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// the wavefront are outstanding (and for nothing else).
#define VBQ_VMCNT_IMM(n) (((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
// s_waitcnt immediate that waits for every LDS/scalar-memory operation only.
#define VBQ_LGKMCNT0_IMM (15 | (3 << 14) | (7 << 4))

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Raw buffer descriptor (base, no stride, size in bytes): loads past `bytes`
// return zeros instead of touching memory.
__device__ inline u32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu);
  r.z = __builtin_amdgcn_readfirstlane(bytes);
  r.w = 0x00020000u;
  return r;
}

__device__ inline uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(p));
}

// Buffer-to-LDS copy: the active lane l reads 16 bytes at byte offset voff of
// the buffer and writes them to LDS address lds + 16 l. It is written as
// assembly so that the compiler does not treat it as a pending LDS store: it
// would otherwise wait for every copy in flight before any LDS read.
// Completion is tracked by explicit load-count waits instead. The
// instruction has no register result, so nothing is left pending in registers.
__device__ inline void dma16(const u32x4& rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// ---- Launch descriptions ---------------------------------------------------------
// One matrix of a GEMV launch. A launch runs one workgroup of four
// wavefronts per row-tile of each matrix; the wavefronts share each tile.
struct GemvMat {
  // the fields every workgroup needs first, in the first 64 bytes (read in
  // one scalar load)
  const uint32_t* tiles;
  const uint8_t* stream;
  const uint16_t* x;       // [B][K] fp16
  int32_t n_rows;
  int32_t n_groups;        // K / 64
  int32_t row_tiles;       // ceil(N / 32)
  int32_t k_tiles;         // ceil(G / 64)
  uint32_t stream_bytes;   // size of the stream, for the buffer range checks
  int32_t split;           // 1: a workgroup per (row-tile, tile); partial row sums meet in the scratch
  int32_t shared;          // 1: a workgroup per row-tile (k-tiles, levels or residual shared by its waves)
  int32_t levels;          // matrices summed into one output (levels), this one and the next levels-1
  int32_t unit_base;       // first partial-sum slot of this matrix in the scratch (split)
  int32_t ctr_base;        // first row-tile counter of this matrix in the scratch (split)
  // the rest
  float* y;                // [B][N]
  const uint16_t* resid;   // [N][K] fp16 or null
  const int8_t* cell;      // [N][K] compact in-cell residual fractions or null
  int32_t wg_begin;        // first workgroup of this matrix in the launch
  int32_t pad_;
};
static_assert(sizeof(GemvMat) == 96, "GemvMat layout");
constexpr int kMaxMats = VBQ_MAX_LAUNCH_MATS;
constexpr int kGemvWaves = 4;
constexpr int kGemvMaxNb = 4;   // batch rows per pass (two with a residual)
constexpr int kGemvMaxNbResid = 2;
// Residual kinds of a launch: none, fp16 per weight, int8 cell fractions;
// and residual levels of one matrix at one batch row, taken two tiles at a
// time (no residual).
constexpr int kModePlain = 0, kModeResid16 = 1, kModeCell8 = 2, kModeLevelPairs = 3;

struct GemvLaunch {
  int32_t wg_begin[kMaxMats];   // first workgroup of each matrix (non-decreasing; INT32_MAX past n_mats)
  GemvMat mats[kMaxMats];
  int32_t n_mats;
  float* partials;         // split matrices: [slot][NB][32] row sums of one tile
  uint32_t* counters;      // split matrices: tiles finished per row-tile (back to 0 when all are)
};
static_assert(sizeof(GemvLaunch) <= 4096, "kernel arguments are limited to 4 KiB");

// Host-side launch helpers.
hipError_t launch_pack(const float* W, const uint8_t* widths, const vbq_matrix& m, hipStream_t s);
hipError_t launch_gemv(const GemvLaunch& L, int nb, int mode, int n_wg, hipStream_t s);
// The scratch of the split GEMV on the current device: partial row sums and
// row-tile counters (sizes in elements).
constexpr size_t kScratchPartials = 1u << 18;   // 1 MiB of float
constexpr size_t kScratchCounters = 1u << 14;   // 64 KiB of uint32
hipError_t gemv_scratch(float** partials, uint32_t** counters);
size_t gemv_lds_bytes(int nb, int mode);
hipError_t launch_verify(const vbq_matrix& m, const uint16_t* resid, uint64_t* result, uint32_t* requant,
                         hipStream_t s);
hipError_t launch_residual_error(const vbq_matrix& m, const float* E_in, float* E_out, hipStream_t s);
hipError_t launch_cell8_encode(const vbq_matrix& m, const uint16_t* r16, int8_t* f, hipStream_t s);
hipError_t launch_cell8_decode(const vbq_matrix& m, const int8_t* f, uint16_t* r16, hipStream_t s);
hipError_t launch_drift(const vbq_matrix& m, const uint16_t* x, int B, float* bound, hipStream_t s);
hipError_t launch_gemm(const vbq_matrix& m, const uint16_t* x, int M, float* y, hipStream_t s);

}  // namespace vbq
