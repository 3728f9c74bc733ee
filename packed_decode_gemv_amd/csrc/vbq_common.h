// Internal definitions shared by the HIP sources of the library (not public).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vbq.h"

namespace vbq {

constexpr int kGroup = VBQ_GROUP;
constexpr int kTile = VBQ_TILE_ROWS;
constexpr int kTileGroups = VBQ_TILE_GROUPS;
constexpr int kWave = 64;

// Error flags in the totals entry of the tile table.
constexpr uint32_t kFlagInvalidWidth = 1u;
constexpr uint32_t kFlagCapacity = 2u;
constexpr uint32_t kFlagTileSize = 4u;

__host__ __device__ inline int row_tiles(int N) { return (N + kTile - 1) / kTile; }
__host__ __device__ inline int k_tiles(int G) { return (G + kTileGroups - 1) / kTileGroups; }

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__host__ __device__ inline int class_of_width(int b) {
  return b == 1 ? 0 : b == 2 ? 1 : b == 4 ? 2 : b == 8 ? 3 : -1;
}

// ---- Block geometry of the byte stream ------------------------------------
// Records per block of width class c. A wavefront decodes one block at a time,
// lane L taking the code bytes [L * cb, (L + 1) * cb) of the block with
// cb = 32, 16, 32, 16 for c = 0..3: four 1-bit records, one 2-bit record, one
// 4-bit record, or a quarter of an 8-bit record.
__host__ __device__ constexpr uint32_t block_records(int c) { return c == 0 ? 256u : c == 3 ? 16u : 64u; }
__host__ __device__ constexpr uint32_t up16(uint32_t v) { return (v + 15u) & ~15u; }
__host__ __device__ constexpr uint32_t codes_area(int c, uint32_t m) { return c == 0 ? up16(8u * m) : (8u << c) * m; }
__host__ __device__ constexpr uint32_t so_area(uint32_t m) { return up16(4u * m); }
__host__ __device__ constexpr uint32_t meta_area(uint32_t m) { return up16(2u * m); }
__host__ __device__ constexpr uint32_t block_bytes(int c, uint32_t m) {
  return codes_area(c, m) + so_area(m) + meta_area(m);
}
// Bytes of class segment c holding n records: full blocks, then the rest.
__host__ __device__ inline uint64_t seg_bytes(int c, uint64_t n) {
  const uint32_t br = block_records(c);
  const uint64_t full = n / br, rem = n - full * br;
  return full * block_bytes(c, br) + (rem ? block_bytes(c, (uint32_t)rem) : 0u);
}
__host__ __device__ inline uint64_t tile_bytes(uint32_t n0, uint32_t n1, uint32_t n2, uint32_t n3) {
  return seg_bytes(0, n0) + seg_bytes(1, n1) + seg_bytes(2, n2) + seg_bytes(3, n3);
}
__host__ __device__ inline uint32_t seg_blocks(int c, uint32_t n) {
  return (n + block_records(c) - 1) / block_records(c);
}

// ---- Device helpers shared by the kernels -----------------------------------
// s_waitcnt immediate that waits until at most n vector-memory operations of
// the wavefront are outstanding (and for nothing else).
#define VBQ_VMCNT_IMM(n) (((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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
// Completion is tracked by the explicit load-count waits instead. The
// instruction has no register result, so nothing is left pending in registers.
__device__ inline void dma16(const u32x4& rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// Host-side launch helpers.
hipError_t launch_pack(const float* W, const uint8_t* widths, const vbq_matrix& m, hipStream_t s);

// One matrix of a GEMV launch. Its workgroups are laid out k-tile column by
// k-tile column: workgroup j of the matrix takes column kt = j / wg_per_col and
// row-tiles [rt0, rt0 + rt_per_wg) with rt0 = (j % wg_per_col) * rt_per_wg.
struct GemvMat {
  const uint32_t* tiles;
  const uint8_t* stream;
  const uint16_t* x;       // [B][K] fp16
  const uint16_t* resid;   // [N][K] fp16 or null
  float* y;                // [B][N]
  float* part;             // [KT][B][N] partial rows (k_tiles > 1), else null
  uint32_t* counters;      // [wg_per_col] arrival counts (k_tiles > 1), zero between calls
  int32_t n_rows;
  int32_t n_groups;        // K / 64
  int32_t row_tiles;       // ceil(N / 16)
  int32_t k_tiles;         // ceil(G / 64)
  int32_t rt_per_wg;       // row-tiles per workgroup
  int32_t wg_per_col;      // workgroups per k-tile column
  int32_t wg_begin;        // first workgroup index of this matrix in the launch
  uint32_t stream_bytes;   // size of the stream, for the buffer range checks
};

constexpr int kMaxMats = 32;   // matrices per launch (about 3 KiB of kernel arguments)
constexpr int kMaxWgTiles = 64;   // tiles of one workgroup (one per lane)

struct GemvLaunch {
  GemvMat mats[kMaxMats];
  int32_t n_mats;
  int32_t rt_per_wg;       // largest row-tiles per workgroup (LDS row sums)
  uint32_t ring_bytes;     // LDS ring of each wavefront (multiple of 1024)
};
static_assert(sizeof(GemvLaunch) <= 4096, "kernel arguments are limited to 4 KiB");

// x of one k-tile in LDS: pairs of a k-group take 32 dwords plus 4 of padding,
// so neighbouring k-groups start 144 bytes apart, which spreads lanes that read
// different k-groups over the LDS banks while every read keeps an immediate
// offset; plus 4 bias constants and the sum per k-group.
constexpr int kXStride = 36;
constexpr int kXBytesPerGroup = kXStride * 4 + 5 * 4;

int gemv_waves(int nb);
int gemv_wgs_per_cu(int nb);
hipError_t launch_gemv(const GemvLaunch& L, int nb, bool resid, int n_wg, size_t lds, hipStream_t s);
size_t gemv_lds_bytes(int nb, int rt_per_wg, uint32_t ring_bytes);
uint32_t gemv_ring_min_bytes();

hipError_t launch_verify(const vbq_matrix& m, const uint16_t* resid, uint64_t* result, uint32_t* requant,
                         hipStream_t s);
hipError_t launch_residual_error(const vbq_matrix& m, const float* E_in, float* E_out, hipStream_t s);
hipError_t launch_sum_levels(const float* parts, int count, size_t n, float* y, hipStream_t s);
hipError_t launch_drift(const vbq_matrix& m, const uint16_t* x, int B, float* bound, hipStream_t s);
hipError_t launch_gemm(const vbq_matrix& m, const uint16_t* x, int M, float* y, hipStream_t s);

}  // namespace vbq
