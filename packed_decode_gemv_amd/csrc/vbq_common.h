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
constexpr int kBlock = 64;  // records per layout block (one per lane)

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

// Byte size of the code segment of class c holding n records.
__host__ __device__ inline uint64_t seg_bytes(int c, uint64_t n) {
  return c == 0 ? ((8 * n + 15) / 16) * 16 : n * (8ull << c);
}

// Byte size of a tile's code area.
__host__ __device__ inline uint64_t tile_code_bytes(uint32_t n0, uint32_t n1, uint32_t n2, uint32_t n3) {
  return seg_bytes(0, n0) + seg_bytes(1, n1) + seg_bytes(2, n2) + seg_bytes(3, n3);
}

// Host-side launch helpers (defined in api.cpp).
hipError_t launch_pack(const float* W, const uint8_t* widths, const vbq_matrix& m, hipStream_t s);

struct GemvMat {
  const uint32_t* tiles;
  const uint32_t* so;
  const uint16_t* meta;
  const uint32_t* codes;
  const uint16_t* x;       // [B][K] fp16
  const uint16_t* resid;   // [N][K] fp16 or null
  float* y;                // [B][N]
  int32_t n_rows;
  int32_t n_groups;        // K / 64
  int32_t row_tiles;       // ceil(N / 16)
  int32_t k_tiles;         // ceil(G / 64)
  int32_t rt_per_wg;       // row-tiles per workgroup
  int32_t wg_begin;        // first workgroup index of this matrix in the launch
  uint32_t so_bytes;       // sizes of so / meta / codes, for buffer range checks
  uint32_t meta_bytes;
  uint32_t code_bytes;
};

constexpr int kMaxMats = 8;

struct GemvLaunch {
  GemvMat mats[kMaxMats];
  int32_t n_mats;
  int32_t rt_per_wg;       // largest row-tiles per workgroup (LDS row sums)
  uint32_t ring_bytes;     // LDS ring of each wavefront (multiple of 16)
};

hipError_t launch_gemv(const GemvLaunch& L, int nb, bool resid, int n_wg, size_t lds, hipStream_t s);
size_t gemv_lds_bytes(int nb, int rt_per_wg, uint32_t ring_bytes);
uint32_t gemv_ring_min_bytes();

hipError_t launch_verify(const vbq_matrix& m, const uint16_t* resid, uint64_t* result, uint32_t* requant,
                         hipStream_t s);
hipError_t launch_gemm(const vbq_matrix& m, const uint16_t* x, int M, float* y, hipStream_t s);

}  // namespace vbq
