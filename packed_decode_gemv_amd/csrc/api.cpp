// C ABI entry points: argument checks, sizing and kernel dispatch.
// Every check happens before anything is enqueued; no C++ exception leaves
// these functions.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "vbq_common.h"

using namespace vbq;

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

vbq_status check_shape(int32_t N, int32_t K) {
  if (N < 1 || K < kGroup || K % kGroup != 0 || K / kGroup > VBQ_MAX_GROUPS) return VBQ_ERR_SHAPE;
  return VBQ_OK;
}

vbq_status check_matrix(const vbq_matrix* m) {
  if (!m) return VBQ_ERR_INVALID_ARG;
  vbq_status st = check_shape(m->n_rows, m->n_cols);
  if (st != VBQ_OK) return st;
  const int G = m->n_cols / kGroup;
  if (m->n_tiles != (int64_t)row_tiles(m->n_rows) * k_tiles(G)) return VBQ_ERR_CAPACITY;
  if (m->max_tile_records < 1 || m->max_tile_records > (int64_t)kTile * kTileGroups) return VBQ_ERR_CAPACITY;
  if (m->max_tile_code16 < 1 || m->max_tile_code16 > (int64_t)kTile * kTileGroups * 4) return VBQ_ERR_CAPACITY;
  if (m->n_records != (int64_t)m->n_rows * (m->n_cols / kGroup)) return VBQ_ERR_CAPACITY;
  if (m->n_code16 < 1 || m->n_code16 > 0x07FFFFFFll) return VBQ_ERR_CAPACITY;   // < 2 GiB of codes
  if (m->n_records > 0x1FFFFFFFll) return VBQ_ERR_SHAPE;                           // < 2 GiB of scales
  if (!m->tiles || !m->so || !m->meta || !m->codes) return VBQ_ERR_INVALID_ARG;
  if (!aligned(m->tiles, 16) || !aligned(m->so, 4) || !aligned(m->meta, 4) || !aligned(m->codes, 16))
    return VBQ_ERR_ALIGNMENT;
  return VBQ_OK;
}

vbq_status from_hip(hipError_t e) { return e == hipSuccess ? VBQ_OK : VBQ_ERR_HIP; }

constexpr size_t kLdsLimit = 160 * 1024;


// Tiles per workgroup: x is staged once per 4096-column window per workgroup,
// so several tiles per workgroup amortise it, while the launch should still
// hold several workgroups per CU. VBQ_TILES_PER_WG overrides the target
// (tuning knob).
int target_tiles_per_wg() {
  static int env = -1;
  if (env < 0) {
    const char* e = getenv("VBQ_TILES_PER_WG");
    env = e ? std::max(0, atoi(e)) : 0;
  }
  return env > 0 ? env : 4;
}

// Per-wavefront LDS ring: as large as the budget of two workgroups per CU
// allows (80 KiB each), at least one 8-bit block.
uint32_t pick_ring_bytes(int nb, int rpw) {
  static int env = -1;
  if (env < 0) {
    const char* e = getenv("VBQ_RING_BYTES");
    env = e ? std::max(0, atoi(e)) : 0;
  }
  if (env > 0) return (uint32_t)env & ~15u;
  const size_t fixed = gemv_lds_bytes(nb, rpw, 0);
  size_t budget = 80 * 1024;
  if (fixed + 8 * (size_t)gemv_ring_min_bytes() > budget) budget = kLdsLimit;
  size_t ring = fixed < budget ? (budget - fixed) / 8 : 0;
  ring = std::min<size_t>(ring, 16384) & ~(size_t)15;
  return (uint32_t)ring;
}
}  // namespace

extern "C" {

int vbq_abi_version(void) { return VBQ_ABI_VERSION; }

const char* vbq_status_string(int s) {
  switch (s) {
    case VBQ_OK: return "ok";
    case VBQ_ERR_INVALID_ARG: return "invalid argument";
    case VBQ_ERR_SHAPE: return "bad shape";
    case VBQ_ERR_BITWIDTH: return "width not in {1,2,4,8}";
    case VBQ_ERR_ALIGNMENT: return "misaligned buffer";
    case VBQ_ERR_UNSUPPORTED: return "unsupported size";
    case VBQ_ERR_CAPACITY: return "layout does not match its buffers";
    case VBQ_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

vbq_status vbq_pack_query(const uint8_t* widths_host, int32_t N, int32_t K, vbq_layout_sizes* out) {
  if (!widths_host || !out) return VBQ_ERR_INVALID_ARG;
  vbq_status st = check_shape(N, K);
  if (st != VBQ_OK) return st;
  const int G = K / kGroup;
  const int RT = row_tiles(N), KT = k_tiles(G);
  int64_t code16 = 0, bits = 0, byw[4] = {0, 0, 0, 0}, max_c = 0, max_r = 0;
  for (int rt = 0; rt < RT; ++rt)
    for (int kt = 0; kt < KT; ++kt) {
      uint32_t n[4] = {0, 0, 0, 0};
      const int r1 = std::min((rt + 1) * kTile, N), g1 = std::min((kt + 1) * kTileGroups, G);
      for (int r = rt * kTile; r < r1; ++r)
        for (int g = kt * kTileGroups; g < g1; ++g) {
          const uint8_t w = widths_host[(int64_t)r * G + g];
          const int c = class_of_width(w);
          if (c < 0) return VBQ_ERR_BITWIDTH;
          n[c]++;
          bits += 64 * w;
        }
      for (int c = 0; c < 4; ++c) byw[c] += n[c];
      const int64_t tc = (int64_t)(tile_code_bytes(n[0], n[1], n[2], n[3]) / 16);
      code16 += tc;
      max_c = std::max(max_c, tc);
      max_r = std::max<int64_t>(max_r, (int64_t)n[0] + n[1] + n[2] + n[3]);
    }
  out->n_tiles = (int64_t)RT * KT;
  out->n_records = (int64_t)N * G;
  out->n_code16 = code16;
  out->max_tile_code16 = max_c;
  out->max_tile_records = max_r;
  out->code_bits = bits;
  for (int c = 0; c < 4; ++c) out->groups_by_width[c] = byw[c];
  return VBQ_OK;
}

vbq_status vbq_pack(const float* W, const uint8_t* widths, const vbq_matrix* m, hipStream_t stream) {
  if (!W || !widths) return VBQ_ERR_INVALID_ARG;
  vbq_status st = check_matrix(m);
  if (st != VBQ_OK) return st;
  if (!aligned(W, 16)) return VBQ_ERR_ALIGNMENT;
  return from_hip(launch_pack(W, widths, *m, stream));
}

vbq_status vbq_matrix_check(const vbq_matrix* m, hipStream_t stream) {
  vbq_status st = check_matrix(m);
  if (st != VBQ_OK) return st;
  uint32_t tot[4] = {0, 0, 0, 0};
  if (hipMemcpyAsync(tot, m->tiles + 4 * m->n_tiles, sizeof(tot), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return VBQ_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return VBQ_ERR_HIP;
  if (tot[3] & kFlagInvalidWidth) return VBQ_ERR_BITWIDTH;
  if (tot[3] & (kFlagCapacity | kFlagTileSize)) return VBQ_ERR_CAPACITY;
  if ((int64_t)tot[0] != m->n_records || (int64_t)tot[1] != m->n_code16) return VBQ_ERR_CAPACITY;
  return VBQ_OK;
}

static vbq_status gemv_impl(int32_t count, const vbq_matrix* ms, const uint16_t* const* xs, const uint16_t* resid,
                            float* const* ys, int32_t B, hipStream_t stream) {
  if (count < 1 || !ms || !xs || !ys) return VBQ_ERR_INVALID_ARG;
  if (B < 1 || B > VBQ_MAX_BATCH) return VBQ_ERR_UNSUPPORTED;
  if (resid && count != 1) return VBQ_ERR_INVALID_ARG;
  const int target = target_tiles_per_wg();
  for (int i = 0; i < count; ++i) {
    vbq_status st = check_matrix(&ms[i]);
    if (st != VBQ_OK) return st;
    if (!xs[i] || !ys[i]) return VBQ_ERR_INVALID_ARG;
    if (!aligned(xs[i], 16) || !aligned(ys[i], 4)) return VBQ_ERR_ALIGNMENT;
  }
  if (resid && !aligned(resid, 16)) return VBQ_ERR_ALIGNMENT;
  // Row-tiles per workgroup of each matrix: about `target` tiles per workgroup.
  std::vector<int> rpw(count);
  int rpw_max = 1;
  for (int i = 0; i < count; ++i) {
    const int KT = k_tiles(ms[i].n_cols / kGroup);
    rpw[i] = std::max(1, std::min(row_tiles(ms[i].n_rows), (target + KT - 1) / KT));
    rpw_max = std::max(rpw_max, rpw[i]);
  }
  const uint32_t ring = pick_ring_bytes(B, rpw_max);
  const size_t lds = gemv_lds_bytes(B, rpw_max, ring);
  if (ring < gemv_ring_min_bytes() || lds > kLdsLimit) return VBQ_ERR_UNSUPPORTED;
  // Split into launches of at most kMaxMats matrices.
  for (int base = 0; base < count; base += kMaxMats) {
    GemvLaunch L;
    memset(&L, 0, sizeof(L));
    const int nm = std::min(kMaxMats, count - base);
    int wg = 0;
    for (int i = 0; i < nm; ++i) {
      const vbq_matrix& m = ms[base + i];
      GemvMat& g = L.mats[i];
      g.tiles = m.tiles;
      g.so = m.so;
      g.meta = m.meta;
      g.codes = m.codes;
      g.x = xs[base + i];
      g.resid = resid;
      g.y = ys[base + i];
      g.n_rows = m.n_rows;
      g.n_groups = m.n_cols / kGroup;
      g.row_tiles = row_tiles(m.n_rows);
      g.k_tiles = k_tiles(g.n_groups);
      g.rt_per_wg = rpw[base + i];
      g.wg_begin = wg;
      g.so_bytes = (uint32_t)(m.n_records * 4);
      g.meta_bytes = (uint32_t)((m.n_records + 1) / 2 * 4);   // whole 4-byte words
      g.code_bytes = (uint32_t)(m.n_code16 * 16);
      wg += (g.row_tiles + g.rt_per_wg - 1) / g.rt_per_wg;
    }
    L.n_mats = nm;
    L.rt_per_wg = rpw_max;
    L.ring_bytes = ring;
    hipError_t e = launch_gemv(L, B, resid != nullptr, wg, lds, stream);
    if (e != hipSuccess) return VBQ_ERR_HIP;
  }
  return VBQ_OK;
}

vbq_status vbq_gemv(const vbq_matrix* m, const uint16_t* x, int32_t B, const uint16_t* residual, float* y,
                    hipStream_t stream) {
  return gemv_impl(1, m, &x, residual, &y, B, stream);
}

vbq_status vbq_gemv_batched(int32_t count, const vbq_matrix* ms, const uint16_t* const* xs, float* const* ys,
                            int32_t B, hipStream_t stream) {
  return gemv_impl(count, ms, xs, nullptr, ys, B, stream);
}

vbq_status vbq_gemm(const vbq_matrix* m, const uint16_t* x_bf16, int32_t M, float* y, hipStream_t stream) {
  vbq_status st = check_matrix(m);
  if (st != VBQ_OK) return st;
  if (!x_bf16 || !y) return VBQ_ERR_INVALID_ARG;
  if (M < 1) return VBQ_ERR_SHAPE;
  if (!aligned(x_bf16, 16) || !aligned(y, 16)) return VBQ_ERR_ALIGNMENT;
  hipError_t e = launch_gemm(*m, x_bf16, M, y, stream);
  if (e == hipErrorNotSupported) return VBQ_ERR_UNSUPPORTED;
  return from_hip(e);
}

vbq_status cell_requant_verify(const vbq_matrix* m, const uint16_t* residual, uint64_t* result,
                               uint32_t* requant_codes, hipStream_t stream) {
  vbq_status st = check_matrix(m);
  if (st != VBQ_OK) return st;
  if (!residual || !result) return VBQ_ERR_INVALID_ARG;
  if (!aligned(residual, 16) || !aligned(result, 8)) return VBQ_ERR_ALIGNMENT;
  if (requant_codes && !aligned(requant_codes, 16)) return VBQ_ERR_ALIGNMENT;
  return from_hip(launch_verify(*m, residual, result, requant_codes, stream));
}

}  // extern "C"
