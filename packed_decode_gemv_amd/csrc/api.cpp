// C ABI entry points: argument checks, sizing and kernel dispatch.
// Every check happens before anything is enqueued; no C++ exception leaves
// these functions, and nothing here allocates device memory.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "vbq_common.h"

using namespace vbq;

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Largest stream, in 16-byte units: 2 GiB - 16 bytes.
constexpr int64_t kMaxStream16 = 0x07FFFFFFll;

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
  // Stream byte offsets are 32-bit on the device, and offsets from 2 GiB up
  // are the GEMV's "no record" loads.
  if (m->n_bytes16 < 1) return VBQ_ERR_CAPACITY;
  if (m->n_bytes16 > kMaxStream16) return VBQ_ERR_UNSUPPORTED;
  if (!m->tiles || !m->stream) return VBQ_ERR_INVALID_ARG;
  if (!aligned(m->tiles, 16) || !aligned(m->stream, 16)) return VBQ_ERR_ALIGNMENT;
  return VBQ_OK;
}

vbq_status from_hip(hipError_t e) { return e == hipSuccess ? VBQ_OK : VBQ_ERR_HIP; }

int cu_count() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Bytes of one tile from the widths (host): the same rules the pack kernel
// and the GEMV follow (see vbq.h).
uint64_t host_tile_bytes(const uint8_t* widths, int N, int G, int rt, int kt, bool* bad) {
  const int r0 = rt * kTileRows, R = std::min(kTileRows, N - r0);
  const int g0 = kt * kTileGroups, Gt = std::min(kTileGroups, G - g0);
  uint32_t n[4] = {0, 0, 0, 0};
  for (int r = 0; r < R; ++r)
    for (int l = 0; l < Gt; ++l) {
      const int c = class_of_width(widths[(int64_t)(r0 + r) * G + g0 + l]);
      if (c < 0) {
        *bad = true;
        return 0;
      }
      n[c]++;
    }
  uint64_t bytes = map_bytes((uint32_t)Gt);
  for (int c = 0; c < 4; ++c) bytes += class_bytes(c, n[c]);
  return bytes;
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
  int64_t bytes = 0, bits = 0, byw[4] = {0, 0, 0, 0}, max_b = 0;
  for (int64_t i = 0; i < (int64_t)N * G; ++i) {
    const int c = class_of_width(widths_host[i]);
    if (c < 0) return VBQ_ERR_BITWIDTH;
    byw[c]++;
    bits += 64 * (int64_t)widths_host[i];
  }
  for (int kt = 0; kt < KT; ++kt)
    for (int rt = 0; rt < RT; ++rt) {
      bool bad = false;
      const int64_t tb = (int64_t)host_tile_bytes(widths_host, N, G, rt, kt, &bad);
      if (bad) return VBQ_ERR_BITWIDTH;
      bytes += tb;
      max_b = std::max(max_b, tb / 16);
    }
  if (bytes / 16 > kMaxStream16) return VBQ_ERR_UNSUPPORTED;
  out->n_tiles = (int64_t)RT * KT;
  out->n_records = (int64_t)N * G;
  out->n_bytes16 = bytes / 16;
  out->max_tile_bytes16 = max_b;
  out->code_bits = bits;
  for (int c = 0; c < 4; ++c) out->groups_by_width[c] = byw[c];
  return VBQ_OK;
}

vbq_status vbq_pack(const float* W, const uint8_t* widths, const vbq_matrix* m, hipStream_t stream) {
  if (!W || !widths) return VBQ_ERR_INVALID_ARG;
  vbq_status st = check_matrix(m);
  if (st != VBQ_OK) return st;
  if (!aligned(W, 16)) return VBQ_ERR_ALIGNMENT;
  if (m->n_tiles > 0x7FFFFFFFll) return VBQ_ERR_UNSUPPORTED;
  return from_hip(launch_pack(W, widths, *m, stream));
}

vbq_status vbq_matrix_check(const vbq_matrix* m, hipStream_t stream) {
  vbq_status st = check_matrix(m);
  if (st != VBQ_OK) return st;
  uint32_t tot[4] = {0, 0, 0, 0};
  if (hipMemcpyAsync(tot, m->tiles + 4 * m->n_tiles, sizeof(tot), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return VBQ_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return VBQ_ERR_HIP;
  if (tot[2] & kFlagInvalidWidth) return VBQ_ERR_BITWIDTH;
  if (tot[2] & kFlagCapacity) return VBQ_ERR_CAPACITY;
  if ((int64_t)tot[0] != m->n_bytes16) return VBQ_ERR_CAPACITY;
  return VBQ_OK;
}

// One GEMV launch sequence: `count` matrices (independent outputs), or with
// levels > 1 one output summed over `count` levels, or one matrix with a
// residual (fp16 per weight, or int8 cell fractions). Batches above two rows
// run as passes of up to two rows.
static vbq_status gemv_impl(int32_t count, const vbq_matrix* ms, const uint16_t* const* xs, const uint16_t* resid,
                            const int8_t* cell, float* const* ys, int32_t B, bool levels, hipStream_t stream,
                            bool split = false) {
  if (count < 1 || count > kMaxMats || !ms || !xs || !ys) return VBQ_ERR_INVALID_ARG;
  if (B < 1 || B > VBQ_MAX_BATCH) return VBQ_ERR_UNSUPPORTED;
  if ((resid || cell) && (count != 1 || levels)) return VBQ_ERR_INVALID_ARG;
  if (resid && cell) return VBQ_ERR_INVALID_ARG;
  for (int i = 0; i < count; ++i) {
    vbq_status st = check_matrix(&ms[i]);
    if (st != VBQ_OK) return st;
    if (!xs[i] || !ys[i]) return VBQ_ERR_INVALID_ARG;
    if (!aligned(xs[i], 16) || !aligned(ys[i], 4)) return VBQ_ERR_ALIGNMENT;
    if (levels && (ms[i].n_rows != ms[0].n_rows || ms[i].n_cols != ms[0].n_cols)) return VBQ_ERR_SHAPE;
  }
  if (resid && !aligned(resid, 16)) return VBQ_ERR_ALIGNMENT;
  if (cell && !aligned(cell, 16)) return VBQ_ERR_ALIGNMENT;
  const int mode = resid ? kModeResid16 : cell ? kModeCell8 : levels ? kModeLevelPairs : kModePlain;
  const int max_nb = (mode == kModePlain || mode == kModeLevelPairs) ? kGemvMaxNb : kGemvMaxNbResid;
  float* partials = nullptr;
  uint32_t* counters = nullptr;
  if (split) {
    // Every matrix with several tiles per row-tile takes a slot of partial
    // sums per tile and a counter per row-tile in the scratch.
    int64_t units = 0, ctrs = 0;
    for (int i = 0; i < count; ++i) {
      const int KT = k_tiles(ms[i].n_cols / kGroup);
      if (KT > 1) {
        units += (int64_t)row_tiles(ms[i].n_rows) * KT;
        ctrs += row_tiles(ms[i].n_rows);
      }
    }
    if (units * std::min(B, max_nb) * kTileRows > (int64_t)kScratchPartials || ctrs > (int64_t)kScratchCounters)
      return VBQ_ERR_UNSUPPORTED;
    if (gemv_scratch(&partials, &counters) != hipSuccess) return VBQ_ERR_HIP;
  }
  for (int b0 = 0; b0 < B; b0 += max_nb) {
    const int nb = std::min(max_nb, B - b0);
    GemvLaunch L;
    memset(&L, 0, sizeof(L));
    L.partials = partials;
    L.counters = counters;
    // Matrices whose workgroups share a row-tile (several k-tiles) take the
    // first workgroups: each of those does more work, so it starts first.
    int order[kMaxMats], no = 0;
    for (int pass = 0; pass < 2; ++pass)
      for (int i = 0; i < count; ++i) {
        const bool shared = levels || resid || k_tiles(ms[i].n_cols / kGroup) > 1;
        if (shared == (pass == 0)) order[no++] = i;
      }
    if (levels) {
      for (int i = 0; i < count; ++i) order[i] = i;   // levels stay together, in order
    }
    int64_t wg = 0, unit = 0, ctr = 0;
    for (int pos = 0; pos < count; ++pos) {
      const int i = order[pos];
      const vbq_matrix& m = ms[i];
      GemvMat& g = L.mats[pos];
      const int G = m.n_cols / kGroup;
      g.tiles = m.tiles;
      g.stream = reinterpret_cast<const uint8_t*>(m.stream);
      g.x = xs[i] + (size_t)b0 * m.n_cols;
      g.resid = resid;
      g.cell = cell;
      g.y = (levels ? ys[0] : ys[i]) + (size_t)b0 * m.n_rows;
      g.n_rows = m.n_rows;
      g.n_groups = G;
      g.row_tiles = row_tiles(m.n_rows);
      g.k_tiles = k_tiles(G);
      g.shared = (levels || resid || g.k_tiles > 1) ? 1 : 0;
      g.levels = (levels && pos == 0) ? count : 1;
      g.stream_bytes = (uint32_t)(m.n_bytes16 * 16);
      g.wg_begin = (int32_t)wg;
      g.split = (split && g.k_tiles > 1) ? 1 : 0;
      g.unit_base = (int32_t)unit;
      g.ctr_base = (int32_t)ctr;
      if (g.split) {
        wg += (int64_t)g.row_tiles * g.k_tiles;
        unit += (int64_t)g.row_tiles * g.k_tiles;
        ctr += g.row_tiles;
      } else if (!levels || pos == 0) {
        wg += g.row_tiles;
      }
    }
    if (wg > 0x7FFFFFFF) return VBQ_ERR_UNSUPPORTED;
    L.n_mats = count;
    for (int i = 0; i < kMaxMats; ++i) L.wg_begin[i] = i < count ? L.mats[i].wg_begin : INT32_MAX;
    if (launch_gemv(L, nb, mode, (int)wg, stream) != hipSuccess) return VBQ_ERR_HIP;
  }
  return VBQ_OK;
}

vbq_status vbq_gemv(const vbq_matrix* m, const uint16_t* x, int32_t B, const uint16_t* residual, float* y,
                    hipStream_t stream) {
  return gemv_impl(1, m, &x, residual, nullptr, &y, B, false, stream);
}

vbq_status vbq_gemv_cell8(const vbq_matrix* m, const uint16_t* x, int32_t B, const int8_t* cell, float* y,
                          hipStream_t stream) {
  if (!cell) return VBQ_ERR_INVALID_ARG;
  return gemv_impl(1, m, &x, nullptr, cell, &y, B, false, stream);
}

vbq_status cell8_encode(const vbq_matrix* m, const uint16_t* residual, int8_t* cell, hipStream_t stream) {
  vbq_status st = check_matrix(m);
  if (st != VBQ_OK) return st;
  if (!residual || !cell) return VBQ_ERR_INVALID_ARG;
  if (!aligned(residual, 16) || !aligned(cell, 16)) return VBQ_ERR_ALIGNMENT;
  return from_hip(launch_cell8_encode(*m, residual, cell, stream));
}

vbq_status cell8_decode(const vbq_matrix* m, const int8_t* cell, uint16_t* residual, hipStream_t stream) {
  vbq_status st = check_matrix(m);
  if (st != VBQ_OK) return st;
  if (!residual || !cell) return VBQ_ERR_INVALID_ARG;
  if (!aligned(residual, 16) || !aligned(cell, 16)) return VBQ_ERR_ALIGNMENT;
  return from_hip(launch_cell8_decode(*m, cell, residual, stream));
}

vbq_status vbq_gemv_batched(int32_t count, const vbq_matrix* ms, const uint16_t* const* xs, float* const* ys,
                            int32_t B, hipStream_t stream) {
  return gemv_impl(count, ms, xs, nullptr, nullptr, ys, B, false, stream);
}

vbq_status vbq_gemv_batched_static(int32_t count, const vbq_matrix* ms, const uint16_t* const* xs,
                                   float* const* ys, int32_t B, hipStream_t stream) {
  return gemv_impl(count, ms, xs, nullptr, nullptr, ys, B, false, stream, true);
}

vbq_status vbq_gemv_levels(int32_t count, const vbq_matrix* ms, const uint16_t* x, int32_t B, float* y,
                           hipStream_t stream) {
  if (count < 1 || count > kMaxMats || !ms || !x || !y) return VBQ_ERR_INVALID_ARG;
  std::vector<const uint16_t*> xs(count, x);
  std::vector<float*> ys(count, y);
  return gemv_impl(count, ms, xs.data(), nullptr, nullptr, ys.data(), B, true, stream);
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

vbq_status vbq_residual_error(const vbq_matrix* m, const float* E_in, float* E_out, hipStream_t stream) {
  vbq_status st = check_matrix(m);
  if (st != VBQ_OK) return st;
  if (!E_in || !E_out) return VBQ_ERR_INVALID_ARG;
  if (!aligned(E_in, 8) || !aligned(E_out, 8)) return VBQ_ERR_ALIGNMENT;
  return from_hip(launch_residual_error(*m, E_in, E_out, stream));
}

vbq_status cell_drift_bound(const vbq_matrix* m, const uint16_t* x, int32_t B, float* bound, hipStream_t stream) {
  vbq_status st = check_matrix(m);
  if (st != VBQ_OK) return st;
  if (!x || !bound) return VBQ_ERR_INVALID_ARG;
  if (B < 1 || B > VBQ_MAX_BATCH) return VBQ_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(bound, 4)) return VBQ_ERR_ALIGNMENT;
  return from_hip(launch_drift(*m, x, B, bound, stream));
}

}  // extern "C"
