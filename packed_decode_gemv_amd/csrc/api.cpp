// C ABI entry points: argument checks, sizing, workspace and kernel dispatch.
// Every check happens before anything is enqueued; no C++ exception leaves
// these functions.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "vbq_common.h"

using namespace vbq;

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

vbq_status check_shape(int32_t N, int32_t K) {
  if (N < 1 || K < kGroup || K % kGroup != 0 || K / kGroup > VBQ_MAX_GROUPS) return VBQ_ERR_SHAPE;
  return VBQ_OK;
}

// Largest possible tile: 1024 eight-bit records in full blocks of 16 plus the
// partial blocks of every class.
constexpr int64_t kMaxTileBytes16 = 8192;

vbq_status check_matrix(const vbq_matrix* m) {
  if (!m) return VBQ_ERR_INVALID_ARG;
  vbq_status st = check_shape(m->n_rows, m->n_cols);
  if (st != VBQ_OK) return st;
  const int G = m->n_cols / kGroup;
  if (m->n_tiles != (int64_t)row_tiles(m->n_rows) * k_tiles(G)) return VBQ_ERR_CAPACITY;
  if (m->n_records != (int64_t)m->n_rows * G) return VBQ_ERR_CAPACITY;
  if (m->max_tile_bytes16 < 1 || m->max_tile_bytes16 > kMaxTileBytes16) return VBQ_ERR_CAPACITY;
  // Stream byte offsets are 32-bit on the device.
  if (m->n_bytes16 < 1 || m->n_bytes16 > 0x0FFFFFFFll) return VBQ_ERR_CAPACITY;
  if (!m->tiles || !m->stream) return VBQ_ERR_INVALID_ARG;
  if (!aligned(m->tiles, 16) || !aligned(m->stream, 16)) return VBQ_ERR_ALIGNMENT;
  return VBQ_OK;
}

vbq_status from_hip(hipError_t e) { return e == hipSuccess ? VBQ_OK : VBQ_ERR_HIP; }

constexpr size_t kLdsLimit = 160 * 1024 - 64;   // dynamic LDS (a few static bytes besides)

int env_int(const char* name) {
  const char* e = getenv(name);
  return e ? std::max(0, atoi(e)) : 0;
}

// Tiles per workgroup: the launch's tiles spread over the workgroups that are
// resident at once (gemv_wgs_per_cu per CU), at most 16 per workgroup.
// VBQ_TILES_PER_WG overrides the target (tuning knob).
int tiles_per_wg(int64_t total_tiles, int slots) {
  static const int env = env_int("VBQ_TILES_PER_WG");
  if (env > 0) return std::min(env, kMaxWgTiles - 1);
  const int64_t t = (total_tiles + slots - 1) / slots;
  return (int)std::max<int64_t>(1, std::min<int64_t>(16, t));
}

// Per-wavefront LDS ring: a power of two of 1 KiB slots, as large as fits next
// to the x table and the row sums in a workgroup's share of the LDS, at most
// 16 KiB (the limit of the block descriptors). VBQ_RING_BYTES overrides it
// (rounded down to a power of two).
uint32_t pow2_floor(size_t v) {
  uint32_t p = 1;
  while ((size_t)p * 2 <= v && p < (1u << 30)) p *= 2;
  return v ? p : 0;
}

size_t wg_lds_budget(int nb) { return kLdsLimit / gemv_wgs_per_cu(nb) / 256 * 256; }

uint32_t pick_ring_bytes(int nb, int rpw) {
  static const int env = env_int("VBQ_RING_BYTES");
  if (env > 0) return pow2_floor(std::min<size_t>((size_t)env, 16384));
  const size_t fixed = gemv_lds_bytes(nb, rpw, 0), budget = wg_lds_budget(nb);
  if (fixed >= budget) return 0;
  return pow2_floor(std::min<size_t>((budget - fixed) / gemv_waves(nb), 16384));
}

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

// Device workspace per (device, stream) for matrices with K > 4096: partial
// rows, and arrival counters, one per row range. Every counter is zero
// between calls (the kernel rearms the ones it used), so counter memory is
// zeroed only when it is created. Both only grow; growing waits for the stream.
struct Buffer {
  void* base = nullptr;
  size_t bytes = 0;
};
struct Workspace {
  Buffer partials, counters;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

hipError_t grow(Buffer& b, size_t bytes, bool zero, hipStream_t stream) {
  if (b.bytes >= bytes) return hipSuccess;
  hipError_t e;
  const size_t want = std::max<size_t>(bytes, 1 << 16);
  if (b.base) {
    if ((e = hipStreamSynchronize(stream)) != hipSuccess) return e;
    if ((e = hipFree(b.base)) != hipSuccess) return e;
    b = Buffer();
  }
  if ((e = hipMalloc(&b.base, want)) != hipSuccess) return e;
  if (zero && (e = hipMemsetAsync(b.base, 0, want, stream)) != hipSuccess) {
    (void)hipFree(b.base);
    b = Buffer();
    return e;
  }
  b.bytes = want;
  return hipSuccess;
}

hipError_t workspace(hipStream_t stream, size_t partial_bytes, size_t counter_bytes, float** partials,
                     uint32_t** counters) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  Workspace& w = g_ws[{dev, stream}];
  if ((e = grow(w.partials, partial_bytes, false, stream)) != hipSuccess) return e;
  if ((e = grow(w.counters, counter_bytes, true, stream)) != hipSuccess) return e;
  *partials = static_cast<float*>(w.partials.base);
  *counters = static_cast<uint32_t*>(w.counters.base);
  return hipSuccess;
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
  int64_t bytes16 = 0, bits = 0, byw[4] = {0, 0, 0, 0}, max_b = 0, max_r = 0;
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
      const int64_t tb = (int64_t)(tile_bytes(n[0], n[1], n[2], n[3]) / 16);
      bytes16 += tb;
      max_b = std::max(max_b, tb);
      max_r = std::max<int64_t>(max_r, (int64_t)n[0] + n[1] + n[2] + n[3]);
    }
  out->n_tiles = (int64_t)RT * KT;
  out->n_records = (int64_t)N * G;
  out->n_bytes16 = bytes16;
  out->max_tile_bytes16 = max_b;
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
  if ((int64_t)tot[0] != m->n_records || (int64_t)tot[1] != m->n_bytes16) return VBQ_ERR_CAPACITY;
  return VBQ_OK;
}

static vbq_status gemv_impl(int32_t count, const vbq_matrix* ms, const uint16_t* const* xs, const uint16_t* resid,
                            float* const* ys, int32_t B, hipStream_t stream) {
  if (count < 1 || !ms || !xs || !ys) return VBQ_ERR_INVALID_ARG;
  if (B < 1 || B > VBQ_MAX_BATCH) return VBQ_ERR_UNSUPPORTED;
  if (resid && count != 1) return VBQ_ERR_INVALID_ARG;
  int64_t total_tiles = 0;
  for (int i = 0; i < count; ++i) {
    vbq_status st = check_matrix(&ms[i]);
    if (st != VBQ_OK) return st;
    if (!xs[i] || !ys[i]) return VBQ_ERR_INVALID_ARG;
    if (!aligned(xs[i], 16) || !aligned(ys[i], 4)) return VBQ_ERR_ALIGNMENT;
    total_tiles += ms[i].n_tiles;
  }
  if (resid && !aligned(resid, 16)) return VBQ_ERR_ALIGNMENT;
  // Row-tiles per workgroup, then the largest ring that fits; with a large
  // batch the row sums may have to shrink to leave room for a ring.
  int target = tiles_per_wg(total_tiles, cu_count() * gemv_wgs_per_cu(B));
  uint32_t ring = pick_ring_bytes(B, target);
  while (ring < gemv_ring_min_bytes() && target > 1) ring = pick_ring_bytes(B, --target);
  if (ring < gemv_ring_min_bytes() || gemv_lds_bytes(B, target, ring) > kLdsLimit) return VBQ_ERR_UNSUPPORTED;
  std::vector<int> rpw(count), wpc(count);
  int rpw_max = 1;
  size_t n_partials = 0, n_counters = 0;
  std::vector<size_t> p_off(count, 0), c_off(count, 0);
  for (int i = 0; i < count; ++i) {
    const int RT = row_tiles(ms[i].n_rows), KT = k_tiles(ms[i].n_cols / kGroup);
    rpw[i] = std::max(1, std::min(RT, target));
    wpc[i] = (RT + rpw[i] - 1) / rpw[i];
    rpw_max = std::max(rpw_max, rpw[i]);
    if (KT > 1) {
      p_off[i] = n_partials;
      n_partials += ((size_t)KT * B * ms[i].n_rows + 63) / 64 * 64;
      c_off[i] = n_counters;
      n_counters += ((size_t)wpc[i] + 63) / 64 * 64;
    }
  }
  const size_t lds = gemv_lds_bytes(B, rpw_max, ring);
  if (lds > kLdsLimit) return VBQ_ERR_UNSUPPORTED;
  float* partials = nullptr;
  uint32_t* counters = nullptr;
  if (n_partials > 0 && workspace(stream, n_partials * 4, n_counters * 4, &partials, &counters) != hipSuccess)
    return VBQ_ERR_HIP;
  // Split into launches of at most kMaxMats matrices.
  for (int base = 0; base < count; base += kMaxMats) {
    GemvLaunch L;
    memset(&L, 0, sizeof(L));
    const int nm = std::min(kMaxMats, count - base);
    // Matrices with several k-tiles take the first workgroups: those start
    // first, so their cross-workgroup finish overlaps the others' streaming.
    int order[kMaxMats], no = 0;
    for (int pass = 0; pass < 2; ++pass)
      for (int i = 0; i < nm; ++i)
        if ((k_tiles(ms[base + i].n_cols / kGroup) > 1) == (pass == 0)) order[no++] = i;
    int wg = 0;
    for (int pos = 0; pos < nm; ++pos) {
      const int i = order[pos];
      const vbq_matrix& m = ms[base + i];
      GemvMat& g = L.mats[pos];
      g.tiles = m.tiles;
      g.stream = reinterpret_cast<const uint8_t*>(m.stream);
      g.x = xs[base + i];
      g.resid = resid;
      g.y = ys[base + i];
      g.n_rows = m.n_rows;
      g.n_groups = m.n_cols / kGroup;
      g.row_tiles = row_tiles(m.n_rows);
      g.k_tiles = k_tiles(g.n_groups);
      g.rt_per_wg = rpw[base + i];
      g.wg_per_col = wpc[base + i];
      g.wg_begin = wg;
      g.stream_bytes = (uint32_t)(m.n_bytes16 * 16);
      if (g.k_tiles > 1) {
        g.part = partials + p_off[base + i];
        g.counters = counters + c_off[base + i];
      }
      wg += g.k_tiles * g.wg_per_col;
    }
    L.n_mats = nm;
    L.rt_per_wg = rpw_max;
    L.ring_bytes = ring;
    if (launch_gemv(L, B, resid != nullptr, wg, lds, stream) != hipSuccess) return VBQ_ERR_HIP;
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

vbq_status vbq_residual_error(const vbq_matrix* m, const float* E_in, float* E_out, hipStream_t stream) {
  vbq_status st = check_matrix(m);
  if (st != VBQ_OK) return st;
  if (!E_in || !E_out) return VBQ_ERR_INVALID_ARG;
  if (!aligned(E_in, 4) || !aligned(E_out, 4)) return VBQ_ERR_ALIGNMENT;
  return from_hip(launch_residual_error(*m, E_in, E_out, stream));
}

vbq_status vbq_gemv_levels(int32_t count, const vbq_matrix* ms, const uint16_t* x, int32_t B, float* scratch,
                           float* y, hipStream_t stream) {
  if (count < 1 || !ms || !x || !scratch || !y) return VBQ_ERR_INVALID_ARG;
  for (int i = 0; i < count; ++i) {
    vbq_status st = check_matrix(&ms[i]);
    if (st != VBQ_OK) return st;
    if (ms[i].n_rows != ms[0].n_rows || ms[i].n_cols != ms[0].n_cols) return VBQ_ERR_SHAPE;
  }
  if (B < 1 || B > VBQ_MAX_BATCH) return VBQ_ERR_UNSUPPORTED;
  if (!aligned(scratch, 4) || !aligned(y, 4)) return VBQ_ERR_ALIGNMENT;
  const size_t per = (size_t)B * (size_t)ms[0].n_rows;
  std::vector<const uint16_t*> xs(count, x);
  std::vector<float*> ys(count);
  for (int i = 0; i < count; ++i) ys[i] = scratch + (size_t)i * per;
  vbq_status st = gemv_impl(count, ms, xs.data(), nullptr, ys.data(), B, stream);
  if (st != VBQ_OK) return st;
  return from_hip(launch_sum_levels(scratch, count, per, y, stream));
}

vbq_status cell_drift_bound(const vbq_matrix* m, const uint16_t* x, int32_t B, float* bound, hipStream_t stream) {
  vbq_status st = check_matrix(m);
  if (st != VBQ_OK) return st;
  if (!x || !bound) return VBQ_ERR_INVALID_ARG;
  if (B < 1 || B > VBQ_MAX_BATCH) return VBQ_ERR_UNSUPPORTED;
  if (!aligned(x, 2) || !aligned(bound, 4)) return VBQ_ERR_ALIGNMENT;
  return from_hip(launch_drift(*m, x, B, bound, stream));
}

}  // extern "C"
