// Batched dequantise-and-multiply on the matrix cores (many tokens at once).
//
// The fused dequantise-and-multiply of the VBQ abstract (page "In-Cell
// Learning: Language Models That Update Their Own Weights in Sequence Without
// Changing the File They Ship") for a batch of M tokens: with enough tokens
// the product is compute-bound, so W is decoded on the fly to bfloat16 and
// contracted on MFMA with fp32 accumulation:
//   y[m][n] = sum_k x[m][k] * bf16(f32(s*q) + o)      (x bfloat16)
//
// A workgroup (4 wavefronts) owns 128 tokens x 128 weight rows (8 row-tiles)
// of y and walks K one 64-weight group at a time. Per group it stages
// x[128 tokens][64] and the 128 rows' decoded weights W[128 rows][64] in LDS
// (bf16, rows padded to 72 elements so the 16-byte operand reads of 16
// consecutive lanes hit disjoint banks), and each wavefront runs 2 x 2
// v_mfma_f32_32x32x16_bf16 tiles over the group: 64 tokens x 64 rows.
//
// Finding a row's record for a given k-group: the layout keeps a tile's
// records by width class, then (row, k-group). At every k-tile the workgroup
// reads the meta of all its records once and builds, per k-group, the list of
// its 128 rows' records sorted by width class (LDS, 64 KiB). The decode of a
// group then gives lane pairs consecutive entries of that list, so a
// wavefront mostly decodes a single width without divergence.
//
// The next group's x and codes are loaded into registers while the current
// group's MFMAs run; LDS is double-buffered.
#include <atomic>

#include "vbq_common.h"

namespace vbq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;              // tokens per workgroup
constexpr int kBN = 128;              // weight rows per workgroup
constexpr int kRowTilesPerWg = kBN / kTile;
constexpr int kStride = 72;           // bf16 elements per LDS row
constexpr int kThreads = 256;

struct GemmArgs {
  const uint32_t* tiles;
  const uint8_t* stream;
  const uint16_t* x;     // [M][K] bf16
  float* y;              // [M][N]
  int32_t M, N, G, RT;
  int32_t m_tiles, n_tiles;
};

struct GemmSmem {
  uint2 ent[kTileGroups][kBN];        // per k-group: {offset/8 | row << 17 | class << 24, scale|offset}
  uint32_t cnt[kTileGroups][4];       // records per (k-group, class), then placement cursors
  __bf16 xs[2][kBM][kStride];
  __bf16 ws[2][kBN][kStride];
};

__device__ inline void gemm_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): LDS traffic of this wavefront done
  __builtin_amdgcn_s_barrier();
}

// Stream position of record `idx` of class c in a tile whose class segments
// start at seg[c]: byte offsets (from the tile) of its codes and of its meta.
__device__ inline void record_offsets(int c, uint32_t idx, uint32_t n_c, uint32_t seg, uint32_t& codes,
                                      uint32_t& so, uint32_t& meta) {
  const uint32_t br = block_records(c);
  const uint32_t k = idx / br, l = idx - k * br;
  const uint32_t m = min(br, n_c - k * br);
  const uint32_t base = seg + k * block_bytes(c, br);
  codes = base + (8u << c) * l;
  so = base + codes_area(c, m) + 4u * l;
  meta = base + codes_area(c, m) + so_area(m) + 2u * l;
}

// Builds the per-k-group record lists of k-tile kt for row-tiles
// [rt0, rt0 + nrt). Offsets are relative to the first byte of tile (kt, rt0).
__device__ void build_index(const GemmArgs& a, GemmSmem& S, int kt, int rt0, int nrt, uint32_t base16, int tid) {
  for (int i = tid; i < kTileGroups * 4; i += kThreads) (&S.cnt[0][0])[i] = 0;
  gemm_barrier();
  for (int pass = 0; pass < 2; ++pass) {
    for (int r = 0; r < nrt; ++r) {
      const int t = kt * a.RT + rt0 + r;
      const uint4 h = *reinterpret_cast<const uint4*>(a.tiles + 4 * (size_t)t);
      const uint32_t n[4] = {h.z & 0xFFFFu, h.z >> 16, h.w & 0xFFFFu, h.w >> 16};
      const uint32_t tb = (h.y - base16) * 16u;   // tile start, relative
      uint32_t seg[4];
      seg[0] = tb;
      seg[1] = seg[0] + (uint32_t)seg_bytes(0, n[0]);
      seg[2] = seg[1] + (uint32_t)seg_bytes(1, n[1]);
      seg[3] = seg[2] + (uint32_t)seg_bytes(2, n[2]);
      const uint32_t total = n[0] + n[1] + n[2] + n[3];
      const uint8_t* wg_bytes = a.stream + (size_t)base16 * 16u;
      for (uint32_t i = tid; i < total; i += kThreads) {
        int c = 0;
        uint32_t idx = i;
        while (c < 3 && idx >= n[c]) {
          idx -= n[c];
          ++c;
        }
        uint32_t co, so, mo;
        record_offsets(c, idx, n[c], seg[c], co, so, mo);
        const uint32_t meta = *reinterpret_cast<const uint16_t*>(wg_bytes + mo);
        const int kgl = (int)(meta >> 4) & 63;
        if (pass == 0) {
          atomicAdd(&S.cnt[kgl][c], 1u);
        } else {
          const uint32_t sov = *reinterpret_cast<const uint32_t*>(wg_bytes + so);
          const uint32_t slot = atomicAdd(&S.cnt[kgl][c], 1u);
          const uint32_t row = (uint32_t)r * kTile + (meta & 15u);
          S.ent[kgl][slot] = make_uint2((co >> 3) | (row << 17) | ((uint32_t)c << 24), sov);
        }
      }
    }
    gemm_barrier();
    if (pass == 0) {
      if (tid < kTileGroups) {   // class c of k-group kgl starts after the narrower classes
        uint32_t s = 0;
        for (int c = 0; c < 4; ++c) {
          const uint32_t v = S.cnt[tid][c];
          S.cnt[tid][c] = s;
          s += v;
        }
      }
      gemm_barrier();
    }
  }
}

// The half (32 codes) of one record a lane decodes, as loaded from HBM.
struct CodeRegs {
  uint4 lo, hi;       // up to 8 words
  uint32_t sov;       // scale | offset << 16
  int32_t row;        // row within the workgroup, or -1
  int32_t c;          // width class
};

__device__ inline void load_codes(const GemmArgs& a, const GemmSmem& S, uint32_t base16, int kgl, int nvalid,
                                  int tid, CodeRegs& R) {
  const int slot = tid >> 1, half = tid & 1;
  R.row = -1;
  R.c = 0;
  R.lo = make_uint4(0, 0, 0, 0);
  R.hi = make_uint4(0, 0, 0, 0);
  R.sov = 0;
  if (slot >= nvalid) return;
  const uint2 e = S.ent[kgl][slot];
  R.c = (int)(e.x >> 24) & 3;
  R.row = (int)(e.x >> 17) & 127;
  R.sov = e.y;
  // half h of a record of width b is its words [h*b, h*b + b)
  const uint8_t* p = a.stream + (size_t)base16 * 16u + ((e.x & 0x1FFFFu) << 3) + (uint32_t)half * (4u << R.c);
  switch (R.c) {
    case 0: R.lo.x = *reinterpret_cast<const uint32_t*>(p); break;
    case 1: {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      R.lo.x = v.x;
      R.lo.y = v.y;
      break;
    }
    case 2: R.lo = *reinterpret_cast<const uint4*>(p); break;
    default:
      R.lo = *reinterpret_cast<const uint4*>(p);
      R.hi = *reinterpret_cast<const uint4*>(p + 16);
      break;
  }
}

__device__ inline uint32_t pack_bf16(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Word i (< 8) of the loaded half.
__device__ inline uint32_t word(const CodeRegs& R, int i) {
  const uint4& v = i < 4 ? R.lo : R.hi;
  const int j = i & 3;
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// Decodes 32 codes of width 2^C into 16 bf16 pairs (natural k order): pair p
// of the half sits in word p / H, code 2p at bit (p % H) * b, code 2p+1 at
// bit 16 + (p % H) * b.
template <int C>
__device__ inline void decode_half(const CodeRegs& R, float s, float o, uint32_t out[16]) {
  constexpr int B = 1 << C, H = 16 / B;
  constexpr uint32_t L = (1u << B) - 1u;
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    const uint32_t w = word(R, p / H);
    const int sh = (p % H) * B;
    const float q0 = (float)((w >> sh) & L);
    const float q1 = (float)((w >> (16 + sh)) & L);
    out[p] = pack_bf16(__builtin_fmaf(s, q0, o), __builtin_fmaf(s, q1, o));
  }
}

__device__ inline void store_weights(GemmSmem& S, int buf, const CodeRegs& R, int tid) {
  if (R.row < 0) return;
  const float s = __half2float(__ushort_as_half((unsigned short)(R.sov & 0xFFFFu)));
  const float o = __half2float(__ushort_as_half((unsigned short)(R.sov >> 16)));
  uint32_t out[16];
  switch (R.c) {
    case 0: decode_half<0>(R, s, o, out); break;
    case 1: decode_half<1>(R, s, o, out); break;
    case 2: decode_half<2>(R, s, o, out); break;
    default: decode_half<3>(R, s, o, out); break;
  }
  uint4* dst = reinterpret_cast<uint4*>(&S.ws[buf][R.row][32 * (tid & 1)]);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
}

struct XRegs {
  uint4 v[4];
};

__device__ inline void load_x(const GemmArgs& a, int m0, int g, int tid, XRegs& X) {
  const int row = tid >> 1, half = tid & 1;
  const int m = m0 + row;
  if (m < a.M) {
    const uint4* p = reinterpret_cast<const uint4*>(a.x + (size_t)m * (size_t)a.G * kGroup + (size_t)g * kGroup +
                                                    32 * half);
#pragma unroll
    for (int i = 0; i < 4; ++i) X.v[i] = p[i];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) X.v[i] = make_uint4(0, 0, 0, 0);
  }
}

__device__ inline void store_x(GemmSmem& S, int buf, const XRegs& X, int tid) {
  uint4* dst = reinterpret_cast<uint4*>(&S.xs[buf][tid >> 1][32 * (tid & 1)]);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = X.v[i];
}

__global__ __launch_bounds__(kThreads) void k_gemm(const GemmArgs a) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  GemmSmem& S = *reinterpret_cast<GemmSmem*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Workgroups that share weight rows (same n-tile) go to the same XCD
  // (workgroups are dealt to the 8 XCDs round-robin), so the second reads the
  // codes from that XCD's L2.
  const int total = a.m_tiles * a.n_tiles;
  int t = (int)blockIdx.x;
  if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);
  const int nt = t / a.m_tiles, mt = t - nt * a.m_tiles;
  const int m0 = mt * kBM;
  const int rt0 = nt * kRowTilesPerWg;
  const int nrt = min(kRowTilesPerWg, a.RT - rt0);
  const int nvalid = min(kBN, a.N - rt0 * kTile);

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int wm = wave >> 1, wn = wave & 1;
  uint32_t base16 = a.tiles[4 * (size_t)rt0 + 1];   // tile (0, rt0)
  build_index(a, S, 0, rt0, nrt, base16, tid);

  CodeRegs R;
  XRegs X;
  load_codes(a, S, base16, 0, nvalid, tid, R);
  load_x(a, m0, 0, tid, X);
  store_weights(S, 0, R, tid);
  store_x(S, 0, X, tid);
  gemm_barrier();

  for (int g = 0; g < a.G; ++g) {
    const int buf = g & 1;
    const bool more = g + 1 < a.G;
    if (more) {
      const int gn = g + 1;
      if ((gn & (kTileGroups - 1)) == 0) {   // next k-tile: new record lists
        const int kt = gn / kTileGroups;
        base16 = a.tiles[4 * (size_t)(kt * a.RT + rt0) + 1];
        build_index(a, S, kt, rt0, nrt, base16, tid);
      }
      load_codes(a, S, base16, gn & (kTileGroups - 1), nvalid, tid, R);
      load_x(a, m0, gn, tid, X);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        av[i] = *reinterpret_cast<const bf16x8*>(&S.xs[buf][wm * 64 + 32 * i + (lane & 31)][16 * kk + 8 * (lane >> 5)]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bv[j] = *reinterpret_cast<const bf16x8*>(&S.ws[buf][wn * 64 + 32 * j + (lane & 31)][16 * kk + 8 * (lane >> 5)]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      store_weights(S, buf ^ 1, R, tid);
      store_x(S, buf ^ 1, X, tid);
    }
    gemm_barrier();
  }

  // acc[i][j][r]: token wm*64 + 32i + 8(r/4) + 4(lane/32) + r%4, row wn*64 + 32j + lane%32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = rt0 * kTile + wn * 64 + 32 * j + (lane & 31);
      if (n >= a.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < a.M) a.y[(size_t)m * a.N + n] = acc[i][j][r];
      }
    }
}

std::atomic<uint64_t> g_gemm_attr{0};   // devices whose LDS limit is raised

}  // namespace

hipError_t launch_gemm(const vbq_matrix& m, const uint16_t* x, int M, float* y, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(g_gemm_attr.load() & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)sizeof(GemmSmem));
    if (e != hipSuccess) return e;
    g_gemm_attr.fetch_or(bit);
  }
  GemmArgs a;
  a.tiles = m.tiles;
  a.stream = reinterpret_cast<const uint8_t*>(m.stream);
  a.x = x;
  a.y = y;
  a.M = M;
  a.N = m.n_rows;
  a.G = m.n_cols / kGroup;
  a.RT = row_tiles(m.n_rows);
  a.m_tiles = (M + kBM - 1) / kBM;
  a.n_tiles = (a.RT + kRowTilesPerWg - 1) / kRowTilesPerWg;
  const int64_t n_wg = (int64_t)a.m_tiles * a.n_tiles;
  if (n_wg <= 0 || n_wg > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_gemm, dim3((unsigned)n_wg), dim3(kThreads), sizeof(GemmSmem), s, a);
  return hipGetLastError();
}

}  // namespace vbq
