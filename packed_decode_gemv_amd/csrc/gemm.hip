// Batched dequantise-and-multiply on the matrix cores (many tokens at once).
//
// The fused dequantise-and-multiply of the VBQ abstract (page "In-Cell
// Learning: Language Models That Update Their Own Weights in Sequence Without
// Changing the File They Ship") for a batch of M tokens: with enough tokens
// the product is compute-bound, so W is decoded on the fly to bfloat16 and
// contracted on MFMA with fp32 accumulation:
//   y[m][n] = sum_k x[m][k] * bf16(fma(s, q, o))      (x bfloat16; fma rounds s*q + o once)
//
// A workgroup owns 128 tokens x 128 weight rows (8 row-tiles) of y and walks
// K one 64-weight group at a time. Four producer wavefronts load the codes
// and decode the weights; four consumer wavefronts copy x into an LDS ring
// with buffer-to-LDS loads and run the MFMAs. Per group the workgroup stages
// x[128 tokens][64] (rows XOR-swizzled by 16-byte column) and the 128 rows'
// decoded weights W[128 rows][64] in LDS (bf16, rows padded to 72 elements so
// the 16-byte operand reads of 16 consecutive lanes hit disjoint banks), and
// each consumer wavefront runs 2 x 2 v_mfma_f32_32x32x16_bf16 tiles over the
// group: 64 tokens x 64 rows.
//
// Finding a row's record for a given k-group: the layout keeps a tile's
// records by width class, then (row, k-group). At every k-tile the workgroup
// reads the meta of all its records once and builds, per k-group, the list of
// its 128 rows' records grouped by width class (LDS, 64 KiB). The decode of a
// group then gives lane pairs consecutive entries of that list, so a
// wavefront decodes one or two widths.
//
// Producers load groups into registers three ahead of the one being
// multiplied (covering the load latency) and decode into the other half of
// double-buffered LDS while the consumers run the MFMAs.
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
constexpr int kThreads = 512;           // 4 producer + 4 consumer wavefronts
constexpr int kProducers = 256;         // threads that load and decode

struct GemmArgs {
  const uint32_t* tiles;
  const uint8_t* stream;
  const uint16_t* x;     // [M][K] bf16
  float* y;              // [M][N]
  int32_t M, N, G, RT;
  int32_t m_tiles, n_tiles;
};

constexpr int kXSlots = 3;            // x of groups g, g + 1, g + 2
constexpr int kXRow = kGroup * 2;     // bytes of one token's x per group

struct GemmSmem {
  uint2 ent[kTileGroups][kBN];        // per k-group: {offset/8 | row << 17 | class << 24, scale|offset}
  uint32_t cnt[kTileGroups][4];       // records per (k-group, class), then placement cursors
  __bf16 ws[2][kBN][kStride];         // decoded weights, double-buffered
  uint8_t xs[kXSlots][kBM * kXRow];   // x rows of 128 bytes, 16-byte columns swizzled
};

// x tile of one group in LDS: token row R at R * 128 bytes, its 16-byte column
// c at position c ^ ((R >> 1) & 7). Sixteen consecutive rows read at one
// column then cover all 64 banks once (two rows per 256-byte bank cycle, eight
// column positions).
__device__ inline uint32_t x_offset(int R, int c) { return (uint32_t)R * kXRow + 16u * (uint32_t)(c ^ ((R >> 1) & 7)); }

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
// Every thread owns up to 4 records of each of the 8 tiles; all their meta and
// scale/offset loads are issued together (two memory round trips in all),
// then the lists are built in LDS: count per (k-group, class), turn counts
// into starts, place.
constexpr int kRecPerThread = kTile * kTileGroups / kThreads;   // 4 per tile

__device__ __attribute__((always_inline)) inline void build_index(const GemmArgs& a, GemmSmem& S, int kt, int rt0, int nrt,
                                                                  uint32_t base16, int tid) {
  constexpr int kHalf = kRowTilesPerWg / 2;
  for (int i = tid; i < kTileGroups * 4; i += kThreads) (&S.cnt[0][0])[i] = 0;
  const uint8_t* wg_bytes = a.stream + (size_t)base16 * 16u;
  // per record slot: tag = codes offset / 8 | row << 17 | class << 24 | k-group << 26
  uint32_t tag[kRowTilesPerWg][kRecPerThread], sov[kRowTilesPerWg][kRecPerThread];
  uint32_t valid = 0;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {   // four tiles at a time keeps the registers in flight bounded
    uint4 hdr[kHalf];
#pragma unroll
    for (int rr = 0; rr < kHalf; ++rr) {
      const int r = hh * kHalf + rr;
      hdr[rr] = r < nrt ? *reinterpret_cast<const uint4*>(a.tiles + 4 * (size_t)(kt * a.RT + rt0 + r))
                        : make_uint4(0, 0, 0, 0);
    }
    uint32_t meta[kHalf][kRecPerThread], co[kHalf][kRecPerThread], cls[kHalf][kRecPerThread];
#pragma unroll
    for (int rr = 0; rr < kHalf; ++rr) {
      const int r = hh * kHalf + rr;
      const uint4 h = hdr[rr];
      const uint32_t n[4] = {h.z & 0xFFFFu, h.z >> 16, h.w & 0xFFFFu, h.w >> 16};
      const uint32_t total = n[0] + n[1] + n[2] + n[3];
      uint32_t seg[4];
      seg[0] = (h.y - base16) * 16u;   // tile start, relative
      seg[1] = seg[0] + (uint32_t)seg_bytes(0, n[0]);
      seg[2] = seg[1] + (uint32_t)seg_bytes(1, n[1]);
      seg[3] = seg[2] + (uint32_t)seg_bytes(2, n[2]);
#pragma unroll
      for (int it = 0; it < kRecPerThread; ++it) {
        // every slot issues its two loads, a slot without a record from the
        // workgroup's first byte (always inside the stream; a row-tile past
        // the matrix has no header to take a position from), and nothing
        // reads them before all are issued
        const uint32_t i = (uint32_t)(tid + it * kThreads);
        const bool has = i < total;
        int c = 0;
        uint32_t idx = has ? i : 0u;
        while (c < 3 && idx >= n[c]) {
          idx -= n[c];
          ++c;
        }
        uint32_t so = 0, mo = 0;
        co[rr][it] = 0;
        if (has) record_offsets(c, idx, n[c], seg[c], co[rr][it], so, mo);
        meta[rr][it] = *reinterpret_cast<const uint16_t*>(wg_bytes + mo);
        sov[r][it] = *reinterpret_cast<const uint32_t*>(wg_bytes + so);
        cls[rr][it] = (uint32_t)c;
        valid |= has ? 1u << (r * kRecPerThread + it) : 0u;
      }
    }
#pragma unroll
    for (int rr = 0; rr < kHalf; ++rr)
#pragma unroll
      for (int it = 0; it < kRecPerThread; ++it) {
        const uint32_t mt = meta[rr][it];
        const uint32_t row = (uint32_t)(hh * kHalf + rr) * kTile + (mt & 15u);
        tag[hh * kHalf + rr][it] = (co[rr][it] >> 3) | (row << 17) | (cls[rr][it] << 24) | (((mt >> 4) & 63u) << 26);
      }
  }
  gemm_barrier();   // counters zeroed
#pragma unroll
  for (int r = 0; r < kRowTilesPerWg; ++r)
#pragma unroll
    for (int it = 0; it < kRecPerThread; ++it)
      if (valid >> (r * kRecPerThread + it) & 1u) atomicAdd(&S.cnt[tag[r][it] >> 26][(tag[r][it] >> 24) & 3u], 1u);
  gemm_barrier();
  if (tid < kTileGroups) {
    // Class order in a k-group's list: 8-bit, 1-bit, 2-bit, 4-bit. Producer
    // wavefronts take 32 consecutive entries each and run one decode path
    // per class they hold, so the short classes are kept apart: with the
    // usual mixes (mostly 1-bit) no wavefront holds more than two classes.
    constexpr int kOrder[4] = {3, 0, 1, 2};
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t v = S.cnt[tid][kOrder[i]];
      S.cnt[tid][kOrder[i]] = sum;
      sum += v;
    }
  }
  gemm_barrier();
#pragma unroll
  for (int r = 0; r < kRowTilesPerWg; ++r)
#pragma unroll
    for (int it = 0; it < kRecPerThread; ++it)
      if (valid >> (r * kRecPerThread + it) & 1u) {
        const uint32_t tg = tag[r][it];
        const uint32_t slot = atomicAdd(&S.cnt[tg >> 26][(tg >> 24) & 3u], 1u);
        S.ent[tg >> 26][slot] = make_uint2(tg & 0x3FFFFFFu, sov[r][it]);
      }
  gemm_barrier();
}

// The half (32 codes) of one record a lane decodes, as loaded from HBM.
struct CodeRegs {
  uint4 lo, hi;       // up to 8 words
  uint32_t sov;       // scale | offset << 16
  int32_t row;        // row within the workgroup, or -1
  int32_t c;          // width class
};

// Every thread issues the same two 16-byte loads for every group, whatever the
// width (and also for rows past N, from the workgroup's first byte), so that
// the compiler's load-count waits are exact: a wait for an older stage never
// has to assume fewer loads in flight and drain the newer ones. Reading 32
// bytes from a record's half stays inside its block: the scale/offset and meta
// areas (at least 32 bytes) follow the codes.
__device__ inline void load_codes(const GemmArgs& a, const GemmSmem& S, uint32_t base16, int kgl, int nvalid,
                                  int tid, CodeRegs& R) {
  const int slot = tid >> 1, half = tid & 1;
  uint2 e = make_uint2(0, 0);
  if (slot < nvalid) e = S.ent[kgl][slot];
  R.c = (int)(e.x >> 24) & 3;
  R.row = slot < nvalid ? (int)(e.x >> 17) & 127 : -1;
  R.sov = e.y;
  // half h of a record of width b is its words [h*b, h*b + b)
  const uint32_t off = slot < nvalid ? ((e.x & 0x1FFFFu) << 3) + (uint32_t)half * (4u << R.c) : 0u;
  const uint8_t* p = a.stream + (size_t)base16 * 16u + off;
  R.lo = *reinterpret_cast<const uint4*>(p);
  R.hi = *reinterpret_cast<const uint4*>(p + 16);
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

// One consumer wavefront copies the 32 token rows [r0, r0 + 32) of group g
// into slot `slot`: four copies of 1 KiB (eight rows each), lane l taking
// row r0 + 8i + l / 8, stored column l % 8. Rows past M read as zeros (the
// buffer ends at M rows).
constexpr int kXCopies = 4;   // copies per consumer wavefront and group

__device__ inline void copy_x(const GemmArgs& a, const u32x4& rsrc, uint32_t slot_lds, int m0, int r0, int g,
                              int lane) {
  const uint32_t K2 = (uint32_t)a.G * kXRow;   // bytes per token row of x
#pragma unroll
  for (int i = 0; i < kXCopies; ++i) {
    const int R = r0 + 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ ((R >> 1) & 7);
    dma16(rsrc, slot_lds + (uint32_t)(r0 + 8 * i) * kXRow,
          (uint32_t)(m0 + R) * K2 + (uint32_t)g * kXRow + 16u * (uint32_t)c);
  }
}

__global__ __launch_bounds__(kThreads) void k_gemm(const GemmArgs a) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  GemmSmem& S = *reinterpret_cast<GemmSmem*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool producer = wave < kProducers / kWave;   // wavefront-uniform role

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

  const int cw = wave - kProducers / kWave;   // consumer wavefront 0..3
  const int wm = (cw >> 1) & 1, wn = cw & 1;
  // Per k-tile: build the record lists, then run the pipeline over its
  // groups, one barrier per group:
  //  - producers hold the codes of groups g+1..g+3 in three register stages:
  //    they load group g + 3 and decode group g + 1 into the free weight
  //    buffer while the consumers multiply group g;
  //  - each consumer wavefront also copies a quarter of x of group g + 2
  //    into the free x slot (buffer-to-LDS, no registers) and, before the
  //    barrier, waits until its copy of group g + 1 has landed.
  // Producers issue only register loads and consumers only copies, so the
  // compiler's load-count waits in the producers are exact and the copies
  // are waited for explicitly. Every step issues the same loads (group
  // indices clamped to the k-tile's last), steps past the end only keep the
  // barrier schedule.
  const bool x_loader = !producer;
  const int xr0 = cw * 32;   // this wavefront's x rows
  const u32x4 xrsrc = make_rsrc(a.x, (uint32_t)a.M * (uint32_t)a.G * kXRow);
  const uint32_t xs_lds = lds_addr(&S.xs[0][0]);
  const int KT = (a.G + kTileGroups - 1) / kTileGroups;
  for (int kt = 0; kt < KT; ++kt) {
    const int g0 = kt * kTileGroups, g1 = min(a.G, g0 + kTileGroups);
    const uint32_t base16 = a.tiles[4 * (size_t)(kt * a.RT + rt0) + 1];
    build_index(a, S, kt, rt0, nrt, base16, tid);
    CodeRegs st0, st1, st2;
    if (producer) {
      load_codes(a, S, base16, g0 & (kTileGroups - 1), nvalid, tid, st0);
      load_codes(a, S, base16, min(g0 + 1, g1 - 1) & (kTileGroups - 1), nvalid, tid, st1);
      load_codes(a, S, base16, min(g0 + 2, g1 - 1) & (kTileGroups - 1), nvalid, tid, st2);
      store_weights(S, g0 & 1, st0, tid);
    } else if (x_loader) {
      copy_x(a, xrsrc, xs_lds + (uint32_t)(g0 % kXSlots) * kBM * kXRow, m0, xr0, g0, lane);
      copy_x(a, xrsrc, xs_lds + (uint32_t)((g0 + 1) % kXSlots) * kBM * kXRow, m0, xr0, min(g0 + 1, g1 - 1),
             lane);
      __builtin_amdgcn_s_waitcnt(VBQ_VMCNT_IMM(kXCopies));   // group g0 landed
    }
    gemm_barrier();
    auto step = [&](int g, CodeRegs& reload, const CodeRegs& next) {
      const int buf = g & 1;
      if (producer) {
        load_codes(a, S, base16, min(g + 3, g1 - 1) & (kTileGroups - 1), nvalid, tid, reload);
        if (g + 1 < g1) store_weights(S, buf ^ 1, next, tid);
      } else {
        if (g < g1) {
          // All operands of the group are read from LDS before the first
          // MFMA, so the wavefront waits for LDS once per group, not per step.
          const uint8_t* xslot = S.xs[g % kXSlots];
          bf16x8 av[4][2], bv[4][2];
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              const int R = wm * 64 + 32 * i + (lane & 31);
              av[kk][i] = *reinterpret_cast<const bf16x8*>(xslot + x_offset(R, 2 * kk + (lane >> 5)));
            }
#pragma unroll
            for (int j = 0; j < 2; ++j)
              bv[kk][j] = *reinterpret_cast<const bf16x8*>(
                  &S.ws[buf][wn * 64 + 32 * j + (lane & 31)][16 * kk + 8 * (lane >> 5)]);
          }
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
              for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[kk][i], bv[kk][j], acc[i][j], 0, 0, 0);
        }
        // The copy of group g + 2 goes out after the MFMAs are issued, so a
        // copy that waits for the memory pipeline does not hold them back;
        // its slot was last read in the previous step, before the barrier.
        if (x_loader)
          copy_x(a, xrsrc, xs_lds + (uint32_t)((g + 2) % kXSlots) * kBM * kXRow, m0, xr0, min(g + 2, g1 - 1),
                 lane);
        if (x_loader) __builtin_amdgcn_s_waitcnt(VBQ_VMCNT_IMM(kXCopies));   // group g + 1 landed
      }
      gemm_barrier();
    };
    for (int g = g0; g < g1; g += 3) {
      step(g, st0, st1);
      step(g + 1, st1, st2);
      step(g + 2, st2, st0);
    }
    if (x_loader) __builtin_amdgcn_s_waitcnt(VBQ_VMCNT_IMM(0));   // no copy left in flight
  }
  if (producer) return;

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
  if ((int64_t)M * m.n_cols * 2 >= (int64_t)1 << 32) return hipErrorNotSupported;   // x addressed with 32-bit offsets
  const int64_t n_wg = (int64_t)a.m_tiles * a.n_tiles;
  if (n_wg <= 0 || n_wg > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_gemm, dim3((unsigned)n_wg), dim3(kThreads), sizeof(GemmSmem), s, a);
  return hipGetLastError();
}

}  // namespace vbq
