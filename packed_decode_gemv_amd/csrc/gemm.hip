// Batched dequantise-and-multiply on the matrix cores (many tokens at once).
//
// The fused dequantise-and-multiply of the VBQ abstract (page "In-Cell
// Learning: Language Models That Update Their Own Weights in Sequence Without
// Changing the File They Ship") for a batch of M tokens: with enough tokens
// the product is compute-bound, so W is decoded on the fly to bfloat16 and
// contracted on MFMA with fp32 accumulation:
//   y[m][n] = sum_k x[m][k] * bf16(fma(s, q, o))      (x bfloat16; fma rounds s*q + o once)
//
// A workgroup owns 256 tokens x 64 weight rows (4 row-tiles) of y and walks K
// one 64-weight group at a time, so at up to 256 tokens every weight is
// decoded once. Four producer wavefronts load the codes and decode the
// weights; four consumer wavefronts copy x into an LDS ring with
// buffer-to-LDS loads and run the MFMAs. Per group the workgroup stages
// x[256 tokens][64] (rows XOR-swizzled by 16-byte column) and the 64 rows'
// decoded weights W[64 rows][64] in LDS (bf16, rows padded to 72 elements so
// the 16-byte operand reads of 16 consecutive lanes hit disjoint banks), and
// each consumer wavefront runs 2 x 2 v_mfma_f32_32x32x16_bf16 tiles over the
// group: its 64 tokens x the 64 rows.
//
// Finding a row's record for a given k-group: the workgroup's 64 rows are two
// layout tiles. At every k-tile the workgroup reads the two tiles' width maps,
// counts the records per (k-group, width), walks the tiles' blocks (lane l on
// column l, which gives each record's row) and builds, per k-group, the list
// of its 64 rows' records grouped by width class (LDS, 32 KiB); then it loads
// every listed record's scale/offset at once. The decode of a group then gives
// four consecutive lanes one entry of that list (a quarter of the record
// each, 16 codes), so a wavefront decodes one or two widths.
// A quarter decodes without per-code conversions where the width is small:
// a 1- or 2-bit record has only 2 or 4 distinct weights, computed once as
// bf16(fma(s, q, o)) and looked up per code pair with a byte permute; 4- and
// 8-bit codes are spread to bytes and converted with the byte-to-float
// conversions.
//
// Producers load groups into registers four ahead of the one being
// multiplied (covering the load latency) and decode into the other half of
// double-buffered LDS while the consumers run the MFMAs.
#include <atomic>

#include "vbq_common.h"

namespace vbq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 256;              // tokens per workgroup
constexpr int kBN = 64;               // weight rows per workgroup
constexpr int kRowTilesPerWg = kBN / kTileRows;
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
  uint32_t cnt[kRowTilesPerWg][kTileGroups][4];   // records per (row-tile, k-group, class)
  __bf16 ws[2][kBN][kStride];         // decoded weights, double-buffered
  uint8_t xs[kXSlots][kBM * kXRow];   // x rows of 128 bytes, 16-byte columns swizzled
};

static_assert(sizeof(GemmSmem) <= 160 * 1024, "LDS of one workgroup");

// x tile of one group in LDS: token row R at R * 128 bytes, its 16-byte column
// c at position c ^ ((R >> 1) & 7). Sixteen consecutive rows read at one
// column then cover all 64 banks once (two rows per 256-byte bank cycle, eight
// column positions).
__device__ inline uint32_t x_offset(int R, int c) { return (uint32_t)R * kXRow + 16u * (uint32_t)(c ^ ((R >> 1) & 7)); }

__device__ inline void gemm_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): LDS traffic of this wavefront done
  __builtin_amdgcn_s_barrier();
}

// Builds the per-k-group record lists of k-tile kt for row-tiles
// [rt0, rt0 + nrt). Code offsets are relative to the first byte of tile
// (kt, rt0) (the two tiles are consecutive in the stream).
//   1. wavefront r < 2 reads the map of tile (kt, rt0 + r) (none past nrt),
//      lane l on column l, and writes its per-class row counts to
//      cnt[r][l][class];
//   2. each of those wavefronts forms, for its lane's k-group, where its
//      records of each class start in the group's list: class order 8, 1,
//      2, 4-bit, and within a class row-tile 0's records before row-tile
//      1's. No list position depends on another wavefront's progress, so the
//      placement needs no atomics and the lists come out the same every call;
//   3. the same wavefronts walk their tile's blocks and place every record
//      (codes offset, row, class; the scale/offset's stream offset for now);
//   4. every thread loads the scale/offset words of eight list entries, all
//      at once, and writes them into the entries.
__device__ __attribute__((always_inline)) inline void build_index(const GemmArgs& a, GemmSmem& S, int kt, int rt0, int nrt,
                                                                  uint32_t base16, int tid) {
  const int wave = tid >> 6, lane = tid & 63;
  const int g0 = kt * kTileGroups, Gt = min(kTileGroups, a.G - g0);
  const bool mine = wave < nrt;
  const bool live = mine && lane < Gt;
  uint32_t tbase = 0, w2 = 0, w3 = 0;
  ClassMasks km = class_masks(0u, 0u, 0);
  if (mine) {
    const int rt = rt0 + wave;
    const uint4 h = *reinterpret_cast<const uint4*>(a.tiles + 4 * (size_t)(kt * a.RT + rt));
    tbase = (h.x - base16) * 16u;
    w2 = h.z;
    w3 = h.w;
    const int R = min(kTileRows, a.N - rt * kTileRows);
    const uint2 mp = live ? *reinterpret_cast<const uint2*>(a.stream + (size_t)h.x * 16u + 8u * (uint32_t)lane)
                          : make_uint2(0u, 0u);
    km = class_masks(mp.x, mp.y, live ? R : 0);
  }
  if (wave < kRowTilesPerWg)
#pragma unroll
    for (int c = 0; c < 4; ++c) S.cnt[wave][lane][c] = (uint32_t)__popc(km.m[c]);
  gemm_barrier();   // per-wavefront counts written
  if (mine) {
    // Class order in a k-group's list: 8-bit, 1-bit, 2-bit, 4-bit. Producer
    // wavefronts take 32 consecutive entries each and run one decode path
    // per class they hold, so the short classes are kept apart: with the
    // usual mixes (mostly 1-bit) no wavefront holds more than two classes.
    constexpr int kOrder[4] = {3, 0, 1, 2};
    uint32_t start[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = kOrder[i];
      const uint32_t n0 = S.cnt[0][lane][c], n1 = S.cnt[1][lane][c];
      start[c] = sum + (wave == 1 ? n0 : 0u);
      sum += n0 + n1;
    }
    uint32_t cbase = tbase + map_bytes((uint32_t)Gt);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t n = class_count(w2, w3, c);
      uint32_t mask = km.m[c];
      uint32_t e = wave_excl_scan((uint32_t)__popc(mask), (uint32_t)lane);
      uint32_t slot = start[c];
      for (; mask; mask &= mask - 1u, ++e, ++slot) {
        const uint32_t row = (uint32_t)wave * kTileRows + (uint32_t)__builtin_ctz(mask);
        const RecPos rp = record_pos(c, n, cbase, e);
        S.ent[lane][slot] = make_uint2((rp.codes >> 3) | (row << 17) | ((uint32_t)c << 24), rp.so);
      }
      cbase += class_bytes(c, n);
    }
  }
  gemm_barrier();
  // Each k-group lists one record per row of the workgroup.
  const int nvalid = min(kBN, a.N - rt0 * kTileRows);
  constexpr int kPer = kTileGroups * kBN / kThreads;   // entries per thread: 8
  uint32_t sov[kPer];
  const uint8_t* wg_bytes = a.stream + (size_t)base16 * 16u;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int idx = tid + e * kThreads, kg = idx / kBN, slot = idx % kBN;
    const bool has = kg < Gt && slot < nvalid;
    const uint32_t off = has ? S.ent[kg][slot].y : 0u;
    sov[e] = *reinterpret_cast<const uint32_t*>(wg_bytes + off);
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int idx = tid + e * kThreads, kg = idx / kBN, slot = idx % kBN;
    if (kg < Gt && slot < nvalid) S.ent[kg][slot].y = sov[e];
  }
  gemm_barrier();
}

// The quarter (16 codes) of one record a lane decodes, as loaded from HBM.
struct CodeRegs {
  uint4 v;            // the 16-byte aligned window holding the quarter's code words
  uint32_t sov;       // scale | offset << 16
  uint32_t info;      // row | class << 6 | first word in v << 8 | valid << 10
};

// Every thread issues the same 16-byte load for every group, whatever the
// width (and also for rows past N, from the workgroup's first byte), so that
// the compiler's load-count waits are exact: a wait for an older stage never
// has to assume fewer loads in flight and drain the newer ones.
//
// Quarter Q of a record (codes 16Q .. 16Q + 15) lies in half Q / 2, pairs
// 8 (Q % 2) .. + 7 of it. Its code words start at record word Q * b / 2 for
// b >= 2 (b / 2 words); a 1-bit quarter is bits 8 (Q % 2) + [0, 8) and
// 16 + 8 (Q % 2) + [0, 8) of word Q / 2. Records are 8 << class bytes and
// blocks 16-byte aligned, so those words never cross a 16-byte boundary, and
// the window stays inside the record's block (its scale/offset area follows
// the codes).
__device__ inline uint2 list_entry(const GemmSmem& S, int kgl, int nvalid, int tid) {
  const int slot = tid >> 2;
  return slot < nvalid ? S.ent[kgl][slot] : make_uint2(0, 0);
}

__device__ inline void load_codes(const GemmArgs& a, uint32_t base16, uint2 e, int nvalid, int tid, CodeRegs& R) {
  const int slot = tid >> 2, qtr = tid & 3;
  const bool has = slot < nvalid;
  const uint32_t c = (e.x >> 24) & 3u;
  const uint32_t wi = c == 0 ? (uint32_t)(qtr >> 1) : (uint32_t)qtr << (c - 1);
  const uint32_t byte = ((e.x & 0x1FFFFu) << 3) + 4u * wi;
  R.sov = e.y;
  R.info = has ? (((e.x >> 17) & 63u) | (c << 6) | (((byte >> 2) & 3u) << 8) | (1u << 10)) : 0u;
  const uint32_t off = has ? (byte & ~15u) : 0u;
  R.v = *reinterpret_cast<const uint4*>(a.stream + (size_t)base16 * 16u + off);
}

__device__ inline uint32_t pack_bf16(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ inline uint32_t word_at(const uint4& v, uint32_t j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// 1- and 2-bit quarters: the 2 or 4 weights bf16(fma(s, q, o)) of the record
// form a table of bf16 in bytes 0..7 of {hi, lo}; the pair of codes (e, o) of
// pair p, at bits p << C and 16 + (p << C) of the quarter's word, selects
// bytes {2e, 2e + 1, 2o, 2o + 1} of it.
template <int C>
__device__ inline void decode_table(const CodeRegs& R, uint32_t j, int qtr, float s, float o, uint32_t out[8]) {
  const uint32_t w = word_at(R.v, j);
  const uint32_t lo = pack_bf16(__builtin_fmaf(s, 0.0f, o), __builtin_fmaf(s, 1.0f, o));
  const uint32_t hi = C == 1 ? pack_bf16(__builtin_fmaf(s, 2.0f, o), __builtin_fmaf(s, 3.0f, o)) : 0u;
  constexpr uint32_t M = C == 0 ? 0x00010001u : 0x00030003u;
  const uint32_t ws = C == 0 ? w >> (8 * (qtr & 1)) : w;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const uint32_t t = (ws >> (p << C)) & M;
    out[p] = __builtin_amdgcn_perm(hi, lo, t * 0x202u + 0x01000100u);
  }
}

// 4-bit quarter: two words of four pairs, pair m of a word holding its even
// code at bit 4m and its odd code at bit 16 + 4m; masking the word and the
// word shifted by 4 with 0x0F0F0F0F puts every code in a byte of its own.
__device__ inline void decode_4bit(const CodeRegs& R, uint32_t j, float s, float o, uint32_t out[8]) {
  const uint32_t w[2] = {j == 0 ? R.v.x : R.v.z, j == 0 ? R.v.y : R.v.w};
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t e = w[k] & 0x0F0F0F0Fu, d = (w[k] >> 4) & 0x0F0F0F0Fu;
    // pair 0: bytes 0, 2 of e; pair 1: of d; pair 2: bytes 1, 3 of e; pair 3: of d
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t src = (m & 1) ? d : e;
      const int b0 = (m >> 1) * 8;
      const float q0 = (float)((src >> b0) & 0xFFu), q1 = (float)((src >> (16 + b0)) & 0xFFu);
      out[4 * k + m] = pack_bf16(__builtin_fmaf(s, q0, o), __builtin_fmaf(s, q1, o));
    }
  }
}

// 8-bit quarter: four words of two pairs, pair m of a word at bytes m and 2 + m.
__device__ inline void decode_8bit(const CodeRegs& R, float s, float o, uint32_t out[8]) {
  const uint32_t w[4] = {R.v.x, R.v.y, R.v.z, R.v.w};
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const uint32_t x = w[p >> 1];
    const int b0 = (p & 1) * 8;
    const float q0 = (float)((x >> b0) & 0xFFu), q1 = (float)((x >> (16 + b0)) & 0xFFu);
    out[p] = pack_bf16(__builtin_fmaf(s, q0, o), __builtin_fmaf(s, q1, o));
  }
}

__device__ inline void store_weights(GemmSmem& S, int buf, const CodeRegs& R, int tid) {
  if (!((R.info >> 10) & 1u)) return;
  const int qtr = tid & 3;
  const uint32_t row = R.info & 63u, c = (R.info >> 6) & 3u, j = (R.info >> 8) & 3u;
  const float s = __half2float(__ushort_as_half((unsigned short)(R.sov & 0xFFFFu)));
  const float o = __half2float(__ushort_as_half((unsigned short)(R.sov >> 16)));
  uint32_t out[8];
  switch (c) {
    case 0: decode_table<0>(R, j, qtr, s, o, out); break;
    case 1: decode_table<1>(R, j, qtr, s, o, out); break;
    case 2: decode_4bit(R, j, s, o, out); break;
    default: decode_8bit(R, s, o, out); break;
  }
  uint4* dst = reinterpret_cast<uint4*>(&S.ws[buf][row][16 * qtr]);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
}

// One consumer wavefront copies the 64 token rows [r0, r0 + 64) of group g
// into slot `slot`: eight copies of 1 KiB (eight rows each), lane l taking
// row r0 + 8i + l / 8, stored column l % 8. Rows past M read as zeros (the
// buffer ends at M rows).
constexpr int kXCopies = 8;   // copies per consumer wavefront and group

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
  const int nvalid = min(kBN, a.N - rt0 * kTileRows);

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int cw = wave - kProducers / kWave;   // consumer wavefront 0..3
  const int wm = cw;   // tokens [64 wm, 64 wm + 64) of the workgroup, all its rows
  // Per k-tile: build the record lists, then run the pipeline over its
  // groups, one barrier per group:
  //  - producers hold the codes of groups g+1..g+4 in four register stages:
  //    they load group g + 4 and decode group g + 1 into the free weight
  //    buffer while the consumers multiply group g;
  //  - each consumer wavefront also copies its quarter of x of group g + 2
  //    into the free x slot (buffer-to-LDS, no registers) at the start of
  //    the step and, before the barrier, waits until its copy of group g + 1
  //    has landed.
  // Producers issue only register loads and consumers only copies, so the
  // compiler's load-count waits in the producers are exact and the copies
  // are waited for explicitly. Every step issues the same loads (group
  // indices clamped to the k-tile's last), steps past the end only keep the
  // barrier schedule.
  const int xr0 = cw * 64;   // this wavefront's x rows
  const u32x4 xrsrc = make_rsrc(a.x, (uint32_t)a.M * (uint32_t)a.G * kXRow);
  const uint32_t xs_lds = lds_addr(&S.xs[0][0]);
  const int KT = (a.G + kTileGroups - 1) / kTileGroups;
  for (int kt = 0; kt < KT; ++kt) {
    const int g0 = kt * kTileGroups, g1 = min(a.G, g0 + kTileGroups);
    const uint32_t base16 = a.tiles[4 * (size_t)(kt * a.RT + rt0) + 0];
    // The consumers' copies of x for the k-tile's first two groups need no
    // record list, so they go out before the lists are built (every x slot
    // is free here: the previous k-tile ended with a barrier after its last
    // reads).
    if (!producer) {
      copy_x(a, xrsrc, xs_lds + (uint32_t)(g0 % kXSlots) * kBM * kXRow, m0, xr0, g0, lane);
      copy_x(a, xrsrc, xs_lds + (uint32_t)((g0 + 1) % kXSlots) * kBM * kXRow, m0, xr0, min(g0 + 1, g1 - 1),
             lane);
    }
    build_index(a, S, kt, rt0, nrt, base16, tid);
    // The two roles run loops of their own with the same barrier schedule:
    // in one shared loop body the compiler merges their load-count state and
    // waits for every load in flight where a register of one role's load is
    // reused by the other.
    if (producer) {
      // The list entry of a group is read from LDS one step before its codes
      // are loaded, so the load goes out right after the barrier.
      auto entry = [&](int g) { return list_entry(S, min(g, g1 - 1) & (kTileGroups - 1), nvalid, tid); };
      CodeRegs st0, st1, st2, st3;
      load_codes(a, base16, entry(g0), nvalid, tid, st0);
      load_codes(a, base16, entry(g0 + 1), nvalid, tid, st1);
      load_codes(a, base16, entry(g0 + 2), nvalid, tid, st2);
      load_codes(a, base16, entry(g0 + 3), nvalid, tid, st3);
      uint2 ahead = entry(g0 + 4);
      store_weights(S, g0 & 1, st0, tid);
      gemm_barrier();
      auto step = [&](int g, CodeRegs& reload, const CodeRegs& next) {
        load_codes(a, base16, ahead, nvalid, tid, reload);   // group g + 4
        ahead = entry(g + 5);
        if (g + 1 < g1) store_weights(S, (g & 1) ^ 1, next, tid);
        gemm_barrier();
      };
      for (int g = g0; g < g1; g += 4) {
        step(g, st0, st1);
        step(g + 1, st1, st2);
        step(g + 2, st2, st3);
        step(g + 3, st3, st0);
      }
    } else {
      __builtin_amdgcn_s_waitcnt(VBQ_VMCNT_IMM(kXCopies));   // group g0 landed
      gemm_barrier();
      auto step = [&](int g) {
        // The copy of group g + 2 goes out first: its slot was last read in
        // the previous step, before the barrier, and the copy then has two
        // steps to land.
        copy_x(a, xrsrc, xs_lds + (uint32_t)((g + 2) % kXSlots) * kBM * kXRow, m0, xr0, min(g + 2, g1 - 1),
               lane);
        if (g < g1) {
          // All operands of the group are read from LDS before the first
          // MFMA, so the wavefront waits for LDS once per group, not per step.
          const uint8_t* xslot = S.xs[g % kXSlots];
          const int buf = g & 1;
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
                  &S.ws[buf][32 * j + (lane & 31)][16 * kk + 8 * (lane >> 5)]);
          }
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
              for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[kk][i], bv[kk][j], acc[i][j], 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(VBQ_VMCNT_IMM(kXCopies));   // group g + 1 landed
        gemm_barrier();
      };
      for (int g = g0; g < g1; g += 4) {
        step(g);
        step(g + 1);
        step(g + 2);
        step(g + 3);
      }
      __builtin_amdgcn_s_waitcnt(VBQ_VMCNT_IMM(0));   // no copy left in flight
    }
  }
  if (producer) return;

  // acc[i][j][r]: token wm*64 + 32i + 8(r/4) + 4(lane/32) + r%4, row 32j + lane%32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = rt0 * kTileRows + 32 * j + (lane & 31);
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
