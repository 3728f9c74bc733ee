// Fused dequantise-and-multiply GEMV over the tiled stream of a packed matrix.
//
// Follows the VBQ abstract (page "In-Cell Learning: Language Models That
// Update Their Own Weights in Sequence Without Changing the File They Ship"):
// 64-weight groups with widths {1,2,4,8}, packed storage, and a kernel that
// dequantises and multiplies in one pass for memory-bandwidth-bound decode.
// The optional residual term follows the CellFill abstract (page "Nothing
// Changed but the Model: CellFill -- Bounded In-Cell Learning for
// Bit-Identical, Revocable Updates to Quantized LLMs"): the served weight is
// the dequantised code plus a per-weight residual, and dropping the residual
// revokes the update. Several residual levels of one matrix (RRQ abstract on
// page thelatestinai.com/papers/2512.18934) are summed in the same launch.
//
// Per group g of row n and batch row b:
//   y[b][n] += s_g * sum_k q_k x_k + o_g * sum_k x_k        (k in the group)
// The inner sum never materialises weights: a code field is OR-ed into the
// mantissa of an fp16 whose exponent makes the field's unit exactly 1, so the
// fp16 value is bias + q with bias = 2^(10-p) for a field at mantissa bit p.
// Four such values and their four activations go to the matrix cores as one
// 16-block v_mfma_f32_4x4x4f16, whose result holds each lane's own
// four-term dot product in one of its four registers (the VALU only builds
// the operands). The bias part, sum_j bias_j (x_2j + x_2j+1), depends only on
// x and the width, so it is computed once per (k-group, width) and
// subtracted per record.
//
// Work split: the four wavefronts of a workgroup decode one tile (32 rows x
// 64 k-groups) together; the steps are described at coop_tile. The tile's
// activations are copied into LDS once, every record's position is a closed
// form of the tile header's class counts (records of a width class are listed
// column by column, 64 to a block), and each record's value goes to an LDS
// slot of its (column, row), so the row sums are added in a fixed order and
// results repeat bit for bit with no atomics. A matrix with one k-tile takes a
// workgroup per tile; a longer one either has a workgroup walk its row-tile's
// k-tiles (and residual levels, then residual rows) in order, or, in the
// launches that may not allocate, a workgroup per tile whose row sums meet in
// a static device array and are added in k-tile order by the last one to
// finish. With a compact in-cell residual the workgroup has four more
// wavefronts that stream the residual bytes while the tile is decoded.
#include <utility>

#include "vbq_common.h"

namespace vbq {

// ---- Decoding ----------------------------------------------------------------
// Field placement of pair-field index f (pair p of a word: f = p % (16/b)) per
// width class c. shift kind: 0 none, 1 right by 6, 2 right by 8.
__host__ __device__ constexpr int shift_kind(int c, int f) {
  return c == 0 ? (f < 10 ? 0 : 1) : c == 1 ? (f < 5 ? 0 : 1) : c == 2 ? (f < 2 ? 0 : 2) : (f < 1 ? 0 : 2);
}
// Mantissa bit of the field after the shift.
__host__ __device__ constexpr int field_pos(int c, int f) {
  return c == 0 ? (f < 10 ? f : f - 6) : c == 1 ? (f < 5 ? 2 * f : 2 * f - 6) : c == 2 ? ((f & 1) ? 4 : 0) : 0;
}
__host__ __device__ constexpr uint32_t field_mask(int c, int p) {
  return (((1u << (1 << c)) - 1u) << p) * 0x00010001u;
}
// fp16 with exponent field 25 - p: the mantissa bit p has weight 1.
__host__ __device__ constexpr uint32_t field_magic(int p) { return (uint32_t)((25 - p) << 10) * 0x00010001u; }
// The fp16 pair (2^(10-p), 2^(10-p)): the bias of both codes of a field at bit p.
__host__ __device__ constexpr uint32_t field_bias_pair(int p) { return (uint32_t)((25 - p) << 10) * 0x00010001u; }

template <int KIND>
__device__ inline uint32_t shifted(uint32_t w) {
  return KIND == 0 ? w : KIND == 1 ? (w >> 6) : (w >> 8);
}

// A constant materialised in a VGPR that the compiler cannot fold back into a
// literal (VOP3 forms such as v_and_or_b32 take no literal operands).
template <uint32_t V>
__device__ inline uint32_t vconst() {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "n"(V));
  return r;
}

__device__ inline half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}

// Masks and exponent patterns of one width class, held in VGPRs for the
// class's blocks (entries a class never uses are dead and cost nothing).
template <int C>
struct Consts {
  uint32_t mask[10], magic[10];
};

template <int C, int... P>
__device__ inline Consts<C> make_consts_impl(std::integer_sequence<int, P...>) {
  Consts<C> k;
  if constexpr (C == 3) {
    k.magic[0] = vconst<0x64646464u>();
  } else {
    ((k.mask[P] = vconst<field_mask(C, P)>(), k.magic[P] = field_magic(P)), ...);
  }
  return k;
}

template <int C>
__device__ inline Consts<C> make_consts() {
  return make_consts_impl<C>(std::make_integer_sequence<int, 10>{});
}

// The fp16 pair (bias + q_2P, bias + q_2P+1) of pair P of a record. Eight-bit
// codes take one byte permute: bytes q_2P and q_2P+1 of the word, each under
// the exponent byte 0x64 (fp16 1024 + q); narrower codes take an AND-OR of
// the field, shifted down first when it lies above the mantissa.
template <int C, int P>
__device__ inline uint32_t pair_h2(const Consts<C>& k, const uint32_t* w) {
  constexpr int H = 16 >> C, F = P % H, FP = field_pos(C, F);
  if constexpr (C == 3) {
    return __builtin_amdgcn_perm(k.magic[0], w[P / H], F ? 0x04030401u : 0x04020400u);
  } else {
    const uint32_t src = shifted<shift_kind(C, F)>(w[P / H]);
    return (src & k.mask[FP]) | k.magic[FP];
  }
}

// The multiply-accumulate of a record on the matrix cores: two code pairs
// (four weights) and their four activations go to one 16-block
// v_mfma_f32_4x4x4f16, whose block of lanes 4b..4b+3 multiplies the four
// lanes' codes by the four lanes' activations: lane l's own four-term dot
// product lands in register l % 4 of its result (the other registers hold
// products with the other lanes' activations and are not used). Two
// accumulators take the record's 16 MFMAs in turn.
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ inline half4_t as_h4(uint32_t lo, uint32_t hi) {
  u32x2 v;
  v.x = lo;
  v.y = hi;
  return __builtin_bit_cast(half4_t, v);
}

template <int C, int NB, int H, int... Q>
__device__ inline void record_mfma(const Consts<C>& k, const uint32_t* w, const uint32_t (&xr)[NB][32],
                                   f32x4_t (&acc)[NB][2], std::integer_sequence<int, Q...>) {
  (
      [&] {
        constexpr int P = H + 2 * Q;
        const half4_t a = as_h4(pair_h2<C, P>(k, w), pair_h2<C, P + 1>(k, w));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[nb][Q & 1] =
              __builtin_amdgcn_mfma_f32_4x4x4f16(a, as_h4(xr[nb][P], xr[nb][P + 1]), acc[nb][Q & 1], 0, 0, 0);
      }(),
      ...);
}

// Register l % 4 of v (the lane's own dot product of a record_mfma), picked
// by the two low bits of the lane index.
__device__ inline float own_dot(const f32x4_t& v, bool b0, bool b1) {
  const float lo = b0 ? v.y : v.x, hi = b0 ? v.w : v.z;
  return b1 ? hi : lo;
}

// sum over the record's pairs of bias(field) * (x_2P + x_2P+1).
template <int C, int NB, int... P>
__device__ inline void class_bias(const uint32_t (&xr)[NB][32], float (&bias)[NB], std::integer_sequence<int, P...>) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    ((a[P & 3] = dot2(xr[nb][P], field_bias_pair(field_pos(C, P % (16 >> C))), a[P & 3])), ...);
    bias[nb] = (a[0] + a[1]) + (a[2] + a[3]);
  }
}

// ---- Cooperative tile -------------------------------------------------------------
// The four wavefronts of a workgroup process one tile together. Every record
// position is a closed form of the tile header (records of a width class are
// listed column by column, 64 to a block), so every load of a tile goes out
// as soon as its header is known:
//  1. Wavefront 0 copies the activations of the tile's 64 columns into LDS
//     with buffer-to-LDS loads; every wavefront loads the width map of its
//     lane's column and issues its first chunks of every class (chunk j of a
//     class = its records 64 j .. 64 j + 63; wavefront w takes chunks w,
//     w + 4, ...).
//  2. Wavefront 0 forms, per column, the bias sum of every class and the sum
//     of the activations; wavefronts 1-3 list the (column, row) of every
//     record in an LDS table (wavefront 1 class 0, 2 class 1, 3 classes 2
//     and 3; lane l writes the entries of its column's rows). Barrier.
//  3. The wavefronts decode their chunks class by class; lane e of a chunk
//     takes record 64 j + e, reads its column and row from the table and the
//     column's activations from LDS (in two halves, to bound the registers),
//     and puts s (dot) + o sum(x) at the slot of its (column, row). Later
//     chunks of a class are loaded D ahead. Barrier.
//  4. Wavefront w adds the slots of rows 8w..8w+7 over the 64 columns in a
//     fixed order and clears them.
constexpr int kSlotPitch = 33;                            // slot (column l, row r) at l * 33 + r; 32 is spare
// Words from one batch row's slots to the next: 2112 and a 16-word skew, so
// that the four lanes of an MFMA block in a four-row pass, which write the
// same slot for their four batch rows, hit four different LDS banks.
constexpr int kSlotWords = kWave * kSlotPitch + 16;
// Activations of a tile's 64 columns: per column 64 fp16 (32 words) and 4
// words of sums, 144 bytes apart, so that the 16-byte reads of lanes on
// different columns fall on different LDS banks. The sums are sum(x) and
// -bias of classes 0, 1, 2 (the bias of 8-bit codes is 1024 sum(x)).
constexpr int kXPitch = 36;                               // words per column
constexpr int kXSum = 32;                                 // word of sum(x) in a column; -bias of class c at 33 + c
constexpr int kXWords = kTileGroups * kXPitch;
constexpr int kMaxRecs = kTileRows * kTileGroups;         // 2048 table entries

template <int NB>
struct LdsMap {
  static constexpr int x = 0;                             // [NB][64][36] fp16 pairs and the column's sums
  // words from one batch row's activations to the next: with four rows a
  // 64-byte skew (16 banks) puts the same column of the four rows on
  // different banks (the four lanes of an MFMA block read one row each), and
  // with the 36-word column pitch, blocks on columns fewer than four apart
  // land on other banks as well
  static constexpr int xrow = NB >= 4 ? kXWords + 16 : kXWords;
  static constexpr int xbuf = NB * xrow;                  // words per activation buffer
  static constexpr int table = x + xbuf;                  // [2048] u32: slot byte << 16 | column byte (from S)
  static constexpr int slots = table + kMaxRecs;          // [NB][64][33]
  static constexpr int ys = slots + NB * kSlotWords;      // [NB][32] residual row sums
  static constexpr int words = ys + NB * kTileRows;
  // With a compact in-cell residual: the scale of slot (column, row) and the
  // residual dot of slot (column, row) per batch row, same pitch as the slots.
  static constexpr int sc = words;
  static constexpr int cd = sc + kSlotWords;
  static constexpr int words_cell = cd + NB * kSlotWords;
};

// Buffer offset that lies outside every stream: loads from it return zeros
// without touching memory.
constexpr uint32_t kNoRecord = 0x80000000u;

// One record in flight: its words and its scale/offset word.
template <int C>
struct Rec {
  uint32_t w[2 << C];
  uint32_t so;
  uint32_t ent;   // four-row passes: the record's quad entry
};

// Chunks of a class each wavefront has in flight: issued at the tile's start
// and refilled while the class is decoded.
template <int C, int NB>
__host__ __device__ constexpr int depth() {
  // (four-row passes run eight wavefronts per tile, each holding one row's
  // activations per lane: together they keep as many chunks in flight as four
  // wavefronts at the one-row depths)
  return NB == 4 ? (C == 0 ? 2 : 1)
                 : C == 0 ? (NB >= 4 ? 1 : 4 / NB) : C == 1 ? (NB >= 2 ? 1 : 2) : 1;   // at least one
}

struct TileRef {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t base;      // byte offset of the tile in the stream
  uint32_t n[4];      // records per class
  uint32_t cb[4];     // byte (from the tile's start) of each class's first block
  uint32_t t0[4];     // first table entry of each class
  int R, Gt, g0;
};

__device__ inline uint4 tile_header(const GemvMat& T, int rt, int kt) {
  return *reinterpret_cast<const uint4*>(T.tiles + 4 * ((size_t)kt * T.row_tiles + rt));
}

__device__ inline TileRef tile_ref_from(const GemvMat& T, int rt, int kt, const uint4 hdr) {
  TileRef t;
  t.base = __builtin_amdgcn_readfirstlane(hdr.x) * 16u;
  const uint32_t w2 = __builtin_amdgcn_readfirstlane(hdr.z), w3 = __builtin_amdgcn_readfirstlane(hdr.w);
  t.R = min(kTileRows, T.n_rows - rt * kTileRows);
  t.g0 = kt * kTileGroups;
  t.Gt = min(kTileGroups, T.n_groups - t.g0);
  uint32_t cb = map_bytes((uint32_t)t.Gt), e = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    t.n[c] = class_count(w2, w3, c);
    t.cb[c] = cb;
    t.t0[c] = e;
    cb += class_bytes(c, t.n[c]);
    e += t.n[c];
  }
  t.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(T.stream), (short)0, (int)T.stream_bytes, 0x00020000);
  return t;
}

__device__ inline TileRef tile_ref(const GemvMat& T, int rt, int kt) { return tile_ref_from(T, rt, kt, tile_header(T, rt, kt)); }

// The width map of the lane's column (columns past the tile repeat its last).
__device__ inline u32x2 map_load(const TileRef& t, uint32_t lane) {
  const int lc = min((int)lane, t.Gt - 1);
  return __builtin_amdgcn_raw_buffer_load_b64(t.rs, (int)(t.base + 8u * (uint32_t)lc), 0, 0);
}

// Issues the loads of chunk j of class C (records 64 j + lane); lanes past
// the class's last record load from kNoRecord.
template <int C>
__device__ inline void issue_chunk(const TileRef& t, uint32_t j, Rec<C>& r, uint32_t lane) {
  constexpr uint32_t RB = 8u << C;
  const uint32_t e = 64u * j + lane;
  uint32_t oc = kNoRecord, os = kNoRecord;
  if (e < t.n[C]) {
    const RecPos rp = record_pos(C, t.n[C], t.cb[C], e);
    oc = t.base + rp.codes;
    os = t.base + rp.so;
  }
  if constexpr (C == 0) {
    const u32x2 u = __builtin_amdgcn_raw_buffer_load_b64(t.rs, (int)oc, 0, 0);
    r.w[0] = u.x;
    r.w[1] = u.y;
  } else {
#pragma unroll
    for (int h = 0; h < (int)RB / 16; ++h) {
      const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(t.rs, (int)(oc + 16u * h), 0, 0);
      r.w[4 * h + 0] = u.x;
      r.w[4 * h + 1] = u.y;
      r.w[4 * h + 2] = u.z;
      r.w[4 * h + 3] = u.w;
    }
  }
  r.so = __builtin_amdgcn_raw_buffer_load_b32(t.rs, (int)os, 0, 0);
}

// Chunks of a class with n records that wavefront w of W takes (chunks w,
// w + W, ...).
template <int W = kGemvWaves>
__device__ inline uint32_t wave_chunks(uint32_t n, int wave) {
  const uint32_t J = (n + 63u) >> 6;
  return J > (uint32_t)wave ? (J - (uint32_t)wave + W - 1) / W : 0u;
}

template <int C, int NB>
struct Flight {
  Rec<C> r[depth<C, NB>()];
};

template <int C, int NB>
__device__ inline void issue_first(const TileRef& t, int wave, Flight<C, NB>& f, uint32_t lane) {
  const uint32_t nS = wave_chunks(t.n[C], wave);
#pragma unroll
  for (int d = 0; d < depth<C, NB>(); ++d)
    issue_chunk<C>(t, (uint32_t)d < nS ? (uint32_t)wave + kGemvWaves * d : 0x3FFFFFFu, f.r[d], lane);
}

// Table entries of class c: lane l writes those of its column's rows, in
// row order, after the entries of the columns before it.
template <int NB>
__device__ inline void table_class(const TileRef& t, int c, uint32_t p0, uint32_t p1, uint32_t valid, uint32_t* S,
                                   uint32_t lane, int buf) {
  uint32_t mask = ((c & 1) ? p0 : ~p0) & ((c & 2) ? p1 : ~p1) & valid;
  const uint32_t first = (c > 0 ? t.n[0] : 0u) + (c > 1 ? t.n[1] : 0u) + (c > 2 ? t.n[2] : 0u);
  uint32_t e = first + wave_excl_scan((uint32_t)__builtin_popcount(mask), lane);
  uint32_t* tab = S + LdsMap<NB>::table;
  const uint32_t xb = 4u * (LdsMap<NB>::x + buf * LdsMap<NB>::xbuf + lane * kXPitch);
  const uint32_t sb = 4u * (LdsMap<NB>::slots + lane * kSlotPitch);
  for (; mask; mask &= mask - 1u, ++e) tab[e] = ((sb + 4u * (uint32_t)__builtin_ctz(mask)) << 16) | xb;
}

// Table entry of the lanes past a class's last record: column 31, spare row 32.
template <int NB>
__host__ __device__ constexpr uint32_t spare_entry() {
  return ((4u * (LdsMap<NB>::slots + 31 * kSlotPitch + 32)) << 16) | (4u * (LdsMap<NB>::x + 31 * kXPitch));
}

// ---- Four batch rows: record quads ----------------------------------------------
// A pass of four batch rows puts the rows in the four B columns of the 4x4x4
// MFMA: lane c of a block supplies batch row c's activations, and the block's
// result holds the dot products of its four lanes' records with all four rows
// (register q of lane c: the record of lane 4 (l / 4) + q with batch row c).
// The four records of a block must then share a column (a k-group), so in
// such a pass the records of a class are taken column by column in quads:
// each column's records of the class in row order, padded with empty entries
// to a multiple of four. Lane p of chunk j takes padded entry 64 j + p. The
// record table holds the padded entries (u16: valid << 15 | column << 5 |
// row); a record's index in the class, and with it its position in the
// stream, is the number of the class's records in the columns before it plus
// its rank among its column's rows.
constexpr int kQuadWaves = 8;                            // wavefronts of a four-row workgroup
constexpr uint32_t kQuadPad = 3 * kTileGroups;          // padding entries of a class at most
constexpr uint32_t kQuadTab = kMaxRecs + 4 * kQuadPad;  // 2816 entries
struct QuadMap {   // words from LdsMap<4>::table
  static constexpr int tab = 0;                          // u16 [2816]
  static constexpr int masks = kQuadTab / 2;             // u32 [4][64]: each class's rows per column
  static constexpr int pre = masks + 4 * kTileGroups;    // u16 [4][64]: the class's records in the columns before
  static constexpr int cnt = pre + 2 * kTileGroups;      // u32 [4]: padded entries per class
  static constexpr int words = cnt + 4;
};
static_assert(QuadMap::words <= kMaxRecs, "record quads fit the record table");

// First padded entry of class c: worst-case regions, so that every wavefront
// places them from the tile header alone.
__device__ inline uint32_t quad_base(const TileRef& t, int c) {
  return (c > 0 ? t.n[0] + kQuadPad : 0u) + (c > 1 ? t.n[1] + kQuadPad : 0u) + (c > 2 ? t.n[2] + kQuadPad : 0u);
}

// The padded entries, row masks and record counts of class c; lane l on
// column l.
__device__ inline void quad_class(const TileRef& t, int c, uint32_t p0, uint32_t p1, uint32_t valid, uint32_t* S,
                                  uint32_t lane) {
  const uint32_t mask = ((c & 1) ? p0 : ~p0) & ((c & 2) ? p1 : ~p1) & valid;
  const uint32_t n = (uint32_t)__builtin_popcount(mask), np = (n + 3u) & ~3u;
  const uint32_t pre = wave_excl_scan(n, lane), ppre = wave_excl_scan(np, lane);
  uint32_t* Q = S + LdsMap<4>::table;
  Q[QuadMap::masks + c * kTileGroups + lane] = mask;
  reinterpret_cast<uint16_t*>(Q + QuadMap::pre)[c * kTileGroups + lane] = (uint16_t)pre;
  if (lane == 63u) Q[QuadMap::cnt + c] = ppre + np;
  uint16_t* tab = reinterpret_cast<uint16_t*>(Q + QuadMap::tab) + quad_base(t, c) + ppre;
  uint32_t m = mask, k = 0;
  for (; m; m &= m - 1u, ++k) tab[k] = (uint16_t)(0x8000u | (lane << 5) | (uint32_t)__builtin_ctz(m));
  for (; k < np; ++k) tab[k] = (uint16_t)(lane << 5);
}

// Step 2.
template <int NB>
__device__ inline void tile_prepare(const TileRef& t, int wave, const u32x2 mp, uint32_t* S, uint32_t lane, int buf) {
  if (wave == 0) {
    // The activation copies of this wavefront were issued before its width
    // map load, and loads complete in order: once the map has arrived (the
    // wait the compiler inserts for this use of it) the copies are in LDS.
    asm volatile("" ::"v"(mp.x), "v"(mp.y));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      uint32_t xr[1][32];
      const uint32_t* xs =
          S + LdsMap<NB>::x + buf * LdsMap<NB>::xbuf + nb * LdsMap<NB>::xrow + lane * (uint32_t)kXPitch;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint4 v = *reinterpret_cast<const uint4*>(xs + 4 * i);
        xr[0][4 * i + 0] = v.x;
        xr[0][4 * i + 1] = v.y;
        xr[0][4 * i + 2] = v.z;
        xr[0][4 * i + 3] = v.w;
      }
      float b[3][1];
      class_bias<0, 1>(xr, b[0], std::make_integer_sequence<int, 32>{});
      class_bias<1, 1>(xr, b[1], std::make_integer_sequence<int, 32>{});
      class_bias<2, 1>(xr, b[2], std::make_integer_sequence<int, 32>{});
      float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < 32; ++p) a[p & 3] = dot2(xr[0][p], 0x3C003C00u, a[p & 3]);
      float* sums = reinterpret_cast<float*>(S + LdsMap<NB>::x + buf * LdsMap<NB>::xbuf + nb * LdsMap<NB>::xrow +
                                             lane * (uint32_t)kXPitch + kXSum);
      *reinterpret_cast<float4*>(sums) = make_float4((a[0] + a[1]) + (a[2] + a[3]), -b[0][0], -b[1][0], -b[2][0]);
    }
  } else {
    const bool live = (int)lane < t.Gt;
    const uint32_t p0 = live ? mp.x : 0u, p1 = live ? mp.y : 0u;
    const uint32_t valid = !live ? 0u : t.R >= 32 ? 0xFFFFFFFFu : ((1u << t.R) - 1u);
    if constexpr (NB == 4) {
      quad_class(t, wave - 1, p0, p1, valid, S, lane);
      if (wave == 3) quad_class(t, 3, p0, p1, valid, S, lane);
    } else {
      table_class<NB>(t, wave - 1, p0, p1, valid, S, lane, buf);
      if (wave == 3) table_class<NB>(t, 3, p0, p1, valid, S, lane, buf);
    }
  }
}

// Decodes lane's record of chunk j: the dot starts from -bias, so it ends as
// sum_k q_k x_k; the slot of (column, row) gets s * dot + o * sum(x). Lanes
// past the class's last record write the spare slot of column 31.
template <int C, int NB, bool CELL>
__device__ inline void decode_chunk(const Consts<C>& k, const Rec<C>& r, const TileRef& t, uint32_t j, uint32_t* S,
                                    uint32_t lane) {
  const uint32_t e = 64u * j + lane;
  const bool valid = 64u * (j + 1u) <= t.n[C] || e < t.n[C];
  const uint32_t ent = valid ? S[LdsMap<NB>::table + t.t0[C] + e] : spare_entry<NB>();
  const uint32_t xoff = ent & 0xFFFFu, soff = ent >> 16;   // byte offsets from S
  const float s = __half2float(__ushort_as_half((unsigned short)(r.so & 0xFFFFu)));
  const float o = __half2float(__ushort_as_half((unsigned short)(r.so >> 16)));
  float* slot = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(S) + soff);
  if (CELL) slot[LdsMap<NB>::sc - LdsMap<NB>::slots] = s;
  // each code pair is decoded once and multiplied with every batch row's
  // activations (read in two halves, to bound the registers)
  const uint32_t* xs0 = reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(S) + xoff);
  float xsum[NB], a0[NB];
  f32x4_t acc[NB][2];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float* sums = reinterpret_cast<const float*>(xs0 + nb * LdsMap<NB>::xrow) + kXSum;
    xsum[nb] = sums[0];
    a0[nb] = C == 3 ? -1024.f * xsum[nb] : sums[1 + C];   // -bias: the dot ends as sum_k q_k x_k
    acc[nb][0] = acc[nb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    uint32_t xr[NB][32];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = *reinterpret_cast<const uint4*>(xs0 + nb * LdsMap<NB>::xrow + 16 * half + 4 * i);
        xr[nb][16 * half + 4 * i + 0] = v.x;
        xr[nb][16 * half + 4 * i + 1] = v.y;
        xr[nb][16 * half + 4 * i + 2] = v.z;
        xr[nb][16 * half + 4 * i + 3] = v.w;
      }
    if (half == 0) record_mfma<C, NB, 0>(k, r.w, xr, acc, std::make_integer_sequence<int, 8>{});
    else record_mfma<C, NB, 16>(k, r.w, xr, acc, std::make_integer_sequence<int, 8>{});
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float dot = a0[nb] + own_dot(acc[nb][0] + acc[nb][1], (lane & 1u) != 0, (lane & 2u) != 0);
    slot[nb * kSlotWords] = __builtin_fmaf(s, dot, o * xsum[nb]);
  }
}

// Step 3 for class C: the chunks in flight are decoded in turn and each
// slot is refilled with the chunk D further on.
template <int C, int NB, bool CELL>
__device__ inline void run_class(const TileRef& t, Flight<C, NB>& f, uint32_t* S, int wave, uint32_t lane) {
  constexpr int D = depth<C, NB>();
  const uint32_t nS = wave_chunks(t.n[C], wave);
  if (nS == 0) return;
  const Consts<C> k = make_consts<C>();
  for (uint32_t s0 = 0; s0 < nS; s0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const uint32_t sq = s0 + d;
      if (sq >= nS) break;
      decode_chunk<C, NB, CELL>(k, f.r[d], t, (uint32_t)wave + kGemvWaves * sq, S, lane);
      const uint32_t sn = sq + D;
      if (sn < nS) issue_chunk<C>(t, (uint32_t)wave + kGemvWaves * sn, f.r[d], lane);
    }
  }
}

// Issues the loads of the record of padded entry 64 j + lane of class C (a
// four-row pass); empty entries and lanes past the class load from
// kNoRecord. The entry is kept with the record for the decode.
template <int C>
__device__ inline void issue_quad(const TileRef& t, uint32_t j, uint32_t cnt, Rec<C>& r, const uint32_t* S,
                                  uint32_t lane) {
  constexpr uint32_t RB = 8u << C;
  const uint32_t p = 64u * j + lane;
  const uint32_t* Q = S + LdsMap<4>::table;
  const uint32_t ent = p < cnt ? (uint32_t)reinterpret_cast<const uint16_t*>(Q + QuadMap::tab)[quad_base(t, C) + p] : 0u;
  uint32_t oc = kNoRecord, os = kNoRecord;
  if (ent & 0x8000u) {
    const uint32_t col = (ent >> 5) & 63u, row = ent & 31u;
    const uint32_t mask = Q[QuadMap::masks + C * kTileGroups + col];
    const uint32_t e = (uint32_t)reinterpret_cast<const uint16_t*>(Q + QuadMap::pre)[C * kTileGroups + col] +
                       (uint32_t)__builtin_popcount(mask & ((1u << row) - 1u));
    const RecPos rp = record_pos(C, t.n[C], t.cb[C], e);
    oc = t.base + rp.codes;
    os = t.base + rp.so;
  }
  r.ent = ent;
  if constexpr (C == 0) {
    const u32x2 u = __builtin_amdgcn_raw_buffer_load_b64(t.rs, (int)oc, 0, 0);
    r.w[0] = u.x;
    r.w[1] = u.y;
  } else {
#pragma unroll
    for (int h = 0; h < (int)RB / 16; ++h) {
      const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(t.rs, (int)(oc + 16u * h), 0, 0);
      r.w[4 * h + 0] = u.x;
      r.w[4 * h + 1] = u.y;
      r.w[4 * h + 2] = u.z;
      r.w[4 * h + 3] = u.w;
    }
  }
  r.so = __builtin_amdgcn_raw_buffer_load_b32(t.rs, (int)os, 0, 0);
}

// v of lane 4 (l / 4) + q (a quad broadcast).
template <int Q>
__device__ inline uint32_t quad_bcast(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, Q | (Q << 2) | (Q << 4) | (Q << 6), 0xF, 0xF, false);
}

// Decodes the record of lane l against batch row l % 4 of its quad's column
// and writes the slots of the quad's records for that row: slot (column, row
// of the record of lane 4 (l / 4) + q) of batch row l % 4 gets
// s_q (dot_q - bias) + o_q sum(x), with the same operations in the same order
// as a single-row pass.
template <int C>
__device__ inline void decode_quad(const Consts<C>& k, const Rec<C>& r, uint32_t* S, uint32_t lane) {
  const uint32_t c = lane & 3u;
  const uint32_t col = (r.ent >> 5) & 63u;   // the quad's column (empty entries carry it too)
  const uint32_t* xs0 = S + LdsMap<4>::x + c * LdsMap<4>::xrow + col * kXPitch;
  const float* sums = reinterpret_cast<const float*>(xs0) + kXSum;
  const float xsum = sums[0];
  const float a0 = C == 3 ? -1024.f * xsum : sums[1 + C];
  f32x4_t acc[1][2];
  acc[0][0] = acc[0][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    uint32_t xr[1][32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = *reinterpret_cast<const uint4*>(xs0 + 16 * half + 4 * i);
      xr[0][16 * half + 4 * i + 0] = v.x;
      xr[0][16 * half + 4 * i + 1] = v.y;
      xr[0][16 * half + 4 * i + 2] = v.z;
      xr[0][16 * half + 4 * i + 3] = v.w;
    }
    if (half == 0) record_mfma<C, 1, 0>(k, r.w, xr, acc, std::make_integer_sequence<int, 8>{});
    else record_mfma<C, 1, 16>(k, r.w, xr, acc, std::make_integer_sequence<int, 8>{});
  }
  const f32x4_t d = acc[0][0] + acc[0][1];
  float* slot = reinterpret_cast<float*>(S + LdsMap<4>::slots) + c * kSlotWords + col * kSlotPitch;
  // each lane converts its own record's scale and offset once; the block's
  // four are then broadcast as floats. Empty entries write the spare row 32
  // of the column's slots (never folded) instead of branching.
  const float s_own = __half2float(__ushort_as_half((unsigned short)(r.so & 0xFFFFu)));
  const float o_own = __half2float(__ushort_as_half((unsigned short)(r.so >> 16)));
  const uint32_t row_own = (r.ent & 0x8000u) ? (r.ent & 31u) : 32u;
  const uint32_t rows[4] = {quad_bcast<0>(row_own), quad_bcast<1>(row_own), quad_bcast<2>(row_own),
                            quad_bcast<3>(row_own)};
  const uint32_t sb = __float_as_uint(s_own), ob = __float_as_uint(o_own);
  const float sq[4] = {__uint_as_float(quad_bcast<0>(sb)), __uint_as_float(quad_bcast<1>(sb)),
                       __uint_as_float(quad_bcast<2>(sb)), __uint_as_float(quad_bcast<3>(sb))};
  const float oq[4] = {__uint_as_float(quad_bcast<0>(ob)), __uint_as_float(quad_bcast<1>(ob)),
                       __uint_as_float(quad_bcast<2>(ob)), __uint_as_float(quad_bcast<3>(ob))};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float dot = a0 + d[q];
    slot[rows[q]] = __builtin_fmaf(sq[q], dot, oq[q] * xsum);
  }
}

template <int C>
__device__ inline void issue_first_quad(const TileRef& t, int wave, Flight<C, 4>& f, uint32_t cnt, const uint32_t* S,
                                        uint32_t lane) {
  const uint32_t nS = wave_chunks<kQuadWaves>(cnt, wave);
#pragma unroll
  for (int d = 0; d < depth<C, 4>(); ++d)
    issue_quad<C>(t, (uint32_t)d < nS ? (uint32_t)wave + kQuadWaves * d : 0x3FFFFFFu, cnt, f.r[d], S, lane);
}

// Step 3 of a four-row pass for class C.
template <int C>
__device__ inline void run_class_quad(const TileRef& t, Flight<C, 4>& f, uint32_t cnt, uint32_t* S, int wave,
                                      uint32_t lane) {
  constexpr int D = depth<C, 4>();
  const uint32_t nS = wave_chunks<kQuadWaves>(cnt, wave);
  if (nS == 0) return;
  const Consts<C> k = make_consts<C>();
  for (uint32_t s0 = 0; s0 < nS; s0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const uint32_t sq = s0 + d;
      if (sq >= nS) break;
      decode_quad<C>(k, f.r[d], S, lane);
      const uint32_t sn = sq + D;
      if (sn < nS) issue_quad<C>(t, (uint32_t)wave + kQuadWaves * sn, cnt, f.r[d], S, lane);
    }
  }
}

// Step 4: rows 8w..8w+7; lane = 8 r + g adds columns 8g..8g+7 of row 8w + r,
// the eight partial sums are combined by a fixed butterfly (every lane of the
// group ends with the same value), and the slots are cleared for the next
// tile.
template <int NB>
__device__ inline void fold_rows(uint32_t* S, int wave, float (&yacc)[NB], uint32_t lane) {
  const uint32_t r = lane >> 3, g = lane & 7u, row = 8u * wave + r;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float* sl = reinterpret_cast<float*>(S + LdsMap<NB>::slots) + nb * kSlotWords + (8u * g) * kSlotPitch + row;
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      v += sl[q * kSlotPitch];
      sl[q * kSlotPitch] = 0.f;
    }
    v += __shfl_xor(v, 1, kWave);
    v += __shfl_xor(v, 2, kWave);
    v += __shfl_xor(v, 4, kWave);
    yacc[nb] += v;
  }
}

// ---- Compact in-cell residual ---------------------------------------------------
// Weight (n, k) of group g carries f[n][k] (int8, |f| <= 127), the residual
// s_g f / 256. Per (row, column) of a tile the slot gets s / 256 times
// D = sum_k f_k x_k on top of the record's value. Byte f ^ 0x80 = f + 128
// under the fp16 exponent byte 0x64 reads as 1152 + f, so two byte permutes
// and two v_dot2 take four weights, and the dot starts from -1152 sum(x).
// D needs no scale, so four more wavefronts of the workgroup form it while
// the first four decode the tile: cell wavefront c takes rows 8c..8c+7, lane
// l its column l (the lane's 64 activations stay in registers for the eight
// rows, and a row's 64 bytes per lane are one 4 KiB contiguous stretch per
// wavefront), and leaves D in LDS. After the decode barrier it adds
// s / 256 D to the slots of its rows, whose scales the decode left in LDS,
// and folds those rows.
template <int NB>
__host__ __device__ constexpr int cell_depth() {
  return NB == 1 ? 3 : 2;   // rows of fractions in flight per wavefront
}

struct CellRows {
  __amdgpu_buffer_rsrc_t rs;   // from the wavefront's first row, column g0
  uint32_t pitch;              // K bytes
  int rows;                    // rows of the tile this wavefront takes (may be <= 0)
  bool live;                   // lane's column inside the matrix
};

__device__ inline CellRows cell_rows_of(const GemvMat& T, int rt, int kt, int cw, uint32_t lane) {
  CellRows c;
  const uint32_t K = (uint32_t)T.n_groups * kGroup;
  const int R = min(kTileRows, T.n_rows - rt * kTileRows);
  const int g0 = kt * kTileGroups, Gt = min(kTileGroups, T.n_groups - g0);
  c.pitch = K;
  c.rows = min(8, R - 8 * cw);
  c.live = (int)lane < Gt;
  const int rows = max(c.rows, 1);
  const size_t first = (size_t)(rt * kTileRows + 8 * cw) * K + (size_t)g0 * kGroup;
  // the fractions this wavefront may read: its rows, columns g0 .. g0 + Gt - 1
  const uint32_t extent = (uint32_t)(rows - 1) * K + (uint32_t)Gt * kGroup;
  c.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(T.cell) + (c.rows > 0 ? first : 0), (short)0,
                                           (int)extent, 0x00020000);
  return c;
}

__device__ inline void cell_issue(const CellRows& c, int i, u32x4 (&v)[4], uint32_t lane) {
  const uint32_t off = (c.live && i < c.rows) ? (uint32_t)i * c.pitch + lane * kGroup : kNoRecord;
#pragma unroll
  for (int h = 0; h < 4; ++h) v[h] = __builtin_amdgcn_raw_buffer_load_b128(c.rs, (int)(off + 16u * h), 0, 0);
}

template <int NB>
struct CellFlight {
  u32x4 v[cell_depth<NB>()][4];
};

// D of rows 8c..8c+7 of the lane's column, to LDS (rows of the tile only).
template <int NB>
__device__ inline void cell_dots(const CellRows& c, CellFlight<NB>& f, uint32_t* S, int cw, uint32_t lane) {
  constexpr int D = cell_depth<NB>();
  uint32_t xr[NB][32];
  float base[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const uint32_t* xs = S + LdsMap<NB>::x + nb * LdsMap<NB>::xrow + lane * (uint32_t)kXPitch;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 v = *reinterpret_cast<const uint4*>(xs + 4 * i);
      xr[nb][4 * i + 0] = v.x;
      xr[nb][4 * i + 1] = v.y;
      xr[nb][4 * i + 2] = v.z;
      xr[nb][4 * i + 3] = v.w;
    }
    base[nb] = -1152.f * reinterpret_cast<const float*>(xs)[kXSum];
  }
  const uint32_t magic = vconst<0x64646464u>();
  float* cd = reinterpret_cast<float*>(S + LdsMap<NB>::cd) + lane * kSlotPitch + 8 * cw;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i >= c.rows) break;
    const u32x4(&v)[4] = f.v[i % D];
    float a[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      a[nb][0] = base[nb];
      a[nb][1] = 0.f;
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint32_t w[4] = {v[h].x, v[h].y, v[h].z, v[h].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t u = w[q] ^ 0x80808080u;
        const uint32_t lo = __builtin_amdgcn_perm(magic, u, 0x04010400u);
        const uint32_t hi = __builtin_amdgcn_perm(magic, u, 0x04030402u);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          a[nb][0] = dot2(lo, xr[nb][8 * h + 2 * q], a[nb][0]);
          a[nb][1] = dot2(hi, xr[nb][8 * h + 2 * q + 1], a[nb][1]);
        }
      }
    }
    if (i + D < 8) cell_issue(c, i + D, f.v[i % D], lane);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) cd[nb * kSlotWords + i] = a[nb][0] + a[nb][1];
  }
}

// After the decode barrier: slot (l, 8c + i) += s / 256 D_i for the lane's
// column (columns past the matrix hold no record and stay zero).
template <int NB>
__device__ inline void cell_apply(const CellRows& c, uint32_t* S, int cw, uint32_t lane) {
  if (!c.live) return;
  const float* sc = reinterpret_cast<const float*>(S + LdsMap<NB>::sc) + lane * kSlotPitch + 8 * cw;
  const float* cd = reinterpret_cast<const float*>(S + LdsMap<NB>::cd) + lane * kSlotPitch + 8 * cw;
  float* slot = reinterpret_cast<float*>(S + LdsMap<NB>::slots) + lane * kSlotPitch + 8 * cw;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i >= c.rows) break;
    const float s256 = sc[i] * (1.f / 256.f);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      slot[nb * kSlotWords + i] = __builtin_fmaf(s256, cd[nb * kSlotWords + i], slot[nb * kSlotWords + i]);
  }
}

// Step 1, first part (wavefront 0): the activations of the tile's columns into
// LDS. It needs no tile header, so it goes out before the header is read.
template <int NB>
__device__ inline void copy_x(const GemvMat& T, int kt, uint32_t* S, uint32_t lane, int buf) {
  const int g0 = kt * kTileGroups;
  // copy i writes LDS chunk m = 64 i + lane, i.e. chunk m % 9
  // of column m / 9 (144 bytes per column); chunks 0-7 of a column are its
  // 128 bytes of x, chunk 8 is the gap and loads from outside the buffer
  // (zeros), as do columns past the matrix's last group
  const size_t K = (size_t)T.n_groups * kGroup;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const u32x4 xrs = make_rsrc(T.x + nb * K, (uint32_t)(K * 2));
    const uint32_t lds = lds_addr(S + LdsMap<NB>::x + buf * LdsMap<NB>::xbuf + nb * LdsMap<NB>::xrow);
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      // (the empty asm keeps the compiler from hoisting these lane-only
      // offsets out of the tile loop, where they would hold registers
      // through the decode)
      uint32_t m = 64u * i + lane;
      asm volatile("" : "+v"(m));
      const uint32_t c = m / 9u, p = m - 9u * c;
      dma16(xrs, lds + 1024u * i, p < 8u ? ((uint32_t)g0 + c) * 128u + 16u * p : kNoRecord);
    }
  }
}

// The rest of steps 1 and 2 for the decoding wavefronts: the width map, the
// first loads of every class, the biases and the record table.
template <int NB>
__device__ inline void tile_start(const GemvMat& T, const TileRef& t, uint32_t* S, int wave, Flight<0, NB>& f0,
                                  Flight<1, NB>& f1, Flight<2, NB>& f2, Flight<3, NB>& f3, uint32_t lane) {
  const u32x2 mp = map_load(t, lane);
  issue_first<0, NB>(t, wave, f0, lane);
  issue_first<1, NB>(t, wave, f1, lane);
  issue_first<2, NB>(t, wave, f2, lane);
  issue_first<3, NB>(t, wave, f3, lane);
  tile_prepare<NB>(t, wave, mp, S, lane, 0);
}

// One tile, all steps; the caller has passed a barrier since the last fold.
// With a compact in-cell residual (CELL) the workgroup has eight wavefronts:
// 0-3 decode, 4-7 form the residual dots and then fold the rows. Every
// wavefront meets the same two barriers, at the same points of the code
// (only the work between them depends on the wavefront's role), and nothing
// of one role's work stays in registers across a barrier.
template <int NB, bool CELL>
__device__ inline void coop_tile(const GemvMat& T, int rt, int kt, uint32_t* S, int wave, float (&yacc)[NB],
                                 uint32_t lane) {
  if constexpr (NB == 4 && !CELL) {
    // Four batch rows: the records go in quads (see issue_quad); their loads
    // follow the record table, so they go out after the first barrier.
    TileRef t;
    Flight<0, 4> f0;
    Flight<1, 4> f1;
    Flight<2, 4> f2;
    Flight<3, 4> f3;
    if (wave == 0) copy_x<4>(T, kt, S, lane, 0);
    t = tile_ref(T, rt, kt);
    // wavefronts 0-3 copy the activations and build the record table,
    // 4-7 only decode
    if (wave < kGemvWaves) tile_prepare<4>(t, wave, map_load(t, lane), S, lane, 0);
    __syncthreads();
    const uint32_t* Q = S + LdsMap<4>::table;
    const uint32_t c0 = __builtin_amdgcn_readfirstlane(Q[QuadMap::cnt + 0]);
    const uint32_t c1 = __builtin_amdgcn_readfirstlane(Q[QuadMap::cnt + 1]);
    const uint32_t c2 = __builtin_amdgcn_readfirstlane(Q[QuadMap::cnt + 2]);
    const uint32_t c3 = __builtin_amdgcn_readfirstlane(Q[QuadMap::cnt + 3]);
    issue_first_quad<0>(t, wave, f0, c0, S, lane);
    issue_first_quad<1>(t, wave, f1, c1, S, lane);
    issue_first_quad<2>(t, wave, f2, c2, S, lane);
    issue_first_quad<3>(t, wave, f3, c3, S, lane);
    run_class_quad<0>(t, f0, c0, S, wave, lane);
    run_class_quad<1>(t, f1, c1, S, wave, lane);
    run_class_quad<2>(t, f2, c2, S, wave, lane);
    run_class_quad<3>(t, f3, c3, S, wave, lane);
    __syncthreads();
    if (wave < kGemvWaves) fold_rows<4>(S, wave, yacc, lane);
    return;
  }
  const bool cell_wave = CELL && wave >= kGemvWaves;
  TileRef t;
  Flight<0, NB> f0;
  Flight<1, NB> f1;
  Flight<2, NB> f2;
  Flight<3, NB> f3;
  if (!cell_wave) {
    if (wave == 0) copy_x<NB>(T, kt, S, lane, 0);
    t = tile_ref(T, rt, kt);
    tile_start<NB>(T, t, S, wave, f0, f1, f2, f3, lane);
  }
  __syncthreads();
  if (!cell_wave) {
    run_class<0, NB, CELL>(t, f0, S, wave, lane);
    run_class<1, NB, CELL>(t, f1, S, wave, lane);
    run_class<2, NB, CELL>(t, f2, S, wave, lane);
    run_class<3, NB, CELL>(t, f3, S, wave, lane);
  } else if constexpr (CELL) {
    const int cw = wave - kGemvWaves;
    const CellRows c = cell_rows_of(T, rt, kt, cw, lane);
    CellFlight<NB> cf;
#pragma unroll
    for (int i = 0; i < cell_depth<NB>(); ++i) cell_issue(c, i, cf.v[i], lane);
    cell_dots<NB>(c, cf, S, cw, lane);
  }
  __syncthreads();
  if constexpr (CELL) {
    if (cell_wave) {
      const int cw = wave - kGemvWaves;
      cell_apply<NB>(cell_rows_of(T, rt, kt, cw, lane), S, cw, lane);
      fold_rows<NB>(S, cw, yacc, lane);
    }
  } else {
    fold_rows<NB>(S, wave, yacc, lane);
  }
}


// Sum over the 64 lanes (the total lands in every lane).
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

// Residual rows r = part, part + 4, ... of row-tile rt over all k-tiles:
// sum_k x[k] r[n][k], lane l on column l of each k-tile (64 fp16 of the
// row). The row sums go to Y[nb][r] (one wavefront per row).
template <int NB>
__device__ inline void residual_rows(const GemvMat& M, int rt, int part, float* Y, uint32_t lane) {
  const int r0 = rt * kTileRows, R = min(kTileRows, M.n_rows - r0);
  const size_t K = (size_t)M.n_groups * kGroup;
  constexpr int kRows = kTileRows / kGemvWaves;
  float acc[NB][kRows];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < kRows; ++i) acc[nb][i] = 0.f;
  for (int kt = 0; kt < M.k_tiles; ++kt) {
    const int g0 = kt * kTileGroups, Gt = min(kTileGroups, M.n_groups - g0);
    // Piece i of lane l is weights 8 (l % 8) .. + 7 of column 8 i + l / 8:
    // the (64 i + l)-th 16 bytes of the tile's stretch of x and of a
    // residual row, so consecutive lanes read consecutive bytes.
    uint32_t xr[NB][32];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint4* xp = reinterpret_cast<const uint4*>(M.x + nb * K + (size_t)g0 * kGroup);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool has = 8 * i + (int)(lane >> 3) < Gt;
        const uint4 v = has ? xp[64 * i + lane] : make_uint4(0u, 0u, 0u, 0u);
        xr[nb][4 * i + 0] = v.x;
        xr[nb][4 * i + 1] = v.y;
        xr[nb][4 * i + 2] = v.z;
        xr[nb][4 * i + 3] = v.w;
      }
    }
    // two rows' pieces in flight at a time
#pragma unroll
    for (int i = 0; i < kRows; i += 2) {
      const int ra = part + kGemvWaves * i, rb = ra + kGemvWaves;
      if (ra >= R) break;
      uint4 cur[2][8];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = h ? rb : ra;
        const uint4* rp =
            reinterpret_cast<const uint4*>(M.resid + (size_t)(r0 + min(r, R - 1)) * K + (size_t)g0 * kGroup);
#pragma unroll
        for (int q = 0; q < 8; ++q)
          cur[h][q] = (8 * q + (int)(lane >> 3) < Gt && r < R) ? rp[64 * q + lane] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if ((h ? rb : ra) >= R) break;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            a[0] = dot2(cur[h][q].x, xr[nb][4 * q + 0], a[0]);
            a[1] = dot2(cur[h][q].y, xr[nb][4 * q + 1], a[1]);
            a[2] = dot2(cur[h][q].z, xr[nb][4 * q + 2], a[2]);
            a[3] = dot2(cur[h][q].w, xr[nb][4 * q + 3], a[3]);
          }
          acc[nb][i + h] += wave_sum((a[0] + a[1]) + (a[2] + a[3]));
        }
      }
    }
  }
  if (lane == 0)
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      const int r = part + kGemvWaves * i;
      if (r < R)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) Y[nb * kTileRows + r] = acc[nb][i];
    }
}

// One workgroup per row-tile of every matrix of the launch. A matrix with one
// k-tile and no residual or levels is one tile per workgroup; otherwise the
// workgroup takes the row-tile's k-tiles (of every level) in order, then the
// residual's rows, at a raised wavefront priority (those workgroups come
// first in the launch and carry several tiles' work).
template <int NB, int MODE>
__host__ __device__ constexpr int gemv_waves() {
  return (MODE == kModeCell8 || MODE == kModeLevelPairs) ? 2 * kGemvWaves
         : (NB == 4 && MODE == kModePlain)              ? kQuadWaves
                                                        : kGemvWaves;
}

// (the second bound is the minimum of wavefronts per SIMD: four caps a
// wavefront at 128 VGPRs)
template <int NB, int MODE>
__host__ __device__ constexpr int gemv_min_waves() {
  return (NB == 1 || gemv_waves<NB, MODE>() == kQuadWaves) ? 4 : 2;
}

template <int NB, int MODE>
__global__ __launch_bounds__((gemv_waves<NB, MODE>() * 64), (gemv_min_waves<NB, MODE>())) void k_gemv(
    const GemvLaunch L) {
  constexpr bool RESID = MODE == kModeResid16, CELL = MODE == kModeCell8, PAIRS = MODE == kModeLevelPairs;
  extern __shared__ __align__(16) uint32_t S[];
  const int tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the workgroup's matrix: the last whose first workgroup is at or before
  // this one (the start table is read in one go)
  int mi = 0, wb = 0;
#pragma unroll
  for (int i = 1; i < 16; ++i) {
    const int b = L.wg_begin[i];
    mi = ((int)blockIdx.x >= b) ? i : mi;
    wb = ((int)blockIdx.x >= b) ? b : wb;
  }
  if (mi == 15) {
#pragma unroll
    for (int i = 16; i < kMaxMats; ++i) {
      const int b = L.wg_begin[i];
      mi = ((int)blockIdx.x >= b) ? i : mi;
      wb = ((int)blockIdx.x >= b) ? b : wb;
    }
  }
  // the fields the first steps need are read together (one wait instead of
  // a wait per field)
  const GemvMat& M = L.mats[mi];
  asm volatile("" ::"s"(M.tiles), "s"(M.stream), "s"(M.x), "s"(M.n_groups), "s"(M.row_tiles), "s"(M.k_tiles),
               "s"(M.stream_bytes), "s"(M.split), "s"(M.shared));
  const int j = (int)blockIdx.x - wb;
  for (int i = tid; i < NB * kSlotWords; i += gemv_waves<NB, MODE>() * kWave) {
    S[LdsMap<NB>::slots + i] = 0u;
    if (PAIRS) S[LdsMap<NB>::words + LdsMap<NB>::slots + i] = 0u;   // the second tile's slots
  }
  float yacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) yacc[nb] = 0.f;
  // the wavefronts that fold rows (the first four, or the four cell
  // wavefronts) hold row 8 fw + lane / 8 in lanes 8 r
  const int fw = CELL ? wave - kGemvWaves : wave;
  const bool folds = fw >= 0 && fw < kGemvWaves;
  const int row = 8 * fw + (int)(lane >> 3);
  if constexpr (PAIRS) {
    // Levels of one matrix at one batch row: the row-tile's tiles (levels in
    // order, k-tiles in order within a level) two at a time, wavefronts 0-3
    // on tile p with the first half of LDS, 4-7 on tile p + 1 with the
    // second. Each half's fold starts from -0 (which adds nothing), and the
    // rows get the first tile's sum, then the second's: the order of the
    // one-tile-at-a-time walk. With an odd count the second half repeats the
    // last tile and its sum is dropped.
    const int rt = j, grp = wave >> 2, gw = wave & 3;
    uint32_t* Sg = S + grp * LdsMap<NB>::words;
    float* xch = reinterpret_cast<float*>(S + 2 * LdsMap<NB>::words);   // [NB][32]: the second tile's row sums
    __builtin_amdgcn_s_setprio(2);
    const int tiles = M.levels * M.k_tiles;
    for (int p = 0; p < tiles; p += 2) {
      const int mp = min(p + grp, tiles - 1);
      const int lv = mp / M.k_tiles, kt = mp - lv * M.k_tiles;
      float part[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) part[nb] = -0.0f;
      coop_tile<NB, false>(L.mats[mi + lv], rt, kt, Sg, gw, part, lane);
      if (grp == 1 && (lane & 7u) == 0)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          xch[nb * kTileRows + row - 8 * kGemvWaves] = p + 1 < tiles ? part[nb] : -0.0f;
      __syncthreads();
      if (grp == 0)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) yacc[nb] = (yacc[nb] + part[nb]) + xch[nb * kTileRows + row];
    }
    const int r0 = rt * kTileRows, R = min(kTileRows, M.n_rows - r0);
    if (folds && (lane & 7u) == 0 && row < R)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) M.y[(size_t)nb * M.n_rows + r0 + row] = yacc[nb];
    return;
  }
  if (M.split) {
    // One tile of a row-tile with several: its row sums go to the scratch;
    // the workgroup that finishes the row-tile's last tile adds them in tile
    // order (the order the sequential path uses) and resets the counter.
    // (split launches have one level per matrix)
    const int tiles = M.k_tiles;
    const int rt = j / tiles, p = j - rt * tiles;
    coop_tile<NB, CELL>(M, rt, p, S, wave, yacc, lane);
    // The partial sums are device-scope atomic stores, which write through
    // the caches, so once they are complete (the wait before the barrier)
    // the counter may count this tile; the last workgroup reads them with
    // device-scope atomic loads. No cache-wide write-back is needed.
    float* part = L.partials + (size_t)(M.unit_base + rt * tiles) * NB * kTileRows;
    if (folds && (lane & 7u) == 0)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        __hip_atomic_store(&part[((size_t)p * NB + nb) * kTileRows + row], yacc[nb], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(VBQ_VMCNT_IMM(0));
    __syncthreads();
    __shared__ uint32_t last;
    if (tid == 0)
      last = __hip_atomic_fetch_add(&L.counters[M.ctr_base + rt], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     (uint32_t)(tiles - 1)
                 ? 1u
                 : 0u;
    __syncthreads();
    if (!last) return;
    const int r0 = rt * kTileRows, R = min(kTileRows, M.n_rows - r0);
    if (folds && (lane & 7u) == 0 && row < R)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float v = 0.f;
        for (int q = 0; q < tiles; ++q)
          v += __hip_atomic_load(&part[((size_t)q * NB + nb) * kTileRows + row], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        M.y[(size_t)nb * M.n_rows + r0 + row] = v;
      }
    if (tid == 0) __hip_atomic_store(&L.counters[M.ctr_base + rt], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int rt = j;
  if (!M.shared) {
    coop_tile<NB, CELL>(M, rt, 0, S, wave, yacc, lane);
  } else {
    __builtin_amdgcn_s_setprio(2);
    const int tiles = M.levels * M.k_tiles;
    for (int p = 0; p < tiles; ++p) {
      const int lv = p / M.k_tiles, kt = p - lv * M.k_tiles;
      coop_tile<NB, CELL>(L.mats[mi + lv], rt, kt, S, wave, yacc, lane);
    }
    if (RESID && M.resid) {
      float* Y = reinterpret_cast<float*>(S + LdsMap<NB>::ys);
      residual_rows<NB>(M, rt, wave, Y, lane);
      __syncthreads();
      const uint32_t row = 8u * wave + (lane >> 3);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) yacc[nb] += Y[nb * kTileRows + row];
    }
  }
  const int r0 = rt * kTileRows, R = min(kTileRows, M.n_rows - r0);
  if (folds && (lane & 7u) == 0 && row < R)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) M.y[(size_t)nb * M.n_rows + r0 + row] = yacc[nb];
}

// Scratch of the split GEMV, one copy per device: partial row sums, then
// row-tile counters. Counters start at zero (static storage) and the last
// workgroup of each row-tile sets its counter back to zero.
static __device__ __align__(256) uint8_t scratch[kScratchPartials * 4 + kScratchCounters * 4];

hipError_t gemv_scratch(float** partials, uint32_t** counters) {
  static void* ptr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr[dev] = p;
  }
  *partials = reinterpret_cast<float*>(ptr[dev]);
  *counters = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(ptr[dev]) + kScratchPartials * 4);
  return hipSuccess;
}

size_t gemv_lds_bytes(int nb, int mode) {
  if (mode == kModeLevelPairs) return 4u * (2 * LdsMap<1>::words + kTileRows);   // one batch row only
  const bool cell = mode == kModeCell8;
  switch (nb) {
    case 1: return 4u * (cell ? LdsMap<1>::words_cell : LdsMap<1>::words);
    case 2: return 4u * (cell ? LdsMap<2>::words_cell : LdsMap<2>::words);
    case 3: return 4u * LdsMap<3>::words;
    default: return 4u * LdsMap<4>::words;
  }
}

template <int NB, int MODE>
static hipError_t launch_one(const GemvLaunch& L, int n_wg, hipStream_t s) {
  const size_t lds = gemv_lds_bytes(NB, MODE);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv<NB, MODE>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((k_gemv<NB, MODE>), dim3(n_wg), dim3(gemv_waves<NB, MODE>() * kWave), lds, s, L);
  return hipGetLastError();
}

hipError_t launch_gemv(const GemvLaunch& L, int nb, int mode, int n_wg, hipStream_t s) {
  // passes of up to four batch rows without a residual, two with one
#define VBQ_CASE(N)                                                                      \
  case N:                                                                                \
    return mode == kModeResid16  ? launch_one<N, kModeResid16>(L, n_wg, s)               \
           : mode == kModeCell8 ? launch_one<N, kModeCell8>(L, n_wg, s)                  \
                                : launch_one<N, kModePlain>(L, n_wg, s);
  if (mode == kModeLevelPairs) {
    if (nb == 1) return launch_one<1, kModeLevelPairs>(L, n_wg, s);
    mode = kModePlain;   // several batch rows: one tile at a time
  }
  switch (nb) {
    VBQ_CASE(1)
    VBQ_CASE(2)
    case 3:
      return mode == kModePlain ? launch_one<3, kModePlain>(L, n_wg, s) : hipErrorInvalidValue;
    case 4:
      return mode == kModePlain ? launch_one<4, kModePlain>(L, n_wg, s) : hipErrorInvalidValue;
    default:
      return hipErrorInvalidValue;
  }
#undef VBQ_CASE
}

}  // namespace vbq
