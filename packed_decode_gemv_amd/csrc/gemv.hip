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
// v_dot2_f32_f16 multiplies two such values by two activations at once. The
// bias part, sum_j bias_j (x_2j + x_2j+1), depends only on x and the width,
// so it is computed once per (k-group, width) and subtracted per record.
//
// Work split: one wavefront decodes one tile (32 rows x 64 k-groups). Lane l
// owns the tile's column l, i.e. k-group 64 kt + l, and keeps that group's 64
// activations (per batch row) in registers for the whole tile. The tile's
// blocks each hold one record per active column, all of one width, so a
// wavefront decodes without divergence and without reading x from LDS. The
// lane finds its record's row from the column's 2-bit width map: the rows of
// one class, taken from a rotation that starts at row l, one per block. Each
// record adds s (dot - bias) + o sum(x) to its row in the wavefront's LDS row
// slice; the rotation spreads the lanes of one block over different rows.
// The blocks stream from HBM into a private LDS ring in 1 KiB pieces with
// buffer-to-LDS loads, so several kilobytes are in flight per wavefront
// without spending registers; the wait before a block is a closed form of its
// stream position. A workgroup of four wavefronts takes four row-tiles of a
// matrix with one k-tile, or one row-tile whose k-tiles (and levels) its
// wavefronts share, with a residual wavefronts 1-3 take the residual's rows;
// the wavefront slices are added in a fixed order at the end, so results are
// identical from run to run and no memory outside the workgroup is needed.
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
    ((k.mask[P] = vconst<field_mask(C, P)>(), k.magic[P] = vconst<field_magic(P)>()), ...);
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

// acc[nb][P % 2] += (bias + q_2P) x_2P + (bias + q_2P+1) x_2P+1 for pair P of
// the record (two accumulators split the dependent chain).
template <int C, int NB, int... P>
__device__ inline void record_dot(const Consts<C>& k, const uint32_t* w, const uint32_t (&xr)[NB][32], float (&a)[NB][2],
                                  std::integer_sequence<int, P...>) {
  (
      [&] {
        const uint32_t hv = pair_h2<C, P>(k, w);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) a[nb][P & 1] = dot2(hv, xr[nb][P], a[nb][P & 1]);
      }(),
      ...);
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

// ---- One tile -------------------------------------------------------------------
template <int NB>
struct TileX {
  uint32_t xr[NB][32];   // x pairs (x_2p, x_2p+1) of the lane's k-group, per batch row
  float xsum[NB];        // sum of the group's 64 activations
};

// Per-wavefront row slots: the record of column l in row r puts its value at
// slot l * kSlotPitch + r (each (row, column) pair has exactly one record per
// tile, so plain stores suffice); slot 32 of a column takes the stores of
// blocks the column has no record in. The pitch of 33 words puts the 32 rows
// read at one column on different banks.
constexpr int kSlotPitch = 33;
constexpr int kSlotWords = kWave * kSlotPitch;   // per batch row: 2112 words, 8448 bytes

// Buffer offset that lies outside every stream: loads from it return zeros
// without touching memory.
constexpr uint32_t kNoRecord = 0x80000000u;

// The record of the lane in one block.
template <int C>
struct Rec {
  uint32_t w[2 << C];
  uint32_t so;
};

// Blocks of a class whose records are in flight while one is decoded: about
// 6-9 KiB per wavefront at one batch row, fewer at more rows (their
// activations take the registers).
template <int C, int NB>
__host__ __device__ constexpr int depth() {
  return (16 >> C) / NB < 2 ? 2 : (16 >> C) / NB;
}

// Issues the loads of the lane's record in block i of a class whose stream
// position is ipos (advanced past the block). A column takes part in block i
// when it holds more than i records of the class; its record is the kk-th of
// the block, kk counting the taking-part columns below it. Columns that do
// not take part (and every column past the class's last block) load from
// kNoRecord, so every block issues the same loads and the count waits stay
// fixed.
template <int C>
__device__ inline void issue_block(__amdgpu_buffer_rsrc_t rs, uint32_t& ipos, uint32_t i, uint32_t n, Rec<C>& r) {
  constexpr uint32_t RB = 8u << C;
  const bool act = n > i;
  const uint64_t bal = __ballot(act);
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)__popcll(bal));
  const uint32_t kk = __mbcnt_hi((uint32_t)(bal >> 32), __mbcnt_lo((uint32_t)bal, 0u));
  const uint32_t ca = codes_area(C, m);
  const uint32_t oc = act ? ipos + RB * kk : kNoRecord;
  const uint32_t os = act ? ipos + ca + 4u * kk : kNoRecord;
  if constexpr (C == 0) {
    const u32x2 u = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)oc, 0, 0);
    r.w[0] = u.x;
    r.w[1] = u.y;
  } else {
#pragma unroll
    for (int h = 0; h < (int)RB / 16; ++h) {
      const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(oc + 16u * h), 0, 0);
      r.w[4 * h + 0] = u.x;
      r.w[4 * h + 1] = u.y;
      r.w[4 * h + 2] = u.z;
      r.w[4 * h + 3] = u.w;
    }
  }
  r.so = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)os, 0, 0);
  ipos += ca + up16(4u * m);
}

// Decodes the lane's record of one block into its row slot: the dot starts
// from -bias, so it ends as sum_k q_k x_k; the slot gets s * dot + o * sum(x).
template <int C, int NB>
__device__ inline void decode_block(const Consts<C>& k, const Rec<C>& r, const TileX<NB>& X, const float (&bias)[NB],
                                    bool act, uint32_t& rot, float* slot, uint32_t lane) {
  float a[NB][2];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    a[nb][0] = -bias[nb];
    a[nb][1] = 0.f;
  }
  record_dot<C, NB>(k, r.w, X.xr, a, std::make_integer_sequence<int, 32>{});
  // rot is empty exactly when the column sits the block out; then the slot
  // is the spare one and the row is not used.
  const uint32_t j = (uint32_t)__builtin_ctz(rot);
  rot &= rot - 1u;
  const uint32_t row = act ? ((j + lane) & 31u) : 32u;
  const float s = __half2float(__ushort_as_half((unsigned short)(r.so & 0xFFFFu)));
  const float o = __half2float(__ushort_as_half((unsigned short)(r.so >> 16)));
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) slot[nb * kSlotWords + row] = __builtin_fmaf(s, a[nb][0] + a[nb][1], o * X.xsum[nb]);
}

// The blocks of class C of a tile (I of them, starting at stream position
// pos): the loads of block i + D go out as block i is decoded, so D blocks
// are in flight. The loop is unrolled D times so that every block in flight
// has registers of its own.
template <int C, int NB>
__device__ inline void run_class(__amdgpu_buffer_rsrc_t rs, uint32_t I, uint32_t mask, const TileX<NB>& X,
                                 uint32_t& pos, float* slot, uint32_t lane) {
  constexpr int D = depth<C, NB>();
  const Consts<C> k = make_consts<C>();
  float bias[NB];
  class_bias<C, NB>(X.xr, bias, std::make_integer_sequence<int, 32>{});
  uint32_t rot = rotate_rows(mask, lane);
  const uint32_t n = (uint32_t)__builtin_popcount(mask);
  Rec<C> R[D];
#pragma unroll
  for (int d = 0; d < D; ++d) issue_block<C>(rs, pos, (uint32_t)d, n, R[d]);
  for (uint32_t i0 = 0; i0 < I; i0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const uint32_t i = i0 + d;
      if (i >= I) break;
      decode_block<C, NB>(k, R[d], X, bias, n > i, rot, slot, lane);
      issue_block<C>(rs, pos, i + D, n, R[d]);
    }
  }
}

// Adds tile (rt, kt) of matrix T into the lanes' row sums yacc (lane r < 32
// holds row r of the tile). S: this wavefront's slots, NB * kSlotWords.
template <int NB>
__device__ inline void packed_tile(const GemvMat& T, int rt, int kt, float (&yacc)[NB], float* S, uint32_t lane) {
  const int t = kt * T.row_tiles + rt;
  const uint4 hdr = *reinterpret_cast<const uint4*>(T.tiles + 4 * (size_t)t);
  const uint32_t base = __builtin_amdgcn_readfirstlane(hdr.x) * 16u;
  const uint32_t iw = __builtin_amdgcn_readfirstlane(hdr.z);
  const int R = min(kTileRows, T.n_rows - rt * kTileRows);
  const int g0 = kt * kTileGroups, Gt = min(kTileGroups, T.n_groups - g0);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(T.stream), (short)0, (int)T.stream_bytes, 0x00020000);
  const int lc = min((int)lane, Gt - 1);
  const bool live = (int)lane < Gt;
  const u32x2 mp = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)(base + 8u * (uint32_t)lc), 0, 0);
  TileX<NB> X;
  const size_t K = (size_t)T.n_groups * kGroup;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const uint4* xp = reinterpret_cast<const uint4*>(T.x + nb * K + (size_t)(g0 + lc) * kGroup);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 v = xp[i];
      X.xr[nb][4 * i + 0] = v.x;
      X.xr[nb][4 * i + 1] = v.y;
      X.xr[nb][4 * i + 2] = v.z;
      X.xr[nb][4 * i + 3] = v.w;
    }
  }
  // A full tile writes every slot once; a partial one clears them first, so
  // the rows and columns it lacks add zero.
  if (R < kTileRows || Gt < kTileGroups)
    for (uint32_t i = lane; i < NB * kSlotWords / 4; i += kWave)
      reinterpret_cast<float4*>(S)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  const ClassMasks km = class_masks(live ? mp.x : 0u, live ? mp.y : 0u, live ? R : 0);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 32; ++p) a[p & 3] = dot2(X.xr[nb][p], 0x3C003C00u, a[p & 3]);
    X.xsum[nb] = (a[0] + a[1]) + (a[2] + a[3]);
  }
  float* slot = S + lane * kSlotPitch;
  uint32_t pos = base + map_bytes((uint32_t)Gt);
  uint32_t I;
  if ((I = iw & 0xFFu)) run_class<0, NB>(rs, I, km.m[0], X, pos, slot, lane);
  if ((I = (iw >> 8) & 0xFFu)) run_class<1, NB>(rs, I, km.m[1], X, pos, slot, lane);
  if ((I = (iw >> 16) & 0xFFu)) run_class<2, NB>(rs, I, km.m[2], X, pos, slot, lane);
  if ((I = (iw >> 24) & 0xFFu)) run_class<3, NB>(rs, I, km.m[3], X, pos, slot, lane);
  // Row sums: lanes r and r + 32 add the slots of columns 0-31 and 32-63 of
  // row r, in column order, then combine.
  const uint32_t r = lane & 31u, h = lane >> 5;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float* col = S + nb * kSlotWords + h * 32u * kSlotPitch + r;
    float v = 0.f;
#pragma unroll 8
    for (int l = 0; l < 32; ++l) v += col[l * kSlotPitch];
    v += __shfl_xor(v, 32, kWave);
    yacc[nb] += v;
  }
}

// Sum over the 64 lanes (the total lands in every lane).
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

// Residual rows r = part, part + 3, ... of row-tile rt over all k-tiles:
// y += sum_k x[k] r[n][k], lane l on column l of each k-tile (64 fp16 of the
// row), the next row's loads issued before the current row is summed.
template <int NB>
__device__ inline void residual_rows(const GemvMat& M, int rt, int part, float* Y, uint32_t lane) {
  const int r0 = rt * kTileRows, R = min(kTileRows, M.n_rows - r0);
  const size_t K = (size_t)M.n_groups * kGroup;
  for (int kt = 0; kt < M.k_tiles; ++kt) {
    const int g0 = kt * kTileGroups, Gt = min(kTileGroups, M.n_groups - g0);
    const int lc = min((int)lane, Gt - 1);
    const bool live = (int)lane < Gt;
    uint32_t xr[NB][32];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint4* xp = reinterpret_cast<const uint4*>(M.x + nb * K + (size_t)(g0 + lc) * kGroup);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint4 v = xp[i];
        xr[nb][4 * i + 0] = live ? v.x : 0u;
        xr[nb][4 * i + 1] = live ? v.y : 0u;
        xr[nb][4 * i + 2] = live ? v.z : 0u;
        xr[nb][4 * i + 3] = live ? v.w : 0u;
      }
    }
    auto load_row = [&](int r, uint4 (&d)[8]) {
      const uint4* rp = reinterpret_cast<const uint4*>(M.resid + (size_t)(r0 + r) * K + (size_t)(g0 + lc) * kGroup);
#pragma unroll
      for (int i = 0; i < 8; ++i) d[i] = rp[i];
    };
    if (part >= R) continue;
    uint4 cur[8], nxt[8];
    load_row(part, cur);
    for (int r = part; r < R; r += 3) {
      const bool more = r + 3 < R;
      if (more) load_row(r + 3, nxt);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          a[0] = dot2(cur[i].x, xr[nb][4 * i + 0], a[0]);
          a[1] = dot2(cur[i].y, xr[nb][4 * i + 1], a[1]);
          a[2] = dot2(cur[i].z, xr[nb][4 * i + 2], a[2]);
          a[3] = dot2(cur[i].w, xr[nb][4 * i + 3], a[3]);
        }
        const float v = wave_sum((a[0] + a[1]) + (a[2] + a[3]));
        if (lane == 0) Y[nb * kTileRows + r] += v;
      }
      if (more) {
#pragma unroll
        for (int i = 0; i < 8; ++i) cur[i] = nxt[i];
      }
    }
  }
}

template <int NB, bool RESID>
__global__ __launch_bounds__(kGemvWaves * 64) void k_gemv(const GemvLaunch L) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int mi = 0;
  for (int i = 1; i < L.n_mats; ++i) mi = ((int)blockIdx.x >= L.mats[i].wg_begin) ? i : mi;
  const GemvMat& M = L.mats[mi];
  const int j = (int)blockIdx.x - M.wg_begin;
  // LDS: the wavefronts' row sums [waves][NB][32], then per wavefront its
  // slots (NB * kSlotWords words).
  float* Ys = reinterpret_cast<float*>(smem);
  float* S = reinterpret_cast<float*>(smem + kGemvWaves * NB * kTileRows * 4) + wave * NB * kSlotWords;
  float yacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) yacc[nb] = 0.f;

  if (!M.shared) {
    // Four row-tiles of a matrix with one k-tile: the wavefronts are independent.
    const int rt = j * kGemvWaves + wave;
    if (rt >= M.row_tiles) return;
    packed_tile<NB>(M, rt, 0, yacc, S, lane);
    const int r0 = rt * kTileRows, R = min(kTileRows, M.n_rows - r0);
    if ((int)lane < R)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) M.y[(size_t)nb * M.n_rows + r0 + lane] = yacc[nb];
    return;
  }

  // One row-tile: its k-tiles (of every level) spread over the wavefronts, or
  // with a residual the packed k-tiles on wavefront 0 and the residual's rows
  // on wavefronts 1-3.
  const int rt = j;
  float* Y = Ys + wave * NB * kTileRows;
  if (RESID && M.resid) {
    if (wave == 0) {
      for (int kt = 0; kt < M.k_tiles; ++kt) packed_tile<NB>(M, rt, kt, yacc, S, lane);
      if (lane < 32)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) Y[nb * kTileRows + lane] = yacc[nb];
    } else {
      for (int i = (int)lane; i < NB * kTileRows; i += kWave) Y[i] = 0.f;
      residual_rows<NB>(M, rt, wave - 1, Y, lane);
    }
  } else {
    const int pairs = M.levels * M.k_tiles;
    for (int p = wave; p < pairs; p += kGemvWaves) {
      const int lv = p / M.k_tiles, kt = p - lv * M.k_tiles;
      packed_tile<NB>(L.mats[mi + lv], rt, kt, yacc, S, lane);
    }
    if (lane < 32)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) Y[nb * kTileRows + lane] = yacc[nb];
  }
  __syncthreads();
  const int r0 = rt * kTileRows, R = min(kTileRows, M.n_rows - r0);
  for (int i = tid; i < NB * kTileRows; i += kGemvWaves * kWave) {
    const int nb = i / kTileRows, r = i - nb * kTileRows;
    float v = Ys[i];
#pragma unroll
    for (int w = 1; w < kGemvWaves; ++w) v += Ys[w * NB * kTileRows + i];
    if (r < R) M.y[(size_t)nb * M.n_rows + r0 + r] = v;
  }
}

size_t gemv_lds_bytes(int nb) {
  return (size_t)kGemvWaves * ((size_t)nb * kTileRows * 4 + (size_t)nb * kSlotWords * 4);
}

template <int NB, bool RESID>
static hipError_t launch_one(const GemvLaunch& L, int n_wg, hipStream_t s) {
  const size_t lds = gemv_lds_bytes(NB);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv<NB, RESID>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 64);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((k_gemv<NB, RESID>), dim3(n_wg), dim3(kGemvWaves * kWave), lds, s, L);
  return hipGetLastError();
}

hipError_t launch_gemv(const GemvLaunch& L, int nb, bool resid, int n_wg, hipStream_t s) {
#define VBQ_CASE(N)                                                                        \
  case N:                                                                                  \
    return resid ? launch_one<N, true>(L, n_wg, s) : launch_one<N, false>(L, n_wg, s);
  switch (nb) {
    VBQ_CASE(1)
    VBQ_CASE(2)
    VBQ_CASE(3)
    VBQ_CASE(4)
    default:
      return hipErrorInvalidValue;
  }
#undef VBQ_CASE
}

}  // namespace vbq
