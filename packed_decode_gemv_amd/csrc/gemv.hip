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
  ((k.mask[P] = vconst<field_mask(C, P)>(), k.magic[P] = vconst<field_magic(P)>()), ...);
  return k;
}

template <int C>
__device__ inline Consts<C> make_consts() {
  return make_consts_impl<C>(std::make_integer_sequence<int, 10>{});
}

// acc[nb][P % 4] += (bias + q_2P) x_2P + (bias + q_2P+1) x_2P+1 for pair P of
// the record (four accumulators split the dependent chain).
template <int C, int P, int NB>
__device__ inline void pair_step(const Consts<C>& k, const uint32_t* w, const uint32_t (&xr)[NB][32],
                                 float (&a)[NB][4]) {
  constexpr int H = 16 >> C, F = P % H, FP = field_pos(C, F);
  const uint32_t src = shifted<shift_kind(C, F)>(w[P / H]);
  const uint32_t hv = (src & k.mask[FP]) | k.magic[FP];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) a[nb][P & 3] = dot2(hv, xr[nb][P], a[nb][P & 3]);
}

template <int C, int NB, int... P>
__device__ inline void record_dot(const Consts<C>& k, const uint32_t* w, const uint32_t (&xr)[NB][32], float (&a)[NB][4],
                                  std::integer_sequence<int, P...>) {
  (pair_step<C, P, NB>(k, w, xr, a), ...);
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

// ---- Synchronisation helpers ---------------------------------------------------

// Waits until at most n vector-memory instructions of this wavefront are
// outstanding (n is wavefront-uniform, clamped to [0, 63]). Loads complete in
// issue order, so this waits for everything issued before the last n.
// s_waitcnt takes its count as an immediate, so this jumps into a table of
// 64 (wait, branch) pairs of 8 bytes each: s_getpc_b64 yields the address of
// the next instruction and the table starts four 4-byte instructions later.
__device__ inline void wait_vmcnt(int n) {
  n = n < 0 ? 0 : (n > 63 ? 63 : n);
  asm volatile(
      "s_getpc_b64 s[94:95]\n\t"
      "s_lshl3_add_u32 s96, %0, 16\n\t"
      "s_add_u32 s94, s94, s96\n\t"
      "s_addc_u32 s95, s95, 0\n\t"
      "s_setpc_b64 s[94:95]\n\t"
      "s_waitcnt vmcnt(0)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(1)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(2)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(3)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(4)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(5)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(6)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(7)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(8)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(9)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(10)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(11)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(12)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(13)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(14)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(15)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(16)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(17)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(18)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(19)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(20)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(21)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(22)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(23)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(24)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(25)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(26)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(27)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(28)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(29)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(30)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(31)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(32)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(33)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(34)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(35)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(36)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(37)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(38)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(39)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(40)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(41)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(42)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(43)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(44)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(45)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(46)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(47)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(48)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(49)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(50)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(51)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(52)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(53)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(54)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(55)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(56)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(57)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(58)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(59)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(60)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(61)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(62)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      "s_waitcnt vmcnt(63)\n\ts_branch .Lvbq_wait_end_%=\n\t"
      ".Lvbq_wait_end_%=:"
      :
      : "s"(__builtin_amdgcn_readfirstlane(n))
      : "s94", "s95", "s96", "scc", "memory");
}

// ---- Streaming ring --------------------------------------------------------------
// A wavefront streams bytes [src, src + span) of a matrix's stream into its
// LDS ring in 1 KiB pieces: piece p (stream bytes [1024 p, 1024 p + 1024) of
// the span) goes to ring slot p mod S. Piece p is issued once every block
// ending before byte 1024 (p - S + 1) of the span is decoded, i.e. up to
// floor(pos / 1024) + S pieces are out after the blocks before pos; a block
// ending at e needs the first ceil(e / 1024). A block holds at most 4352
// bytes (64 eight-bit records and their scale/offset words), so it spans at
// most six pieces and S >= 8 always has them in the ring at once.
struct Ring {
  u32x4 rsrc;
  uint32_t lds;       // LDS address of slot 0
  uint32_t slots;     // S (a power of two)
  uint32_t src;       // stream byte of the first piece
  uint32_t np;        // pieces of the span
  uint32_t issued;    // pieces issued so far
};

__device__ inline void ring_issue(Ring& r, uint32_t upto, uint32_t lane16) {
  upto = min(upto, r.np);
  for (; r.issued < upto; ++r.issued)
    dma16(r.rsrc, r.lds + ((r.issued & (r.slots - 1u)) << 10), r.src + (r.issued << 10) + lane16);
}

// ---- One tile -------------------------------------------------------------------
template <int NB>
struct TileX {
  uint32_t xr[NB][32];   // x pairs (x_2p, x_2p+1) of the lane's k-group, per batch row
  float xsum[NB];        // sum of the group's 64 activations
};

// Decodes the blocks of class C of a tile: I blocks, the lane's column holding
// n records of the class (rows in mask, visited from the rotation at row l).
template <int C, int NB>
__device__ inline void run_class(Ring& rg, const uint8_t* ring, uint32_t ring_mask, uint32_t I, uint32_t n,
                                 uint32_t mask, const TileX<NB>& X, uint32_t& pos, float* Y, uint32_t lane) {
  constexpr int B = 1 << C;
  const Consts<C> k = make_consts<C>();
  float bias[NB];
  class_bias<C, NB>(X.xr, bias, std::make_integer_sequence<int, 32>{});
  uint32_t rot = rotate_rows(mask, lane);
  const uint32_t lane16 = 16u * lane;
  for (uint32_t i = 0; i < I; ++i) {
    const bool act = n > i;
    const uint64_t bal = __ballot(act);
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)__popcll(bal));
    const uint32_t kk = __mbcnt_hi((uint32_t)(bal >> 32), __mbcnt_lo((uint32_t)bal, 0u));
    const uint32_t ca = codes_area(C, m), bytes = ca + up16(4u * m);
    wait_vmcnt((int)rg.issued - (int)((pos + bytes + 1023u) >> 10));
    if (act) {
      uint32_t w[2 * B];
      const uint32_t cb = pos + (8u * B) * kk;
      if constexpr (C == 0) {
        const uint2 u = *reinterpret_cast<const uint2*>(ring + (cb & ring_mask));
        w[0] = u.x;
        w[1] = u.y;
      } else {
#pragma unroll
        for (int h = 0; h < B / 2; ++h) {
          const uint4 u = *reinterpret_cast<const uint4*>(ring + ((cb + 16u * h) & ring_mask));
          w[4 * h + 0] = u.x;
          w[4 * h + 1] = u.y;
          w[4 * h + 2] = u.z;
          w[4 * h + 3] = u.w;
        }
      }
      const uint32_t so = *reinterpret_cast<const uint32_t*>(ring + ((pos + ca + 4u * kk) & ring_mask));
      const uint32_t j = (uint32_t)__builtin_ctz(rot);
      rot &= rot - 1u;
      const uint32_t row = (j + lane) & 31u;
      float a[NB][4];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) a[nb][0] = a[nb][1] = a[nb][2] = a[nb][3] = 0.f;
      record_dot<C, NB>(k, w, X.xr, a, std::make_integer_sequence<int, 32>{});
      const float s = __half2float(__ushort_as_half((unsigned short)(so & 0xFFFFu)));
      const float o = __half2float(__ushort_as_half((unsigned short)(so >> 16)));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float dot = (a[nb][0] + a[nb][1]) + (a[nb][2] + a[nb][3]);
        atomicAdd(&Y[nb * kTileRows + row], __builtin_fmaf(s, dot - bias[nb], o * X.xsum[nb]));
      }
    }
    pos += bytes;
    // Refill the freed ring slots once this block's LDS reads are complete.
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    ring_issue(rg, (pos >> 10) + rg.slots, lane16);
  }
}

// Adds tile (rt, kt) of matrix T into the wavefront's row slice Y [NB][32].
template <int NB>
__device__ inline void packed_tile(const GemvMat& T, int rt, int kt, float* Y, const uint8_t* ring, uint32_t ring_bytes,
                                   uint32_t lane) {
  const int t = kt * T.row_tiles + rt;
  const uint4 hdr = *reinterpret_cast<const uint4*>(T.tiles + 4 * (size_t)t);
  const uint32_t base = __builtin_amdgcn_readfirstlane(hdr.x) * 16u;
  const uint32_t size = __builtin_amdgcn_readfirstlane(hdr.y) * 16u;
  const uint32_t iw = __builtin_amdgcn_readfirstlane(hdr.z);
  const int R = min(kTileRows, T.n_rows - rt * kTileRows);
  const int g0 = kt * kTileGroups, Gt = min(kTileGroups, T.n_groups - g0);
  const uint32_t mb = map_bytes((uint32_t)Gt);
  Ring rg;
  rg.rsrc = make_rsrc(T.stream, T.stream_bytes);
  rg.lds = lds_addr(ring);
  rg.slots = ring_bytes >> 10;
  rg.src = base + mb;
  rg.np = (size - mb + 1023u) >> 10;
  rg.issued = 0;
  // The first pieces go out before the map and x loads: those loads complete
  // in order after the pieces, so once x is in registers the pieces are in
  // the ring as well.
  ring_issue(rg, rg.slots, 16u * lane);
  const int lc = min((int)lane, Gt - 1);
  const bool live = (int)lane < Gt;
  const uint2 mp = *reinterpret_cast<const uint2*>(T.stream + base + 8u * (uint32_t)lc);
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
  const ClassMasks km = class_masks(live ? mp.x : 0u, live ? mp.y : 0u, live ? R : 0);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 32; ++p) a[p & 3] = dot2(X.xr[nb][p], 0x3C003C00u, a[p & 3]);
    X.xsum[nb] = (a[0] + a[1]) + (a[2] + a[3]);
  }
  const uint32_t ring_mask = ring_bytes - 1u;
  uint32_t pos = 0;
  uint32_t I;
  if ((I = iw & 0xFFu)) run_class<0, NB>(rg, ring, ring_mask, I, __popc(km.m[0]), km.m[0], X, pos, Y, lane);
  if ((I = (iw >> 8) & 0xFFu)) run_class<1, NB>(rg, ring, ring_mask, I, __popc(km.m[1]), km.m[1], X, pos, Y, lane);
  if ((I = (iw >> 16) & 0xFFu)) run_class<2, NB>(rg, ring, ring_mask, I, __popc(km.m[2]), km.m[2], X, pos, Y, lane);
  if ((I = (iw >> 24) & 0xFFu)) run_class<3, NB>(rg, ring, ring_mask, I, __popc(km.m[3]), km.m[3], X, pos, Y, lane);
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
  float* Ys = reinterpret_cast<float*>(smem);                       // [waves][NB][32]
  float* Y = Ys + wave * NB * kTileRows;
  const uint8_t* ring = smem + kGemvWaves * NB * kTileRows * 4 + wave * L.ring_bytes;
  for (int i = (int)lane; i < NB * kTileRows; i += kWave) Y[i] = 0.f;

  if (!M.shared) {
    // Four row-tiles of a matrix with one k-tile: the wavefronts are independent.
    const int rt = j * kGemvWaves + wave;
    if (rt >= M.row_tiles) return;
    packed_tile<NB>(M, rt, 0, Y, ring, L.ring_bytes, lane);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the row slice is complete
    const int r0 = rt * kTileRows, R = min(kTileRows, M.n_rows - r0);
    for (int i = (int)lane; i < NB * kTileRows; i += kWave) {
      const int nb = i / kTileRows, r = i - nb * kTileRows;
      if (r < R) M.y[(size_t)nb * M.n_rows + r0 + r] = Y[i];
    }
    return;
  }

  // One row-tile: its k-tiles (of every level) spread over the wavefronts, or
  // with a residual the packed k-tiles on wavefront 0 and the residual's rows
  // on wavefronts 1-3.
  const int rt = j;
  if (RESID && M.resid) {
    if (wave == 0) {
      for (int kt = 0; kt < M.k_tiles; ++kt) packed_tile<NB>(M, rt, kt, Y, ring, L.ring_bytes, lane);
    } else {
      residual_rows<NB>(M, rt, wave - 1, Y, lane);
    }
  } else {
    const int pairs = M.levels * M.k_tiles;
    for (int p = wave; p < pairs; p += kGemvWaves) {
      const int lv = p / M.k_tiles, kt = p - lv * M.k_tiles;
      packed_tile<NB>(L.mats[mi + lv], rt, kt, Y, ring, L.ring_bytes, lane);
    }
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

size_t gemv_lds_bytes(int nb, uint32_t ring_bytes) {
  return (size_t)kGemvWaves * ((size_t)nb * kTileRows * 4 + ring_bytes);
}

template <int NB, bool RESID>
static hipError_t launch_one(const GemvLaunch& L, int n_wg, hipStream_t s) {
  const size_t lds = gemv_lds_bytes(NB, L.ring_bytes);
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
