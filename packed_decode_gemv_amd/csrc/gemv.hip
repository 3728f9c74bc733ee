// Fused dequantise-and-multiply GEMV over the block stream of a packed matrix.
//
// Follows the VBQ abstract (page "In-Cell Learning: Language Models That
// Update Their Own Weights in Sequence Without Changing the File They Ship"):
// 64-weight groups with widths {1,2,4,8}, packed storage, and a fused
// dequantise-and-multiply for memory-bandwidth-bound decode. The optional
// residual term follows the CellFill abstract (page "Nothing Changed but the
// Model: CellFill -- Bounded In-Cell Learning for Bit-Identical, Revocable
// Updates to Quantized LLMs"): the served weight is the dequantised code plus a
// per-weight residual, and dropping the residual revokes the update.
//
// Per group g of row n and batch row b:
//   y[b][n] += s_g * sum_k q_k x_k + o_g * sum_k x_k        (k in the group)
// The inner sum never materialises weights: a code field is OR-ed into the
// mantissa of an fp16 whose exponent makes the field's unit exactly 1, so the
// fp16 value is bias + q with bias = 2^(10-p) for a field at mantissa bit p.
// v_dot2_f32_f16 multiplies two such values by two activations at once. The
// bias part, sum_j bias_j (x_2j + x_2j+1), depends only on x and the field
// positions of the width, so it is computed once per (k-group, width) in LDS
// and subtracted per group. Fields sit at mantissa bits 0..9 where they
// already are in the word, so most need no shift; masks and exponent patterns
// live in registers so that building one fp16 pair is a single v_and_or_b32.
//
// Work split: a workgroup owns a range of row-tiles of one k-tile column of
// one matrix (several matrices per launch for batched calls). Those tiles are
// consecutive in the stream, so the workgroup's data is one contiguous byte
// range; its blocks are split evenly over the wavefronts, and each wavefront
// streams its own sub-range from HBM into a private LDS ring in 1 KiB pieces
// with buffer-to-LDS loads, keeping several kilobytes in flight without
// spending registers. Because a wavefront's bytes are one stream, the wait
// before decoding a block is a closed form (pieces issued minus pieces that
// cover the block's end). Each block holds records of a single width, so a
// wavefront decodes without divergence; neighbouring lanes mostly share a
// k-group, so their x reads are broadcasts. Wavefronts accumulate rows in
// their own LDS slices, summed in a fixed order at the end; with several
// k-tiles, the last workgroup of a row range to finish adds the partial rows
// in k-tile order. Results are therefore identical from run to run.
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
__host__ __device__ constexpr float field_bias(int c, int f) { return (float)(1 << (10 - field_pos(c, f))); }

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

template <int E>
__device__ inline uint32_t lane_of(const uint4& v) {
  return E == 0 ? v.x : E == 1 ? v.y : E == 2 ? v.z : v.w;
}

// Masks and exponent patterns of one width class, held in VGPRs for the whole
// block loop (entries a class never uses are dead and cost nothing).
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

// Decode geometry of class C: pairs per word, words of one record (part) a
// lane decodes at a time and its pairs, records per lane (1-bit: four
// consecutive records) and lanes per record (8-bit: four quarters).
template <int C>
struct Geo {
  static constexpr int H = 16 >> C;                              // pairs per word
  static constexpr int NW = C == 0 ? 2 : C == 2 ? 8 : 4;         // words per record part
  static constexpr int NP = NW * H;                              // pairs per part: 32, 32, 32, 8
  static constexpr int RPL = C == 0 ? 4 : 1;                     // records per lane
  static constexpr int LPR = C == 3 ? 4 : 1;                     // lanes per record
};

template <int C, int J, int NB>
__device__ inline void pair_step(const Consts<C>& k, const uint32_t* w, const uint4 (&xv)[NB], float (&acc)[NB]) {
  constexpr int H = Geo<C>::H, F = J % H, P = field_pos(C, F);
  const uint32_t src = shifted<shift_kind(C, F)>(w[J / H]);
  const uint32_t hv = (src & k.mask[P]) | k.magic[P];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = dot2(hv, lane_of<J & 3>(xv[nb]), acc[nb]);
}

template <int C, int CH, int NB>
__device__ inline void chunk_compute(const Consts<C>& k, const uint32_t* w, const uint4 (&xv)[NB], float (&acc)[NB]) {
  pair_step<C, 4 * CH + 0, NB>(k, w, xv, acc);
  pair_step<C, 4 * CH + 1, NB>(k, w, xv, acc);
  pair_step<C, 4 * CH + 2, NB>(k, w, xv, acc);
  pair_step<C, 4 * CH + 3, NB>(k, w, xv, acc);
}

template <int C, int NB, int CH0, int G, int... g>
__device__ inline void compute_group(const Consts<C>& k, const uint32_t* w, const uint4 (&xv)[G][NB], float (&acc)[NB],
                                     std::integer_sequence<int, g...>) {
  (chunk_compute<C, CH0 + g, NB>(k, w, xv[g], acc), ...);
}

// acc[nb] += sum_j (bias_j + q_2j) x_2j + (bias_j + q_2j+1) x_2j+1 over the
// lane's pairs. xk points at the lane's first pair in the x table of batch
// row 0; batch rows are xstride dwords apart. The x chunks of a group (all of
// them for one batch row) are loaded into registers before any is used, so a
// record waits for LDS once rather than once per chunk; the scheduling
// barrier keeps the compiler from interleaving loads and uses again.
template <int C, int NB, int CH0>
__device__ inline void dot_from(const Consts<C>& k, const uint32_t* w, const uint32_t* xk, int xstride,
                                float (&acc)[NB]) {
  constexpr int NCH = Geo<C>::NP / 4;
  if constexpr (CH0 < NCH) {
    constexpr int GMAX = 8 / NB > 1 ? 8 / NB : 1;
    constexpr int G = NCH - CH0 < GMAX ? NCH - CH0 : GMAX;
    uint4 xv[G][NB];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) xv[g][nb] = *reinterpret_cast<const uint4*>(xk + nb * xstride + 4 * (CH0 + g));
    __builtin_amdgcn_sched_barrier(0);
    compute_group<C, NB, CH0, G>(k, w, xv, acc, std::make_integer_sequence<int, G>{});
    dot_from<C, NB, CH0 + G>(k, w, xk, xstride, acc);
  }
}

// ---- Synchronisation helpers ---------------------------------------------------

// Waits until at most n vector-memory instructions of this wavefront are
// outstanding (n is wavefront-uniform, clamped to [0, 63]). Loads complete in
// issue order, so this waits for everything issued before the last n.
// s_waitcnt takes its count as an immediate, so this jumps into a table of
// 64 (wait, branch) pairs of 8 bytes each: s_getpc_b64 yields the address of
// the next instruction and the table starts four 4-byte instructions later.
// A switch over the 64 counts compiles into a long chain of scalar branches.
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

// Workgroup barrier for data written with ordinary LDS stores. It waits for
// this wavefront's LDS operations only: a full __syncthreads() would also wait
// for every buffer-to-LDS copy in flight (they count as memory loads), which
// drains the rings. Ring data is covered by the count waits instead.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---- Workgroup tile list -------------------------------------------------------
// Lane i (< nt) of every wavefront holds the header of tile i of the
// workgroup (consecutive tiles of one k-tile column) and the number of blocks
// before it; lane nt holds the header of the next tile, whose byte base ends
// the workgroup's range.
struct TileLanes {
  uint32_t byte0, n01, n23, pre, cpre;   // per lane
  int nt, total;                         // tiles, blocks (uniform)
  uint32_t cost;                         // decode cost of all blocks (uniform)
};

__device__ inline uint32_t tile_blocks(uint32_t n01, uint32_t n23) {
  return seg_blocks(0, n01 & 0xFFFF) + seg_blocks(1, n01 >> 16) + seg_blocks(2, n23 & 0xFFFF) +
         seg_blocks(3, n23 >> 16);
}

// Relative decode cost of one block per width class (VALU instructions of a
// wavefront: a 1-bit block holds four records per lane, the others one).
__host__ __device__ constexpr uint32_t block_cost(int c) { return c == 0 ? 6u : c == 3 ? 1u : 2u; }

__device__ inline uint32_t tile_cost(uint32_t n01, uint32_t n23) {
  return block_cost(0) * seg_blocks(0, n01 & 0xFFFF) + block_cost(1) * seg_blocks(1, n01 >> 16) +
         block_cost(2) * seg_blocks(2, n23 & 0xFFFF) + block_cost(3) * seg_blocks(3, n23 >> 16);
}

// Exclusive sum over the 64 lanes (DPP row shifts, then row broadcasts).
__device__ inline uint32_t wave_excl_sum(uint32_t v) {
  uint32_t inc = v;
  inc += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)inc, 0x111, 0xF, 0xF, false);
  inc += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)inc, 0x112, 0xF, 0xF, false);
  inc += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)inc, 0x114, 0xF, 0xF, false);
  inc += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)inc, 0x118, 0xF, 0xF, false);
  inc += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)inc, 0x142, 0xA, 0xF, false);
  inc += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)inc, 0x143, 0xC, 0xF, false);
  return inc - v;
}

// h: the header loaded by this lane (zeros past the end of the list).
__device__ inline TileLanes make_tile_lanes(const uint4& h, int nt, uint32_t lane) {
  TileLanes T;
  T.nt = nt;
  T.byte0 = h.y * 16u;
  T.n01 = (int)lane < nt ? h.z : 0u;
  T.n23 = (int)lane < nt ? h.w : 0u;
  const uint32_t nb = tile_blocks(T.n01, T.n23), cb = tile_cost(T.n01, T.n23);
  T.pre = wave_excl_sum(nb);
  T.cpre = wave_excl_sum(cb);
  T.total = __builtin_amdgcn_readlane(T.pre + nb, nt - 1);
  T.cost = __builtin_amdgcn_readlane(T.cpre + cb, nt - 1);
  return T;
}

// First block of the workgroup whose cost prefix (the summed block_cost of
// the blocks before it) is at least `target` (< the workgroup's total cost),
// as wavefront-uniform (block index, byte offset). Blocks of a class are laid
// out back to back and all but the last are full, so the search is a ballot
// over the tiles' cost prefixes and closed forms per class.
__device__ inline void first_block_at(const TileLanes& T, uint32_t target, uint32_t lane, uint32_t& j_out,
                                      uint32_t& byte_out) {
  const int t = __builtin_popcountll(__builtin_amdgcn_ballot_w64((int)lane < T.nt && T.cpre <= target)) - 1;
  const uint32_t n01 = __builtin_amdgcn_readlane(T.n01, t), n23 = __builtin_amdgcn_readlane(T.n23, t);
  const uint32_t n[4] = {n01 & 0xFFFFu, n01 >> 16, n23 & 0xFFFFu, n23 >> 16};
  uint32_t s = __builtin_amdgcn_readlane(T.byte0, t), j = __builtin_amdgcn_readlane(T.pre, t);
  uint32_t cs = __builtin_amdgcn_readlane(T.cpre, t);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (target <= cs) break;   // the class (or the next tile) starts at or after the target
    constexpr uint32_t kFull[4] = {block_bytes(0, block_records(0)), block_bytes(1, block_records(1)),
                                   block_bytes(2, block_records(2)), block_bytes(3, block_records(3))};
    const uint32_t kc = seg_blocks(c, n[c]);
    const uint32_t k = (target - cs + block_cost(c) - 1u) / block_cost(c);
    if (k < kc) {
      j += k;
      s += k * kFull[c];
      break;
    }
    cs += block_cost(c) * kc;
    s += (uint32_t)seg_bytes(c, n[c]);
    j += kc;
  }
  j_out = j;
  byte_out = s;
}

// ---- Per-lane block lookup ---------------------------------------------------------
// Where block j of the workgroup (j < total) sits, computed with vector
// instructions so that a whole wavefront finds its blocks at once.
struct BlockInfo {
  uint32_t byte, size, m;
  int c, t;
};

__device__ inline uint32_t sel4(int c, uint32_t a, uint32_t b, uint32_t d, uint32_t e) {
  return c == 0 ? a : c == 1 ? b : c == 2 ? d : e;
}

// Tile holding block j when the same j is in every lane (wavefront-uniform).
__device__ inline int tile_of(const TileLanes& T, uint32_t j, uint32_t lane) {
  return __builtin_popcountll(__builtin_amdgcn_ballot_w64((int)lane < T.nt && T.pre <= j)) - 1;
}

// Block j of lane (j in [j_lo, j_hi], both wavefront-uniform).
__device__ inline BlockInfo block_info(const TileLanes& T, uint32_t j, uint32_t j_lo, uint32_t j_hi, uint32_t lane) {
  BlockInfo r;
  // the tile: the last one whose first block is at or before j; only the
  // tiles between those of j_lo and j_hi can hold it
  const int t_lo = tile_of(T, j_lo, lane), t_hi = tile_of(T, j_hi, lane);
  int t = t_lo;
  for (int tt = t_lo + 1; tt <= t_hi; ++tt) t += j >= (uint32_t)__builtin_amdgcn_readlane(T.pre, tt) ? 1 : 0;
  const uint32_t byte0 = __shfl(T.byte0, t, kWave), n01 = __shfl(T.n01, t, kWave);
  const uint32_t n23 = __shfl(T.n23, t, kWave), pre = __shfl(T.pre, t, kWave);
  const uint32_t n0 = n01 & 0xFFFF, n1 = n01 >> 16, n2 = n23 & 0xFFFF, n3 = n23 >> 16;
  const uint32_t k0 = seg_blocks(0, n0), k01 = k0 + seg_blocks(1, n1), k012 = k01 + seg_blocks(2, n2);
  const uint32_t jb = j - pre;
  const int c = (jb >= k0) + (jb >= k01) + (jb >= k012);
  const uint32_t kb = sel4(c, 0u, k0, k01, k012);
  const uint32_t s1 = (uint32_t)seg_bytes(0, n0), s2 = s1 + (uint32_t)seg_bytes(1, n1);
  const uint32_t sb = sel4(c, 0u, s1, s2, s2 + (uint32_t)seg_bytes(2, n2));
  const uint32_t bi = jb - kb;
  const uint32_t n = sel4(c, n0, n1, n2, n3);
  const uint32_t br = sel4(c, block_records(0), block_records(1), block_records(2), block_records(3));
  const uint32_t full = sel4(c, block_bytes(0, block_records(0)), block_bytes(1, block_records(1)),
                             block_bytes(2, block_records(2)), block_bytes(3, block_records(3)));
  r.m = min(br, n - bi * br);
  r.byte = byte0 + sb + bi * full;
  r.size = (c == 0 ? up16(8u * r.m) : (8u << c) * r.m) + up16(4u * r.m) + up16(2u * r.m);
  r.c = c;
  r.t = t;
  return r;
}

// ---- LDS layout and block decode ---------------------------------------------------
struct AllConsts {
  Consts<0> k0;
  Consts<1> k1;
  Consts<2> k2;
  Consts<3> k3;
};

struct Smem {
  uint32_t* xs;    // [NB][64][36] pairs (x_2p, x_2p+1) of the k-tile
  float* cx;       // [NB][4][64] bias constants per width class
  float* xsum;     // [NB][64] sum of x over the group
  float* yw;       // [waves][NB][nrow] per-wavefront row sums
  const uint8_t* ring;   // this wavefront's ring
  uint32_t ring_mask;    // ring bytes - 1 (a power of two)
};

// Inclusive sum over the 64 lanes of a wavefront with DPP row shifts and row
// broadcasts (lanes without a source add zero).
__device__ inline float wave_incl_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x111, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x112, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false));
  return v;
}

// Contribution of one record part: s * (sum of decoded pairs * x - bias) +
// o * sum(x) (the bias and the offset term only on the record's first part).
template <int C, int NB>
__device__ inline void record_part(const Consts<C>& k, const Smem& S, const uint32_t* w, uint32_t so, int kgl, int q,
                                   float (&v)[NB]) {
  float acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = q == 0 ? -S.cx[(nb * 4 + C) * kTileGroups + kgl] : 0.0f;
  const uint32_t* xk = S.xs + kgl * kXStride + q * (uint32_t)Geo<C>::NP;
  dot_from<C, NB, 0>(k, w, xk, kTileGroups * kXStride, acc);
  const float s = __half2float(__ushort_as_half((unsigned short)(so & 0xFFFF)));
  const float o = q == 0 ? __half2float(__ushort_as_half((unsigned short)(so >> 16))) : 0.0f;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) v[nb] = __builtin_fmaf(s, acc[nb], o * S.xsum[nb * kTileGroups + kgl]);
}

// Decodes one block of class C (m records) at ring offset `boff` and adds each
// record's contribution to its row. Records run in (row, k-group) order, so
// rows are sorted along the lanes. Each lane ends with one (row, value) pair:
// the row of its last record and the sum over its records of that row (a
// 1-bit lane first adds its other rows straight into the row sums). Runs of
// equal rows across lanes are then closed with one inclusive wavefront scan P:
// the last lane of a run adds P to its row and subtracts P from the next
// run's row, which leaves every row with the sum of its own run.
template <int C, int NB>
__device__ inline void compute_block(const Consts<C>& k, const Smem& S, uint32_t boff, uint32_t m, int rl, int nrow,
                                     int wave, uint32_t lane) {
  constexpr int LPR = Geo<C>::LPR, NW = Geo<C>::NW;
  const uint32_t mask = S.ring_mask;
  const uint32_t ca = codes_area(C, m), sa = so_area(m);
  float* yw = S.yw + wave * NB * nrow + rl * kTile;
  float v[NB];
  int key = kTile;                            // lanes past the block form their own last run
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) v[nb] = 0.0f;
  if constexpr (C == 0) {
    if (4u * lane < m) {
      const uint4 c01 = *reinterpret_cast<const uint4*>(S.ring + ((boff + 32u * lane) & mask));
      const uint4 c23 = *reinterpret_cast<const uint4*>(S.ring + ((boff + 32u * lane + 16u) & mask));
      const uint4 so4 = *reinterpret_cast<const uint4*>(S.ring + ((boff + ca + 16u * lane) & mask));
      const uint2 mt4 = *reinterpret_cast<const uint2*>(S.ring + ((boff + ca + sa + 8u * lane) & mask));
      const uint32_t mts[4] = {mt4.x & 0xFFFFu, mt4.x >> 16, mt4.y & 0xFFFFu, mt4.y >> 16};
      const uint32_t sos[4] = {so4.x, so4.y, so4.z, so4.w};
      const uint32_t ws[8] = {c01.x, c01.y, c01.z, c01.w, c23.x, c23.y, c23.z, c23.w};
      const uint32_t n_here = min(4u, m - 4u * lane);
      const int first = (int)(mts[0] & 15u);
      key = (int)((n_here == 4u ? mts[3] : n_here == 3u ? mts[2] : n_here == 2u ? mts[1] : mts[0]) & 15u);
      float head[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) head[nb] = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if ((uint32_t)i < n_here) {
          float r[NB];
          record_part<0, NB>(k, S, ws + 2 * i, sos[i], (int)(mts[i] >> 4) & (kTileGroups - 1), 0, r);
          const int row = (int)(mts[i] & 15u);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            if (row == key) v[nb] += r[nb];
            else if (row == first) head[nb] += r[nb];
            else atomicAdd(&yw[nb * nrow + row], r[nb]);   // a row wholly inside this lane
          }
        }
      }
      if (first != key) {   // the lane's first row continues the run of earlier lanes
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) atomicAdd(&yw[nb * nrow + first], head[nb]);
      }
    }
  } else {
    const uint32_t l = lane / LPR, q = lane % LPR;
    if (l < m) {
      uint32_t w[NW];
      const uint32_t cb = 4u * NW;   // code bytes per lane
#pragma unroll
      for (int h = 0; h < NW / 4; ++h) {
        const uint4 u = *reinterpret_cast<const uint4*>(S.ring + ((boff + cb * lane + 16u * h) & mask));
        w[4 * h + 0] = u.x;
        w[4 * h + 1] = u.y;
        w[4 * h + 2] = u.z;
        w[4 * h + 3] = u.w;
      }
      const uint32_t so = *reinterpret_cast<const uint32_t*>(S.ring + ((boff + ca + 4u * l) & mask));
      const uint32_t mt = *reinterpret_cast<const uint16_t*>(S.ring + ((boff + ca + sa + 2u * l) & mask));
      key = (int)(mt & 15u);
      record_part<C, NB>(k, S, w, so, (int)(mt >> 4) & (kTileGroups - 1), (int)q, v);
    }
  }
  const int next = __builtin_amdgcn_update_dpp(kTile, key, 0x130, 0xF, 0xF, false);   // lane + 1 (wave shift)
  const bool end = key != next && key < kTile;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float p = wave_incl_sum(v[nb]);
    if (end) {   // distinct rows: the end lanes of different runs never share an address
      atomicAdd(&yw[nb * nrow + key], p);
      if (next < kTile) atomicAdd(&yw[nb * nrow + next], -p);
    }
  }
}

template <int NB>
__device__ inline void compute_any(const AllConsts& K, const Smem& S, int c, uint32_t boff, uint32_t m, int rl,
                                   int nrow, int wave, uint32_t lane) {
  switch (c) {
    case 0: compute_block<0, NB>(K.k0, S, boff, m, rl, nrow, wave, lane); break;
    case 1: compute_block<1, NB>(K.k1, S, boff, m, rl, nrow, wave, lane); break;
    case 2: compute_block<2, NB>(K.k2, S, boff, m, rl, nrow, wave, lane); break;
    default: compute_block<3, NB>(K.k3, S, boff, m, rl, nrow, wave, lane); break;
  }
}

// x of k-groups [g0, g0 + ng): four threads per (batch row, k-group), each
// owning 8 of the 32 pairs. The loads are issued first, together with the
// tile headers, and waited for once.
template <int NB, int WAVES>
struct XItems {
  static constexpr int N = (NB * kTileGroups * 4 + WAVES * kWave - 1) / (WAVES * kWave);
  uint4 lo[N], hi[N];
};

template <int NB, int WAVES>
__device__ inline void load_x(const GemvMat& M, XItems<NB, WAVES>& X, int g0, int ng, int tid) {
  const int K = M.n_groups * kGroup;
#pragma unroll
  for (int it = 0; it < XItems<NB, WAVES>::N; ++it) {
    const int i = tid + it * WAVES * kWave;
    X.lo[it] = make_uint4(0, 0, 0, 0);
    X.hi[it] = make_uint4(0, 0, 0, 0);
    if (i < NB * ng * 4) {
      const int nb = i / (ng * 4), rem = i - nb * ng * 4, kgl = rem >> 2, qt = rem & 3;
      const uint16_t* xr = M.x + (size_t)nb * K + (size_t)(g0 + kgl) * kGroup + 16 * qt;
      X.lo[it] = *reinterpret_cast<const uint4*>(xr);        // pairs 8qt .. 8qt+3
      X.hi[it] = *reinterpret_cast<const uint4*>(xr + 8);    // pairs 8qt+4 .. 8qt+7
    }
  }
}

// Writes the pairs (x_2p, x_2p+1) to LDS with the per-group sums and bias
// constants, reduced across the four threads of a (batch row, k-group).
template <int NB, int WAVES>
__device__ inline void stage_x(const Smem& S, const XItems<NB, WAVES>& X, int ng, int tid) {
#pragma unroll
  for (int it = 0; it < XItems<NB, WAVES>::N; ++it) {
    const int i = tid + it * WAVES * kWave;
    // uniform per wavefront: no item for any lane of it in this round
    if (it * WAVES * kWave + (tid & ~(kWave - 1)) >= NB * ng * 4) break;
    const int nb = i / (ng * 4), rem = i - nb * ng * 4, kgl = rem >> 2, qt = rem & 3;
    const bool live = i < NB * ng * 4;
    const uint32_t p[8] = {X.lo[it].x, X.lo[it].y, X.lo[it].z, X.lo[it].w,
                           X.hi[it].x, X.hi[it].y, X.hi[it].z, X.hi[it].w};
    if (live) {
      uint32_t* xk = S.xs + (nb * kTileGroups + kgl) * kXStride + 8 * qt;
      *reinterpret_cast<uint4*>(xk) = X.lo[it];
      *reinterpret_cast<uint4*>(xk + 4) = X.hi[it];
    }
    float Xs = 0.f, c0 = 0.f, c1 = 0.f, c2 = 0.f, c3 = 0.f;
    const bool odd = qt & 1;   // pair index 8qt + e: f = pair % 16 for 1-bit, pair % 8 for 2-bit
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const half2_t h = as_h2(p[e]);
      const float sj = (float)h.x + (float)h.y;
      Xs += sj;
      c0 += (odd ? field_bias(0, 8 + e) : field_bias(0, e)) * sj;
      c1 += field_bias(1, e) * sj;
      c2 += field_bias(2, e % 4) * sj;
      c3 += field_bias(3, e % 2) * sj;
    }
#pragma unroll
    for (int d = 1; d <= 2; d <<= 1) {
      Xs += __shfl_xor(Xs, d, kWave);
      c0 += __shfl_xor(c0, d, kWave);
      c1 += __shfl_xor(c1, d, kWave);
      c2 += __shfl_xor(c2, d, kWave);
      c3 += __shfl_xor(c3, d, kWave);
    }
    if (live && qt == 0) {
      S.cx[(nb * 4 + 0) * kTileGroups + kgl] = c0;
      S.cx[(nb * 4 + 1) * kTileGroups + kgl] = c1;
      S.cx[(nb * 4 + 2) * kTileGroups + kgl] = c2;
      S.cx[(nb * 4 + 3) * kTileGroups + kgl] = c3;
      S.xsum[nb * kTileGroups + kgl] = Xs;
    }
  }
}

// y[b][n] += sum_k x[b][k] r[n][k] over the workgroup's k-tile, one row per
// wavefront at a time (all copies are consumed by then, so plain loads wait
// for nothing else).
template <int NB, int WAVES>
__device__ inline void residual_rows(const GemvMat& M, const Smem& S, int r0, int nrow, int g0, int ng, int wave,
                                     uint32_t lane) {
  const int K = M.n_groups * kGroup;
  for (int ri = wave; ri < nrow; ri += WAVES) {
    const int row = r0 + ri;
    if (row >= M.n_rows) break;
    const uint4* rr = reinterpret_cast<const uint4*>(M.resid + (size_t)row * K + (size_t)g0 * kGroup);
    float acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = 0.f;
    const int n16 = ng * 8;                                  // 16-byte chunks in the window
    uint4 rv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = (int)lane + kWave * u;
      rv[u] = c < n16 ? rr[c] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = (int)lane + kWave * u;
      if (c < n16) {
        const int kgl = c >> 3, qq = c & 7;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint4 xv = *reinterpret_cast<const uint4*>(S.xs + (nb * kTileGroups + kgl) * kXStride + 4 * qq);
          acc[nb] = dot2(rv[u].x, xv.x, acc[nb]);
          acc[nb] = dot2(rv[u].y, xv.y, acc[nb]);
          acc[nb] = dot2(rv[u].z, xv.z, acc[nb]);
          acc[nb] = dot2(rv[u].w, xv.w, acc[nb]);
        }
      }
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float v = acc[nb];
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
      if (lane == 0) S.yw[(wave * NB + nb) * nrow + ri] += v;
    }
  }
}

// ---- Split-K finish -------------------------------------------------------------
// Partial rows of a matrix with several k-tiles meet in a workspace that every
// XCD of the device sees. Only device-scope read-modify-write atomics touch
// it: they are performed at the device's coherence point, not in an XCD's own
// L2, so no L2 write-back or invalidate is needed. A workgroup swaps its
// partial rows in, waits until those atomics are acknowledged, then counts
// itself in for its row range; the one that counts last reads every k-tile's
// partial rows back (again by atomics), adds them in k-tile order and writes
// y, then rearms the counter for the next call on the stream. Nothing waits
// on another workgroup, and the sum order is fixed.
// The swap returns the old value (kept live below), so its completion, which
// the waits count, means the new value is in place at the coherence point.
__device__ inline void swap_agent(float* p, float v) {
  const uint32_t old = __hip_atomic_exchange(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("" ::"v"(old));
}

__device__ inline float read_agent(float* p) {
  return __uint_as_float(
      __hip_atomic_fetch_or(reinterpret_cast<uint32_t*>(p), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

template <int NB, int WAVES>
__device__ inline void finish_split(const GemvMat& M, const Smem& S, int kt, int cj, int r0, int nrow, int tid) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(VBQ_VMCNT_IMM(0));   // this lane's swaps are performed
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  lds_barrier();                                  // ... and every lane's
  uint32_t* flag = reinterpret_cast<uint32_t*>(S.cx);
  if (tid == 0) {
    const uint32_t before =
        __hip_atomic_fetch_add(&M.counters[cj], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = before == (uint32_t)(M.k_tiles - 1);
  }
  lds_barrier();
  if (!*flag) return;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  for (int i = tid; i < NB * nrow; i += WAVES * kWave) {
    const int nb = i / nrow, ri = i - nb * nrow;
    const int row = r0 + ri;
    if (row < M.n_rows) {
      float v = 0.f;
      for (int t = 0; t < M.k_tiles; ++t) v += read_agent(&M.part[((size_t)t * NB + nb) * M.n_rows + row]);
      M.y[(size_t)nb * M.n_rows + row] = v;
    }
  }
  if (tid == 0) __hip_atomic_exchange(&M.counters[cj], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Descriptor of one block of a wavefront, built by one lane, read back with
// v_readlane in the block loop:
//   bits 0-9 ring offset / 16 (rings up to 16 KiB), 10-11 width class,
//   12-19 records - 1, 20-24 copies that may still be outstanding when the
//   block is decoded (fewer than the 16 slots), 25-29 copies to issue after it.
// The block's tile goes in a second per-lane word.
// With pieces of 1 KiB at stream offset 1024 p going to ring slot p mod S, and
// piece p issued as soon as every block before stream offset 1024 (p - S + 1)
// is decoded, the pieces issued before block j are min(np, pos_j / 1024 + S)
// and the block needs the first ceil((pos_j + size_j) / 1024): both closed
// forms of the block's stream position. A block spans at most five pieces
// (3584 bytes at an odd start), so S >= 5 keeps all of them in the ring.
// Only kFirstPieces go out before the first block (at stream offset 0, so it
// needs at most four): a wavefront starts decoding as soon as its first block
// has landed, and issues the rest of its ring after that block.
constexpr uint32_t kFirstPieces = 4;

__device__ inline uint32_t make_desc(const BlockInfo& b, uint32_t B0, uint32_t np, uint32_t slots, uint32_t ring_mask) {
  const uint32_t pos = b.byte - B0;
  const uint32_t need = (pos + b.size + 1023u) >> 10;
  const uint32_t before = min(np, pos == 0 ? kFirstPieces : (pos >> 10) + slots);
  const uint32_t after = min(np, ((pos + b.size) >> 10) + slots);
  return ((pos & ring_mask) >> 4) | ((uint32_t)b.c << 10) | ((b.m - 1u) << 12) | ((before - need) << 20) |
         ((after - before) << 25);
}

template <int NB, int WAVES, bool RESID>
__global__ __launch_bounds__(WAVES * 64) void k_gemv(const GemvLaunch L) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keeps block bookkeeping scalar
  int mi = 0;
  for (int i = 1; i < L.n_mats; ++i) mi = ((int)blockIdx.x >= L.mats[i].wg_begin) ? i : mi;
  const GemvMat& M = L.mats[mi];
  const int j = (int)blockIdx.x - M.wg_begin;
  const int kt = j / M.wg_per_col, cj = j - kt * M.wg_per_col;
  const int rt0 = cj * M.rt_per_wg;
  const int nrl = min(M.rt_per_wg, M.row_tiles - rt0);
  const int nrow = nrl * kTile, r0 = rt0 * kTile;
  const int g0 = kt * kTileGroups, ng = min(kTileGroups, M.n_groups - g0);

  Smem S;
  S.xs = reinterpret_cast<uint32_t*>(smem);
  S.cx = reinterpret_cast<float*>(S.xs + NB * kTileGroups * kXStride);
  S.xsum = S.cx + NB * 4 * kTileGroups;
  S.yw = S.xsum + NB * kTileGroups;
  uint8_t* rings = reinterpret_cast<uint8_t*>(S.yw + WAVES * NB * L.rt_per_wg * kTile);
  const uint32_t ring = L.ring_bytes;
  S.ring = rings + wave * ring;
  S.ring_mask = ring - 1u;
  const uint32_t ring_lds = lds_addr(S.ring);
  const uint32_t slots = ring >> 10;
  const u32x4 rsrc = make_rsrc(M.stream, M.stream_bytes);

  // Ordinary loads (x, tile headers) come before the first copy and are
  // waited for once, on every path: waiting for them later would also wait
  // for every copy in flight.
  XItems<NB, WAVES> X;
  load_x<NB, WAVES>(M, X, g0, ng, tid);
  uint4 h = make_uint4(0, 0, 0, 0);
  if ((int)lane <= nrl) h = *reinterpret_cast<const uint4*>(M.tiles + 4 * (size_t)(kt * M.row_tiles + rt0 + (int)lane));
  __builtin_amdgcn_s_waitcnt(VBQ_VMCNT_IMM(0));
  const TileLanes T = make_tile_lanes(h, nrl, lane);

  // This wavefront's blocks [b0, b1) and their bytes [B0, B1): the blocks
  // whose cost prefix falls in its equal share of the workgroup's decode cost.
  // They stream in pieces of 1 KiB; the first pieces go out before anything
  // else is set up.
  uint32_t ub0, B0, ub1, B1;
  first_block_at(T, (uint32_t)(((uint64_t)T.cost * wave) / WAVES), lane, ub0, B0);
  if (wave == WAVES - 1) {
    ub1 = (uint32_t)T.total;
    B1 = __builtin_amdgcn_readlane(T.byte0, T.nt);
  } else {
    first_block_at(T, (uint32_t)(((uint64_t)T.cost * (wave + 1)) / WAVES), lane, ub1, B1);
  }
  const int b0 = (int)ub0, b1 = (int)ub1;
  const uint32_t span = b0 < b1 ? B1 - B0 : 0u, np = (span + 1023u) >> 10;
  uint32_t issued = 0;
  const uint32_t lane16 = 16u * lane;
  auto issue = [&](uint32_t upto) {
    for (; issued < upto; ++issued) {
      const uint32_t piece = issued << 10;
      const uint32_t lds = ring_lds + ((issued & (slots - 1u)) << 10);
      if (span - piece >= 1024u) {
        dma16(rsrc, lds, B0 + piece + lane16);
      } else if (lane16 < span - piece) {   // the last piece: lanes past the range stay idle
        dma16(rsrc, lds, B0 + piece + lane16);
      }
    }
  };
  issue(min(np, kFirstPieces));   // first, so that the setup below overlaps the copies

  stage_x<NB, WAVES>(S, X, ng, tid);
  for (int i = tid; i < WAVES * NB * nrow; i += WAVES * kWave) S.yw[i] = 0.0f;
  AllConsts K;
  K.k0 = make_consts<0>();
  K.k1 = make_consts<1>();
  K.k2 = make_consts<2>();
  K.k3 = make_consts<3>();
  lds_barrier();                              // x table and zeroed row sums visible

  for (int base = b0; base < b1; base += kWave) {
    const uint32_t jhi = (uint32_t)min(b1 - 1, base + kWave - 1);
    const uint32_t jl = min((uint32_t)(base + (int)lane), jhi);
    const BlockInfo bi = block_info(T, jl, (uint32_t)base, jhi, lane);
    const uint32_t desc = make_desc(bi, B0, np, slots, S.ring_mask);
    const int n_here = min(kWave, b1 - base);
    for (int k = 0; k < n_here; ++k) {
      const uint32_t d = __builtin_amdgcn_readlane(desc, k);
      const int t = __builtin_amdgcn_readlane(bi.t, k);
      wait_vmcnt((int)((d >> 20) & 31u));
      compute_any<NB>(K, S, (int)((d >> 10) & 3u), (d & 1023u) << 4, ((d >> 12) & 255u) + 1u, t, nrow, wave, lane);
      // Refill the freed ring slots; the decode's LDS reads are complete first.
      __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0)
      issue(issued + ((d >> 25) & 31u));
    }
  }
  if constexpr (RESID) residual_rows<NB, WAVES>(M, S, r0, nrow, g0, ng, wave, lane);
  lds_barrier();

  // Rows of this workgroup: sum the wavefront slices in a fixed order.
  const bool split = M.k_tiles > 1;
  for (int i = tid; i < NB * nrow; i += WAVES * kWave) {
    const int nb = i / nrow, ri = i - nb * nrow;
    const int row = r0 + ri;
    if (row < M.n_rows) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) v += S.yw[(w * NB + nb) * nrow + ri];
      if (split)
        swap_agent(&M.part[((size_t)kt * NB + nb) * M.n_rows + row], v);
      else
        M.y[(size_t)nb * M.n_rows + row] = v;
    }
  }
  if (split) finish_split<NB, WAVES>(M, S, kt, cj, r0, nrow, tid);
}

// Eight wavefronts per workgroup. With one batch row the x table is small,
// so two workgroups (with 8 KiB rings) share a CU: one's start-up and final
// reduction overlap the other's streaming.
int gemv_waves(int) { return 8; }
int gemv_wgs_per_cu(int nb) { return nb <= 1 ? 2 : 1; }

size_t gemv_lds_bytes(int nb, int rt_per_wg, uint32_t ring_bytes) {
  const int waves = gemv_waves(nb);
  size_t b = (size_t)nb * kTileGroups * kXStride * 4;   // x pairs
  b += (size_t)nb * 4 * kTileGroups * 4;                // bias constants
  b += (size_t)nb * kTileGroups * 4;                    // x sums
  b += (size_t)waves * nb * rt_per_wg * kTile * 4;      // per-wavefront row sums
  b += (size_t)waves * ring_bytes;                      // rings
  return b;
}

// The ring is a power of two of at least five 1 KiB slots: a block spans at
// most five pieces (3584 bytes at an odd start).
uint32_t gemv_ring_min_bytes() { return 8u * 1024u; }

template <int NB, int WAVES, bool RESID>
static hipError_t launch_one(const GemvLaunch& L, int n_wg, size_t lds, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv<NB, WAVES, RESID>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 64);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((k_gemv<NB, WAVES, RESID>), dim3(n_wg), dim3(WAVES * kWave), lds, s, L);
  return hipGetLastError();
}

hipError_t launch_gemv(const GemvLaunch& L, int nb, bool resid, int n_wg, size_t lds, hipStream_t s) {
#define VBQ_CASE(N)                                                                                  \
  case N:                                                                                            \
    return resid ? launch_one<N, 8, true>(L, n_wg, lds, s)                           \
                 : launch_one<N, 8, false>(L, n_wg, lds, s);
  switch (nb) {
    VBQ_CASE(1)
    VBQ_CASE(2)
    VBQ_CASE(3)
    VBQ_CASE(4)
    VBQ_CASE(5)
    VBQ_CASE(6)
    VBQ_CASE(7)
    VBQ_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef VBQ_CASE
}

}  // namespace vbq
