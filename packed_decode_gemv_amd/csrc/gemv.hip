// Fused dequantise-and-multiply GEMV over the tiled mixed-width layout.
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
// bias part, sum_j bias_j (x_j + x_{32+j}), depends only on x and the field
// positions of the width, so it is computed once per (k-group, width) in LDS
// and subtracted per group. Masks and exponent patterns live in registers so
// that building one fp16 pair is a single v_and_or_b32.
//
// Work split: a workgroup (8 wavefronts) owns a range of 16-row row-tiles of
// one matrix (several matrices per launch for batched calls) and walks its
// tiles k-tile by k-tile, staging the matching 4096-column window of x in LDS.
// Inside a tile the records are grouped by width in blocks of 64, so every
// block is decoded by one wavefront with a single width: no divergence, and
// neighbouring lanes mostly share a k-group, so their x reads are broadcasts.
// Each wavefront copies its own upcoming blocks from HBM straight into a
// private LDS ring with buffer-to-LDS loads, keeping several kilobytes in
// flight without spending registers, and waits on exact load counts before it
// decodes a block. Wavefronts accumulate rows in their own LDS slices, summed
// in a fixed order at the end, so results are identical from run to run.
#include <utility>

#include "vbq_common.h"

namespace vbq {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;

// Field placement of pair index f within a word, per width class c.
// shift kind: 0 none, 1 left by 4, 2 right by 2, 3 right by 8.
__host__ __device__ constexpr int shift_kind(int c, int f) {
  return c == 0 ? (f < 6 ? 1 : f < 12 ? 2 : 3)
       : c == 1 ? (f < 3 ? 1 : f < 6 ? 2 : 3)
       : c == 2 ? (f < 2 ? 0 : 3)
       : (f < 1 ? 0 : 3);
}
// Mantissa bit of the field after the shift.
__host__ __device__ constexpr int field_pos(int c, int f) {
  return c == 0 ? (f < 6 ? f + 4 : f < 12 ? f - 2 : f - 8)
       : c == 1 ? (f < 3 ? 4 + 2 * f : f < 6 ? 4 + 2 * (f - 3) : 4 + 2 * (f - 6))
       : c == 2 ? ((f & 1) ? 4 : 0)
       : 0;
}
__host__ __device__ constexpr uint32_t field_mask(int c, int p) {
  return (((1u << (1 << c)) - 1u) << p) * 0x00010001u;
}
// fp16 with exponent field 25 - p: the mantissa bit p has weight 1.
__host__ __device__ constexpr uint32_t field_magic(int p) { return (uint32_t)((25 - p) << 10) * 0x00010001u; }
__host__ __device__ constexpr float field_bias(int c, int f) { return (float)(1 << (10 - field_pos(c, f))); }

template <int KIND>
__device__ inline uint32_t shifted(uint32_t w) {
  return KIND == 0 ? w : KIND == 1 ? (w << 4) : KIND == 2 ? (w >> 2) : (w >> 8);
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

template <int C, int J, int NB>
__device__ inline void pair_step(const Consts<C>& k, const uint32_t* w, const uint4 (&xv)[NB], float (&acc)[NB]) {
  constexpr int H = 16 >> C, F = J % H, P = field_pos(C, F);
  const uint32_t src = shifted<shift_kind(C, F)>(w[J / H]);
  const uint32_t hv = (src & k.mask[P]) | k.magic[P];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = dot2(hv, lane_of<J & 3>(xv[nb]), acc[nb]);
}

template <int C, int CH, int NB>
__device__ inline void chunk_step(const Consts<C>& k, const uint32_t* w, const uint32_t* xk, int xstride,
                                  float (&acc)[NB]) {
  uint4 xv[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) xv[nb] = *reinterpret_cast<const uint4*>(xk + nb * xstride + 4 * CH);
  pair_step<C, 4 * CH + 0, NB>(k, w, xv, acc);
  pair_step<C, 4 * CH + 1, NB>(k, w, xv, acc);
  pair_step<C, 4 * CH + 2, NB>(k, w, xv, acc);
  pair_step<C, 4 * CH + 3, NB>(k, w, xv, acc);
}

// acc[nb] += sum_j (bias_j + q_j) x_j + (bias_j + q_{32+j}) x_{32+j} over the
// 32 pairs of one record. xk points at the record's k-group in the x table of
// batch row 0; batch rows are xstride dwords apart.
template <int C, int NB, int... CH>
__device__ inline void dot_record_impl(const Consts<C>& k, const uint32_t* w, const uint32_t* xk, int xstride,
                                       float (&acc)[NB], std::integer_sequence<int, CH...>) {
  (chunk_step<C, CH, NB>(k, w, xk, xstride, acc), ...);
}

// x pairs of one k-group take 32 dwords plus 4 of padding: neighbouring
// k-groups start 144 bytes apart, which spreads lanes that read different
// k-groups over the LDS banks while every read keeps an immediate offset.
constexpr int kXStride = 36;
// Ring bytes of one block: codes (64 records of 8b bytes), scale/offset
// (64 x 4 bytes), meta (64 x 2 bytes plus one halfword of alignment slack).
__host__ __device__ constexpr uint32_t ring_block_bytes(int c) { return (512u << c) + 256u + 144u; }
constexpr uint32_t kRingMinBytes = ring_block_bytes(3);

typedef __attribute__((address_space(3))) void lds_void;

struct Rsrc {
  __amdgpu_buffer_rsrc_t so, meta, codes;
};

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Waits until at most n vector-memory instructions of this wavefront are
// outstanding (n is wavefront-uniform). Loads complete in issue order, so this
// waits for everything issued before the last n.
#define VBQ_VMCNT_IMM(n) (((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
#define VBQ_W(n) case n: __builtin_amdgcn_s_waitcnt(VBQ_VMCNT_IMM(n)); break;
__device__ inline void wait_vmcnt(int n) {
  switch (n < 63 ? n : 63) {
    VBQ_W(0) VBQ_W(1) VBQ_W(2) VBQ_W(3) VBQ_W(4) VBQ_W(5) VBQ_W(6) VBQ_W(7)
    VBQ_W(8) VBQ_W(9) VBQ_W(10) VBQ_W(11) VBQ_W(12) VBQ_W(13) VBQ_W(14) VBQ_W(15)
    VBQ_W(16) VBQ_W(17) VBQ_W(18) VBQ_W(19) VBQ_W(20) VBQ_W(21) VBQ_W(22) VBQ_W(23)
    VBQ_W(24) VBQ_W(25) VBQ_W(26) VBQ_W(27) VBQ_W(28) VBQ_W(29) VBQ_W(30) VBQ_W(31)
    VBQ_W(32) VBQ_W(33) VBQ_W(34) VBQ_W(35) VBQ_W(36) VBQ_W(37) VBQ_W(38) VBQ_W(39)
    VBQ_W(40) VBQ_W(41) VBQ_W(42) VBQ_W(43) VBQ_W(44) VBQ_W(45) VBQ_W(46) VBQ_W(47)
    VBQ_W(48) VBQ_W(49) VBQ_W(50) VBQ_W(51) VBQ_W(52) VBQ_W(53) VBQ_W(54) VBQ_W(55)
    VBQ_W(56) VBQ_W(57) VBQ_W(58) VBQ_W(59) VBQ_W(60) VBQ_W(61) VBQ_W(62)
    default: __builtin_amdgcn_s_waitcnt(VBQ_VMCNT_IMM(63)); break;
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);   // keep LDS reads of the landed data after the wait
}
#undef VBQ_W

// Position of a wavefront in its block sequence. A workgroup owns row-tiles
// [rt0, rt0 + nrl) of one matrix; its blocks are ordered (k-tile, row-tile,
// width class, block) -- the storage order inside each tile -- and wavefront w
// takes every kWaves-th block starting at w. All fields are wavefront-uniform.
struct Cur {
  int kt, rl, c, bi;
  uint32_t rec0, code0, n[4];
  bool valid;
};

__device__ inline int nblk_of(uint32_t n) { return (int)((n + kBlock - 1) / kBlock); }

__device__ inline void cur_tile(Cur& q, const GemvMat& M, int rt0) {
  const uint4 th = *reinterpret_cast<const uint4*>(M.tiles + 4 * ((rt0 + q.rl) * M.k_tiles + q.kt));
  q.rec0 = th.x;
  q.code0 = th.y;
  q.n[0] = th.z & 0xFFFF;
  q.n[1] = th.z >> 16;
  q.n[2] = th.w & 0xFFFF;
  q.n[3] = th.w >> 16;
}

// Moves forward k blocks (k >= 0) in the workgroup's sequence.
__device__ inline void cur_advance(Cur& q, const GemvMat& M, int rt0, int nrl, int k) {
  while (q.valid) {
    const int left = nblk_of(q.n[q.c]) - q.bi;
    if (k < left) {
      q.bi += k;
      return;
    }
    k -= left;
    q.bi = 0;
    if (++q.c == 4) {
      q.c = 0;
      if (++q.rl == nrl) {
        q.rl = 0;
        if (++q.kt == M.k_tiles) {
          q.valid = false;
          return;
        }
      }
      cur_tile(q, M, rt0);
    }
  }
}

__device__ inline Cur cur_first(const GemvMat& M, int rt0, int nrl, int wave) {
  Cur q;
  q.kt = 0;
  q.rl = 0;
  q.c = 0;
  q.bi = 0;
  q.valid = true;
  cur_tile(q, M, rt0);
  cur_advance(q, M, rt0, nrl, wave);
  return q;
}

__device__ inline uint32_t cur_m(const Cur& q) { return min((uint32_t)kBlock, q.n[q.c] - (uint32_t)q.bi * kBlock); }

__device__ inline uint32_t cur_rec(const Cur& q) {
  uint32_t r = q.rec0 + (uint32_t)q.bi * kBlock;
  for (int c = 0; c < q.c; ++c) r += q.n[c];
  return r;
}

__device__ inline uint32_t cur_code(const Cur& q) {
  uint32_t o = q.code0 * 16u + (uint32_t)q.bi * (kBlock * 8u << q.c);
  for (int c = 0; c < q.c; ++c) o += (uint32_t)seg_bytes(c, q.n[c]);
  return o;
}

// Number of DMA instructions one block issues (codes pieces of 1 KiB, one for
// the scale/offset words, one for the meta halfwords).
__device__ inline int block_dma_count(int c, uint32_t m) { return (int)((8u * (1u << c) * m + 1023u) / 1024u) + 2; }

// Ring placement: blocks take consecutive ring bytes; a block that would
// straddle the end of the ring starts again at offset 0.
__device__ inline uint32_t ring_place(uint32_t& pos, uint32_t bytes, uint32_t ring) {
  const uint32_t off = pos % ring;
  if (off + bytes > ring) pos += ring - off;
  const uint32_t at = pos % ring;
  pos += bytes;
  return at;
}

// Copies one block of class C from HBM into the wavefront's ring at byte
// offset `at` of the LDS: codes (1 KiB per instruction, 16 bytes per lane),
// scale/offset words and meta halfwords (4 bytes per lane). Lanes past the
// block's data are inactive, so nothing beyond it is read or written.
template <int C>
__device__ inline void dma_block(const Rsrc& R, uint8_t* lds, uint32_t at, uint32_t code_src, uint32_t rec_src,
                                 uint32_t m, uint32_t lane) {
  constexpr uint32_t B = 1u << C;
  const uint32_t cbytes = 8u * B * m;
  const int pieces = (int)((cbytes + 1023u) / 1024u);
  for (int p = 0; p < pieces; ++p) {
    if (1024u * p + 16u * lane < cbytes)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(R.codes, (lds_void*)(lds + at + 1024u * p), 16,
                                               code_src + 1024u * p + 16u * lane, 0, 0, 0);
  }
  const uint32_t so_at = at + (512u << C);
  if (lane < m)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(R.so, (lds_void*)(lds + so_at), 4, (rec_src + lane) * 4u, 0, 0, 0);
  const uint32_t d = rec_src & 1u;                       // meta starts at an odd halfword
  if (lane < (m + d + 1u) / 2u)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(R.meta, (lds_void*)(lds + so_at + 256u), 4,
                                             (rec_src - d) * 2u + 4u * lane, 0, 0, 0);
}

__device__ inline int issue_block(const Rsrc& R, uint8_t* lds, uint32_t at, const Cur& q, uint32_t lane) {
  const uint32_t m = cur_m(q), code = cur_code(q), rec = cur_rec(q);
  switch (q.c) {
    case 0: dma_block<0>(R, lds, at, code, rec, m, lane); break;
    case 1: dma_block<1>(R, lds, at, code, rec, m, lane); break;
    case 2: dma_block<2>(R, lds, at, code, rec, m, lane); break;
    default: dma_block<3>(R, lds, at, code, rec, m, lane); break;
  }
  return block_dma_count(q.c, m);
}

struct AllConsts {
  Consts<0> k0;
  Consts<1> k1;
  Consts<2> k2;
  Consts<3> k3;
};

struct Smem {
  uint32_t* xs;    // [NB][64][36] pairs (x_2p, x_2p+1) of the current 4096-column window
  float* cx;       // [NB][4][64] bias constants per width class
  float* xsum;     // [NB][64] sum of x over the group
  float* yw;       // [kWaves][NB][nrl*16] per-wavefront row sums
  uint8_t* ring;   // this wavefront's ring
};

// Decodes one block of class C from the ring at byte offset `at`.
template <int C, int NB>
__device__ inline void compute_block(const Consts<C>& k, const Smem& S, uint32_t at, uint32_t rec_src, uint32_t m,
                                     int kt, int rl, int nrow, int wave, uint32_t lane) {
  if (lane < m) {
    constexpr int B = 1 << C;
    const uint8_t* blk = S.ring + at;
    uint32_t w[2 * B];
    if constexpr (B == 1) {
      const uint2 v = *reinterpret_cast<const uint2*>(blk + 8u * lane);
      w[0] = v.x;
      w[1] = v.y;
    } else {
#pragma unroll
      for (int q = 0; q < B / 2; ++q) {
        const uint4 v = *reinterpret_cast<const uint4*>(blk + (q * m + lane) * 16u);
        w[4 * q + 0] = v.x;
        w[4 * q + 1] = v.y;
        w[4 * q + 2] = v.z;
        w[4 * q + 3] = v.w;
      }
    }
    const uint8_t* so_p = blk + (512u << C);
    const uint32_t so = *reinterpret_cast<const uint32_t*>(so_p + 4u * lane);
    const uint32_t mt = *reinterpret_cast<const uint16_t*>(so_p + 256u + 2u * ((rec_src & 1u) + lane));
    const int row = mt & 15, kgl = (int)(mt >> 4) - kt * kTileGroups;
    float acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = -S.cx[(nb * 4 + C) * kTileGroups + kgl];   // remove the bias part
    const uint32_t* xk = S.xs + ((kgl << 5) + (kgl << 2));   // kgl * kXStride
    dot_record_impl<C, NB>(k, w, xk, kTileGroups * kXStride, acc, std::make_integer_sequence<int, 8>{});
    const float s = __half2float(__ushort_as_half((unsigned short)(so & 0xFFFF)));
    const float o = __half2float(__ushort_as_half((unsigned short)(so >> 16)));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float v = s * acc[nb] + o * S.xsum[nb * kTileGroups + kgl];
      atomicAdd(&S.yw[(wave * NB + nb) * nrow + rl * kTile + row], v);
    }
  }
}

template <int NB>
__device__ inline void compute_any(const AllConsts& K, const Smem& S, uint32_t at, const Cur& q, int nrow, int wave,
                                   uint32_t lane) {
  const uint32_t m = cur_m(q), rec = cur_rec(q);
  switch (q.c) {
    case 0: compute_block<0, NB>(K.k0, S, at, rec, m, q.kt, q.rl, nrow, wave, lane); break;
    case 1: compute_block<1, NB>(K.k1, S, at, rec, m, q.kt, q.rl, nrow, wave, lane); break;
    case 2: compute_block<2, NB>(K.k2, S, at, rec, m, q.kt, q.rl, nrow, wave, lane); break;
    default: compute_block<3, NB>(K.k3, S, at, rec, m, q.kt, q.rl, nrow, wave, lane); break;
  }
}

// Stages the x window of k-tile kt into LDS as pairs (x_2p, x_2p+1) with the
// per-group sums and bias constants: four threads per (batch row, k-group),
// each owning 8 of the 32 pairs, reduced across the four lanes.
template <int NB>
__device__ inline void stage_x(const GemvMat& M, const Smem& S, int kt, int tid) {
  const int G = M.n_groups, K = G * kGroup;
  const int g0 = kt * kTileGroups, ng = min(kTileGroups, G - g0);
  for (int i = tid; i < NB * kTileGroups * 4; i += kThreads) {
    const int nb = i / (kTileGroups * 4), rem = i - nb * kTileGroups * 4, kgl = rem >> 2, qt = rem & 3;
    uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
    if (kgl < ng) {
      const uint16_t* xr = M.x + (size_t)nb * K + (size_t)(g0 + kgl) * kGroup + 16 * qt;
      lo = *reinterpret_cast<const uint4*>(xr);        // pairs 8qt .. 8qt+3
      hi = *reinterpret_cast<const uint4*>(xr + 8);    // pairs 8qt+4 .. 8qt+7
    }
    uint32_t* xk = S.xs + (nb * kTileGroups + kgl) * kXStride + 8 * qt;
    *reinterpret_cast<uint4*>(xk) = lo;
    *reinterpret_cast<uint4*>(xk + 4) = hi;
    const uint32_t p[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    float X = 0.f, c0 = 0.f, c1 = 0.f, c2 = 0.f, c3 = 0.f;
    const bool odd = qt & 1;   // pair index 8qt + e; for 1-bit fields f = pair % 16
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const half2_t h = as_h2(p[e]);
      const float sj = (float)h.x + (float)h.y;
      X += sj;
      c0 += (odd ? field_bias(0, 8 + e) : field_bias(0, e)) * sj;
      c1 += field_bias(1, e) * sj;
      c2 += field_bias(2, e % 4) * sj;
      c3 += field_bias(3, e % 2) * sj;
    }
#pragma unroll
    for (int d = 1; d <= 2; d <<= 1) {
      X += __shfl_xor(X, d, kWave);
      c0 += __shfl_xor(c0, d, kWave);
      c1 += __shfl_xor(c1, d, kWave);
      c2 += __shfl_xor(c2, d, kWave);
      c3 += __shfl_xor(c3, d, kWave);
    }
    if (qt == 0) {
      S.cx[(nb * 4 + 0) * kTileGroups + kgl] = c0;
      S.cx[(nb * 4 + 1) * kTileGroups + kgl] = c1;
      S.cx[(nb * 4 + 2) * kTileGroups + kgl] = c2;
      S.cx[(nb * 4 + 3) * kTileGroups + kgl] = c3;
      S.xsum[nb * kTileGroups + kgl] = X;
    }
  }
}

template <int NB, bool RESID>
__global__ __launch_bounds__(kThreads) void k_gemv(const GemvLaunch L) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keeps block bookkeeping scalar
  int mi = 0;
  for (int i = 1; i < L.n_mats; ++i) mi = ((int)blockIdx.x >= L.mats[i].wg_begin) ? i : mi;
  const GemvMat& M = L.mats[mi];
  const int rt0 = ((int)blockIdx.x - M.wg_begin) * M.rt_per_wg;
  const int nrl = min(M.rt_per_wg, M.row_tiles - rt0);
  const int nrow = nrl * kTile;

  Smem S;
  S.xs = reinterpret_cast<uint32_t*>(smem);
  S.cx = reinterpret_cast<float*>(S.xs + NB * kTileGroups * kXStride);
  S.xsum = S.cx + NB * 4 * kTileGroups;
  S.yw = S.xsum + NB * kTileGroups;
  uint8_t* rings = reinterpret_cast<uint8_t*>(S.yw + kWaves * NB * L.rt_per_wg * kTile);
  const uint32_t ring = L.ring_bytes;
  S.ring = rings + wave * ring;

  Rsrc R;
  R.so = make_rsrc(M.so, M.so_bytes);
  R.meta = make_rsrc(M.meta, M.meta_bytes);
  R.codes = make_rsrc(M.codes, M.code_bytes);

  // Fill the ring before anything else, so HBM latency overlaps the staging.
  Cur iq = cur_first(M, rt0, nrl, wave);      // next block to copy
  Cur cq = iq;                                // next block to decode
  uint32_t ipos = 0, cpos = 0;                // ring byte counters (copy / decode side)
  int issued = 0, consumed = 0;               // DMA instructions issued / belonging to decoded blocks
  int pending = 0;                            // blocks copied but not decoded yet
  // A block may be copied when it ends within one ring length of the oldest
  // pending block; with nothing pending it always fits (at offset 0 at worst).
  while (iq.valid) {
    const uint32_t bytes = ring_block_bytes(iq.c);
    uint32_t p = ipos;
    const uint32_t at = ring_place(p, bytes, ring);
    if (pending > 0 && p - cpos > ring) break;
    ipos = p;
    issued += issue_block(R, S.ring, at, iq, lane);
    ++pending;
    cur_advance(iq, M, rt0, nrl, kWaves);
  }

  for (int i = tid; i < kWaves * NB * nrow; i += kThreads) S.yw[i] = 0.0f;
  AllConsts K;
  K.k0 = make_consts<0>();
  K.k1 = make_consts<1>();
  K.k2 = make_consts<2>();
  K.k3 = make_consts<3>();

  for (int kt = 0; kt < M.k_tiles; ++kt) {
    if (kt > 0) __syncthreads();              // everyone is done with the previous x window
    stage_x<NB>(M, S, kt, tid);
    __syncthreads();
    while (cq.valid && cq.kt == kt) {
      const uint32_t bytes = ring_block_bytes(cq.c);
      const uint32_t at = ring_place(cpos, bytes, ring);
      consumed += block_dma_count(cq.c, cur_m(cq));
      wait_vmcnt(issued - consumed);
      compute_any<NB>(K, S, at, cq, nrow, wave, lane);
      cur_advance(cq, M, rt0, nrl, kWaves);
      --pending;
      // Refill the freed ring space; the decode's LDS reads are complete first.
      __builtin_amdgcn_s_waitcnt(0xC07F);       // lgkmcnt(0)
      while (iq.valid) {
        const uint32_t ib = ring_block_bytes(iq.c);
        uint32_t p = ipos;
        const uint32_t iat = ring_place(p, ib, ring);
        if (pending > 0 && p - cpos > ring) break;
        ipos = p;
        issued += issue_block(R, S.ring, iat, iq, lane);
        ++pending;
        cur_advance(iq, M, rt0, nrl, kWaves);
      }
    }
    if constexpr (RESID) {
      // y[b][n] += sum_k x[b][k] r[n][k] over this window, one row per wavefront.
      const int K = M.n_groups * kGroup;
      const int g0 = kt * kTileGroups, ng = min(kTileGroups, M.n_groups - g0);
      for (int ri = wave; ri < nrow; ri += kWaves) {
        const int row = rt0 * kTile + ri;
        if (row >= M.n_rows) break;
        const uint4* rr = reinterpret_cast<const uint4*>(M.resid + (size_t)row * K + (size_t)g0 * kGroup);
        float acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = 0.f;
        for (int c = lane; c < ng * 8; c += kWave) {           // 16-byte chunks of the window
          const uint4 rv = rr[c];
          const int kgl = c >> 3, q = c & 7;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const uint4 xv = *reinterpret_cast<const uint4*>(S.xs + (nb * kTileGroups + kgl) * kXStride + 4 * q);
            acc[nb] = dot2(rv.x, xv.x, acc[nb]);
            acc[nb] = dot2(rv.y, xv.y, acc[nb]);
            acc[nb] = dot2(rv.z, xv.z, acc[nb]);
            acc[nb] = dot2(rv.w, xv.w, acc[nb]);
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
  }
  wait_vmcnt(0);
  __syncthreads();

  for (int i = tid; i < NB * nrow; i += kThreads) {
    const int nb = i / nrow, ri = i - nb * nrow;
    const int row = rt0 * kTile + ri;
    if (row < M.n_rows) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += S.yw[(w * NB + nb) * nrow + ri];
      M.y[(size_t)nb * M.n_rows + row] = v;
    }
  }
}

size_t gemv_lds_bytes(int nb, int rt_per_wg, uint32_t ring_bytes) {
  size_t b = (size_t)nb * kTileGroups * kXStride * 4;   // x window
  b += (size_t)nb * 4 * kTileGroups * 4;                // bias constants
  b += (size_t)nb * kTileGroups * 4;                    // x sums
  b += (size_t)kWaves * nb * rt_per_wg * kTile * 4;     // per-wavefront row sums
  b += (size_t)kWaves * ring_bytes;                     // rings
  return b;
}

uint32_t gemv_ring_min_bytes() { return kRingMinBytes; }

template <int NB, bool RESID>
static hipError_t launch_one(const GemvLaunch& L, int n_wg, size_t lds, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv<NB, RESID>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((k_gemv<NB, RESID>), dim3(n_wg), dim3(kThreads), lds, s, L);
  return hipGetLastError();
}

hipError_t launch_gemv(const GemvLaunch& L, int nb, bool resid, int n_wg, size_t lds, hipStream_t s) {
#define VBQ_CASE(N)                                                              \
  case N:                                                                        \
    return resid ? launch_one<N, true>(L, n_wg, lds, s) : launch_one<N, false>(L, n_wg, lds, s);
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
