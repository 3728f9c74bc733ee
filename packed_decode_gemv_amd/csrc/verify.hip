// Re-quantisation check of an in-cell update.
//
// CellFill abstract (page "Nothing Changed but the Model: CellFill -- Bounded
// In-Cell Learning for Bit-Identical, Revocable Updates to Quantized LLMs"):
// the release's codes and scales are not touched, an update is a per-weight
// residual that must stay within the weight's rounding cell, and rounding the
// updated weights again must reproduce the released codes exactly. For every weight
// this kernel re-quantises the served value (dequantised code + residual)
// against the frozen scale and offset, counts codes that change and residuals
// that leave the cell, keeps the smallest failing index, and optionally writes
// a copy of the byte stream with the re-quantised codes so the artifact can be
// compared byte for byte.
//
// The decision is integer-valued, so the binary32 operation sequence is fixed
// (built with -ffp-contract=off). Residuals under a record-level bound keep
// every code provably (keep_bound_bits); the rest take an estimated quotient
// that decides as the correctly rounded one does (quarter_fast) or the
// correctly rounded quotient itself:
//   deq = f32(s*q) + o;  v = deq + r;  q' = clamp(rint((v - o) / s), 0, L)
//   out of cell: |r| >= 0.5*s  (or r != 0 when s == 0).
#include "vbq_common.h"

namespace vbq {

__global__ void k_verify_init(uint64_t* result) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    result[0] = 0;
    result[1] = 0;
    result[2] = ~0ull;
  }
}

// Re-quantises the 16 weights of a quarter with correctly rounded quotients:
// counts into lm / lo, smallest failing index into lf, re-quantised code words
// into nw. Any scale is handled (zero, negative or not finite).
template <int C>
__device__ inline void quarter_pass(const uint32_t (&w)[4], const uint4 (&rv)[2], float s, float o, int q,
                                    uint64_t lin0, uint32_t& lm, uint32_t& lo, uint64_t& lf, uint32_t (&nw)[4]) {
  constexpr int B = 1 << C, H = 16 / B, L = (1 << B) - 1;
  const int p0 = 8 * q, wbase = p0 / H;
  const float half_s = __fmul_rn(0.5f, s);
  lm = lo = 0;
  lf = ~0ull;
#pragma unroll
  for (int i = 0; i < 4; ++i) nw[i] = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int pr = p0 + j / 2, odd = j & 1;
    const int wi = pr / H - wbase, sh = 16 * odd + (pr % H) * B;
    const uint32_t code = (w[wi] >> sh) & (uint32_t)L;
    const uint4& rr = rv[j / 8];
    const uint32_t rw = ((j / 2) & 3) == 0 ? rr.x : ((j / 2) & 3) == 1 ? rr.y : ((j / 2) & 3) == 2 ? rr.z : rr.w;
    const float r = __half2float(__ushort_as_half((unsigned short)(odd ? (rw >> 16) : (rw & 0xFFFF))));
    const float deq = __fadd_rn(__fmul_rn(s, (float)code), o);
    const float a = __fsub_rn(__fadd_rn(deq, r), o);
    uint32_t qp = 0;
    if (s != 0.0f) {
      float t = rintf(__fdiv_rn(a, s));
      t = t < 0.0f ? 0.0f : t;
      t = t > (float)L ? (float)L : t;
      qp = (uint32_t)t;
    }
    const bool bad_code = qp != code;
    const bool bad_cell = (s > 0.0f) ? (fabsf(r) >= half_s) : (r != 0.0f);
    lm += bad_code;
    lo += bad_cell;
    if ((bad_code || bad_cell) && lin0 + j < lf) lf = lin0 + j;
    nw[wi] |= qp << sh;
  }
}

// The common case, for a finite s > 0: re-quantised code words into nw, and
// true when every weight keeps its code and its residual is inside the cell,
// i.e. the quarter contributes nothing to the counts. False sends the quarter
// to quarter_exact.
//   - s*q is exact in binary32 (at most 11 x 8 significant bits), so
//     fma(s, q, o) rounds exactly like f32(s*q) + o.
//   - The quotient is estimated as t = a * rcp(s), within |a/s| * 2^-22 of
//     the correctly rounded a / s. Only quotients in [0, L] (L <= 255) decide
//     a code, since the clamp maps everything else to 0 or L either way. There
//     the estimate is within 2^-14 of the correctly rounded quotient, so if it
//     is at least 2^-12 away from every half-integer, both round to the same
//     integer. Closer estimates go to the exact path.
template <int C>
__device__ inline bool quarter_fast(const uint32_t (&w)[4], const uint4 (&rv)[2], float s, float o, int q,
                                    uint32_t (&nw)[4]) {
  constexpr int B = 1 << C, H = 16 / B, L = (1 << B) - 1;
  const int p0 = 8 * q, wbase = p0 / H;
  const float half_s = 0.5f * s;   // exact
  const float rs = __builtin_amdgcn_rcpf(s);
  bool ok = true;
#pragma unroll
  for (int i = 0; i < 4; ++i) nw[i] = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int pr = p0 + j / 2, odd = j & 1;
    const int wi = pr / H - wbase, sh = 16 * odd + (pr % H) * B;
    const uint32_t code = (w[wi] >> sh) & (uint32_t)L;
    const uint4& rr = rv[j / 8];
    const uint32_t rw = ((j / 2) & 3) == 0 ? rr.x : ((j / 2) & 3) == 1 ? rr.y : ((j / 2) & 3) == 2 ? rr.z : rr.w;
    const float r = __half2float(__ushort_as_half((unsigned short)(odd ? (rw >> 16) : (rw & 0xFFFF))));
    const float deq = __builtin_fmaf(s, (float)code, o);
    const float a = __fsub_rn(__fadd_rn(deq, r), o);
    const float t = a * rs;
    const float rt = rintf(t);
    const uint32_t qp = (uint32_t)__builtin_amdgcn_fmed3f(rt, 0.0f, (float)L);
    ok = ok && (fabsf(t - rt) < 0.5f - 0x1p-12f) && (qp == code) && (fabsf(r) < half_s);
    nw[wi] |= qp << sh;
  }
  return ok;
}

// The rare quarter that changes a code, leaves its cell, has a quotient near a
// rounding boundary or a scale that is not a finite positive number: redone
// with correctly rounded divisions, out of line (arguments and results by value, so that
// nothing has to live in memory) to keep its registers off the common path.
struct QuarterResult {
  uint32_t lm, lo;
  uint64_t lf;
  uint4 nw;
};

template <int C>
__device__ __attribute__((noinline)) QuarterResult quarter_exact(uint4 w4, uint4 r0v, uint4 r1v, float s, float o,
                                                                 int q, uint64_t lin0) {
  const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
  const uint4 rv[2] = {r0v, r1v};
  QuarterResult res;
  uint32_t nw[4];
  quarter_pass<C>(w, rv, s, o, q, lin0, res.lm, res.lo, res.lf, nw);
  res.nw = make_uint4(nw[0], nw[1], nw[2], nw[3]);
  return res;
}

// Checks one record (its 64 weights as four quarters of 16) of class C:
// w = the record's 2b code words, rv = its 64 residuals (32 pairs), lin0 =
// linear index of its first weight. Counts, first failing index and the
// re-quantised words (nw) are accumulated into the lane's state.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Largest |r| (fp16 bits) that provably keeps every code of a record with a
// finite scale s > 0, offset o and L = 2^b - 1, plus one: 0 when none does.
// With a = ((f32(s q) + o) + r) - o and t = a / s (three roundings and a
// correctly rounded quotient, unit roundoff u = 2^-24) the rounding errors
// add at most u (4 s (L + 1) + 2 |o|) to |t - q| s, so
//   |r| < 0.5 s - 2^-19 (s (L + 2) + |o|)
// gives |t - q| < 0.5: rint(t) = q (inside [0, L], so the clamp keeps it) and
// |r| < s / 2. The threshold is computed in binary32 (its own roundings are
// far inside the eightfold slack of 2^-19 over 4u) and rounded down to fp16.
__device__ inline uint32_t keep_bound_bits(float s, float o, int L) {
  if (!(s > 0.0f && s <= 65504.0f)) return 0u;
  const float thr = 0.5f * s - 0x1p-19f * (s * (float)(L + 2) + fabsf(o));
  if (!(thr > 0.0f)) return 0u;
  uint32_t h = __half_as_ushort(__float2half(thr));
  if (__half2float(__ushort_as_half((unsigned short)h)) > thr) --h;   // round down (h >= 1 here)
  return h;
}

template <int C>
__device__ inline void check_record(const uint32_t* w, const uint4 (&rv)[8], uint32_t so, uint64_t lin0,
                                    uint32_t& mism, uint32_t& ooc, uint64_t& first, uint32_t* nw) {
  constexpr int B = 1 << C, H = 16 / B, NWORD = 2 * B;
  const float s = __half2float(__ushort_as_half((unsigned short)(so & 0xFFFF)));
  const float o = __half2float(__ushort_as_half((unsigned short)(so >> 16)));
  // The common case: every |r| of the record under the bound above, so every
  // code comes back unchanged and every residual is inside its cell. The
  // largest |r| is taken on the fp16 bit patterns (sign cleared; the
  // patterns of non-negative values, infinities and NaNs order as unsigned
  // integers, and NaN or infinite residuals never pass).
  {
    u16x2 mx = {0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t v[4] = {rv[i].x, rv[i].y, rv[i].z, rv[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, v[j] & 0x7FFF7FFFu));
    }
    const uint32_t top = mx.x > mx.y ? mx.x : mx.y;
    if (top < keep_bound_bits(s, o, (1 << B) - 1)) {
#pragma unroll
      for (int i = 0; i < NWORD; ++i) nw[i] = w[i];
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < NWORD; ++i) nw[i] = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int wbase = (8 * q) / H;
    uint32_t win[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) win[i] = (wbase + i < NWORD) ? w[wbase + i < NWORD ? wbase + i : 0] : 0u;
    const uint4 rq[2] = {rv[2 * q], rv[2 * q + 1]};
    uint32_t qw[4];
    const bool fast = s > 0.0f && s <= 65504.0f && quarter_fast<C>(win, rq, s, o, q, qw);
    if (!fast) {
      const QuarterResult e = quarter_exact<C>(make_uint4(win[0], win[1], win[2], win[3]), rq[0], rq[1], s, o, q,
                                               lin0 + 16u * (uint32_t)q);
      qw[0] = e.nw.x;
      qw[1] = e.nw.y;
      qw[2] = e.nw.z;
      qw[3] = e.nw.w;
      mism += e.lm;
      ooc += e.lo;
      first = e.lf < first ? e.lf : first;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (wbase + i < NWORD) nw[(wbase + i) < NWORD ? wbase + i : 0] |= qw[i];
  }
}

// With the re-quantised stream (k_verify): one workgroup of four wavefronts
// per tile, lane l on column l: a column's records of each class are taken in
// row order, wavefront w checking every fourth of them (those with index
// w mod 4 in the column): codes and scale/offset at the record's position,
// the record's 64 residuals from its row, columns 64 (64 kt + l) .. + 63.
// Without it, k_verify_rows (below) reads the residual in row order.
constexpr int kVerifyWaves = 4;

template <int C>
__device__ inline void verify_record(const uint8_t* tb, uint8_t* rb, RecPos rp, const uint16_t* __restrict__ resid,
                                     uint64_t lin0, size_t roff, uint32_t& mism, uint32_t& ooc, uint64_t& first) {
  constexpr int B = 1 << C;
  uint32_t w[2 * B];
  const uint8_t* cp = tb + rp.codes;
  if constexpr (C == 0) {
    const uint2 u = *reinterpret_cast<const uint2*>(cp);
    w[0] = u.x;
    w[1] = u.y;
  } else {
#pragma unroll
    for (int h = 0; h < B / 2; ++h) {
      const uint4 u = reinterpret_cast<const uint4*>(cp)[h];
      w[4 * h + 0] = u.x;
      w[4 * h + 1] = u.y;
      w[4 * h + 2] = u.z;
      w[4 * h + 3] = u.w;
    }
  }
  const uint32_t so = *reinterpret_cast<const uint32_t*>(tb + rp.so);
  uint4 rv[8];
  const uint4* rp16 = reinterpret_cast<const uint4*>(resid + roff);
#pragma unroll
  for (int i = 0; i < 8; ++i) rv[i] = rp16[i];
  uint32_t nw[2 * B];
  check_record<C>(w, rv, so, lin0, mism, ooc, first, nw);
  if (rb) {
    uint8_t* dp = rb + rp.codes;
    if constexpr (C == 0) {
      *reinterpret_cast<uint2*>(dp) = make_uint2(nw[0], nw[1]);
    } else {
#pragma unroll
      for (int h = 0; h < B / 2; ++h)
        reinterpret_cast<uint4*>(dp)[h] = make_uint4(nw[4 * h + 0], nw[4 * h + 1], nw[4 * h + 2], nw[4 * h + 3]);
    }
  }
}

__global__ __launch_bounds__(kVerifyWaves * 64) void k_verify(const uint32_t* __restrict__ tiles,
                                                               const uint8_t* __restrict__ stream, int N, int G,
                                                               int RT, const uint16_t* __restrict__ resid,
                                                               uint64_t* result, uint8_t* requant) {
  __shared__ uint32_t s_mism, s_ooc;
  __shared__ unsigned long long s_first;
  const int t = (int)blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid == 0) {
    s_mism = 0;
    s_ooc = 0;
    s_first = ~0ull;
  }
  const size_t K = (size_t)G * kGroup;
  const int kt = t / RT, rt = t - kt * RT;
  const int r0 = rt * kTileRows, R = min(kTileRows, N - r0);
  const int g0 = kt * kTileGroups, Gt = min(kTileGroups, G - g0);
  const uint64_t tbyte = (uint64_t)tiles[4 * t + 0] * 16;
  const uint32_t size = tiles[4 * t + 1] * 16, w2 = tiles[4 * t + 2], w3 = tiles[4 * t + 3];
  const uint8_t* tb = stream + tbyte;
  uint8_t* rb = requant ? requant + tbyte : nullptr;
  // Copy the tile (map, scales, offsets, padding); codes are rewritten below.
  if (rb)
    for (uint32_t i = tid; i < size / 16; i += kVerifyWaves * 64)
      reinterpret_cast<uint4*>(rb)[i] = reinterpret_cast<const uint4*>(tb)[i];
  __syncthreads();
  const bool live = lane < Gt;
  const uint2 mp = live ? *reinterpret_cast<const uint2*>(tb + 8 * lane) : make_uint2(0u, 0u);
  const ClassMasks km = class_masks(mp.x, mp.y, live ? R : 0);
  uint32_t mism = 0, ooc = 0;
  uint64_t first = ~0ull;
  uint32_t cbase = map_bytes((uint32_t)Gt);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t n = class_count(w2, w3, c);
    uint32_t mask = km.m[c];
    uint32_t e = wave_excl_scan((uint32_t)__popc(mask), (uint32_t)lane);
    for (uint32_t j = 0; mask; mask &= mask - 1u, ++e, ++j) {
      if ((int)(j % kVerifyWaves) != wave) continue;
      const int row = r0 + __builtin_ctz(mask);
      const RecPos rp = record_pos(c, n, cbase, e);
      const size_t roff = (size_t)row * K + (size_t)(g0 + lane) * kGroup;
      const uint64_t lin0 = (uint64_t)roff;
      switch (c) {
        case 0: verify_record<0>(tb, rb, rp, resid, lin0, roff, mism, ooc, first); break;
        case 1: verify_record<1>(tb, rb, rp, resid, lin0, roff, mism, ooc, first); break;
        case 2: verify_record<2>(tb, rb, rp, resid, lin0, roff, mism, ooc, first); break;
        default: verify_record<3>(tb, rb, rp, resid, lin0, roff, mism, ooc, first); break;
      }
    }
    cbase += class_bytes(c, n);
  }
  if (mism) atomicAdd(&s_mism, mism);
  if (ooc) atomicAdd(&s_ooc, ooc);
  if (first != ~0ull) atomicMin(&s_first, (unsigned long long)first);
  __syncthreads();
  if (tid == 0) {
    if (s_mism) atomicAdd(reinterpret_cast<unsigned long long*>(&result[0]), (unsigned long long)s_mism);
    if (s_ooc) atomicAdd(reinterpret_cast<unsigned long long*>(&result[1]), (unsigned long long)s_ooc);
    if (s_first != ~0ull) atomicMin(reinterpret_cast<unsigned long long*>(&result[2]), s_first);
  }
}

// ---- Re-quantisation check without the re-quantised stream --------------------
// The residual is read in row order: a wavefront takes one row of a tile at a
// time, and load i of lane l is the 16 bytes (8 weights) at 16 (64 i + l) of
// the row's 8 KiB stretch, so consecutive lanes read consecutive bytes. That
// piece belongs to the record of column 8 i + l / 8 (weights 8 (l % 8) ..
// + 7). Every weight is decided on its own, so a lane checks its eight
// weights against the record's scale and offset: under the record-level
// bound on |r| all eight keep their codes and stay in their cells; otherwise
// they are redone one by one with correctly rounded quotients (the codes are
// loaded only then). Workgroups of four wavefronts take kVerifyRowsPerWg
// rows of a tile each.
constexpr int kVerifyRowsPerWg = 8;

// Per column of the tile, in LDS: the map planes and, per class, the class's
// records in the columns before it.
struct VerifyCols {
  uint32_t p0[kTileGroups], p1[kTileGroups];
  uint16_t pre[4][kTileGroups];
};

// The exact decision for weights 8m .. 8m + 7 of a record of width b = 2^C
// (any scale): counts into lm / lo and the smallest failing linear index.
template <int C>
__device__ __attribute__((noinline)) void piece_exact(uint2 cw, uint4 rr, float s, float o, int m, uint64_t lin0,
                                                      uint32_t& lm, uint32_t& lo, uint64_t& lf) {
  constexpr int B = 1 << C, H = 16 / B, L = (1 << B) - 1;
  const int w0 = (4 * m) / H;   // first code word of the piece (cw.x; cw.y the next)
  const float half_s = __fmul_rn(0.5f, s);
  const uint32_t rw[4] = {rr.x, rr.y, rr.z, rr.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int k = 8 * m + j, pr = k >> 1, odd = k & 1;
    const int wi = pr / H - w0, sh = 16 * odd + (pr % H) * B;
    const uint32_t code = ((wi == 0 ? cw.x : cw.y) >> sh) & (uint32_t)L;
    const uint32_t h = (rw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
    const float r = __half2float(__ushort_as_half((unsigned short)h));
    const float deq = __fadd_rn(__fmul_rn(s, (float)code), o);
    const float a = __fsub_rn(__fadd_rn(deq, r), o);
    uint32_t qp = 0;
    if (s != 0.0f) {
      float t = rintf(__fdiv_rn(a, s));
      t = t < 0.0f ? 0.0f : t;
      t = t > (float)L ? (float)L : t;
      qp = (uint32_t)t;
    }
    const bool bad_code = qp != code;
    const bool bad_cell = (s > 0.0f) ? (fabsf(r) >= half_s) : (r != 0.0f);
    lm += bad_code;
    lo += bad_cell;
    if ((bad_code || bad_cell) && lin0 + j < lf) lf = lin0 + j;
  }
}

__global__ __launch_bounds__(kVerifyWaves * 64) void k_verify_rows(const uint32_t* __restrict__ tiles,
                                                                    const uint8_t* __restrict__ stream, int N, int G,
                                                                    int RT, const uint16_t* __restrict__ resid,
                                                                    uint64_t* result) {
  __shared__ VerifyCols cols;
  __shared__ uint32_t s_mism, s_ooc;
  __shared__ unsigned long long s_first;
  constexpr int kParts = kTileRows / kVerifyRowsPerWg;
  const int t = (int)blockIdx.x / kParts, part = (int)blockIdx.x % kParts;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const size_t K = (size_t)G * kGroup;
  const int kt = t / RT, rt = t - kt * RT;
  const int r0 = rt * kTileRows, R = min(kTileRows, N - r0);
  const int g0 = kt * kTileGroups, Gt = min(kTileGroups, G - g0);
  const uint8_t* tb = stream + (uint64_t)tiles[4 * t + 0] * 16;
  const uint32_t w2 = tiles[4 * t + 2], w3 = tiles[4 * t + 3];
  if (wave == 0) {
    const bool live = lane < Gt;
    const uint2 mp = live ? *reinterpret_cast<const uint2*>(tb + 8 * lane) : make_uint2(0u, 0u);
    const ClassMasks km = class_masks(mp.x, mp.y, live ? R : 0);
    cols.p0[lane] = mp.x;
    cols.p1[lane] = mp.y;
#pragma unroll
    for (int c = 0; c < 4; ++c) cols.pre[c][lane] = (uint16_t)wave_excl_scan((uint32_t)__popc(km.m[c]), (uint32_t)lane);
  }
  if (tid == 0) {
    s_mism = 0;
    s_ooc = 0;
    s_first = ~0ull;
  }
  uint32_t n[4], cb[4];
  uint32_t cbase = map_bytes((uint32_t)Gt);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    n[c] = class_count(w2, w3, c);
    cb[c] = cbase;
    cbase += class_bytes(c, n[c]);
  }
  __syncthreads();
  uint32_t mism = 0, ooc = 0;
  uint64_t first = ~0ull;
  const int m = lane & 7;   // the lane's eight weights of a record
  const uint32_t valid = R >= 32 ? 0xFFFFFFFFu : ((1u << R) - 1u);
  for (int rr = wave; rr < kVerifyRowsPerWg; rr += kVerifyWaves) {
    const int row = part * kVerifyRowsPerWg + rr;
    if (row >= R) break;
    const uint4* rrow = reinterpret_cast<const uint4*>(resid + (size_t)(r0 + row) * K + (size_t)g0 * kGroup);
    uint4 rv[8];
    uint32_t so[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int g = 8 * i + (lane >> 3);
      so[i] = 0u;
      rv[i] = make_uint4(0u, 0u, 0u, 0u);
      if (g < Gt) {
        rv[i] = rrow[64 * i + lane];
        const uint32_t p0 = cols.p0[g], p1 = cols.p1[g];
        const int c = (int)((p0 >> row) & 1u) | (int)(((p1 >> row) & 1u) << 1);
        const uint32_t mc = ((c & 1) ? p0 : ~p0) & ((c & 2) ? p1 : ~p1) & valid;
        const uint32_t e = (uint32_t)cols.pre[c][g] + (uint32_t)__popc(mc & ((1u << row) - 1u));
        const uint32_t nc = c == 0 ? n[0] : c == 1 ? n[1] : c == 2 ? n[2] : n[3];
        const uint32_t bc = c == 0 ? cb[0] : c == 1 ? cb[1] : c == 2 ? cb[2] : cb[3];
        so[i] = *reinterpret_cast<const uint32_t*>(tb + record_pos(c, nc, bc, e).so);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int g = 8 * i + (lane >> 3);
      if (g >= Gt) continue;
      const uint32_t p0 = cols.p0[g], p1 = cols.p1[g];
      const int c = (int)((p0 >> row) & 1u) | (int)(((p1 >> row) & 1u) << 1);
      const float sc = __half2float(__ushort_as_half((unsigned short)(so[i] & 0xFFFFu)));
      const float of = __half2float(__ushort_as_half((unsigned short)(so[i] >> 16)));
      const uint32_t v[4] = {rv[i].x, rv[i].y, rv[i].z, rv[i].w};
      uint32_t mx = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t a = v[j] & 0x7FFF7FFFu;
        mx = max(mx, max(a & 0xFFFFu, a >> 16));
      }
      if (mx < keep_bound_bits(sc, of, (1 << (1 << c)) - 1)) continue;
      // the rare piece: its code word(s), then the exact decisions
      const uint32_t mc = ((c & 1) ? p0 : ~p0) & ((c & 2) ? p1 : ~p1) & valid;
      const uint32_t e = (uint32_t)cols.pre[c][g] + (uint32_t)__popc(mc & ((1u << row) - 1u));
      const uint32_t nc = c == 0 ? n[0] : c == 1 ? n[1] : c == 2 ? n[2] : n[3];
      const uint32_t bc = c == 0 ? cb[0] : c == 1 ? cb[1] : c == 2 ? cb[2] : cb[3];
      const int h = 16 >> c, w0 = (4 * m) / h;
      const uint32_t* cwp = reinterpret_cast<const uint32_t*>(tb + record_pos(c, nc, bc, e).codes) + w0;
      const uint2 cw = make_uint2(cwp[0], c == 3 ? cwp[1] : 0u);
      const uint64_t lin0 = (uint64_t)(r0 + row) * K + (uint64_t)(g0 + g) * kGroup + 8u * (uint32_t)m;
      switch (c) {
        case 0: piece_exact<0>(cw, rv[i], sc, of, m, lin0, mism, ooc, first); break;
        case 1: piece_exact<1>(cw, rv[i], sc, of, m, lin0, mism, ooc, first); break;
        case 2: piece_exact<2>(cw, rv[i], sc, of, m, lin0, mism, ooc, first); break;
        default: piece_exact<3>(cw, rv[i], sc, of, m, lin0, mism, ooc, first); break;
      }
    }
  }
  if (mism) atomicAdd(&s_mism, mism);
  if (ooc) atomicAdd(&s_ooc, ooc);
  if (first != ~0ull) atomicMin(&s_first, (unsigned long long)first);
  __syncthreads();
  if (tid == 0) {
    if (s_mism) atomicAdd(reinterpret_cast<unsigned long long*>(&result[0]), (unsigned long long)s_mism);
    if (s_ooc) atomicAdd(reinterpret_cast<unsigned long long*>(&result[1]), (unsigned long long)s_ooc);
    if (s_first != ~0ull) atomicMin(reinterpret_cast<unsigned long long*>(&result[2]), s_first);
  }
}

hipError_t launch_verify(const vbq_matrix& m, const uint16_t* resid, uint64_t* result, uint32_t* requant,
                         hipStream_t s) {
  hipLaunchKernelGGL(k_verify_init, dim3(1), dim3(64), 0, s, result);
  if (!requant) {
    constexpr int64_t kParts = kTileRows / kVerifyRowsPerWg;
    if (m.n_tiles * kParts > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_verify_rows, dim3((unsigned)(m.n_tiles * kParts)), dim3(kVerifyWaves * 64), 0, s, m.tiles,
                       reinterpret_cast<const uint8_t*>(m.stream), m.n_rows, m.n_cols / kGroup, row_tiles(m.n_rows),
                       resid, result);
    return hipGetLastError();
  }
  if (m.n_tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_verify, dim3((unsigned)m.n_tiles), dim3(kVerifyWaves * 64), 0, s, m.tiles,
                     reinterpret_cast<const uint8_t*>(m.stream), m.n_rows, m.n_cols / kGroup, row_tiles(m.n_rows),
                     resid, result, reinterpret_cast<uint8_t*>(requant));
  return hipGetLastError();
}

// ---- Drift bound ------------------------------------------------------------
// bound[b][n] = 0.5 * sum_g s[n][g] * X[b][g],  X[b][g] = sum_{k in g} |x[b][k]|:
// with every residual strictly inside half its group's scale, no output moves
// further than this (CellFill abstract: bounded drift). One workgroup of four
// wavefronts per row-tile walks its k-tiles in order. Per k-tile it forms X
// for the tile's groups (fp32, in k order, from 16-byte loads); lane l takes
// the records of column l in rows 8w .. 8w + 7 (wavefront w): a record's
// index in its class follows from the map planes (the class's records in the
// columns before, from a wave scan, plus its rank in its column), so the
// eight scale loads of a lane go out together. Each record puts
// 0.5 s X[b][l] at its (row, column) slot in LDS (a row has exactly one
// record per column); then one thread per (batch row, row) adds its slots in
// column order, so the sum order is fixed. Batches above four rows run as
// passes.
constexpr int kDriftThreads = 256;
constexpr int kDriftNb = 4;

template <int NB>
__global__ __launch_bounds__(kDriftThreads) void k_drift(const uint32_t* __restrict__ tiles,
                                                         const uint8_t* __restrict__ stream,
                                                         const uint16_t* __restrict__ x, int N, int G, int RT,
                                                         float* __restrict__ bound) {
  __shared__ float X[NB][kTileGroups];
  __shared__ float P[NB][kTileRows][kTileGroups + 1];
  const int rt = (int)blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = G * kGroup;
  const int r0 = rt * kTileRows, R = min(kTileRows, N - r0);
  const int b_own = tid / kTileRows, r_own = tid % kTileRows;   // summed by this thread while tid < NB * 32
  float acc = 0.0f;
  const int KT = k_tiles(G);
  constexpr int kRowsPerWave = kTileRows / 4;
  for (int kt = 0; kt < KT; ++kt) {
    const int g0 = kt * kTileGroups, Gt = min(kTileGroups, G - g0);
    // The scale loads need only the tile header and the width map, so they
    // go out before the activation sums are formed.
    const int t = kt * RT + rt;
    const uint8_t* tb = stream + (size_t)tiles[4 * t + 0] * 16;
    const uint32_t w2 = tiles[4 * t + 2], w3 = tiles[4 * t + 3];
    const bool live = lane < Gt;
    const uint2 mp = live ? *reinterpret_cast<const uint2*>(tb + 8 * lane) : make_uint2(0u, 0u);
    const ClassMasks km = class_masks(mp.x, mp.y, live ? R : 0);
    // per class: its record count, first block and the records in the
    // columns before this lane's
    uint32_t n[4], cb[4], pre[4];
    uint32_t cbase = map_bytes((uint32_t)Gt);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      n[c] = class_count(w2, w3, c);
      cb[c] = cbase;
      pre[c] = wave_excl_scan((uint32_t)__popc(km.m[c]), (uint32_t)lane);
      cbase += class_bytes(c, n[c]);
    }
    uint32_t so[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int row = kRowsPerWave * wave + i;
      const uint32_t bit = 1u << row;
      const int c = (int)((mp.x >> row) & 1u) | (int)(((mp.y >> row) & 1u) << 1);
      const uint32_t mc = c == 0 ? km.m[0] : c == 1 ? km.m[1] : c == 2 ? km.m[2] : km.m[3];
      const uint32_t nc = c == 0 ? n[0] : c == 1 ? n[1] : c == 2 ? n[2] : n[3];
      const uint32_t bc = c == 0 ? cb[0] : c == 1 ? cb[1] : c == 2 ? cb[2] : cb[3];
      const uint32_t pc = c == 0 ? pre[0] : c == 1 ? pre[1] : c == 2 ? pre[2] : pre[3];
      so[i] = 0u;
      if (mc & bit) {   // a record (live column, row < R)
        const uint32_t e = pc + (uint32_t)__popc(mc & (bit - 1u));
        so[i] = *reinterpret_cast<const uint32_t*>(tb + record_pos(c, nc, bc, e).so);
      }
    }
    for (int i = tid; i < NB * kTileGroups; i += kDriftThreads) {
      const int b = i / kTileGroups, g = i - b * kTileGroups;
      float sx = 0.0f;
      if (g < Gt) {
        // x rows are 128-byte aligned per group (the caller's buffer is
        // 16-byte aligned and K is a multiple of 64)
        const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)b * K + (size_t)(g0 + g) * kGroup);
        uint4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = xr[j];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            sx += fabsf(__half2float(__ushort_as_half((unsigned short)(w[h] & 0xFFFFu))));
            sx += fabsf(__half2float(__ushort_as_half((unsigned short)(w[h] >> 16))));
          }
        }
      }
      X[b][g] = sx;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int row = kRowsPerWave * wave + i;
      const float hs = 0.5f * __half2float(__ushort_as_half((unsigned short)(so[i] & 0xFFFFu)));
      if (live && row < R)
#pragma unroll
        for (int b = 0; b < NB; ++b) P[b][row][lane] = hs * X[b][lane];
    }
    __syncthreads();
    // the slots of a row in column order; columns past the tile add +0,
    // which leaves the (non-negative) sum unchanged
    if (tid < NB * kTileRows) {
      float v[kTileGroups];
#pragma unroll
      for (int g = 0; g < kTileGroups; ++g) v[g] = g < Gt ? P[b_own][r_own][g] : 0.0f;
#pragma unroll
      for (int g = 0; g < kTileGroups; ++g) acc += v[g];
    }
    __syncthreads();   // X and P are rewritten for the next k-tile
  }
  if (tid < NB * kTileRows && r_own < R) bound[(size_t)b_own * N + r0 + r_own] = acc;
}

hipError_t launch_drift(const vbq_matrix& m, const uint16_t* x, int B, float* bound, hipStream_t s) {
  const int RT = row_tiles(m.n_rows), G = m.n_cols / kGroup;
  const uint8_t* st = reinterpret_cast<const uint8_t*>(m.stream);
  for (int b0 = 0; b0 < B; b0 += kDriftNb) {
    const int nb = B - b0 < kDriftNb ? B - b0 : kDriftNb;
    const uint16_t* xb = x + (size_t)b0 * m.n_cols;
    float* yb = bound + (size_t)b0 * m.n_rows;
#define VBQ_DRIFT(NB)                                                                                        \
  case NB:                                                                                                   \
    hipLaunchKernelGGL(k_drift<NB>, dim3(RT), dim3(kDriftThreads), 0, s, m.tiles, st, xb, m.n_rows, G, RT, yb); \
    break;
    switch (nb) {
      VBQ_DRIFT(1)
      VBQ_DRIFT(2)
      VBQ_DRIFT(3)
      VBQ_DRIFT(4)
      default:
        return hipErrorInvalidValue;
    }
#undef VBQ_DRIFT
  }
  return hipGetLastError();
}

}  // namespace vbq
