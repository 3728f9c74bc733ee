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
// (built with -ffp-contract=off; the quotient decides as the correctly
// rounded one does, see quarter_fast):
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
template <int C>
__device__ inline void check_record(const uint32_t* w, const uint4 (&rv)[8], uint32_t so, uint64_t lin0,
                                    uint32_t& mism, uint32_t& ooc, uint64_t& first, uint32_t* nw) {
  constexpr int B = 1 << C, H = 16 / B, NWORD = 2 * B;
  const float s = __half2float(__ushort_as_half((unsigned short)(so & 0xFFFF)));
  const float o = __half2float(__ushort_as_half((unsigned short)(so >> 16)));
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

// One workgroup of four wavefronts per tile, lane l on column l: a column's
// records of each class are taken in row order, wavefront w checking every
// fourth of them (those with index w mod 4 in the column): codes and
// scale/offset at the record's position, the record's 64 residuals from its
// row, columns 64 (64 kt + l) .. + 63.
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

hipError_t launch_verify(const vbq_matrix& m, const uint16_t* resid, uint64_t* result, uint32_t* requant,
                         hipStream_t s) {
  hipLaunchKernelGGL(k_verify_init, dim3(1), dim3(64), 0, s, result);
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
// for the tile's groups (fp32, in k order); lane l takes the records of
// column l (wavefront w every fourth of them) and each record puts
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
  for (int kt = 0; kt < KT; ++kt) {
    const int g0 = kt * kTileGroups, Gt = min(kTileGroups, G - g0);
    for (int i = tid; i < NB * kTileGroups; i += kDriftThreads) {
      const int b = i / kTileGroups, g = i - b * kTileGroups;
      float sx = 0.0f;
      if (g < Gt) {
        const uint16_t* xr = x + (size_t)b * K + (size_t)(g0 + g) * kGroup;
        for (int j = 0; j < kGroup; ++j) sx += fabsf(__half2float(__ushort_as_half(xr[j])));
      }
      X[b][g] = sx;
    }
    __syncthreads();
    const int t = kt * RT + rt;
    const uint8_t* tb = stream + (size_t)tiles[4 * t + 0] * 16;
    const uint32_t w2 = tiles[4 * t + 2], w3 = tiles[4 * t + 3];
    const bool live = lane < Gt;
    const uint2 mp = live ? *reinterpret_cast<const uint2*>(tb + 8 * lane) : make_uint2(0u, 0u);
    const ClassMasks km = class_masks(mp.x, mp.y, live ? R : 0);
    uint32_t cbase = map_bytes((uint32_t)Gt);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t n = class_count(w2, w3, c);
      uint32_t mask = km.m[c];
      uint32_t e = wave_excl_scan((uint32_t)__popc(mask), (uint32_t)lane);
      for (uint32_t j = 0; mask; mask &= mask - 1u, ++e, ++j) {
        if ((int)(j % 4u) != wave) continue;
        const int row = __builtin_ctz(mask);
        const uint32_t so = *reinterpret_cast<const uint32_t*>(tb + record_pos(c, n, cbase, e).so);
        const float hs = 0.5f * __half2float(__ushort_as_half((unsigned short)(so & 0xFFFFu)));
#pragma unroll
        for (int b = 0; b < NB; ++b) P[b][row][lane] = hs * X[b][lane];
      }
      cbase += class_bytes(c, n);
    }
    __syncthreads();
    if (tid < NB * kTileRows)
      for (int g = 0; g < Gt; ++g) acc += P[b_own][r_own][g];
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
