// Re-quantisation check of an in-cell update.
//
// CellFill abstract (page "Nothing Changed but the Model: CellFill -- Bounded
// In-Cell Learning for Bit-Identical, Revocable Updates to Quantized LLMs"):
// with the integer codes and scales of a release frozen, the update lives in a
// per-weight residual strictly inside each quantisation cell, and
// re-quantisation returns the released artifact bit-for-bit. For every weight
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

// One quarter of a record: 16 consecutive weights (codes 16q .. 16q + 15).
// The pair layout puts them in pairs 8q .. 8q + 7, i.e. in words
// [8q / H, (8q + 7) / H] of the record (H = 16 / b pairs per word): loaded as
// one 16-byte read starting at word 8q / H (reading past the record stays in
// its block, whose scale/offset and meta areas follow the codes).
struct Quarter {
  uint4 w;         // words from 8q / H on
  uint32_t so;     // scale | offset << 16
  uint32_t meta;   // row | k-group << 4
  uint32_t wbyte;  // byte offset of w in the stream
  int c;           // width class, -1 if no record
};

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

template <int C>
__device__ inline void check_quarter(const Quarter& Qr, int q, int r0, int g0, int K, const uint4 (&rv)[2],
                                     uint32_t& mism, uint32_t& ooc, uint64_t& first, uint32_t (&nw)[4]) {
  const uint32_t w[4] = {Qr.w.x, Qr.w.y, Qr.w.z, Qr.w.w};
  const float s = __half2float(__ushort_as_half((unsigned short)(Qr.so & 0xFFFF)));
  const float o = __half2float(__ushort_as_half((unsigned short)(Qr.so >> 16)));
  const bool fast = s > 0.0f && s <= 65504.0f && quarter_fast<C>(w, rv, s, o, q, nw);
  if (!fast) {
    const int row = r0 + (int)(Qr.meta & 15), kg = g0 + (int)(Qr.meta >> 4);
    const uint64_t lin0 = (uint64_t)row * K + (uint64_t)kg * kGroup + 16u * (uint32_t)q;
    const QuarterResult e = quarter_exact<C>(Qr.w, rv[0], rv[1], s, o, q, lin0);
    nw[0] = e.nw.x;
    nw[1] = e.nw.y;
    nw[2] = e.nw.z;
    nw[3] = e.nw.w;
    mism += e.lm;
    ooc += e.lo;
    first = e.lf < first ? e.lf : first;
  }
}

// One workgroup of 256 threads per tile (several resident per CU, so one's
// memory round trips overlap another's arithmetic), four lanes per record (a
// quarter each), sixteen quarters per lane in batches of two (at most 96
// VGPRs: five wavefronts per SIMD). All loads of a batch are issued together:
// the records' codes, scale/offset and meta, then the residuals the meta
// points at.
constexpr int kVerifyThreads = 256;

// Without the re-quantised stream, a tile's records are split over
// kVerifyParts workgroups (more round trips in flight per CU); with it, one
// workgroup per tile copies the tile and rewrites its codes.
constexpr int kVerifyParts = 4;

__global__ __launch_bounds__(kVerifyThreads, 5) void k_verify(const uint32_t* __restrict__ tiles,
                                                           const uint8_t* __restrict__ stream, int G, int RT,
                                                           const uint16_t* __restrict__ resid, uint64_t* result,
                                                           uint8_t* requant, int parts) {
  __shared__ uint32_t s_mism, s_ooc;
  __shared__ unsigned long long s_first;
  const int t = (int)blockIdx.x / parts, part = (int)blockIdx.x - t * parts, tid = threadIdx.x;
  if (tid == 0) {
    s_mism = 0;
    s_ooc = 0;
    s_first = ~0ull;
  }
  const int K = G * kGroup;
  const int kt = t / RT, rt = t - kt * RT;
  const int r0 = rt * kTile, g0 = kt * kTileGroups;
  const uint64_t tb = (uint64_t)tiles[4 * t + 1] * 16;
  const uint32_t a = tiles[4 * t + 2], bb = tiles[4 * t + 3];
  const uint32_t n[4] = {a & 0xFFFF, a >> 16, bb & 0xFFFF, bb >> 16};
  const uint32_t sb[4] = {0, (uint32_t)seg_bytes(0, n[0]), (uint32_t)(seg_bytes(0, n[0]) + seg_bytes(1, n[1])),
                          (uint32_t)(seg_bytes(0, n[0]) + seg_bytes(1, n[1]) + seg_bytes(2, n[2]))};
  const uint32_t size = sb[3] + (uint32_t)seg_bytes(3, n[3]);
  const uint8_t* tbytes = stream + tb;
  uint8_t* rbytes = requant ? requant + tb : nullptr;
  // Copy the tile (scales, offsets, meta, padding); codes are rewritten below.
  if (rbytes)
    for (uint32_t i = tid; i < size / 16; i += kVerifyThreads)
      reinterpret_cast<uint4*>(rbytes)[i] = reinterpret_cast<const uint4*>(tbytes)[i];
  __syncthreads();
  const uint32_t total = n[0] + n[1] + n[2] + n[3];
  const int q = tid & 3;
  uint32_t mism = 0, ooc = 0;
  uint64_t first = ~0ull;
  constexpr int kPer = kTile * kTileGroups * 4 / kVerifyThreads;   // quarters per thread: 16
  constexpr int kBatch = 2;                                         // quarters loaded together
  const int per = kPer / parts;                                     // quarters of this workgroup per thread
  const uint32_t ibase = (uint32_t)(part * per) * (kVerifyThreads / 4);
  for (int b0 = 0; b0 < per; b0 += kBatch) {
    Quarter Q[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const uint32_t i = ibase + (uint32_t)(tid >> 2) + (uint32_t)(b0 + u) * (kVerifyThreads / 4);
      Q[u].c = -1;
      Q[u].wbyte = 0;
      if (i < total) {
        int c = 0;
        uint32_t idx = i;
        while (c < 3 && idx >= n[c]) {
          idx -= n[c];
          ++c;
        }
        const uint32_t br = block_records(c), k = idx / br, l = idx - k * br, m = min(br, n[c] - k * br);
        const uint32_t blk = sb[c] + k * (uint32_t)block_bytes(c, br);
        const uint32_t H = 16u >> c;
        Q[u].c = c;
        Q[u].wbyte = blk + (8u << c) * l + 4u * ((8u * (uint32_t)q) / H);
        Q[u].so = *reinterpret_cast<const uint32_t*>(tbytes + blk + codes_area(c, m) + 4u * l);
        Q[u].meta = *reinterpret_cast<const uint16_t*>(tbytes + blk + codes_area(c, m) + so_area(m) + 2u * l);
        // 4-byte aligned; a 16-byte read from here stays inside the block
        const uint32_t* wp = reinterpret_cast<const uint32_t*>(tbytes + Q[u].wbyte);
        Q[u].w = make_uint4(wp[0], wp[1], wp[2], wp[3]);
      }
    }
    uint4 R[kBatch][2];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      R[u][0] = R[u][1] = make_uint4(0, 0, 0, 0);
      if (Q[u].c >= 0) {
        const int row = r0 + (int)(Q[u].meta & 15), kg = g0 + (int)(Q[u].meta >> 4);
        const uint4* rp =
            reinterpret_cast<const uint4*>(resid + (uint64_t)row * K + (uint64_t)kg * kGroup + 16u * q);
        R[u][0] = rp[0];
        R[u][1] = rp[1];
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int c = Q[u].c;
      uint32_t nw[4];
      if (c == 0) check_quarter<0>(Q[u], q, r0, g0, K, R[u], mism, ooc, first, nw);
      else if (c == 1) check_quarter<1>(Q[u], q, r0, g0, K, R[u], mism, ooc, first, nw);
      else if (c == 2) check_quarter<2>(Q[u], q, r0, g0, K, R[u], mism, ooc, first, nw);
      else if (c == 3) check_quarter<3>(Q[u], q, r0, g0, K, R[u], mism, ooc, first, nw);
      if (c < 0) continue;
      // 1-bit: the two quarters of one code word combine their bits
      if (c == 0) nw[0] |= __shfl_xor(nw[0], 1, kWave);
      if (rbytes) {
        uint32_t* dst = reinterpret_cast<uint32_t*>(rbytes + Q[u].wbyte);
        if (c == 0) {
          if ((q & 1) == 0) dst[0] = nw[0];
        } else {
          const int nword = c == 1 ? 1 : c == 2 ? 2 : 4;
          for (int i = 0; i < nword; ++i) dst[i] = nw[i];
        }
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
  const int parts = requant ? 1 : kVerifyParts;
  if ((int64_t)m.n_tiles * parts > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_verify, dim3((unsigned)(m.n_tiles * parts)), dim3(kVerifyThreads), 0, s, m.tiles,
                     reinterpret_cast<const uint8_t*>(m.stream), m.n_cols / kGroup, row_tiles(m.n_rows), resid,
                     result, reinterpret_cast<uint8_t*>(requant), parts);
  return hipGetLastError();
}

// ---- Drift bound ------------------------------------------------------------
// bound[b][n] = 0.5 * sum_g s[n][g] * X[b][g],  X[b][g] = sum_{k in g} |x[b][k]|:
// with every residual strictly inside half its group's scale, no output moves
// further than this (CellFill abstract: bounded drift). One workgroup per
// row-tile walks its k-tiles in order. Per k-tile it forms X for the tile's
// groups (fp32, in k order); every record puts 0.5 s X[b][g] at its (row,
// group) slot in LDS (a row has exactly one record per group); and one thread
// per (batch row, row) adds its slots in group order, so the sum order is
// fixed.
constexpr int kDriftThreads = 256;

template <int NB>
__global__ __launch_bounds__(kDriftThreads) void k_drift(const uint32_t* __restrict__ tiles,
                                                         const uint8_t* __restrict__ stream,
                                                         const uint16_t* __restrict__ x, int N, int G, int RT,
                                                         float* __restrict__ bound) {
  __shared__ float X[NB][kTileGroups];
  __shared__ float P[NB][kTile][kTileGroups + 1];
  const int rt = (int)blockIdx.x, tid = threadIdx.x;
  const int K = G * kGroup;
  const int b_own = tid / kTile, r_own = tid % kTile;   // summed by this thread while tid < NB * 16
  float acc = 0.0f;
  const int KT = k_tiles(G);
  for (int kt = 0; kt < KT; ++kt) {
    const int g0 = kt * kTileGroups, ng = min(kTileGroups, G - g0);
    for (int i = tid; i < NB * kTileGroups; i += kDriftThreads) {
      const int b = i / kTileGroups, g = i - b * kTileGroups;
      float sx = 0.0f;
      if (g < ng) {
        const uint16_t* xr = x + (size_t)b * K + (size_t)(g0 + g) * kGroup;
        for (int j = 0; j < kGroup; ++j) sx += fabsf(__half2float(__ushort_as_half(xr[j])));
      }
      X[b][g] = sx;
    }
    __syncthreads();
    const int t = kt * RT + rt;
    const uint8_t* tb = stream + (size_t)tiles[4 * t + 1] * 16;
    const uint32_t a = tiles[4 * t + 2], bb = tiles[4 * t + 3];
    const uint32_t n[4] = {a & 0xFFFF, a >> 16, bb & 0xFFFF, bb >> 16};
    const uint32_t s1 = (uint32_t)seg_bytes(0, n[0]), s2 = s1 + (uint32_t)seg_bytes(1, n[1]);
    const uint32_t sb[4] = {0u, s1, s2, s2 + (uint32_t)seg_bytes(2, n[2])};
    const uint32_t total = n[0] + n[1] + n[2] + n[3];
    for (uint32_t i = tid; i < total; i += kDriftThreads) {
      int c = 0;
      uint32_t idx = i;
      while (c < 3 && idx >= n[c]) {
        idx -= n[c];
        ++c;
      }
      const uint32_t br = block_records(c), k = idx / br, l = idx - k * br, m = min(br, n[c] - k * br);
      const uint32_t blk = sb[c] + k * (uint32_t)block_bytes(c, br);
      const uint32_t so = *reinterpret_cast<const uint32_t*>(tb + blk + codes_area(c, m) + 4u * l);
      const uint32_t meta = *reinterpret_cast<const uint16_t*>(tb + blk + codes_area(c, m) + so_area(m) + 2u * l);
      const float hs = 0.5f * __half2float(__ushort_as_half((unsigned short)(so & 0xFFFFu)));
      const int row = (int)(meta & 15u), g = (int)((meta >> 4) & (uint32_t)(kTileGroups - 1));
#pragma unroll
      for (int b = 0; b < NB; ++b) P[b][row][g] = hs * X[b][g];
    }
    __syncthreads();
    if (tid < NB * kTile)
      for (int g = 0; g < ng; ++g) acc += P[b_own][r_own][g];
    __syncthreads();   // X and P are rewritten for the next k-tile
  }
  const int row = rt * kTile + r_own;
  if (tid < NB * kTile && row < N) bound[(size_t)b_own * N + row] = acc;
}

hipError_t launch_drift(const vbq_matrix& m, const uint16_t* x, int B, float* bound, hipStream_t s) {
  const int RT = row_tiles(m.n_rows), G = m.n_cols / kGroup;
  const uint8_t* st = reinterpret_cast<const uint8_t*>(m.stream);
#define VBQ_DRIFT(NB)                                                                                   \
  case NB:                                                                                              \
    hipLaunchKernelGGL(k_drift<NB>, dim3(RT), dim3(kDriftThreads), 0, s, m.tiles, st, x, m.n_rows, G, RT, bound); \
    break;
  switch (B) {
    VBQ_DRIFT(1)
    VBQ_DRIFT(2)
    VBQ_DRIFT(3)
    VBQ_DRIFT(4)
    VBQ_DRIFT(5)
    VBQ_DRIFT(6)
    VBQ_DRIFT(7)
    VBQ_DRIFT(8)
    default:
      return hipErrorInvalidValue;
  }
#undef VBQ_DRIFT
  return hipGetLastError();
}

}  // namespace vbq
