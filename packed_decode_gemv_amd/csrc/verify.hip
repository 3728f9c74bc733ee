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
// (built with -ffp-contract=off; correctly rounded division):
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

// Checks record l of a block of class C holding m records (block at `blk`).
template <int C>
__device__ inline void verify_record(const uint8_t* blk, uint8_t* rq_blk, uint32_t m, uint32_t l, int r0, int g0,
                                     int K, const uint16_t* __restrict__ resid, uint32_t& mism, uint32_t& ooc,
                                     uint64_t& first) {
  constexpr int B = 1 << C, H = 16 / B, L = (1 << B) - 1;
  uint32_t w[2 * B];
  uint32_t off[B > 1 ? B / 2 : 1];
  if constexpr (B == 1) {
    off[0] = 8u * l;
    const uint2 v = *reinterpret_cast<const uint2*>(blk + off[0]);
    w[0] = v.x;
    w[1] = v.y;
  } else {
#pragma unroll
    for (int q = 0; q < B / 2; ++q) {
      off[q] = (l * (B / 2) + (uint32_t)q) * 16u;   // records are contiguous
      const uint4 v = *reinterpret_cast<const uint4*>(blk + off[q]);
      w[4 * q + 0] = v.x;
      w[4 * q + 1] = v.y;
      w[4 * q + 2] = v.z;
      w[4 * q + 3] = v.w;
    }
  }
  const uint32_t sov = *reinterpret_cast<const uint32_t*>(blk + codes_area(C, m) + 4u * l);
  const uint32_t mt = *reinterpret_cast<const uint16_t*>(blk + codes_area(C, m) + so_area(m) + 2u * l);
  const int row = r0 + (int)(mt & 15), kg = g0 + (int)(mt >> 4);
  const float s = __half2float(__ushort_as_half((unsigned short)(sov & 0xFFFF)));
  const float o = __half2float(__ushort_as_half((unsigned short)(sov >> 16)));
  const float half_s = __fmul_rn(0.5f, s);
  const uint64_t lin0 = (uint64_t)row * K + (uint64_t)kg * kGroup;
  const uint4* rp = reinterpret_cast<const uint4*>(resid + lin0);
  uint32_t nw[2 * B];
#pragma unroll
  for (int i = 0; i < 2 * B; ++i) nw[i] = 0;
#pragma unroll
  for (int ch = 0; ch < 8; ++ch) {
    const uint4 rv = rp[ch];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = 8 * ch + e;                     // natural index inside the group
      const int pr = j >> 1, odd = j & 1;           // pair (code 2p, code 2p+1)
      const int wi = pr / H, sh = 16 * odd + (pr % H) * B;
      const uint32_t q = (w[wi] >> sh) & (uint32_t)L;
      const uint32_t rw = (e >> 1) == 0 ? rv.x : (e >> 1) == 1 ? rv.y : (e >> 1) == 2 ? rv.z : rv.w;
      const unsigned short rb = (unsigned short)((e & 1) ? (rw >> 16) : (rw & 0xFFFF));
      const float r = __half2float(__ushort_as_half(rb));
      const float deq = __fadd_rn(__fmul_rn(s, (float)q), o);
      const float v = __fadd_rn(deq, r);
      uint32_t qp = 0;
      if (s != 0.0f) {
        float t = rintf(__fdiv_rn(__fsub_rn(v, o), s));
        t = t < 0.0f ? 0.0f : t;
        t = t > (float)L ? (float)L : t;
        qp = (uint32_t)t;
      }
      const bool bad_code = qp != q;
      const bool bad_cell = (s > 0.0f) ? (fabsf(r) >= half_s) : (r != 0.0f);
      mism += bad_code;
      ooc += bad_cell;
      if ((bad_code || bad_cell) && lin0 + j < first) first = lin0 + j;
      nw[wi] |= qp << sh;
    }
  }
  if (rq_blk) {
    if constexpr (B == 1) {
      *reinterpret_cast<uint2*>(rq_blk + off[0]) = make_uint2(nw[0], nw[1]);
    } else {
#pragma unroll
      for (int q = 0; q < B / 2; ++q)
        *reinterpret_cast<uint4*>(rq_blk + off[q]) = make_uint4(nw[4 * q], nw[4 * q + 1], nw[4 * q + 2], nw[4 * q + 3]);
    }
  }
}

// Record i of class segment C (n records) at `seg`.
template <int C>
__device__ inline void verify_seg_record(const uint8_t* seg, uint8_t* rq_seg, uint32_t n, uint32_t i, int r0, int g0,
                                         int K, const uint16_t* resid, uint32_t& mism, uint32_t& ooc,
                                         uint64_t& first) {
  constexpr uint32_t BR = block_records(C);
  const uint32_t k = i / BR, l = i - k * BR, m = min(BR, n - k * BR);
  const uint64_t bo = (uint64_t)k * block_bytes(C, BR);
  verify_record<C>(seg + bo, rq_seg ? rq_seg + bo : nullptr, m, l, r0, g0, K, resid, mism, ooc, first);
}

__global__ __launch_bounds__(256) void k_verify(const uint32_t* __restrict__ tiles, const uint8_t* __restrict__ stream,
                                                int G, int RT, const uint16_t* __restrict__ resid,
                                                uint64_t* result, uint8_t* requant) {
  __shared__ uint32_t s_mism, s_ooc;
  __shared__ unsigned long long s_first;
  const int t = blockIdx.x, tid = threadIdx.x;
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
  const uint64_t sb[4] = {0, seg_bytes(0, n[0]), seg_bytes(0, n[0]) + seg_bytes(1, n[1]),
                          seg_bytes(0, n[0]) + seg_bytes(1, n[1]) + seg_bytes(2, n[2])};
  const uint64_t size = sb[3] + seg_bytes(3, n[3]);
  const uint8_t* tbytes = stream + tb;
  uint8_t* rbytes = requant ? requant + tb : nullptr;
  // Copy the tile (scales, offsets, meta, padding); codes are rewritten below.
  if (rbytes)
    for (uint64_t i = tid; i < size / 16; i += blockDim.x)
      reinterpret_cast<uint4*>(rbytes)[i] = reinterpret_cast<const uint4*>(tbytes)[i];
  __syncthreads();
  const uint32_t total = n[0] + n[1] + n[2] + n[3];
  uint32_t mism = 0, ooc = 0;
  uint64_t first = ~0ull;
  for (uint32_t i = tid; i < total; i += blockDim.x) {
    int c = 0;
    uint32_t idx = i;
    while (c < 3 && idx >= n[c]) {
      idx -= n[c];
      ++c;
    }
    const uint8_t* seg = tbytes + sb[c];
    uint8_t* rseg = rbytes ? rbytes + sb[c] : nullptr;
    switch (c) {
      case 0: verify_seg_record<0>(seg, rseg, n[0], idx, r0, g0, K, resid, mism, ooc, first); break;
      case 1: verify_seg_record<1>(seg, rseg, n[1], idx, r0, g0, K, resid, mism, ooc, first); break;
      case 2: verify_seg_record<2>(seg, rseg, n[2], idx, r0, g0, K, resid, mism, ooc, first); break;
      default: verify_seg_record<3>(seg, rseg, n[3], idx, r0, g0, K, resid, mism, ooc, first); break;
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
  hipLaunchKernelGGL(k_verify, dim3((unsigned)m.n_tiles), dim3(256), 0, s, m.tiles,
                     reinterpret_cast<const uint8_t*>(m.stream), m.n_cols / kGroup, row_tiles(m.n_rows), resid,
                     result, reinterpret_cast<uint8_t*>(requant));
  return hipGetLastError();
}

}  // namespace vbq
