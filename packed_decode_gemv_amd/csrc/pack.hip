// Device-side packing: per-group round-to-nearest quantisation to fp16
// scale/offset and the tiled (16 rows x 64 k-groups), width-sorted byte
// stream of blocks.
//
// Groups of 64 weights with per-group widths {1,2,4,8} and packed low-bit
// storage: VBQ abstract (page "In-Cell Learning: Language Models That Update
// Their Own Weights in Sequence Without Changing the File They Ship").
// Asymmetric scale + offset: SLQ abstract (page thelatestinai.com/papers/2512.18934).
//
// Three launches on the caller's stream:
//   1. k_pack_count: per tile, how many groups of each width class.
//   2. k_pack_scan : one workgroup scans the tiles into record and byte bases
//                    and writes the totals entry (with error flags).
//   3. k_pack_tiles: per tile, clear its bytes, rank every group inside its
//                    class in (row, k-group) order, quantise it and write its
//                    codes, scale/offset and meta into its block.
// The quantiser's arithmetic must give the same bits on every run and match the
// documented binary32 sequence, so this file is built with -ffp-contract=off and
// uses correctly rounded division and round-half-even conversions.
#include "vbq_common.h"

namespace vbq {

// Tiles are stored k-tile major: t = kt * RT + rt.
__global__ __launch_bounds__(256) void k_pack_count(const uint8_t* __restrict__ widths, int N, int G, int RT,
                                                    uint32_t* __restrict__ tiles) {
  __shared__ uint32_t cnt[5];
  const int t = blockIdx.x;
  if (threadIdx.x < 5) cnt[threadIdx.x] = 0;
  __syncthreads();
  const int kt = t / RT, rt = t - kt * RT;
  const int r0 = rt * kTile, rows = min(kTile, N - r0);
  const int g0 = kt * kTileGroups, ng = min(kTileGroups, G - g0);
  uint32_t c0 = 0, c1 = 0, c2 = 0, c3 = 0, bad = 0;
  for (int i = threadIdx.x; i < rows * ng; i += blockDim.x) {
    const int r = i / ng, g = i - r * ng;
    const int b = widths[(size_t)(r0 + r) * G + g0 + g];
    c0 += b == 1;
    c1 += b == 2;
    c2 += b == 4;
    c3 += b == 8;
    bad += class_of_width(b) < 0;
  }
  atomicAdd(&cnt[0], c0);
  atomicAdd(&cnt[1], c1);
  atomicAdd(&cnt[2], c2);
  atomicAdd(&cnt[3], c3);
  atomicAdd(&cnt[4], bad);
  __syncthreads();
  if (threadIdx.x == 0) {
    tiles[4 * t + 0] = cnt[4];                 // invalid count, replaced by the scan
    tiles[4 * t + 1] = 0;
    tiles[4 * t + 2] = cnt[0] | (cnt[1] << 16);
    tiles[4 * t + 3] = cnt[2] | (cnt[3] << 16);
  }
}

// Inclusive prefix sum over a 64-wide wavefront.
__device__ inline uint64_t wave_incl_scan(uint64_t v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    uint64_t u = __shfl_up(v, d, kWave);
    if (lane >= d) v += u;
  }
  return v;
}

__global__ __launch_bounds__(1024) void k_pack_scan(uint32_t* __restrict__ tiles, int n_tiles,
                                                    uint64_t cap_records, uint64_t cap_bytes16,
                                                    uint64_t cap_tile_bytes16) {
  __shared__ uint64_t wr[16], wc[16];
  __shared__ uint64_t carry_r, carry_c;
  __shared__ uint32_t bad_total, too_big;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    carry_r = 0;
    carry_c = 0;
    bad_total = 0;
    too_big = 0;
  }
  __syncthreads();
  for (int base = 0; base < n_tiles; base += 1024) {
    const int t = base + tid;
    uint64_t nr = 0, nc = 0;
    uint32_t bad = 0;
    if (t < n_tiles) {
      const uint32_t a = tiles[4 * t + 2], b = tiles[4 * t + 3];
      const uint32_t n0 = a & 0xFFFF, n1 = a >> 16, n2 = b & 0xFFFF, n3 = b >> 16;
      nr = (uint64_t)n0 + n1 + n2 + n3;
      nc = tile_bytes(n0, n1, n2, n3) / 16;
      bad = tiles[4 * t + 0];
      if (nc > cap_tile_bytes16) atomicOr(&too_big, 1u);
    }
    const uint64_t ir = wave_incl_scan(nr, lane), ic = wave_incl_scan(nc, lane);
    if (lane == 63) {
      wr[wave] = ir;
      wc[wave] = ic;
    }
    if (bad) atomicAdd(&bad_total, bad);
    __syncthreads();
    uint64_t pr = carry_r, pc = carry_c;
    for (int w = 0; w < wave; ++w) {
      pr += wr[w];
      pc += wc[w];
    }
    if (t < n_tiles) {
      tiles[4 * t + 0] = (uint32_t)(pr + ir - nr);
      tiles[4 * t + 1] = (uint32_t)(pc + ic - nc);
    }
    __syncthreads();
    if (tid == 0) {
      uint64_t sr = 0, sc = 0;
      for (int w = 0; w < 16; ++w) {
        sr += wr[w];
        sc += wc[w];
      }
      carry_r += sr;
      carry_c += sc;
    }
    __syncthreads();
  }
  if (tid == 0) {
    uint32_t flags = 0;
    if (bad_total) flags |= kFlagInvalidWidth;
    if (carry_r != cap_records || carry_c > cap_bytes16 || carry_r > 0xFFFFFFFFull || carry_c > 0xFFFFFFFFull)
      flags |= kFlagCapacity;
    if (too_big) flags |= kFlagTileSize;
    tiles[4 * n_tiles + 0] = (uint32_t)carry_r;
    tiles[4 * n_tiles + 1] = (uint32_t)carry_c;
    tiles[4 * n_tiles + 2] = bad_total;
    tiles[4 * n_tiles + 3] = flags;
  }
}

// Round-to-nearest asymmetric quantiser of one 64-weight group (binary32,
// no contraction): lo/hi by a sequential scan with strict comparisons,
// scale16 = fp16(f32(hi - lo) / L), offset16 = fp16(lo),
// q = s == 0 ? 0 : clamp(rint(f32(w - o) / s), 0, L).
template <int B>
__device__ inline void quantize_pack_group(const float* __restrict__ wg, uint32_t* so_out, uint32_t (&words)[2 * B]) {
  float v[64];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float4 f = reinterpret_cast<const float4*>(wg)[i];
    v[4 * i + 0] = f.x;
    v[4 * i + 1] = f.y;
    v[4 * i + 2] = f.z;
    v[4 * i + 3] = f.w;
  }
  float lo = v[0], hi = v[0];
#pragma unroll
  for (int j = 1; j < 64; ++j) {
    lo = (v[j] < lo) ? v[j] : lo;
    hi = (v[j] > hi) ? v[j] : hi;
  }
  constexpr int L = (1 << B) - 1;
  const float sf = __fdiv_rn(__fsub_rn(hi, lo), (float)L);
  const __half s16 = __float2half_rn(sf);
  const __half o16 = __float2half_rn(lo);
  const float s = __half2float(s16), o = __half2float(o16);
  *so_out = (uint32_t)__half_as_ushort(s16) | ((uint32_t)__half_as_ushort(o16) << 16);
  uint32_t q[64];
#pragma unroll
  for (int j = 0; j < 64; ++j) {
    float r = rintf(__fdiv_rn(__fsub_rn(v[j], o), s));
    r = r < 0.0f ? 0.0f : r;
    r = r > (float)L ? (float)L : r;
    q[j] = (s == 0.0f) ? 0u : (uint32_t)r;
  }
  constexpr int H = 16 / B;   // pair p = (code 2p, code 2p+1) -> word p / H, field p % H
#pragma unroll
  for (int w = 0; w < 2 * B; ++w) {
    uint32_t lo16 = 0, hi16 = 0;
#pragma unroll
    for (int f = 0; f < H; ++f) {
      lo16 |= q[2 * (w * H + f)] << (f * B);
      hi16 |= q[2 * (w * H + f) + 1] << (f * B);
    }
    words[w] = lo16 | (hi16 << 16);
  }
}

// Writes record idx of class segment C (n_c records, segment at `seg`).
template <int C>
__device__ inline void write_record(const float* __restrict__ wg, uint32_t idx, uint32_t n_c, uint8_t* __restrict__ seg,
                                    uint16_t meta_v) {
  constexpr int B = 1 << C;
  constexpr uint32_t BR = block_records(C);
  uint32_t words[2 * B];
  uint32_t so_v;
  quantize_pack_group<B>(wg, &so_v, words);
  const uint32_t k = idx / BR, l = idx - k * BR;
  const uint32_t m = min(BR, n_c - k * BR);
  uint8_t* blk = seg + (uint64_t)k * block_bytes(C, BR);
  if constexpr (B == 1) {
    *reinterpret_cast<uint2*>(blk + 8u * l) = make_uint2(words[0], words[1]);
  } else {   // records are contiguous: chunk q of record l at (l * B/2 + q) * 16
#pragma unroll
    for (int q = 0; q < B / 2; ++q)
      *reinterpret_cast<uint4*>(blk + (l * (B / 2) + (uint32_t)q) * 16u) =
          make_uint4(words[4 * q + 0], words[4 * q + 1], words[4 * q + 2], words[4 * q + 3]);
  }
  *reinterpret_cast<uint32_t*>(blk + codes_area(C, m) + 4u * l) = so_v;
  *reinterpret_cast<uint16_t*>(blk + codes_area(C, m) + so_area(m) + 2u * l) = meta_v;
}

__global__ __launch_bounds__(256) void k_pack_tiles(const float* __restrict__ W, const uint8_t* __restrict__ widths,
                                                    int N, int G, int RT, const uint32_t* __restrict__ tiles,
                                                    int n_tiles, uint8_t* __restrict__ stream) {
  if (tiles[4 * n_tiles + 3] != 0) return;   // invalid widths or mismatched buffers: write nothing
  __shared__ uint32_t carry[4];
  __shared__ uint32_t wcnt[4][4];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kt = t / RT, rt = t - kt * RT;
  const int r0 = rt * kTile, rows = min(kTile, N - r0);
  const int g0 = kt * kTileGroups, ng = min(kTileGroups, G - g0);
  const size_t K = (size_t)G * kGroup;
  const uint32_t a = tiles[4 * t + 2], bb = tiles[4 * t + 3];
  const uint32_t n[4] = {a & 0xFFFF, a >> 16, bb & 0xFFFF, bb >> 16};
  uint8_t* tile_base = stream + (uint64_t)tiles[4 * t + 1] * 16;
  const uint64_t s1 = seg_bytes(0, n[0]), s2 = s1 + seg_bytes(1, n[1]), s3 = s2 + seg_bytes(2, n[2]);
  const uint64_t tb = s3 + seg_bytes(3, n[3]);
  // Clear the tile (padding must be zero), then write the records over it.
  for (uint64_t i = tid; i < tb / 16; i += blockDim.x)
    reinterpret_cast<uint4*>(tile_base)[i] = make_uint4(0u, 0u, 0u, 0u);
  if (tid < 4) carry[tid] = 0;
  __syncthreads();
  const int total = rows * ng;
  for (int base = 0; base < total; base += 256) {
    const int i = base + tid;
    int c = -1, kl = 0, r = 0;
    if (i < total) {
      r = i / ng;      // (row, k-group) order
      kl = i - r * ng;
      c = class_of_width(widths[(size_t)(r0 + r) * G + g0 + kl]);
    }
    uint32_t rank = 0;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const uint64_t mask = __ballot(c == cc);
      if (c == cc) rank = __mbcnt_hi((uint32_t)(mask >> 32), __mbcnt_lo((uint32_t)mask, 0u));
      if (lane == 0) wcnt[wave][cc] = (uint32_t)__popcll(mask);
    }
    __syncthreads();
    if (c >= 0) {
      uint32_t idx = carry[c] + rank;
      for (int w = 0; w < wave; ++w) idx += wcnt[w][c];
      const float* wg = W + (size_t)(r0 + r) * K + (size_t)(g0 + kl) * kGroup;
      const uint16_t mv = (uint16_t)(r | (kl << 4));
      switch (c) {
        case 0: write_record<0>(wg, idx, n[0], tile_base, mv); break;
        case 1: write_record<1>(wg, idx, n[1], tile_base + s1, mv); break;
        case 2: write_record<2>(wg, idx, n[2], tile_base + s2, mv); break;
        default: write_record<3>(wg, idx, n[3], tile_base + s3, mv); break;
      }
    }
    __syncthreads();
    if (tid < 4) carry[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
    __syncthreads();
  }
}

hipError_t launch_pack(const float* W, const uint8_t* widths, const vbq_matrix& m, hipStream_t s) {
  const int G = m.n_cols / kGroup;
  const int RT = row_tiles(m.n_rows);
  const int T = (int)m.n_tiles;
  hipLaunchKernelGGL(k_pack_count, dim3(T), dim3(256), 0, s, widths, m.n_rows, G, RT, m.tiles);
  hipLaunchKernelGGL(k_pack_scan, dim3(1), dim3(1024), 0, s, m.tiles, T, (uint64_t)m.n_records,
                     (uint64_t)m.n_bytes16, (uint64_t)m.max_tile_bytes16);
  hipLaunchKernelGGL(k_pack_tiles, dim3(T), dim3(256), 0, s, W, widths, m.n_rows, G, RT, m.tiles, T,
                     reinterpret_cast<uint8_t*>(m.stream));
  return hipGetLastError();
}

// ---- Recurrent residual levels ---------------------------------------------------
// Each level after the base is the 2-bit RTN of the error the levels before it
// leave (RRQ abstract on page thelatestinai.com/papers/2512.18934). The error
// a packed level leaves:
//   E_out[n][k] = E_in[n][k] - (f32(s q) + o)
// in binary32 with one rounding per operation (s q is exact). One workgroup
// per tile; each wavefront takes whole records with lane j on code j, so a
// record's 64 weights are one contiguous 256-byte segment of a row. Code j of
// a record lies in half j / 32, pair p = (j % 32) / 2: word h b + p / (16 / b),
// bit 16 (j % 2) + (p % (16 / b)) b. E_out may be E_in.
__global__ __launch_bounds__(256) void k_residual_error(const uint32_t* __restrict__ tiles,
                                                        const uint8_t* __restrict__ stream, int G, int RT,
                                                        const float* E_in, float* E_out) {
  const int t = (int)blockIdx.x, kt = t / RT, rt = t - kt * RT;
  const int wave = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63;
  const size_t K = (size_t)G * kGroup;
  const uint8_t* tb = stream + (size_t)tiles[4 * t + 1] * 16;
  const uint32_t a = tiles[4 * t + 2], bb = tiles[4 * t + 3];
  const uint32_t n[4] = {a & 0xFFFF, a >> 16, bb & 0xFFFF, bb >> 16};
  const uint32_t s1 = (uint32_t)seg_bytes(0, n[0]), s2 = s1 + (uint32_t)seg_bytes(1, n[1]);
  const uint32_t sb[4] = {0u, s1, s2, s2 + (uint32_t)seg_bytes(2, n[2])};
  const uint32_t total = n[0] + n[1] + n[2] + n[3];
  for (uint32_t i = (uint32_t)wave; i < total; i += 4) {
    int c = 0;
    uint32_t idx = i;
    while (c < 3 && idx >= n[c]) {
      idx -= n[c];
      ++c;
    }
    const uint32_t br = block_records(c), k = idx / br, l = idx - k * br, m = min(br, n[c] - k * br);
    const uint32_t blk = sb[c] + k * (uint32_t)block_bytes(c, br);
    const uint32_t* codes = reinterpret_cast<const uint32_t*>(tb + blk + (8u << c) * l);
    const uint32_t so = *reinterpret_cast<const uint32_t*>(tb + blk + codes_area(c, m) + 4u * l);
    const uint32_t meta = *reinterpret_cast<const uint16_t*>(tb + blk + codes_area(c, m) + so_area(m) + 2u * l);
    const int b = 1 << c, H = 16 >> c;
    const int h = lane >> 5, p = (lane & 31) >> 1, odd = lane & 1;
    const uint32_t q = (codes[h * b + p / H] >> (16 * odd + (p % H) * b)) & ((1u << b) - 1u);
    const float sc = __half2float(__ushort_as_half((unsigned short)(so & 0xFFFFu)));
    const float of = __half2float(__ushort_as_half((unsigned short)(so >> 16)));
    const size_t e = (size_t)(rt * kTile + (int)(meta & 15u)) * K +
                     (size_t)(kt * kTileGroups + (int)((meta >> 4) & (uint32_t)(kTileGroups - 1))) * kGroup +
                     (size_t)lane;
    E_out[e] = __fsub_rn(E_in[e], __fadd_rn(__fmul_rn(sc, (float)q), of));
  }
}

// y[i] = sum over levels l in order of parts[l][i] (binary32).
__global__ __launch_bounds__(256) void k_sum_levels(const float* __restrict__ parts, int count, size_t n,
                                                    float* __restrict__ y) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    float v = parts[i];
    for (int l = 1; l < count; ++l) v += parts[(size_t)l * n + i];
    y[i] = v;
  }
}

hipError_t launch_residual_error(const vbq_matrix& m, const float* E_in, float* E_out, hipStream_t s) {
  const int G = m.n_cols / kGroup, RT = row_tiles(m.n_rows);
  hipLaunchKernelGGL(k_residual_error, dim3((unsigned)m.n_tiles), dim3(256), 0, s, m.tiles,
                     reinterpret_cast<const uint8_t*>(m.stream), G, RT, E_in, E_out);
  return hipGetLastError();
}

hipError_t launch_sum_levels(const float* parts, int count, size_t n, float* y, hipStream_t s) {
  const size_t want = (n + 255) / 256;
  const unsigned blocks = (unsigned)(want < 4096 ? (want > 0 ? want : 1) : 4096);
  hipLaunchKernelGGL(k_sum_levels, dim3(blocks), dim3(256), 0, s, parts, count, n, y);
  return hipGetLastError();
}

}  // namespace vbq
