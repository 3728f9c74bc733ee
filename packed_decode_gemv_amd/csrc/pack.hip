// Device-side packing: per-group round-to-nearest quantisation to fp16
// scale/offset and the tiled byte stream (tiles of 32 rows x 64 k-groups,
// a 2-bit width map per column, then per width class its records listed
// column by column in blocks of 64; the exact rules are in vbq.h).
//
// Groups of 64 weights with per-group widths {1,2,4,8} and packed low-bit
// storage: VBQ abstract (page "In-Cell Learning: Language Models That Update
// Their Own Weights in Sequence Without Changing the File They Ship").
// Asymmetric scale + offset: SLQ abstract (page thelatestinai.com/papers/2512.18934).
//
// Three launches on the caller's stream, one wavefront per tile with lane l
// on column l (k-group 64 kt + l):
//   1. k_pack_sizes: class masks per column, records per class, tile size.
//   2. k_pack_scan : one workgroup scans the tile sizes into byte bases and
//                    writes the totals entry (with error flags).
//   3. k_pack_tiles: clears the tile, writes its map, then every lane writes
//                    the records of its column (codes and scale/offset) at
//                    their closed-form positions.
// The quantiser's arithmetic must give the same bits on every run and match the
// documented binary32 sequence, so this file is built with -ffp-contract=off and
// uses correctly rounded division and round-half-even conversions.
#include "vbq_common.h"

namespace vbq {

// Class masks of column g (lane l of tile (rt, kt)) read from the widths;
// also flags widths outside {1,2,4,8}.
struct ColumnInfo {
  ClassMasks k;
  uint32_t p0, p1;
  bool bad;
};

__device__ inline ColumnInfo read_column(const uint8_t* __restrict__ widths, int G, int r0, int R, int g, bool live) {
  ColumnInfo ci;
  ci.p0 = ci.p1 = 0;
  ci.bad = false;
  if (live) {
    for (int r = 0; r < R; ++r) {
      const int c = class_of_width(widths[(size_t)(r0 + r) * G + g]);
      if (c < 0) {
        ci.bad = true;
        continue;
      }
      ci.p0 |= (uint32_t)(c & 1) << r;
      ci.p1 |= (uint32_t)(c >> 1) << r;
    }
  }
  ci.k = class_masks(ci.p0, ci.p1, live ? R : 0);
  return ci;
}

// Tiles are stored k-tile major: t = kt * RT + rt.
__global__ __launch_bounds__(64) void k_pack_sizes(const uint8_t* __restrict__ widths, int N, int G, int RT,
                                                   uint32_t* __restrict__ tiles) {
  const int t = blockIdx.x, lane = threadIdx.x;
  const int kt = t / RT, rt = t - kt * RT;
  const int r0 = rt * kTileRows, R = min(kTileRows, N - r0);
  const int g0 = kt * kTileGroups, Gt = min(kTileGroups, G - g0);
  const ColumnInfo ci = read_column(widths, G, r0, R, g0 + lane, lane < Gt);
  uint32_t bytes = map_bytes((uint32_t)Gt), n[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    n[c] = wave_total((uint32_t)__builtin_popcount(ci.k.m[c]));
    bytes += class_bytes(c, n[c]);
  }
  const uint32_t bad = (uint32_t)__popcll(__ballot(ci.bad));
  if (lane == 0) {
    tiles[4 * t + 0] = bad;                 // invalid count, replaced by the scan
    tiles[4 * t + 1] = bytes / 16;
    tiles[4 * t + 2] = n[0] | (n[1] << 16);
    tiles[4 * t + 3] = n[2] | (n[3] << 16);
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

__global__ __launch_bounds__(1024) void k_pack_scan(uint32_t* __restrict__ tiles, int n_tiles, uint64_t cap_bytes16) {
  __shared__ uint64_t wc[16];
  __shared__ uint64_t carry_c;
  __shared__ uint32_t bad_total;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    carry_c = 0;
    bad_total = 0;
  }
  __syncthreads();
  for (int base = 0; base < n_tiles; base += 1024) {
    const int t = base + tid;
    uint64_t nc = 0;
    uint32_t bad = 0;
    if (t < n_tiles) {
      nc = tiles[4 * t + 1];
      bad = tiles[4 * t + 0];
    }
    const uint64_t ic = wave_incl_scan(nc, lane);
    if (lane == 63) wc[wave] = ic;
    if (bad) atomicAdd(&bad_total, bad);
    __syncthreads();
    uint64_t pc = carry_c;
    for (int w = 0; w < wave; ++w) pc += wc[w];
    if (t < n_tiles) tiles[4 * t + 0] = (uint32_t)(pc + ic - nc);
    __syncthreads();
    if (tid == 0) {
      uint64_t sc = 0;
      for (int w = 0; w < 16; ++w) sc += wc[w];
      carry_c += sc;
    }
    __syncthreads();
  }
  if (tid == 0) {
    uint32_t flags = 0;
    if (bad_total) flags |= kFlagInvalidWidth;
    if (carry_c != cap_bytes16 || carry_c > 0xFFFFFFFFull) flags |= kFlagCapacity;
    tiles[4 * n_tiles + 0] = (uint32_t)carry_c;
    tiles[4 * n_tiles + 1] = bad_total;
    tiles[4 * n_tiles + 2] = flags;
    tiles[4 * n_tiles + 3] = 0;
  }
}

// Round-to-nearest asymmetric quantiser of one 64-weight group (binary32,
// no contraction): lo/hi by a sequential scan with strict comparisons,
// scale16 = fp16(f32(hi - lo) / L), offset16 = fp16(lo),
// q = s == 0 ? 0 : clamp(rint(f32(w - o) / s), 0, L); the codes are packed in
// pairs (code 2p at bit (p % h) b of word p / h, code 2p+1 16 bits higher).
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
  constexpr int H = 16 / B;
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

template <int C>
__device__ inline void write_record(const float* __restrict__ wg, uint8_t* __restrict__ codes, uint32_t* so) {
  constexpr int B = 1 << C;
  uint32_t words[2 * B];
  uint32_t so_v;
  quantize_pack_group<B>(wg, &so_v, words);
  if constexpr (B == 1) {
    *reinterpret_cast<uint2*>(codes) = make_uint2(words[0], words[1]);
  } else {
#pragma unroll
    for (int q = 0; q < B / 2; ++q)
      reinterpret_cast<uint4*>(codes)[q] = make_uint4(words[4 * q + 0], words[4 * q + 1], words[4 * q + 2], words[4 * q + 3]);
  }
  *so = so_v;
}

__global__ __launch_bounds__(64) void k_pack_tiles(const float* __restrict__ W, const uint8_t* __restrict__ widths,
                                                   int N, int G, int RT, const uint32_t* __restrict__ tiles,
                                                   int n_tiles, uint8_t* __restrict__ stream) {
  if (tiles[4 * n_tiles + 2] != 0) return;   // invalid widths or mismatched buffers: write nothing
  const int t = blockIdx.x, lane = threadIdx.x;
  const int kt = t / RT, rt = t - kt * RT;
  const int r0 = rt * kTileRows, R = min(kTileRows, N - r0);
  const int g0 = kt * kTileGroups, Gt = min(kTileGroups, G - g0);
  const size_t K = (size_t)G * kGroup;
  uint8_t* tb = stream + (size_t)tiles[4 * t + 0] * 16;
  const uint32_t tsize = tiles[4 * t + 1] * 16, w2 = tiles[4 * t + 2], w3 = tiles[4 * t + 3];
  // Clear the tile (padding must be zero); the records are written over it
  // after these stores have completed.
  for (uint32_t i = lane; i < tsize / 16; i += kWave) reinterpret_cast<uint4*>(tb)[i] = make_uint4(0u, 0u, 0u, 0u);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  const bool live = lane < Gt;
  const ColumnInfo ci = read_column(widths, G, r0, R, g0 + lane, live);
  if (live) *reinterpret_cast<uint2*>(tb + 8 * lane) = make_uint2(ci.p0, ci.p1);
  uint32_t cbase = map_bytes((uint32_t)Gt);
  const float* wcol = W + (size_t)(g0 + lane) * kGroup;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t n = class_count(w2, w3, c);
    uint32_t mask = ci.k.m[c];
    uint32_t e = wave_excl_scan((uint32_t)__builtin_popcount(mask), (uint32_t)lane);
    for (; mask; mask &= mask - 1u, ++e) {
      const int row = __builtin_ctz(mask);
      const RecPos rp = record_pos(c, n, cbase, e);
      const float* wg = wcol + (size_t)(r0 + row) * K;
      uint8_t* codes = tb + rp.codes;
      uint32_t* so = reinterpret_cast<uint32_t*>(tb + rp.so);
      switch (c) {
        case 0: write_record<0>(wg, codes, so); break;
        case 1: write_record<1>(wg, codes, so); break;
        case 2: write_record<2>(wg, codes, so); break;
        default: write_record<3>(wg, codes, so); break;
      }
    }
    cbase += class_bytes(c, n);
  }
}

hipError_t launch_pack(const float* W, const uint8_t* widths, const vbq_matrix& m, hipStream_t s) {
  const int G = m.n_cols / kGroup;
  const int RT = row_tiles(m.n_rows);
  const int T = (int)m.n_tiles;
  hipLaunchKernelGGL(k_pack_sizes, dim3(T), dim3(64), 0, s, widths, m.n_rows, G, RT, m.tiles);
  hipLaunchKernelGGL(k_pack_scan, dim3(1), dim3(1024), 0, s, m.tiles, T, (uint64_t)m.n_bytes16);
  hipLaunchKernelGGL(k_pack_tiles, dim3(T), dim3(64), 0, s, W, widths, m.n_rows, G, RT, m.tiles, T,
                     reinterpret_cast<uint8_t*>(m.stream));
  return hipGetLastError();
}

// ---- Recurrent residual levels ---------------------------------------------------
// Each level after the base is the 2-bit RTN of the error the levels before it
// leave (RRQ abstract on page thelatestinai.com/papers/2512.18934). The error
// a packed level leaves:
//   E_out[n][k] = E_in[n][k] - (f32(s q) + o)
// in binary32 with one rounding per operation (s q is exact). One wavefront
// per tile; lane l handles the records of its column, and the code pair p of
// a record is pair (p % h) of word p / h.
template <int C>
__device__ inline void residual_record(const uint8_t* codes, uint32_t so, const float* ein, float* eout) {
  constexpr int B = 1 << C, H = 16 / B;
  uint32_t w[2 * B];
#pragma unroll
  for (int i = 0; i < 2 * B; ++i) w[i] = reinterpret_cast<const uint32_t*>(codes)[i];
  const float sc = __half2float(__ushort_as_half((unsigned short)(so & 0xFFFFu)));
  const float of = __half2float(__ushort_as_half((unsigned short)(so >> 16)));
#pragma unroll
  for (int p = 0; p < 32; ++p) {
    const uint32_t word = w[p / H];
    const uint32_t q0 = (word >> ((p % H) * B)) & ((1u << B) - 1u);
    const uint32_t q1 = (word >> (16 + (p % H) * B)) & ((1u << B) - 1u);
    const float2 e = reinterpret_cast<const float2*>(ein)[p];
    float2 o;
    o.x = __fsub_rn(e.x, __fadd_rn(__fmul_rn(sc, (float)q0), of));
    o.y = __fsub_rn(e.y, __fadd_rn(__fmul_rn(sc, (float)q1), of));
    reinterpret_cast<float2*>(eout)[p] = o;
  }
}

__global__ __launch_bounds__(64) void k_residual_error(const uint32_t* __restrict__ tiles,
                                                       const uint8_t* __restrict__ stream, int N, int G, int RT,
                                                       const float* E_in, float* E_out) {
  const int t = blockIdx.x, lane = threadIdx.x;
  const int kt = t / RT, rt = t - kt * RT;
  const int r0 = rt * kTileRows, R = min(kTileRows, N - r0);
  const int g0 = kt * kTileGroups, Gt = min(kTileGroups, G - g0);
  const size_t K = (size_t)G * kGroup;
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
    uint32_t e = wave_excl_scan((uint32_t)__builtin_popcount(mask), (uint32_t)lane);
    for (; mask; mask &= mask - 1u, ++e) {
      const int row = __builtin_ctz(mask);
      const RecPos rp = record_pos(c, n, cbase, e);
      const size_t at = (size_t)(r0 + row) * K + (size_t)(g0 + lane) * kGroup;
      const uint32_t so = *reinterpret_cast<const uint32_t*>(tb + rp.so);
      switch (c) {
        case 0: residual_record<0>(tb + rp.codes, so, E_in + at, E_out + at); break;
        case 1: residual_record<1>(tb + rp.codes, so, E_in + at, E_out + at); break;
        case 2: residual_record<2>(tb + rp.codes, so, E_in + at, E_out + at); break;
        default: residual_record<3>(tb + rp.codes, so, E_in + at, E_out + at); break;
      }
    }
    cbase += class_bytes(c, n);
  }
}

hipError_t launch_residual_error(const vbq_matrix& m, const float* E_in, float* E_out, hipStream_t s) {
  const int G = m.n_cols / kGroup, RT = row_tiles(m.n_rows);
  hipLaunchKernelGGL(k_residual_error, dim3((unsigned)m.n_tiles), dim3(64), 0, s, m.tiles,
                     reinterpret_cast<const uint8_t*>(m.stream), m.n_rows, G, RT, E_in, E_out);
  return hipGetLastError();
}

// ---- Compact in-cell residual ----------------------------------------------------
// CellFill abstract (page "Nothing Changed but the Model: CellFill -- Bounded
// In-Cell Learning for Bit-Identical, Revocable Updates to Quantized LLMs"):
// an update is a residual that stays inside each weight's rounding cell. The
// compact form keeps one signed byte f per weight, standing for s f / 256 with
// s the scale of the weight's group; |f| <= 127 keeps every such residual
// strictly inside its cell. In binary32:
//   encode  f = clamp(rint(f32(r / s) * 256), -127, 127), and 0 where s = 0;
//   decode  r = fp16(s f / 256) (s f / 256 is exact, so one rounding).
// One wavefront per tile; lane l handles the records of its column.
__device__ inline uint32_t cell8_code(uint32_t h, float s) {
  const float r = __half2float(__ushort_as_half((unsigned short)h));
  float t = s != 0.f ? rintf(__fdiv_rn(r, s) * 256.f) : 0.f;
  t = fminf(fmaxf(t, -127.f), 127.f);
  return (uint32_t)(int32_t)t & 0xFFu;
}

// fp16(s f / 256). The conversion is written out as v_cvt_f16_f32: folded into
// a mixed-precision fma with a +0 addend, it would turn the -0 of a zero scale
// times a negative f into +0.
__device__ inline uint32_t cell8_value(uint32_t byte, float s) {
  const float v = (float)(int32_t)(int8_t)(uint8_t)byte;
  const float r = (s * v) * (1.f / 256.f);
  uint32_t h;
  asm("v_cvt_f16_f32 %0, %1" : "=v"(h) : "v"(r));
  return h & 0xFFFFu;
}

// ENCODE: in = fp16 residual [N][K], out = int8 [N][K]; else the reverse.
// Rows are taken in order: a wavefront takes one row of a tile at a time, and
// piece i of lane l is weights 8 (l % 8) .. + 7 of the record of column
// 8 i + l / 8, i.e. the 8 * (64 i + l)-th weight of the row's stretch, so
// consecutive lanes read and write consecutive bytes. A record's index in its
// class follows from the map planes (the class's records in the columns
// before, kept in LDS, plus the row's rank in its column). Workgroups of four
// wavefronts take kCell8RowsPerWg rows of a tile each. Every weight is
// converted on its own with its record's scale, so the order changes no
// result.
constexpr int kCell8Waves = 4;
constexpr int kCell8RowsPerWg = 8;

struct Cell8Cols {
  uint32_t p0[kTileGroups], p1[kTileGroups];
  uint16_t pre[4][kTileGroups];
};

template <bool ENCODE>
__global__ __launch_bounds__(kCell8Waves * 64) void k_cell8(const uint32_t* __restrict__ tiles,
                                                            const uint8_t* __restrict__ stream, int N, int G, int RT,
                                                            const void* in, void* out) {
  __shared__ Cell8Cols cols;
  constexpr int kParts = kTileRows / kCell8RowsPerWg;
  const int t = (int)blockIdx.x / kParts, part = (int)blockIdx.x % kParts;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kt = t / RT, rt = t - kt * RT;
  const int r0 = rt * kTileRows, R = min(kTileRows, N - r0);
  const int g0 = kt * kTileGroups, Gt = min(kTileGroups, G - g0);
  const size_t K = (size_t)G * kGroup;
  const uint8_t* tb = stream + (size_t)tiles[4 * t + 0] * 16;
  const uint32_t w2 = tiles[4 * t + 2], w3 = tiles[4 * t + 3];
  if (wave == 0) {
    const bool live = lane < Gt;
    const uint2 mp = live ? *reinterpret_cast<const uint2*>(tb + 8 * lane) : make_uint2(0u, 0u);
    const ClassMasks km = class_masks(mp.x, mp.y, live ? R : 0);
    cols.p0[lane] = mp.x;
    cols.p1[lane] = mp.y;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      cols.pre[c][lane] = (uint16_t)wave_excl_scan((uint32_t)__builtin_popcount(km.m[c]), (uint32_t)lane);
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
  const uint32_t valid = R >= 32 ? 0xFFFFFFFFu : ((1u << R) - 1u);
  for (int rr = wave; rr < kCell8RowsPerWg; rr += kCell8Waves) {
    const int row = part * kCell8RowsPerWg + rr;
    if (row >= R) break;
    const size_t at = (size_t)(r0 + row) * K + (size_t)g0 * kGroup;   // the row's first weight of the tile
    uint32_t so[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int g = 8 * i + (lane >> 3);
      so[i] = 0u;
      if (g < Gt) {
        const uint32_t p0 = cols.p0[g], p1 = cols.p1[g];
        const int c = (int)((p0 >> row) & 1u) | (int)(((p1 >> row) & 1u) << 1);
        const uint32_t mc = ((c & 1) ? p0 : ~p0) & ((c & 2) ? p1 : ~p1) & valid;
        const uint32_t e = (uint32_t)cols.pre[c][g] + (uint32_t)__builtin_popcount(mc & ((1u << row) - 1u));
        const uint32_t nc = c == 0 ? n[0] : c == 1 ? n[1] : c == 2 ? n[2] : n[3];
        const uint32_t bc = c == 0 ? cb[0] : c == 1 ? cb[1] : c == 2 ? cb[2] : cb[3];
        so[i] = *reinterpret_cast<const uint32_t*>(tb + record_pos(c, nc, bc, e).so);
      }
    }
    if constexpr (ENCODE) {
      const uint4* rp = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(in) + at);
      uint2* fp = reinterpret_cast<uint2*>(reinterpret_cast<int8_t*>(out) + at);
      uint4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 8 * i + (lane >> 3) < Gt ? rp[64 * i + lane] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (8 * i + (lane >> 3) >= Gt) continue;
        const float sc = __half2float(__ushort_as_half((unsigned short)(so[i] & 0xFFFFu)));
        const uint32_t h[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        uint32_t o[2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
          o[j] = cell8_code(h[2 * j] & 0xFFFFu, sc) | (cell8_code(h[2 * j] >> 16, sc) << 8) |
                 (cell8_code(h[2 * j + 1] & 0xFFFFu, sc) << 16) | (cell8_code(h[2 * j + 1] >> 16, sc) << 24);
        fp[64 * i + lane] = make_uint2(o[0], o[1]);
      }
    } else {
      const uint2* fp = reinterpret_cast<const uint2*>(reinterpret_cast<const int8_t*>(in) + at);
      uint4* rp = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + at);
      uint2 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 8 * i + (lane >> 3) < Gt ? fp[64 * i + lane] : make_uint2(0u, 0u);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (8 * i + (lane >> 3) >= Gt) continue;
        const float sc = __half2float(__ushort_as_half((unsigned short)(so[i] & 0xFFFFu)));
        const uint32_t w[2] = {v[i].x, v[i].y};
        uint32_t h[4];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          h[2 * j] = cell8_value(w[j] & 0xFFu, sc) | (cell8_value((w[j] >> 8) & 0xFFu, sc) << 16);
          h[2 * j + 1] = cell8_value((w[j] >> 16) & 0xFFu, sc) | (cell8_value(w[j] >> 24, sc) << 16);
        }
        rp[64 * i + lane] = make_uint4(h[0], h[1], h[2], h[3]);
      }
    }
  }
}

hipError_t launch_cell8_encode(const vbq_matrix& m, const uint16_t* r16, int8_t* f, hipStream_t s) {
  const int G = m.n_cols / kGroup, RT = row_tiles(m.n_rows);
  constexpr int64_t kParts = kTileRows / kCell8RowsPerWg;
  if (m.n_tiles * kParts > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_cell8<true>, dim3((unsigned)(m.n_tiles * kParts)), dim3(kCell8Waves * 64), 0, s, m.tiles,
                     reinterpret_cast<const uint8_t*>(m.stream), m.n_rows, G, RT, (const void*)r16, (void*)f);
  return hipGetLastError();
}

hipError_t launch_cell8_decode(const vbq_matrix& m, const int8_t* f, uint16_t* r16, hipStream_t s) {
  const int G = m.n_cols / kGroup, RT = row_tiles(m.n_rows);
  constexpr int64_t kParts = kTileRows / kCell8RowsPerWg;
  if (m.n_tiles * kParts > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_cell8<false>, dim3((unsigned)(m.n_tiles * kParts)), dim3(kCell8Waves * 64), 0, s, m.tiles,
                     reinterpret_cast<const uint8_t*>(m.stream), m.n_rows, G, RT, (const void*)f, (void*)r16);
  return hipGetLastError();
}

}  // namespace vbq
