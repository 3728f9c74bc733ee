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
// and subtracted per group.
//
// Work split: a workgroup (4 wavefronts) owns a range of 16-row tiles of one
// matrix (several matrices per launch for batched calls). Inside a tile the
// records are grouped by width, so every 64-record block is decoded by one
// wavefront with a single width: no divergence, and neighbouring lanes mostly
// share a k-group, so their x reads from LDS are broadcasts. Each wavefront
// accumulates its rows in its own LDS slice; the slices are summed in a fixed
// order at the end, so results are identical from run to run.
#include "vbq_common.h"

namespace vbq {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;

// Field placement of pair index f within a word, per width class.
// shift kind: 0 none, 1 left by 4, 2 right by 2, 3 right by 8.
__device__ constexpr int shift_kind(int c, int f) {
  return c == 0 ? (f < 6 ? 1 : f < 12 ? 2 : 3)
       : c == 1 ? (f < 3 ? 1 : f < 6 ? 2 : 3)
       : c == 2 ? (f < 2 ? 0 : 3)
       : (f < 1 ? 0 : 3);
}
// Mantissa bit of the field after the shift.
__device__ constexpr int field_pos(int c, int f) {
  return c == 0 ? (f < 6 ? f + 4 : f < 12 ? f - 2 : f - 8)
       : c == 1 ? (f < 3 ? 4 + 2 * f : f < 6 ? 4 + 2 * (f - 3) : 4 + 2 * (f - 6))
       : c == 2 ? ((f & 1) ? 4 : 0)
       : 0;
}
__device__ constexpr uint32_t field_mask(int c, int p) {
  return (((1u << (1 << c)) - 1u) << p) * 0x00010001u;
}
// fp16 with exponent field 25 - p: the mantissa bit p has weight 1.
__device__ constexpr uint32_t field_magic(int p) { return (uint32_t)((25 - p) << 10) * 0x00010001u; }
__device__ constexpr float field_bias(int c, int f) { return (float)(1 << (10 - field_pos(c, f))); }

__device__ inline uint32_t shifted(uint32_t w, int kind) {
  return kind == 0 ? w : kind == 1 ? (w << 4) : kind == 2 ? (w >> 2) : (w >> 8);
}

__device__ inline half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}

// acc[nb] += sum_j (bias_j + q_j) x_j + (bias_j + q_{32+j}) x_{32+j} over the
// 32 pairs of one record. xk points at the record's k-group in the x table of
// batch row 0; batch rows are xstride dwords apart; chunks are XOR-swizzled by swz.
template <int C, int NB>
__device__ inline void dot_record(const uint32_t (&w)[2 << C], const uint32_t* xk, int xstride, int swz,
                                  float (&acc)[NB]) {
  constexpr int H = 16 >> C;   // fields per 16-bit half
#pragma unroll
  for (int ch = 0; ch < 8; ++ch) {
    uint4 xv[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      xv[nb] = *reinterpret_cast<const uint4*>(xk + nb * xstride + ((ch ^ swz) << 2));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = 4 * ch + e;
      const int f = j % H;
      const int p = field_pos(C, f);
      const uint32_t hv = (shifted(w[j / H], shift_kind(C, f)) & field_mask(C, p)) | field_magic(p);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint32_t xe = e == 0 ? xv[nb].x : e == 1 ? xv[nb].y : e == 2 ? xv[nb].z : xv[nb].w;
        acc[nb] = dot2(hv, xe, acc[nb]);
      }
    }
  }
}

struct Smem {
  uint32_t* xs;    // [NB][GS][32] swizzled pairs (x_j, x_{32+j})
  uint32_t* xn;    // [NB][GS][32] natural pairs (x_2i, x_2i+1), residual mode only
  float* cx;       // [NB][4][GS] bias constants per width class
  float* xsum;     // [NB][GS] sum of x over the group
  float* yw;       // [kWaves][NB][nt][16] per-wavefront row sums
  int gs;
};

template <int C, int NB>
__device__ inline void run_class(const GemvMat& M, const Smem& S, uint32_t n, uint32_t rec, uint64_t seg, int& bcount,
                                 int tl, int nt, int wave, int lane) {
  constexpr int B = 1 << C;
  const int nblk = (int)((n + kBlock - 1) / kBlock);
  const int first = ((wave - bcount) % kWaves + kWaves) % kWaves;
  const uint8_t* cbytes = reinterpret_cast<const uint8_t*>(M.codes) + seg;
  for (int bi = first; bi < nblk; bi += kWaves) {
    const uint32_t m = min((uint32_t)kBlock, n - (uint32_t)bi * kBlock);
    if ((uint32_t)lane < m) {
      const uint32_t r = rec + (uint32_t)bi * kBlock + lane;
      const uint32_t sov = M.so[r];
      const uint32_t mt = M.meta[r];
      const int row = mt & 15, kg = (int)(mt >> 4);
      const uint8_t* base = cbytes + (uint64_t)bi * kBlock * 8 * B;
      uint32_t w[2 * B];
      if constexpr (B == 1) {
        const uint2 v = *reinterpret_cast<const uint2*>(base + 8 * lane);
        w[0] = v.x;
        w[1] = v.y;
      } else {
#pragma unroll
        for (int q = 0; q < B / 2; ++q) {
          const uint4 v = *reinterpret_cast<const uint4*>(base + ((uint64_t)q * m + lane) * 16);
          w[4 * q + 0] = v.x;
          w[4 * q + 1] = v.y;
          w[4 * q + 2] = v.z;
          w[4 * q + 3] = v.w;
        }
      }
      float acc[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = 0.0f;
      dot_record<C, NB>(w, S.xs + kg * 32, S.gs * 32, kg & 7, acc);
      const float s = __half2float(__ushort_as_half((unsigned short)(sov & 0xFFFF)));
      const float o = __half2float(__ushort_as_half((unsigned short)(sov >> 16)));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float v = s * (acc[nb] - S.cx[(nb * 4 + C) * S.gs + kg]) + o * S.xsum[nb * S.gs + kg];
        atomicAdd(&S.yw[((wave * NB + nb) * nt + tl) * kTile + row], v);
      }
    }
  }
  bcount += nblk;
}

template <int NB, bool RESID>
__global__ __launch_bounds__(kThreads) void k_gemv(const GemvLaunch L) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int mi = 0;
  for (int i = 1; i < L.n_mats; ++i) mi = ((int)blockIdx.x >= L.mats[i].wg_begin) ? i : mi;
  const GemvMat& M = L.mats[mi];
  const int G = M.n_groups, K = G * kGroup;
  const int t0 = ((int)blockIdx.x - M.wg_begin) * M.tiles_per_wg;
  const int t1 = min(t0 + M.tiles_per_wg, M.n_tiles);
  const int nt = t1 - t0;

  Smem S;
  S.gs = L.max_groups;
  S.xs = reinterpret_cast<uint32_t*>(smem);
  S.xn = S.xs + NB * S.gs * 32;
  S.cx = reinterpret_cast<float*>(S.xn + (RESID ? NB * S.gs * 32 : 0));
  S.xsum = S.cx + NB * 4 * S.gs;
  S.yw = S.xsum + NB * S.gs;

  // Stage x as swizzled (x_j, x_{32+j}) pairs; natural pairs for the residual.
  for (int i = tid; i < NB * G * 32; i += kThreads) {
    const int nb = i / (G * 32), rem = i - nb * G * 32, kg = rem >> 5, j = rem & 31;
    const uint16_t* xr = M.x + (size_t)nb * K + kg * kGroup;
    S.xs[(nb * S.gs + kg) * 32 + (((j >> 2) ^ (kg & 7)) << 2) + (j & 3)] =
        (uint32_t)xr[j] | ((uint32_t)xr[32 + j] << 16);
    if constexpr (RESID)
      S.xn[nb * S.gs * 32 + rem] = reinterpret_cast<const uint32_t*>(M.x + (size_t)nb * K)[rem];
  }
  for (int i = tid; i < kWaves * NB * nt * kTile; i += kThreads) S.yw[i] = 0.0f;
  __syncthreads();

  // Per (batch row, k-group): sum of x and the bias constant of each width.
  for (int i = tid; i < NB * G; i += kThreads) {
    const int nb = i / G, kg = i - nb * G;
    const uint32_t* xk = S.xs + (nb * S.gs + kg) * 32;
    float X = 0.f, c0 = 0.f, c1 = 0.f, c2 = 0.f, c3 = 0.f;
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) {
      const uint4 v = *reinterpret_cast<const uint4*>(xk + ((ch ^ (kg & 7)) << 2));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 4 * ch + e;
        const uint32_t u = e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
        const half2_t h = as_h2(u);
        const float sj = (float)h.x + (float)h.y;
        X += sj;
        c0 += field_bias(0, j % 16) * sj;
        c1 += field_bias(1, j % 8) * sj;
        c2 += field_bias(2, j % 4) * sj;
        c3 += field_bias(3, j % 2) * sj;
      }
    }
    S.cx[(nb * 4 + 0) * S.gs + kg] = c0;
    S.cx[(nb * 4 + 1) * S.gs + kg] = c1;
    S.cx[(nb * 4 + 2) * S.gs + kg] = c2;
    S.cx[(nb * 4 + 3) * S.gs + kg] = c3;
    S.xsum[nb * S.gs + kg] = X;
  }
  __syncthreads();

  int bcount = 0;
  for (int tl = 0; tl < nt; ++tl) {
    const uint32_t* th = M.tiles + 4 * (t0 + tl);
    const uint32_t rec = th[0];
    const uint64_t seg = (uint64_t)th[1] * 16;
    const uint32_t a = th[2], bb = th[3];
    const uint32_t n0 = a & 0xFFFF, n1 = a >> 16, n2 = bb & 0xFFFF, n3 = bb >> 16;
    const uint64_t s1 = seg + seg_bytes(0, n0), s2 = s1 + seg_bytes(1, n1), s3 = s2 + seg_bytes(2, n2);
    run_class<0, NB>(M, S, n0, rec, seg, bcount, tl, nt, wave, lane);
    run_class<1, NB>(M, S, n1, rec + n0, s1, bcount, tl, nt, wave, lane);
    run_class<2, NB>(M, S, n2, rec + n0 + n1, s2, bcount, tl, nt, wave, lane);
    run_class<3, NB>(M, S, n3, rec + n0 + n1 + n2, s3, bcount, tl, nt, wave, lane);
  }

  if constexpr (RESID) {
    // y[b][n] += sum_k x[b][k] r[n][k] over the residual rows of this range.
    const int kc = K / 8;   // 16-byte chunks per row
    for (int ri = wave; ri < nt * kTile; ri += kWaves) {
      const int tl = ri / kTile, r = ri % kTile;
      const int row = (t0 + tl) * kTile + r;
      if (row >= M.n_rows) continue;   // uniform across the wavefront
      const uint4* rr = reinterpret_cast<const uint4*>(M.resid + (size_t)row * K);
      float acc[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = 0.f;
      for (int c = lane; c < kc; c += kWave) {
        const uint4 rv = rr[c];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint4 xv = *reinterpret_cast<const uint4*>(S.xn + nb * S.gs * 32 + 4 * c);
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
        if (lane == 0) S.yw[((wave * NB + nb) * nt + tl) * kTile + r] += v;
      }
    }
  }
  __syncthreads();

  for (int i = tid; i < NB * nt * kTile; i += kThreads) {
    const int nb = i / (nt * kTile), rem = i - nb * nt * kTile;
    const int row = t0 * kTile + rem;
    if (row < M.n_rows) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += S.yw[(w * NB + nb) * nt * kTile + rem];
      M.y[(size_t)nb * M.n_rows + row] = v;
    }
  }
}

size_t gemv_lds_bytes(int nb, int max_groups, bool resid, int tiles_per_wg) {
  const size_t gs = (size_t)max_groups;
  size_t b = (size_t)nb * gs * 128;              // swizzled x pairs
  if (resid) b += (size_t)nb * gs * 128;         // natural x pairs
  b += (size_t)nb * gs * 4 * 4;                  // bias constants
  b += (size_t)nb * gs * 4;                      // x sums
  b += (size_t)kWaves * nb * tiles_per_wg * kTile * 4;
  return b;
}

int gemv_max_tiles_per_wg() { return 8; }

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
