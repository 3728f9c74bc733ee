/*
 * Plain, slow CPU oracle for packed mixed-bit GEMV (TEST INFRASTRUCTURE ONLY).
 *
 * Only tests/, the smoke check and the benchmark's cpu_baseline leg may load
 * this library. The product path never calls it and shares no code with it.
 *
 * What it follows:
 *  - Variable bit-width quantisation (VBQ abstract, page "In-Cell Learning:
 *    Language Models That Update Their Own Weights in Sequence Without
 *    Changing the File They Ship"): every contiguous group of 64 weights along
 *    K carries its own width b in {1,2,4,8}; the widths are stored packed, and
 *    the kernel that dequantises while it multiplies must give the same
 *    result as the plain product with the dequantised matrix.
 *  - Asymmetric quantisation with a scale and an offset (SLQ abstract, page
 *    thelatestinai.com/papers/2512.18934): w = scale*q + offset, q in [0, 2^b-1].
 *  - CellFill (page "Nothing Changed but the Model: CellFill -- Bounded In-Cell
 *    Learning for Bit-Identical, Revocable Updates to Quantized LLMs",
 *    section Abstract): frozen codes and scales, a per-weight residual kept
 *    within its rounding cell, so quantising again gives back identical codes;
 *    removing the residual undoes an update; the output drift has a bound.
 *
 * Where the pages are silent the readings are: scale and offset stored as
 * IEEE binary16; round-to-nearest (min/max) quantiser evaluated in binary32 with
 * round-half-even; codes computed against the fp16-rounded scale and offset;
 * a group whose scale rounds to zero gets all-zero codes.
 *
 * Precision: dequantisation and dot products are fp64 (exact widening of the
 * fp16/bf16 inputs). The quantiser and the re-quantisation check decide
 * integers, so they run in binary32 with the exact operation sequence stated
 * at each function (no FMA contraction; build with -ffp-contract=off).
 *
 * Execution layout written and read here (the format the GPU library uses;
 * this file implements it independently from its written specification):
 *   the matrix is cut into tiles of 32 rows x 64 k-groups (4096 columns),
 *   stored k-tile major: tile t = kt * RT + rt covers rows 32rt.. and k-groups
 *   64kt.., RT = ceil(N/32), KT = ceil(G/64); a tile has R <= 32 rows and
 *   Gt <= 64 columns (k-groups). Width class c = 0..3 for b = 1,2,4,8. The
 *   groups of class c of a tile form a list of N_c records in column-major
 *   order (by column, then by row); records 64k .. 64k+63 of the list make
 *   block k of the class.
 *   A tile is, each area padded with zeros to a multiple of 16 bytes:
 *     map   : per column l, u32 plane0 (bit r = class & 1) then u32 plane1
 *             (bit r = class >> 1);
 *     blocks: for c = 0..3, the class's blocks in order; a block of m
 *             records is a codes area (2b words per record, record j at
 *             byte 8bj) then an so area (u32 scale | offset << 16 at 4j).
 *   Record words: with h = 16/b, pair p = (code 2p, code 2p+1) sits in word
 *   p/h, code 2p at bit (p%h)*b and code 2p+1 at bit 16+(p%h)*b.
 *   Per tile 4 u32: first 16-byte unit, size in 16-byte units,
 *   N_0 | N_1<<16, N_2 | N_3<<16; one extra entry after the last tile holds
 *   (total 16-byte units, 0, 0, 0).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_GROUP 64

#define ORC_TILE_ROWS 32
#define ORC_TILE_GROUPS 64

/* Deliberate-mistake switch used only by the tests that show the pins catch
 * plausible mistakes. 0 = correct oracle. */
static int g_mut = 0;
void orc_set_mutation(int m) { g_mut = m; }
int orc_get_mutation(void) { return g_mut; }

/* ------------------------------------------------------------------ */
/* IEEE 754 binary16 / bfloat16 conversions, written from the format   */
/* definition: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits */
/* ------------------------------------------------------------------ */

/* Round a double to the nearest binary16 value, ties to even. */
uint16_t orc_f64_to_f16(double v) {
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  double a = fabs(v);
  if (isnan(v)) return 0x7E00u;
  if (a >= 65520.0) return sign | 0x7C00u;            /* rounds past 65504 */
  if (a < ldexp(1.0, -14)) {                            /* subnormal range */
    double m = nearbyint(ldexp(a, 24));                 /* units of 2^-24 */
    return sign | (uint16_t)m;                          /* m==1024 -> smallest normal */
  }
  int e2;
  (void)frexp(a, &e2);                                  /* a = f * 2^e2, f in [0.5,1) */
  int E = e2 - 1;                                       /* a in [2^E, 2^(E+1)) */
  double m = nearbyint(ldexp(a, 10 - E));               /* in [1024, 2048] */
  if (m >= 2048.0) { m = 1024.0; E += 1; }
  if (E + 15 >= 31) return sign | 0x7C00u;
  return sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)m - 1024);
}

uint16_t orc_f32_to_f16(float f) { return orc_f64_to_f16((double)f); }

double orc_f16_to_f64(uint16_t h) {
  int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(1024 + m), e - 25);
  return s ? -v : v;
}

float orc_f16_to_f32(uint16_t h) { return (float)orc_f16_to_f64(h); }

double orc_bf16_to_f64(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* ------------------------------------------------------------------ */
/* Round-to-nearest asymmetric quantiser for one 64-weight group       */
/* ------------------------------------------------------------------ */

/* lo = min, hi = max (sequential scan, strict comparisons);
 * L = 2^b - 1; scale16 = f16(f32(f32(hi - lo) / L)); offset16 = f16(lo);
 * s, o = the fp16 values widened to f32;
 * q_j = s == 0 ? 0 : clamp(rint(f32(f32(w_j - o) / s)), 0, L). */
void orc_quantize_group(const float* w, int b, uint16_t* s16, uint16_t* o16, uint8_t* q) {
  float lo = w[0], hi = w[0];
  for (int j = 1; j < ORC_GROUP; ++j) {
    if (w[j] < lo) lo = w[j];
    if (w[j] > hi) hi = w[j];
  }
  int L = (1 << b) - 1;
  float Lf = (float)L;
  if (g_mut == 7) Lf = (float)(L + 1);                 /* mutation: wrong level count */
  float range = hi - lo;
  float sf = range / Lf;
  *s16 = orc_f32_to_f16(sf);
  *o16 = orc_f32_to_f16(lo);
  float s = orc_f16_to_f32(*s16), o = orc_f16_to_f32(*o16);
  for (int j = 0; j < ORC_GROUP; ++j) {
    if (s == 0.0f) { q[j] = 0; continue; }
    float t = (w[j] - o) / s;
    float r = (g_mut == 3) ? floorf(t) : rintf(t);     /* mutation: truncation */
    if (r < 0.0f) r = 0.0f;
    if (r > (float)L) r = (float)L;
    q[j] = (uint8_t)r;
  }
}

/* ------------------------------------------------------------------ */
/* Canonical LSB-first packing of one group: code j at bit (j*b) mod 32 */
/* of word floor(j*b/32); 2b words per group.                           */
/* ------------------------------------------------------------------ */
void orc_pack_group_canonical(const uint8_t* q, int b, uint32_t* words) {
  for (int w = 0; w < 2 * b; ++w) words[w] = 0;
  for (int j = 0; j < ORC_GROUP; ++j) {
    int bit = j * b;
    int sh = bit % 32;
    if (g_mut == 4) sh = 32 - b - sh;                   /* mutation: MSB-first */
    words[bit / 32] |= (uint32_t)q[j] << sh;
  }
}

void orc_unpack_group_canonical(const uint32_t* words, int b, uint8_t* q) {
  uint32_t mask = (1u << b) - 1u;
  for (int j = 0; j < ORC_GROUP; ++j) {
    int bit = j * b;
    q[j] = (uint8_t)((words[bit / 32] >> (bit % 32)) & mask);
  }
}

/* Record word layout (even codes in the low halves, odd codes in the high
 * halves): see the file header. */
void orc_pack_group_record(const uint8_t* q, int b, uint32_t* words) {
  int h = 16 / b;
  for (int w = 0; w < 2 * b; ++w) {
    uint32_t lo = 0, hi = 0;
    for (int f = 0; f < h; ++f) {
      int p = w * h + f;
      lo |= (uint32_t)q[2 * p] << (f * b);
      hi |= (uint32_t)q[2 * p + 1] << (f * b);
    }
    words[w] = (g_mut == 9) ? (hi | (lo << 16)) : (lo | (hi << 16));  /* mutation: halves swapped */
  }
}

void orc_unpack_group_record(const uint32_t* words, int b, uint8_t* q) {
  int h = 16 / b;
  uint32_t mask = (1u << b) - 1u;
  for (int p = 0; p < 32; ++p) {
    uint32_t w = words[p / h];
    q[2 * p] = (uint8_t)((w >> ((p % h) * b)) & mask);
    q[2 * p + 1] = (uint8_t)((w >> (16 + (p % h) * b)) & mask);
  }
}

/* ------------------------------------------------------------------ */
/* Execution layout: sizes, writer, reader                              */
/* ------------------------------------------------------------------ */
static int width_class(int b) {
  switch (b) { case 1: return 0; case 2: return 1; case 4: return 2; case 8: return 3; default: return -1; }
}
static int class_bits(int c) { return 1 << c; }

static int64_t up16(int64_t v) { return (v + 15) / 16 * 16; }

/* Tile geometry: number of row-tiles and k-tiles. */
static void tile_grid(int N, int K, int64_t* RT, int64_t* KT) {
  int G = K / 64;
  *RT = (N + ORC_TILE_ROWS - 1) / ORC_TILE_ROWS;
  *KT = (G + ORC_TILE_GROUPS - 1) / ORC_TILE_GROUPS;
}

/* Everything the layout of one tile depends on: its rows and columns, the
 * class of every group, and per class its records in list order. */
typedef struct {
  int r0, R, g0, Gt;
  int cls[ORC_TILE_ROWS][ORC_TILE_GROUPS];
  int N[4];
  int rec_row[4][ORC_TILE_ROWS * ORC_TILE_GROUPS];
  int rec_col[4][ORC_TILE_ROWS * ORC_TILE_GROUPS];
} orc_tile;

/* Fills T for tile (rt, kt). Returns -1 on an invalid width. */
static int tile_info(const uint8_t* widths, int N, int G, int64_t rt, int64_t kt, orc_tile* T) {
  T->r0 = (int)(rt * ORC_TILE_ROWS);
  T->R = N - T->r0 < ORC_TILE_ROWS ? N - T->r0 : ORC_TILE_ROWS;
  T->g0 = (int)(kt * ORC_TILE_GROUPS);
  T->Gt = G - T->g0 < ORC_TILE_GROUPS ? G - T->g0 : ORC_TILE_GROUPS;
  for (int r = 0; r < T->R; ++r)
    for (int l = 0; l < T->Gt; ++l) {
      T->cls[r][l] = width_class(widths[(int64_t)(T->r0 + r) * G + T->g0 + l]);
      if (T->cls[r][l] < 0) return -1;
    }
  for (int c = 0; c < 4; ++c) {
    int e = 0;
    /* column-major: outer loop over columns, inner over rows (ascending);
     * mutation 8 lists the records row-major instead */
    int outer = (g_mut == 8) ? T->R : T->Gt, inner = (g_mut == 8) ? T->Gt : T->R;
    for (int a = 0; a < outer; ++a)
      for (int b = 0; b < inner; ++b) {
        int l = (g_mut == 8) ? b : a, r = (g_mut == 8) ? a : b;
        if (T->cls[r][l] == c) {
          T->rec_row[c][e] = r;
          T->rec_col[c][e] = l;
          ++e;
        }
      }
    T->N[c] = e;
  }
  return 0;
}

/* Records in block k of a class with n records. */
static int block_records(int n, int k) { return n - 64 * k < 64 ? n - 64 * k : 64; }

static int64_t block_bytes(int c, int m) { return up16(8 * (int64_t)class_bits(c) * m) + up16(4 * (int64_t)m); }

static int64_t tile_bytes(const orc_tile* T) {
  int64_t bytes = up16(8 * (int64_t)T->Gt);
  for (int c = 0; c < 4; ++c)
    for (int k = 0; 64 * k < T->N[c]; ++k) bytes += block_bytes(c, block_records(T->N[c], k));
  return bytes;
}

static uint32_t count_word(const orc_tile* T, int half) {
  return (uint32_t)T->N[2 * half] | ((uint32_t)T->N[2 * half + 1] << 16);
}

/* Counts the sizes of the layout. Returns 0, or -1 for a bad shape or width. */
int orc_layout_sizes(const uint8_t* widths, int N, int K, int64_t* n_tiles, int64_t* n_records,
                     int64_t* n_bytes16) {
  if (N < 1 || K < 64 || K % 64 != 0 || K / 64 >= 4096) return -1;
  int G = K / 64;
  int64_t RT, KT, bytes = 0;
  tile_grid(N, K, &RT, &KT);
  orc_tile* T = (orc_tile*)malloc(sizeof(orc_tile));
  for (int64_t kt = 0; kt < KT; ++kt)
    for (int64_t rt = 0; rt < RT; ++rt) {
      if (tile_info(widths, N, G, rt, kt, T) != 0) { free(T); return -1; }
      bytes += tile_bytes(T);
    }
  free(T);
  *n_tiles = RT * KT;
  *n_records = (int64_t)N * G;
  *n_bytes16 = bytes / 16;
  return 0;
}

/* Quantises W (f32 [N][K]) with the per-group widths and writes the execution
 * layout: tiles [(n_tiles+1)*4] and the byte stream [n_bytes16*4 u32].
 * Returns 0 or -1. */
int orc_pack(const float* W, const uint8_t* widths, int N, int K, uint32_t* tiles, uint32_t* stream) {
  int64_t T_, R_, B16;
  if (orc_layout_sizes(widths, N, K, &T_, &R_, &B16) != 0) return -1;
  int G = K / 64;
  int64_t RT, KT;
  tile_grid(N, K, &RT, &KT);
  memset(stream, 0, (size_t)B16 * 16);
  orc_tile* T = (orc_tile*)malloc(sizeof(orc_tile));
  int64_t byte = 0;
  for (int64_t t = 0; t < T_; ++t) {
    int64_t kt = t / RT, rt = t % RT;                   /* k-tile major */
    tile_info(widths, N, G, rt, kt, T);
    uint8_t* tb = (uint8_t*)stream + byte;
    for (int l = 0; l < T->Gt; ++l) {
      uint32_t p0 = 0, p1 = 0;
      for (int r = 0; r < T->R; ++r) {
        p0 |= (uint32_t)(T->cls[r][l] & 1) << r;
        p1 |= (uint32_t)(T->cls[r][l] >> 1) << r;
      }
      memcpy(tb + 8 * l, &p0, 4);
      memcpy(tb + 8 * l + 4, &p1, 4);
    }
    int64_t pos = up16(8 * (int64_t)T->Gt);
    for (int c = 0; c < 4; ++c) {
      int b = class_bits(c);
      for (int k = 0; 64 * k < T->N[c]; ++k) {
        int m = block_records(T->N[c], k);
        for (int j = 0; j < m; ++j) {
          int e = 64 * k + j, l = T->rec_col[c][e], r = T->rec_row[c][e];
          uint16_t s16, o16;
          uint8_t q[64];
          uint32_t words[16];
          orc_quantize_group(W + (int64_t)(T->r0 + r) * K + 64 * (int64_t)(T->g0 + l), b, &s16, &o16, q);
          orc_pack_group_record(q, b, words);
          memcpy(tb + pos + 8 * (int64_t)b * j, words, 8 * (size_t)b);
          uint32_t so = (uint32_t)s16 | ((uint32_t)o16 << 16);
          memcpy(tb + pos + up16(8 * (int64_t)b * m) + 4 * j, &so, 4);
        }
        pos += block_bytes(c, m);
      }
    }
    tiles[4 * t + 0] = (uint32_t)(byte / 16);
    tiles[4 * t + 1] = (uint32_t)(pos / 16);
    tiles[4 * t + 2] = count_word(T, 0);
    tiles[4 * t + 3] = count_word(T, 1);
    byte += pos;
  }
  free(T);
  tiles[4 * T_ + 0] = (uint32_t)(byte / 16);
  tiles[4 * T_ + 1] = 0;
  tiles[4 * T_ + 2] = 0;
  tiles[4 * T_ + 3] = 0;
  return 0;
}

static int all_zero(const uint8_t* p, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (p[i]) return 0;
  return 1;
}

/* Reads the execution layout back into natural order: codes [N][K], and per
 * group scale16/offset16/width [N][G]. Rows listed in `rows` only (n_rows of
 * them) when rows != NULL; outputs are then [n_rows][...] in that order.
 * The classes come from each tile's map alone. Returns 0, or -1 if the layout
 * is inconsistent (a tile entry that disagrees with its map, a tile that does
 * not end where the next begins, nonzero padding or unused map bits). */
int orc_unpack(const uint32_t* tiles, const uint32_t* stream, int N, int K, const int64_t* rows, int64_t n_rows,
               uint8_t* q_out, uint16_t* s_out, uint16_t* o_out, uint8_t* w_out) {
  if (N < 1 || K < 64 || K % 64 != 0) return -1;
  int G = K / 64;
  int64_t RT, KT;
  tile_grid(N, K, &RT, &KT);
  int64_t nr = rows ? n_rows : N;
  for (int64_t i = 0; i < nr * G; ++i) w_out[i] = 0;
  orc_tile* T = (orc_tile*)malloc(sizeof(orc_tile));
  uint8_t* wmap = (uint8_t*)malloc((size_t)ORC_TILE_ROWS * G);   /* widths of one row-tile, from the maps */
  int rc = 0;
  for (int64_t ri = 0; ri < nr && rc == 0; ++ri) {
    int64_t row = rows ? rows[ri] : ri;
    if (row < 0 || row >= N) { rc = -1; break; }
    int64_t rt = row / ORC_TILE_ROWS;
    for (int64_t kt = 0; kt < KT && rc == 0; ++kt) {
      int64_t t = kt * RT + rt;
      const uint8_t* tb = (const uint8_t*)stream + (int64_t)tiles[4 * t] * 16;
      int r0 = (int)(rt * ORC_TILE_ROWS), R = N - r0 < ORC_TILE_ROWS ? N - r0 : ORC_TILE_ROWS;
      int g0 = (int)(kt * ORC_TILE_GROUPS), Gt = G - g0 < ORC_TILE_GROUPS ? G - g0 : ORC_TILE_GROUPS;
      /* widths of this tile from its map */
      for (int l = 0; l < Gt; ++l) {
        uint32_t p0, p1;
        memcpy(&p0, tb + 8 * l, 4);
        memcpy(&p1, tb + 8 * l + 4, 4);
        if (R < 32 && ((p0 | p1) >> R) != 0) { rc = -1; break; }
        for (int r = 0; r < R; ++r) {
          int c = (int)((p0 >> r) & 1u) | (int)(((p1 >> r) & 1u) << 1);
          wmap[(int64_t)r * G + g0 + l] = (uint8_t)class_bits(c);
        }
      }
      if (rc) break;
      if (!all_zero(tb + 8 * Gt, up16(8 * (int64_t)Gt) - 8 * Gt)) { rc = -1; break; }
      /* the tile as the writer sees it, built from the map's widths */
      tile_info(wmap, R, G, 0, kt, T);
      T->r0 = r0;
      if (tiles[4 * t + 2] != count_word(T, 0) || tiles[4 * t + 3] != count_word(T, 1) ||
          (int64_t)tiles[4 * t + 1] * 16 != tile_bytes(T) || tiles[4 * t + 0] + tiles[4 * t + 1] != tiles[4 * t + 4]) {
        rc = -1;
        break;
      }
      int64_t pos = up16(8 * (int64_t)Gt);
      for (int c = 0; c < 4 && rc == 0; ++c) {
        int b = class_bits(c);
        for (int k = 0; 64 * k < T->N[c] && rc == 0; ++k) {
          int m = block_records(T->N[c], k);
          if (!all_zero(tb + pos + 8 * (int64_t)b * m, up16(8 * (int64_t)b * m) - 8 * (int64_t)b * m) ||
              !all_zero(tb + pos + up16(8 * (int64_t)b * m) + 4 * m, up16(4 * (int64_t)m) - 4 * m)) {
            rc = -1;
            break;
          }
          for (int j = 0; j < m; ++j) {
            int e = 64 * k + j, l = T->rec_col[c][e], r = T->rec_row[c][e];
            if (r0 + r != row) continue;
            uint32_t words[16], so;
            memcpy(words, tb + pos + 8 * (int64_t)b * j, 8 * (size_t)b);
            memcpy(&so, tb + pos + up16(8 * (int64_t)b * m) + 4 * j, 4);
            uint8_t q[64];
            orc_unpack_group_record(words, b, q);
            int64_t g = g0 + l;
            if (w_out[ri * G + g] != 0) { rc = -1; break; }
            memcpy(q_out + ri * K + 64 * g, q, 64);
            s_out[ri * G + g] = (uint16_t)(so & 0xFFFF);
            o_out[ri * G + g] = (uint16_t)(so >> 16);
            w_out[ri * G + g] = (uint8_t)b;
          }
          pos += block_bytes(c, m);
        }
      }
    }
    if (rc == 0)
      for (int g = 0; g < G; ++g)
        if (w_out[ri * G + g] == 0) { rc = -1; break; }
  }
  free(wmap);
  free(T);
  return rc;
}

/* ------------------------------------------------------------------ */
/* Dequantise + dot, fp64, natural k order                              */
/* ------------------------------------------------------------------ */

/* Wdq[n][k] = s_g*q + o_g (+ r[n][k]), exact widening of the fp16 inputs. */
static double dequant(const uint8_t* q, const uint16_t* s16, const uint16_t* o16, const uint16_t* resid,
                      int64_t n, int64_t k, int K) {
  int G = K / 64;
  int64_t g = n * G + k / 64;
  double s = orc_f16_to_f64(s16[g]);
  double o = orc_f16_to_f64(o16[g]);
  if (g_mut == 1) o = 0.0;                              /* mutation: offset dropped */
  double w = s * (double)q[n * K + k] + o;
  if (resid) {
    double r = orc_f16_to_f64(resid[n * K + k]);
    w += (g_mut == 6) ? -r : r;                         /* mutation: residual sign */
  }
  return w;
}

/* y[b][n] = sum_k x[b][k] * Wdq[n][k] for n < N (rows of the natural arrays),
 * x fp16 [B][K] (or bf16 when x_is_bf16), y fp64 [B][N]. */
void orc_gemv(const uint8_t* q, const uint16_t* s16, const uint16_t* o16, int N, int K,
              const uint16_t* x, int B, int x_is_bf16, const uint16_t* resid, double* y) {
  double* xd = (double*)malloc(sizeof(double) * (size_t)B * K);
  for (int64_t i = 0; i < (int64_t)B * K; ++i) xd[i] = x_is_bf16 ? orc_bf16_to_f64(x[i]) : orc_f16_to_f64(x[i]);
  for (int64_t n = 0; n < N; ++n)
    for (int b = 0; b < B; ++b) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        int64_t kx = (g_mut == 2) ? (k ^ 1) : k;        /* mutation: wrong x index */
        acc += xd[(int64_t)b * K + kx] * dequant(q, s16, o16, resid, n, k, K);
      }
      y[(int64_t)b * N + n] = acc;
    }
  free(xd);
}

/* ------------------------------------------------------------------ */
/* bfloat16 weights for the batched (matrix-core) product               */
/* ------------------------------------------------------------------ */

/* Round a binary32 value to bfloat16 (8 significant bits), ties to even:
 * the two candidates are f with its low 16 bits cleared and the next
 * bfloat16 away from zero; the nearer wins, a tie goes to the one whose last
 * kept bit is 0. */
uint16_t orc_f32_to_bf16(float f) {
  uint32_t u, up;
  memcpy(&u, &f, 4);
  if (isnan(f)) return (uint16_t)((u >> 16) | 0x40u);
  uint32_t lo = u & 0xFFFF0000u;
  if (lo == u) return (uint16_t)(u >> 16);
  up = lo + 0x10000u;
  float flo, fup;
  memcpy(&flo, &lo, 4);
  memcpy(&fup, &up, 4);
  double dlo = fabs((double)f - (double)flo), dup = fabs((double)fup - (double)f);
  if (dlo < dup) return (uint16_t)(lo >> 16);
  if (dup < dlo) return (uint16_t)(up >> 16);
  if (g_mut == 10) return (uint16_t)(up >> 16);         /* mutation: ties away from zero */
  return (uint16_t)(((lo >> 16) & 1u) ? (up >> 16) : (lo >> 16));
}

/* Wbf[n][k] = bf16(f32(f32(s) * q) + f32(o)): the product is exact in binary32
 * (11-bit scale times an 8-bit code), the sum is one binary32 rounding, then
 * one rounding to bfloat16. This is the weight a bf16 matrix-core product
 * multiplies; used to separate that rounding from the accumulation order. */
void orc_dequant_bf16(const uint8_t* q, const uint16_t* s16, const uint16_t* o16, int N, int K, uint16_t* out) {
  int G = K / ORC_GROUP;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      float s = orc_f16_to_f32(s16[n * G + k / ORC_GROUP]);
      float o = orc_f16_to_f32(o16[n * G + k / ORC_GROUP]);
      float sq = s * (float)q[n * K + k];
      float v = sq + o;
      out[n * K + k] = orc_f32_to_bf16(v);
    }
}

/* ------------------------------------------------------------------ */
/* In-cell residual and the re-quantisation check (binary32)            */
/* ------------------------------------------------------------------ */

/* r16[n][k] = f16(u[n][k] * s_g) with the product in fp64. */
void orc_make_cell_residual(const double* u, const uint16_t* s16, int N, int K, uint16_t* r16) {
  int G = K / 64;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k)
      r16[n * K + k] = orc_f64_to_f16(u[n * K + k] * orc_f16_to_f64(s16[n * G + k / 64]));
}

/* For every weight, in binary32 with this operation order:
 *   s, o, r = widened fp16; deq = f32(f32(s*q) + o); v = f32(deq + r);
 *   q' = s == 0 ? 0 : clamp(rint(f32(f32(v - o) / s)), 0, L)
 *   mismatch   : q' != q
 *   out of cell: s > 0 ? |r| >= f32(0.5*s) : r != 0
 * Scales and offsets are carried through unchanged (frozen).
 * counts[0] = mismatches, counts[1] = out of cell, counts[2] = smallest linear
 * index n*K+k that has either (UINT64_MAX if none). q_prime (natural order)
 * may be NULL. */
void orc_requant_verify(const uint8_t* q, const uint16_t* s16, const uint16_t* o16, const uint8_t* widths,
                        const uint16_t* r16, int N, int K, uint64_t* counts, uint8_t* q_prime) {
  int G = K / 64;
  uint64_t mism = 0, ooc = 0, first = UINT64_MAX;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      int64_t gi = n * G + k / 64;
      int L = (g_mut == 12) ? 255 : (1 << widths[gi]) - 1;  /* mutation: L not from the group's width */
      float s = orc_f16_to_f32(s16[gi]), o = orc_f16_to_f32(o16[gi]);
      float r = orc_f16_to_f32(r16[n * K + k]);
      float qf = (float)q[n * K + k];
      float sq = s * qf;
      float deq = sq + o;
      float v = deq + r;
      int qp;
      if (s == 0.0f) qp = 0;
      else {
        float d = v - o;
        float t = d / s;
        float rr = rintf(t);
        if (g_mut != 11) {                              /* mutation: clamp dropped */
          if (rr < 0.0f) rr = 0.0f;
          if (rr > (float)L) rr = (float)L;
        }
        qp = (int)rr;
      }
      int bad_code = qp != (int)q[n * K + k];
      int bad_cell;
      if (s > 0.0f) {
        float half = 0.5f * s;
        bad_cell = (g_mut == 5) ? (fabsf(r) > half) : (fabsf(r) >= half);  /* mutation: boundary */
      } else {
        bad_cell = r != 0.0f;
      }
      mism += (uint64_t)bad_code;
      ooc += (uint64_t)bad_cell;
      if ((bad_code || bad_cell) && (uint64_t)(n * K + k) < first) first = (uint64_t)(n * K + k);
      if (q_prime) q_prime[n * K + k] = (uint8_t)qp;
    }
  counts[0] = mism;
  counts[1] = ooc;
  counts[2] = first;
}

/* ------------------------------------------------------------------ */
/* Compact in-cell residual: one byte per weight                        */
/* ------------------------------------------------------------------ */
/* An encoding of the in-cell residual of this library's own (the CellFill
 * page keeps the residual inside the weight's rounding cell but fixes no
 * storage for it): a signed byte f in [-127, 127] per weight stands for
 *   r = s * f / 256        (s = the group's fp16 scale)
 * so |r| <= (127/256) s < s/2: every encoded residual lies inside its cell.
 * Encoding an fp16 residual, in binary32 with one rounding per operation:
 *   f = s == 0 ? 0 : clamp(rint(f32(r / s) * 256), -127, 127)   (ties even) */
void orc_cell8_encode(const uint16_t* r16, const uint16_t* s16, int N, int K, int8_t* f) {
  int G = K / 64;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      float sc = orc_f16_to_f32(s16[n * G + k / 64]);
      float r = orc_f16_to_f32(r16[n * K + k]);
      int v = 0;
      if (sc != 0.0f) {
        float t = (r / sc) * 256.0f;
        float rr = (g_mut == 14) ? truncf(t) : rintf(t);   /* mutation: truncation */
        if (rr < -127.0f) rr = -127.0f;
        if (rr > 127.0f) rr = 127.0f;
        v = (int)rr;
      }
      f[n * K + k] = (int8_t)v;
    }
}

/* The fp16 residual a fraction byte stands for: r = fp16(s f / 256). s f / 256
 * is exact in fp64, so the result is one rounding to nearest even. */
void orc_cell8_decode(const int8_t* f, const uint16_t* s16, int N, int K, uint16_t* r16) {
  int G = K / 64;
  double unit = (g_mut == 15) ? 255.0 : 256.0;          /* mutation: wrong fraction unit in the decode */
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k)
      r16[n * K + k] = orc_f64_to_f16(orc_f16_to_f64(s16[n * G + k / 64]) * (double)f[n * K + k] / unit);
}

/* y[b][n] = sum_k x[b][k] * (s*q + o + s*f/256), fp64 (exact widening; the
 * products and the division by 256 are exact in fp64). */
void orc_gemv_cell8(const uint8_t* q, const uint16_t* s16, const uint16_t* o16, int N, int K, const uint16_t* x,
                    int B, const int8_t* f, double* y) {
  int G = K / 64;
  double* xd = (double*)malloc(sizeof(double) * (size_t)B * K);
  for (int64_t i = 0; i < (int64_t)B * K; ++i) xd[i] = orc_f16_to_f64(x[i]);
  double frac = (g_mut == 13) ? 128.0 : 256.0;          /* mutation: wrong fraction unit */
  for (int64_t n = 0; n < N; ++n)
    for (int b = 0; b < B; ++b) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double sc = orc_f16_to_f64(s16[n * G + k / 64]);
        double w = dequant(q, s16, o16, NULL, n, k, K) + sc * (double)f[n * K + k] / frac;
        acc += xd[(int64_t)b * K + k] * w;
      }
      y[(int64_t)b * N + n] = acc;
    }
  free(xd);
}

/* ------------------------------------------------------------------ */
/* Array helpers for the Python wrapper                                 */
/* ------------------------------------------------------------------ */
void orc_f64_to_f16_array(const double* v, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f64_to_f16(v[i]);
}
void orc_f32_to_f16_array(const float* v, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_f16(v[i]);
}
void orc_f16_to_f64_array(const uint16_t* h, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_to_f64(h[i]);
}
/* Quantises every group of W [N][K] with widths [N][G] into natural-order
 * codes [N][K] and scale16/offset16 [N][G]. Returns 0 or -1. */
int orc_quantize_matrix(const float* W, const uint8_t* widths, int N, int K, uint8_t* q, uint16_t* s16,
                        uint16_t* o16) {
  if (N < 1 || K < 64 || K % 64 != 0) return -1;
  int G = K / 64;
  for (int64_t n = 0; n < N; ++n)
    for (int g = 0; g < G; ++g) {
      int b = widths[n * G + g];
      if (width_class(b) < 0) return -1;
      orc_quantize_group(W + n * K + 64 * g, b, &s16[n * G + g], &o16[n * G + g], q + n * K + 64 * g);
    }
  return 0;
}
