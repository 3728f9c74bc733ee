/* Drives every entry point of the oracle (oracle/vbq_oracle.c) on small
 * random shapes, for a build with AddressSanitizer and UndefinedBehavior-
 * Sanitizer: any out-of-bounds access, leak or undefined operation aborts the
 * run. It also checks the round trips the oracle promises (the layout reads
 * back as the quantiser's output; a zero residual re-quantises to the same
 * codes). Exit status 0 means clean.
 *
 * Inputs are drawn here with a 64-bit linear congruential generator; nothing
 * of the method is computed here besides what the oracle returns. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_quantize_matrix(const float* W, const uint8_t* widths, int N, int K, uint8_t* q, uint16_t* s16,
                        uint16_t* o16);
int orc_layout_sizes(const uint8_t* widths, int N, int K, int64_t* n_tiles, int64_t* n_records,
                     int64_t* n_bytes16);
int orc_pack(const float* W, const uint8_t* widths, int N, int K, uint32_t* tiles, uint32_t* stream);
int orc_unpack(const uint32_t* tiles, const uint32_t* stream, int N, int K, const int64_t* rows, int64_t n_rows,
               uint8_t* q_out, uint16_t* s_out, uint16_t* o_out, uint8_t* w_out);
void orc_gemv(const uint8_t* q, const uint16_t* s16, const uint16_t* o16, int N, int K, const uint16_t* x, int B,
              int x_is_bf16, const uint16_t* resid, double* y);
void orc_make_cell_residual(const double* u, const uint16_t* s16, int N, int K, uint16_t* r16);
void orc_requant_verify(const uint8_t* q, const uint16_t* s16, const uint16_t* o16, const uint8_t* widths,
                        const uint16_t* r16, int N, int K, uint64_t* counts, uint8_t* q_prime);
void orc_pack_group_canonical(const uint8_t* q, int b, uint32_t* words);
void orc_unpack_group_canonical(const uint32_t* words, int b, uint8_t* q);
void orc_pack_group_record(const uint8_t* q, int b, uint32_t* words);
void orc_unpack_group_record(const uint32_t* words, int b, uint8_t* q);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(g_state >> 33);
}
static double unit(void) { return (rnd() + 0.5) / 2147483648.0; }   /* (0, 1) */
static float normal(void) { return (float)(sqrt(-2.0 * log(unit())) * cos(6.283185307179586 * unit())); }

#define CHECK(cond, ...)                  \
  do {                                    \
    if (!(cond)) {                        \
      fprintf(stderr, __VA_ARGS__);       \
      fprintf(stderr, "\n");              \
      return 1;                           \
    }                                     \
  } while (0)

static int one_case(int N, int K) {
  const int G = K / 64;
  float* W = malloc(sizeof(float) * (size_t)N * K);
  uint8_t* widths = malloc((size_t)N * G);
  for (int64_t i = 0; i < (int64_t)N * K; ++i) W[i] = 0.02f * normal();
  for (int64_t i = 0; i < (int64_t)N * G; ++i) widths[i] = (uint8_t)(1u << (rnd() % 4));
  if (N > 2) memset(W + 64, 0, 64 * sizeof(float));   /* a constant group: scale 0 */

  uint8_t* q = malloc((size_t)N * K);
  uint16_t* s16 = malloc(sizeof(uint16_t) * (size_t)N * G);
  uint16_t* o16 = malloc(sizeof(uint16_t) * (size_t)N * G);
  CHECK(orc_quantize_matrix(W, widths, N, K, q, s16, o16) == 0, "quantize failed %dx%d", N, K);

  int64_t T, R, B16;
  CHECK(orc_layout_sizes(widths, N, K, &T, &R, &B16) == 0, "sizes failed");
  uint32_t* tiles = malloc(sizeof(uint32_t) * 4 * (size_t)(T + 1));
  uint32_t* stream = malloc((size_t)B16 * 16);
  CHECK(orc_pack(W, widths, N, K, tiles, stream) == 0, "pack failed");

  uint8_t* q2 = malloc((size_t)N * K);
  uint16_t* s2 = malloc(sizeof(uint16_t) * (size_t)N * G);
  uint16_t* o2 = malloc(sizeof(uint16_t) * (size_t)N * G);
  uint8_t* w2 = malloc((size_t)N * G);
  CHECK(orc_unpack(tiles, stream, N, K, NULL, N, q2, s2, o2, w2) == 0, "unpack failed");
  CHECK(memcmp(q, q2, (size_t)N * K) == 0 && memcmp(s16, s2, 2 * (size_t)N * G) == 0 &&
            memcmp(o16, o2, 2 * (size_t)N * G) == 0 && memcmp(widths, w2, (size_t)N * G) == 0,
        "layout does not read back as the quantiser's output (%dx%d)", N, K);
  int64_t rows[2] = {N - 1, 0};
  uint8_t* qr = malloc(2 * (size_t)K);
  uint16_t* sr = malloc(sizeof(uint16_t) * 2 * (size_t)G);
  uint16_t* orr = malloc(sizeof(uint16_t) * 2 * (size_t)G);
  uint8_t* wr = malloc(2 * (size_t)G);
  CHECK(orc_unpack(tiles, stream, N, K, rows, 2, qr, sr, orr, wr) == 0, "row unpack failed");
  CHECK(memcmp(qr, q + (size_t)(N - 1) * K, (size_t)K) == 0 && memcmp(qr + K, q, (size_t)K) == 0,
        "row subset differs");
  free(qr), free(sr), free(orr), free(wr);

  const int B = 3;
  uint16_t* x = malloc(sizeof(uint16_t) * (size_t)B * K);
  for (int64_t i = 0; i < (int64_t)B * K; ++i) x[i] = (uint16_t)(0x3C00u ^ (rnd() & 0x83FFu));   /* |x| in [1,2) */
  double* y = malloc(sizeof(double) * (size_t)B * N);
  double* u = malloc(sizeof(double) * (size_t)N * K);
  uint16_t* r16 = malloc(sizeof(uint16_t) * (size_t)N * K);
  for (int64_t i = 0; i < (int64_t)N * K; ++i) u[i] = 0.98 * unit() - 0.49;
  orc_make_cell_residual(u, s16, N, K, r16);
  orc_gemv(q, s16, o16, N, K, x, B, 0, NULL, y);
  orc_gemv(q, s16, o16, N, K, x, B, 1, r16, y);
  for (int64_t i = 0; i < (int64_t)B * N; ++i) CHECK(isfinite(y[i]), "non-finite y");

  uint64_t counts[3];
  memset(r16, 0, sizeof(uint16_t) * (size_t)N * K);
  orc_requant_verify(q, s16, o16, widths, r16, N, K, counts, q2);
  CHECK(counts[0] == 0 && counts[1] == 0 && counts[2] == UINT64_MAX, "zero residual fails the check");
  CHECK(memcmp(q2, q, (size_t)N * K) == 0, "zero residual changes a code");
  r16[(size_t)(N / 2) * K + 7] = 0x7C00u;   /* +inf: outside every cell */
  orc_requant_verify(q, s16, o16, widths, r16, N, K, counts, NULL);
  CHECK(counts[1] >= 1, "infinite residual not reported");

  free(W), free(widths), free(q), free(s16), free(o16), free(tiles), free(stream);
  free(q2), free(s2), free(o2), free(w2), free(x), free(y), free(u), free(r16);
  return 0;
}

int main(void) {
  /* per-group packings, every width */
  for (int b = 1; b <= 8; b <<= 1) {
    uint8_t qa[64], qb[64];
    uint32_t words[16];
    for (int i = 0; i < 64; ++i) qa[i] = (uint8_t)(rnd() & ((1u << b) - 1u));
    orc_pack_group_canonical(qa, b, words);
    orc_unpack_group_canonical(words, b, qb);
    CHECK(memcmp(qa, qb, 64) == 0, "canonical round trip, b=%d", b);
    orc_pack_group_record(qa, b, words);
    orc_unpack_group_record(words, b, qb);
    CHECK(memcmp(qa, qb, 64) == 0, "record round trip, b=%d", b);
  }
  const int shapes[][2] = {{1, 64}, {3, 128}, {17, 192}, {16, 4096}, {33, 4160}, {5, 8192 + 64}};
  for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i)
    if (one_case(shapes[i][0], shapes[i][1]) != 0) return 1;
  printf("oracle clean under the sanitizers\n");
  return 0;
}
