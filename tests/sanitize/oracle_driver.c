/* Exercises the CPU oracle on small seeded inputs under AddressSanitizer and
 * UndefinedBehaviorSanitizer: every format's encode / decode / product, the
 * MX target, the KV stream functions, the prefix codes, and decoding of
 * corrupted streams (which must be refused, never read out of bounds).
 * Exit status 0 when every call returned what it should. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "cass_oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) { /* splitmix64 */
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
      return 1;                                                  \
    }                                                            \
  } while (0)

static int weights(int fmt, int64_t R, int64_t C, int64_t k, int m, int64_t B) {
  uint16_t* w = malloc((size_t)(R * C) * 2);
  for (int64_t i = 0; i < R * C; i++) w[i] = (uint16_t)next_u64();
  int64_t sb = 0, vb = 0;
  int st = orc_encode(w, R, C, k, m, B, fmt, NULL, 0, NULL, 0, &sb, &vb);
  if (st == ORC_ERR_OVERFLOW) { free(w); return 0; } /* format 4 refuses long codes */
  CHECK(st == ORC_OK);
  uint8_t* spec = calloc((size_t)sb, 1);
  uint8_t* verif = calloc((size_t)vb, 1);
  st = orc_encode(w, R, C, k, m, B, fmt, spec, sb, verif, vb, &sb, &vb);
  if (st == ORC_ERR_OVERFLOW && fmt == ORC_FMT_C1S) { /* 16-bit superblock offsets exceeded */
    free(w); free(spec); free(verif);
    return 0;
  }
  CHECK(st == ORC_OK);
  uint16_t* out = malloc((size_t)(R * C) * 2);
  CHECK(orc_draft_decode(spec, sb, out) == ORC_OK);
  CHECK(orc_reconstruct(spec, sb, verif, vb, out) == ORC_OK);
  if (fmt != 3) CHECK(memcmp(out, w, (size_t)(R * C) * 2) == 0);
  uint16_t x[2 * 1024];
  for (int i = 0; i < 2 * C; i++) x[i] = (uint16_t)(0x3C00 + (next_u64() & 0x7F)); /* finite */
  double* y = malloc((size_t)(2 * R) * sizeof(double));
  double* ay = malloc((size_t)(2 * R) * sizeof(double));
  CHECK(orc_product(spec, sb, NULL, 0, x, 2, y, ay, 1) == ORC_OK);
  CHECK(orc_product(spec, sb, verif, vb, x, 2, y, ay, 2) == ORC_OK);
  /* corrupted copies: refused or decoded, never read outside the buffers */
  for (int t = 0; t < 64; t++) {
    uint8_t* bad = malloc((size_t)sb);
    memcpy(bad, spec, (size_t)sb);
    bad[next_u64() % (uint64_t)sb] ^= (uint8_t)(1u << (next_u64() & 7));
    /* the output holds the rows x cols the (possibly corrupted) header names */
    int64_t hf[8], so[12], sl[12];
    if (orc_header(bad, sb, ORC_MAGIC_SPEC, hf, so, sl) == ORC_OK && hf[2] * hf[3] <= (1 << 22)) {
      uint16_t* o2 = malloc((size_t)(hf[2] * hf[3] + 1) * 2);
      (void)orc_draft_decode(bad, sb, o2);
      (void)orc_reconstruct(bad, sb, verif, vb, o2);
      free(o2);
    }
    free(bad);
  }
  CHECK(orc_draft_decode(spec, 100, out) == ORC_ERR_CORRUPT); /* truncated */
  free(w); free(spec); free(verif); free(out); free(y); free(ay);
  return 0;
}

int main(void) {
  for (int fmt = 1; fmt <= 4; fmt++) {
    if (weights(fmt, 7, 512, 150, 3, 256)) return 1;
    if (weights(fmt, 3, 256, 0, 0, 64)) return 1;
    if (weights(fmt, 2, 1024, 1024, 7, 128)) return 1;
  }
  uint16_t mx[4 * 256], mt[4 * 256];
  for (int i = 0; i < 4 * 256; i++) mx[i] = (uint16_t)next_u64();
  CHECK(orc_mx_target(mx, 4, 256, mt) == ORC_OK);
  /* KV streams */
  for (int fmt = 1; fmt <= 2; fmt++) {
    const int64_t T = 40, D = 128, k = 38, m = 3, Tm = 48, cc = 48 * 38 * 8, vc = 48 * 90 * 8;
    int64_t so[5], vo[5], sb, vb;
    CHECK(orc_kv_layout(fmt, D, k, m, Tm, cc, vc, so, vo, &sb, &vb) == ORC_OK);
    uint16_t* vec = malloc((size_t)(T * D) * 2);
    /* values of a few binades (the code capacities hold their codes) */
    for (int64_t i = 0; i < T * D; i++) {
      const uint64_t r = next_u64();
      vec[i] = (uint16_t)(((r & 1) << 15) | ((120 + (r >> 1) % 10) << 7) | ((r >> 8) & 0x7F));
    }
    uint8_t* spec = calloc((size_t)sb, 1);
    uint8_t* verif = calloc((size_t)vb, 1);
    uint64_t tails[2];
    CHECK(orc_kv_encode(fmt, vec, T, 16, D, k, m, Tm, cc, vc, spec, verif, tails) == ORC_OK);
    uint16_t* out = malloc((size_t)(T * D) * 2);
    CHECK(orc_kv_decode(fmt, spec, NULL, T, D, k, m, Tm, cc, vc, out) == ORC_OK);
    CHECK(orc_kv_decode(fmt, spec, verif, T, D, k, m, Tm, cc, vc, out) == ORC_OK);
    CHECK(memcmp(out, vec, (size_t)(T * D) * 2) == 0);
    free(vec); free(spec); free(verif); free(out);
  }
  /* prefix codes */
  uint64_t hist[256] = {0};
  for (int i = 0; i < 256; i++) hist[i] = (i % 7 == 0) ? 1 + (next_u64() % 1000) : 0;
  uint8_t len[256];
  uint32_t code[256];
  CHECK(orc_huffman_lengths(hist, 12, len) == ORC_OK);
  CHECK(orc_canonical_codes(len, code) == ORC_OK);
  uint8_t sym[512], back[512];
  for (int i = 0; i < 512; i++) sym[i] = (uint8_t)(7 * (next_u64() % 37));
  uint8_t stream[4096] = {0};
  uint32_t blk[8];
  int64_t bits = 0;
  CHECK(orc_prefix_encode(sym, 512, 64, len, code, stream, sizeof stream, blk, &bits) == ORC_OK);
  CHECK(orc_prefix_decode(stream, sizeof stream, 512, len, code, back) == ORC_OK);
  CHECK(memcmp(sym, back, 512) == 0);
  CHECK(orc_unary_code(hist, len, code) == ORC_OK);
  printf("oracle driver ok\n");
  return 0;
}
