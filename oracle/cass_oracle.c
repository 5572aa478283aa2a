/*
 * CPU oracle for the Cassandra bit-level weight format -- TEST INFRASTRUCTURE.
 * Plain scalar C, written for readability, not speed.  Only tests, the smoke
 * check and the CPU-baseline leg of the benchmark use it.
 *
 * Sources followed (page titles and sections):
 *  [R31] Cassandra review, marsggbo.github.io, section 3.1: weights and KV are
 *        transformed in three steps -- unstructured value pruning by numerical
 *        saliency, mantissa truncation of the kept values, exponent compression --
 *        and split into speculation data (draft) and verification data (rest);
 *        pruned values and chopped mantissa bits go to the verification data;
 *        the draft loads only speculation data, zero-filled back to standard
 *        floating point; the target loads both and reassembles losslessly.
 *  [R32] same page, section 3.2: exponent entropy is low; Cassandra-1 codes
 *        exponents with a unary code where frequent exponents get short codes,
 *        decoded by counting zeros up to the one; Cassandra-2 uses an MX-style
 *        shared exponent.
 *  [MX]  OCP Microscaling Formats (MX) v1.0 specification, cited by the paper:
 *        blocks of 32 elements with one shared 8-bit exponent.
 *  [P4F6] pith.science review of "Cassandra: Enabling Reasoning LLMs at Edge via
 *        Self-Speculative Decoding", Figure 6(a): exponent Shannon entropy.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  saliency = |w| (15 magnitude bits), group = one row, ties -> lower column;
 *  truncation chops (never rounds); zero-fill is +0 (0x0000); rank tables are
 *  per tensor and per stream, ties -> smaller exponent, absent symbols appended
 *  ascending; unary code = r zeros then a one, LSB first; blocks are B original
 *  positions; Cassandra-2 keeps the verification stream lossless and confines
 *  the MX loss to the draft.
 */
#include "cass_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define HDR_BYTES 256
#define MAX_SEC 12

/* ------------------------------------------------------------------ bits */

static void put_bits(uint8_t* buf, uint64_t pos, uint64_t val, int width) {
  for (int t = 0; t < width; t++)
    if ((val >> t) & 1u) buf[(pos + t) >> 3] |= (uint8_t)(1u << ((pos + t) & 7));
}

static uint64_t get_bits(const uint8_t* buf, uint64_t pos, int width) {
  uint64_t v = 0;
  for (int t = 0; t < width; t++)
    v |= (uint64_t)((buf[(pos + t) >> 3] >> ((pos + t) & 7)) & 1u) << t;
  return v;
}

static void put_u16(uint8_t* p, uint16_t v) { p[0] = v & 255; p[1] = v >> 8; }
static void put_u32(uint8_t* p, uint32_t v) { for (int i = 0; i < 4; i++) p[i] = (v >> (8 * i)) & 255; }
static void put_u64(uint8_t* p, uint64_t v) { for (int i = 0; i < 8; i++) p[i] = (v >> (8 * i)) & 255; }
static uint16_t get_u16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static uint32_t get_u32(const uint8_t* p) {
  uint32_t v = 0;
  for (int i = 0; i < 4; i++) v |= (uint32_t)p[i] << (8 * i);
  return v;
}
static uint64_t get_u64(const uint8_t* p) {
  uint64_t v = 0;
  for (int i = 0; i < 8; i++) v |= (uint64_t)p[i] << (8 * i);
  return v;
}

static int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

/* Unary code [R32]: r zeros, then a one. */
static void put_unary(uint8_t* buf, uint64_t pos, int r) { put_bits(buf, pos + (uint64_t)r, 1, 1); }

/* Decode one unary code by counting zeros up to the one; -1 if none within 256. */
static int get_unary(const uint8_t* buf, uint64_t pos, uint64_t end) {
  for (int r = 0; r < 256; r++) {
    if (pos + (uint64_t)r >= end) return -1;
    if (get_bits(buf, pos + (uint64_t)r, 1)) return r;
  }
  return -1;
}

/* bf16 fields */
static int bf_s(uint16_t b) { return b >> 15; }
static int bf_e(uint16_t b) { return (b >> 7) & 0xFF; }
static int bf_f(uint16_t b) { return b & 0x7F; }
static int bf_key(uint16_t b) { return b & 0x7FFF; }

static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* ------------------------------------------------------------- pruning */

typedef struct { int key; int64_t idx; } keyed;

static int cmp_salience(const void* a, const void* b) {
  const keyed* x = (const keyed*)a;
  const keyed* y = (const keyed*)b;
  if (x->key != y->key) return x->key > y->key ? -1 : 1; /* larger |w| first */
  return x->idx < y->idx ? -1 : (x->idx > y->idx); /* then lower column */
}

int orc_select(const uint16_t* w, int64_t R, int64_t C, int64_t k, uint8_t* keep) {
  if (R < 0 || C <= 0 || k < 0 || k > C) return ORC_ERR_INVALID;
  int bad = 0;
  /* rows are independent groups: each row is sorted on its own (threads
   * only split the rows among them) */
#pragma omp parallel reduction(| : bad)
  {
    keyed* order = (keyed*)malloc(sizeof(keyed) * (size_t)C);
    if (!order) bad |= 1;
#pragma omp for schedule(static)
    for (int64_t r = 0; r < R; r++) {
      if (!order) continue;
      for (int64_t j = 0; j < C; j++) {
        order[j].key = bf_key(w[r * C + j]);
        order[j].idx = j;
      }
      qsort(order, (size_t)C, sizeof(keyed), cmp_salience);
      memset(keep + r * C, 0, (size_t)C);
      for (int64_t i = 0; i < k; i++) keep[r * C + order[i].idx] = 1;
    }
    free(order);
  }
  return bad ? ORC_ERR_CAPACITY : ORC_OK;
}

/* --------------------------------------------------- exponent statistics */

int orc_histograms(const uint16_t* w, const uint8_t* keep, int64_t n,
                   uint64_t hist_kept[256], uint64_t hist_pruned[256]) {
  memset(hist_kept, 0, 256 * sizeof(uint64_t));
  memset(hist_pruned, 0, 256 * sizeof(uint64_t));
  for (int64_t i = 0; i < n; i++) {
    if (keep[i]) hist_kept[bf_e(w[i])]++;
    else hist_pruned[bf_e(w[i])]++;
  }
  return ORC_OK;
}

void orc_rank_table(const uint64_t hist[256], uint8_t perm[256]) {
  /* selection sort: the symbol of rank r is the most frequent not yet ranked,
   * smaller symbol first among equal counts */
  int used[256] = {0};
  for (int r = 0; r < 256; r++) {
    int best = -1;
    for (int s = 0; s < 256; s++) {
      if (used[s]) continue;
      if (best < 0 || hist[s] > hist[best]) best = s;
    }
    used[best] = 1;
    perm[r] = (uint8_t)best;
  }
}

/* -------------------------------------------------------------- header */

typedef struct {
  uint32_t magic, version, format, mant;
  int64_t R, C, B, k, total;
  uint32_t nsec;
  uint32_t sblocks; /* format 4: blocks per superblock (the header's u32 at byte 60) */
  int64_t off[MAX_SEC], len[MAX_SEC];
} hdr_t;

static void write_header(uint8_t* buf, const hdr_t* h) {
  memset(buf, 0, HDR_BYTES);
  put_u32(buf + 0, h->magic);
  put_u32(buf + 4, h->version);
  put_u32(buf + 8, h->format);
  put_u32(buf + 12, h->mant);
  put_u64(buf + 16, (uint64_t)h->R);
  put_u64(buf + 24, (uint64_t)h->C);
  put_u64(buf + 32, (uint64_t)h->B);
  put_u64(buf + 40, (uint64_t)h->k);
  put_u64(buf + 48, (uint64_t)h->total);
  put_u32(buf + 56, h->nsec);
  put_u32(buf + 60, h->sblocks);
  for (int s = 0; s < MAX_SEC; s++) {
    put_u64(buf + 64 + 16 * s, (uint64_t)h->off[s]);
    put_u64(buf + 72 + 16 * s, (uint64_t)h->len[s]);
  }
}

static int read_header(const uint8_t* buf, int64_t len, uint32_t magic, hdr_t* h) {
  if (!buf || len < HDR_BYTES) return ORC_ERR_CORRUPT;
  h->magic = get_u32(buf + 0);
  h->version = get_u32(buf + 4);
  h->format = get_u32(buf + 8);
  h->mant = get_u32(buf + 12);
  h->R = (int64_t)get_u64(buf + 16);
  h->C = (int64_t)get_u64(buf + 24);
  h->B = (int64_t)get_u64(buf + 32);
  h->k = (int64_t)get_u64(buf + 40);
  h->total = (int64_t)get_u64(buf + 48);
  h->nsec = get_u32(buf + 56);
  h->sblocks = get_u32(buf + 60);
  if (h->magic != magic || h->version != 1) return ORC_ERR_CORRUPT;
  if (h->format != ORC_FMT_C1 && h->format != ORC_FMT_C2 && h->format != ORC_FMT_C2T &&
      h->format != ORC_FMT_C1S)
    return ORC_ERR_CORRUPT;
  if (h->sblocks != (h->format == ORC_FMT_C1S ? ORC_SUPERBLOCK_BLOCKS : 0u)) return ORC_ERR_CORRUPT;
  if (h->mant > 7 || h->R < 0 || h->C <= 0 || h->B <= 0 || h->C % h->B || h->B % 32 ||
      h->k < 0 || h->k > h->C || h->C > 65536 || h->total > len || h->nsec > MAX_SEC)
    return ORC_ERR_CORRUPT;
  for (int s = 0; s < MAX_SEC; s++) {
    h->off[s] = (int64_t)get_u64(buf + 64 + 16 * s);
    h->len[s] = (int64_t)get_u64(buf + 72 + 16 * s);
    if (h->off[s] < 0 || h->len[s] < 0 || h->off[s] + h->len[s] > h->total)
      return ORC_ERR_CORRUPT;
  }
  return ORC_OK;
}

int orc_header(const uint8_t* buf, int64_t len, uint32_t expect_magic, int64_t out[8],
               int64_t sec_off[12], int64_t sec_len[12]) {
  hdr_t h;
  int st = read_header(buf, len, expect_magic, &h);
  if (st) return st;
  out[0] = h.format; out[1] = h.mant; out[2] = h.R; out[3] = h.C;
  out[4] = h.B; out[5] = h.k; out[6] = h.total; out[7] = h.nsec;
  for (int s = 0; s < MAX_SEC; s++) { sec_off[s] = h.off[s]; sec_len[s] = h.len[s]; }
  return ORC_OK;
}

/* Lay sections out in order after the header.  Each starts on a multiple of
 * 256 bytes and is followed by at least 16 zero bytes before the next one (or
 * the end of the stream), so that a reader fetching whole words past the last
 * bit of a section stays inside the stream. */
static int64_t layout(hdr_t* h, int nsec, const int64_t* lens) {
  int64_t pos = HDR_BYTES;
  h->nsec = (uint32_t)nsec;
  for (int s = 0; s < MAX_SEC; s++) { h->off[s] = 0; h->len[s] = 0; }
  for (int s = 0; s < nsec; s++) {
    h->off[s] = pos;
    h->len[s] = lens[s];
    pos = align256(pos + lens[s] + 16);
  }
  h->total = pos;
  return pos;
}

/* Section indices. */
enum { S1_RANK = 0, S1_BITMAP, S1_ROWBASE, S1_BLKOFF, S1_KEPTB, S1_FIELDS, S1_CODES, S1_N };
enum { V1_RANK = 0, V1_ROWBASE, V1_BLKOFF, V1_LOWMANT, V1_PRUNED, V1_CODES, V1_N };
enum { S2_BITMAP = 0, S2_SHEXP, S2_KEPTB, S2_FIELDS, S2_N };
enum { V2_RANK = 0, V2_ROWBASE_K, V2_BLKOFF_K, V2_RESID, V2_PRUNED, V2_ROWBASE_P,
       V2_BLKOFF_P, V2_CODES, V2_N };
/* format 3: the speculation stream is Cassandra-2's; the verification stream
 * holds the target's group exponents, the kept values' low 7-m bits of t and
 * the pruned values' (sign, t) in 9 bits, all at fixed positions */
enum { V3_GEXP = 0, V3_LOW, V3_PRUNED, V3_N };

/* ----------------------------------------------------- Cassandra-2 helpers */

/* Shared-exponent view of one value [MX]: eff = max(e,1) and the 8-bit
 * significand M with its hidden bit, so that |value| = M * 2^(eff-134). */
static int mx_eff(uint16_t b) { return bf_e(b) > 0 ? bf_e(b) : 1; }
static int mx_sig(uint16_t b) { return ((bf_e(b) > 0) << 7) | bf_f(b); }

/* Draft bf16 bits from (sign, aligned significand a, shared exponent E, m):
 * the value a * 2^(E-127-m), written as a bf16 pattern by normalising a. */
static uint16_t mx_draft_bits(int s, int a, int E, int m) {
  if (a == 0) return 0x0000;
  int p = 0;
  while ((a >> (p + 1)) != 0) p++; /* index of the leading one */
  int e = E - m + p;
  if (e >= 1) return (uint16_t)((s << 15) | (e << 7) | ((a << (7 - p)) & 0x7F));
  return (uint16_t)((s << 15) | (a << (E - m + 6))); /* subnormal result */
}

/* Group exponent of the target: the largest max(e,1) over 32 positions. */
static int mx_group_exp(const uint16_t* g) {
  int X = 0;
  for (int i = 0; i < 32; i++)
    if (mx_eff(g[i]) > X) X = mx_eff(g[i]);
  return X;
}

/* The value's 8-bit significand aligned to the group exponent X, chopped. */
static int mx_target_sig(uint16_t b, int X) {
  int d = X - mx_eff(b);
  return d >= 8 ? 0 : mx_sig(b) >> d;
}

int orc_mx_target(const uint16_t* w, int64_t R, int64_t C, uint16_t* out) {
  if (R < 0 || C <= 0 || C % 32 || (R > 0 && (!w || !out))) return ORC_ERR_INVALID;
  for (int64_t r = 0; r < R; r++)
    for (int64_t g = 0; g < C; g += 32) {
      const uint16_t* src = w + r * C + g;
      int X = mx_group_exp(src);
      for (int i = 0; i < 32; i++)
        out[r * C + g + i] = mx_draft_bits(bf_s(src[i]), mx_target_sig(src[i], X), X, 7);
    }
  return ORC_OK;
}

/* ------------------------------------------------------------------ encode */

int orc_encode(const uint16_t* w, int64_t R, int64_t C, int64_t k, int m, int64_t B,
               int format, uint8_t* spec, int64_t spec_cap, uint8_t* verif,
               int64_t verif_cap, int64_t* spec_bytes, int64_t* verif_bytes) {
  if (R < 0 || C <= 0 || C > 65536 || B < 32 || (B & (B - 1)) || C % B || k < 0 || k > C ||
      m < 0 || m > 7 ||
      (format != ORC_FMT_C1 && format != ORC_FMT_C2 && format != ORC_FMT_C2T && format != ORC_FMT_C1S))
    return ORC_ERR_INVALID;
  /* format 3 shares Cassandra-2's speculation stream; format 4 is Cassandra-1
   * with superblock metadata */
  const int c1 = format == ORC_FMT_C1 || format == ORC_FMT_C1S;
  const int c2 = !c1;
  const int64_t SB = ORC_SUPERBLOCK_BLOCKS, nsb = (C / B + SB - 1) / SB;
  if (R > 0 && !w) return ORC_ERR_INVALID;
  const int64_t n = R * C, nb = C / B;

  /* step 1: pruning by magnitude [R31] */
  uint8_t* keep = (uint8_t*)malloc((size_t)(n ? n : 1));
  if (!keep) return ORC_ERR_CAPACITY;
  orc_select(w, R, C, k, keep);

  /* step 3 statistics and frequency-ranked tables [R32] */
  uint64_t hk[256], hp[256];
  orc_histograms(w, keep, n, hk, hp);
  uint8_t perm_s[256], perm_v[256];
  int rank_s[256], rank_v[256];
  orc_rank_table(hk, perm_s);
  orc_rank_table(hp, perm_v);
  for (int r = 0; r < 256; r++) { rank_s[perm_s[r]] = r; rank_v[perm_v[r]] = r; }

  /* Cassandra-2: shared exponent per 32 positions over the kept values [MX] */
  uint8_t* shexp = NULL;
  if (c2) {
    shexp = (uint8_t*)calloc((size_t)(n / 32 + 1), 1);
    for (int64_t g = 0; g < n / 32; g++) {
      int E = 0;
      for (int64_t j = g * 32; j < g * 32 + 32; j++)
        if (keep[j] && mx_eff(w[j]) > E) E = mx_eff(w[j]);
      shexp[g] = (uint8_t)E;
    }
  }

  /* code lengths per row (step 3 of [R31], codes of [R32]) */
  uint64_t* sbits = (uint64_t*)calloc((size_t)R + 1, 8); /* spec unary bits per row (C-1) */
  uint64_t* vbits = (uint64_t*)calloc((size_t)R + 1, 8); /* verif pruned-exponent bits */
  uint64_t* kbits = (uint64_t*)calloc((size_t)R + 1, 8); /* C-2 kept residue bits */
  for (int64_t r = 0; r < R; r++) {
    for (int64_t j = 0; j < C; j++) {
      uint16_t b = w[r * C + j];
      if (keep[r * C + j]) {
        if (c1) {
          sbits[r] += (uint64_t)rank_s[bf_e(b)] + 1;
        } else if (format == ORC_FMT_C2) {
          int d = shexp[(r * C + j) / 32] - mx_eff(b);
          int wdt = 7 - m + d < 8 ? 7 - m + d : 8;
          kbits[r] += (uint64_t)d + 1 + (uint64_t)wdt;
        }
      } else if (format != ORC_FMT_C2T) {
        vbits[r] += (uint64_t)rank_v[bf_e(b)] + 1;
      }
    }
  }
  uint64_t stot = 0, vtot = 0, ktot = 0;
  for (int64_t r = 0; r < R; r++) { stot += sbits[r]; vtot += vbits[r]; ktot += kbits[r]; }

  hdr_t hs, hv;
  memset(&hs, 0, sizeof hs);
  memset(&hv, 0, sizeof hv);
  hs.magic = ORC_MAGIC_SPEC; hv.magic = ORC_MAGIC_VERIF;
  hs.version = hv.version = 1;
  hs.format = hv.format = (uint32_t)format;
  hs.mant = hv.mant = (uint32_t)m;
  hs.R = hv.R = R; hs.C = hv.C = C; hs.B = hv.B = B; hs.k = hv.k = k;
  if (c1) {
    int64_t ls[S1_N] = {256, n / 8, 8 * R, 4 * R * nb, 2 * R * nb,
                        (R * k * (1 + m) + 7) / 8, (int64_t)((stot + 7) / 8)};
    if (format == ORC_FMT_C1S) { /* u64 per superblock, u16 per block */
      ls[S1_ROWBASE] = 8 * R * nsb;
      ls[S1_BLKOFF] = 2 * R * nb;
      hs.sblocks = hv.sblocks = (uint32_t)SB;
    }
    int64_t lv[V1_N] = {256, 8 * R, 4 * R * nb, (R * k * (7 - m) + 7) / 8, R * (C - k),
                        (int64_t)((vtot + 7) / 8)};
    layout(&hs, S1_N, ls);
    layout(&hv, V1_N, lv);
  } else if (format == ORC_FMT_C2) {
    int64_t ls[S2_N] = {n / 8, n / 32, 2 * R * nb, (R * k * (2 + m) + 7) / 8};
    int64_t lv[V2_N] = {256, 8 * R, 4 * R * nb, (int64_t)((ktot + 7) / 8), R * (C - k),
                        8 * R, 4 * R * nb, (int64_t)((vtot + 7) / 8)};
    layout(&hs, S2_N, ls);
    layout(&hv, V2_N, lv);
  } else {
    int64_t ls[S2_N] = {n / 8, n / 32, 2 * R * nb, (R * k * (2 + m) + 7) / 8};
    int64_t lv[V3_N] = {n / 32, (R * k * (7 - m) + 7) / 8, (R * (C - k) * 9 + 7) / 8};
    layout(&hs, S2_N, ls);
    layout(&hv, V3_N, lv);
  }
  if (spec_bytes) *spec_bytes = hs.total;
  if (verif_bytes) *verif_bytes = hv.total;

  int status = ORC_OK;
  if (spec && verif) {
    if (spec_cap < hs.total || verif_cap < hv.total) {
      status = ORC_ERR_CAPACITY;
    } else {
      memset(spec, 0, (size_t)hs.total);
      memset(verif, 0, (size_t)hv.total);
      write_header(spec, &hs);
      write_header(verif, &hv);
      uint64_t sbase = 0, vbase = 0, kbase = 0, sb_base = 0;
      for (int64_t r = 0; r < R && status == ORC_OK; r++) {
        int64_t kept_i = 0, pr_i = 0;        /* kept / pruned index within the row */
        uint64_t spos = sbase, vpos = vbase, kpos = kbase;
        if (c1) {
          if (format == ORC_FMT_C1) put_u64(spec + hs.off[S1_ROWBASE] + 8 * r, sbase);
          put_u64(verif + hv.off[V1_ROWBASE] + 8 * r, vbase);
        } else if (format == ORC_FMT_C2) {
          put_u64(verif + hv.off[V2_ROWBASE_K] + 8 * r, kbase);
          put_u64(verif + hv.off[V2_ROWBASE_P] + 8 * r, vbase);
        }
        for (int64_t j = 0; j < C; j++) {
          if (j % B == 0) { /* per-block offsets and kept-before counts */
            int64_t blk = r * nb + j / B;
            if (format == ORC_FMT_C1S) {
              /* superblock of SB blocks: u64 base at its first block, u16
               * offsets from that base */
              if ((j / B) % SB == 0) {
                sb_base = spos;
                put_u64(spec + hs.off[S1_ROWBASE] + 8 * (r * nsb + (j / B) / SB), sb_base);
              }
              if (spos - sb_base > 65535) { status = ORC_ERR_OVERFLOW; break; }
              put_u16(spec + hs.off[S1_BLKOFF] + 2 * blk, (uint16_t)(spos - sb_base));
              put_u16(spec + hs.off[S1_KEPTB] + 2 * blk, (uint16_t)kept_i);
              put_u32(verif + hv.off[V1_BLKOFF] + 4 * blk, (uint32_t)(vpos - vbase));
            } else if (format == ORC_FMT_C1) {
              put_u32(spec + hs.off[S1_BLKOFF] + 4 * blk, (uint32_t)(spos - sbase));
              put_u16(spec + hs.off[S1_KEPTB] + 2 * blk, (uint16_t)kept_i);
              put_u32(verif + hv.off[V1_BLKOFF] + 4 * blk, (uint32_t)(vpos - vbase));
            } else {
              put_u16(spec + hs.off[S2_KEPTB] + 2 * blk, (uint16_t)kept_i);
              if (format == ORC_FMT_C2) {
                put_u32(verif + hv.off[V2_BLKOFF_K] + 4 * blk, (uint32_t)(kpos - kbase));
                put_u32(verif + hv.off[V2_BLKOFF_P] + 4 * blk, (uint32_t)(vpos - vbase));
              }
            }
          }
          /* format 3: the target's group exponent, once per 32 positions */
          const int X = format == ORC_FMT_C2T ? mx_group_exp(w + r * C + j / 32 * 32) : 0;
          if (format == ORC_FMT_C2T && j % 32 == 0) verif[hv.off[V3_GEXP] + (r * C + j) / 32] = (uint8_t)X;
          uint16_t b = w[r * C + j];
          int s = bf_s(b), e = bf_e(b), f = bf_f(b);
          if (keep[r * C + j]) {
            int64_t kin = r * k + kept_i; /* kept index in the tensor */
            if (c1) {
              /* step 2: top m mantissa bits with the sign to spec, the rest to verif */
              put_bits(spec + hs.off[S1_BITMAP], (uint64_t)(r * C + j), 1, 1);
              int ft = f >> (7 - m), fl = f & ((1 << (7 - m)) - 1);
              put_bits(spec + hs.off[S1_FIELDS], (uint64_t)kin * (1 + m),
                       (uint64_t)((s << m) | ft), 1 + m);
              put_unary(spec + hs.off[S1_CODES], spos, rank_s[e]);
              spos += (uint64_t)rank_s[e] + 1;
              put_bits(verif + hv.off[V1_LOWMANT], (uint64_t)kin * (7 - m), (uint64_t)fl, 7 - m);
            } else {
              put_bits(spec + hs.off[S2_BITMAP], (uint64_t)(r * C + j), 1, 1);
              int E = shexp[(r * C + j) / 32];
              int d = E - mx_eff(b), M = mx_sig(b);
              int shift = 7 - m + d;
              int a = shift >= 8 ? 0 : M >> shift;
              int wdt = shift < 8 ? shift : 8;
              put_bits(spec + hs.off[S2_FIELDS], (uint64_t)kin * (2 + m),
                       (uint64_t)((s << (m + 1)) | a), 2 + m);
              if (format == ORC_FMT_C2) {
                put_unary(verif + hv.off[V2_RESID], kpos, d);
                kpos += (uint64_t)d + 1;
                put_bits(verif + hv.off[V2_RESID], kpos, (uint64_t)(M & ((1 << wdt) - 1)), wdt);
                kpos += (uint64_t)wdt;
              } else {
                /* the target's t; its top m+1 bits are the draft's a (X == E here) */
                int t = mx_target_sig(b, X);
                put_bits(verif + hv.off[V3_LOW], (uint64_t)kin * (7 - m),
                         (uint64_t)(t & ((1 << (7 - m)) - 1)), 7 - m);
              }
            }
            kept_i++;
          } else if (format == ORC_FMT_C2T) {
            /* pruned, format 3: sign and t aligned to the group exponent */
            int64_t pin = r * (C - k) + pr_i;
            put_bits(verif + hv.off[V3_PRUNED], (uint64_t)pin * 9,
                     (uint64_t)((s << 8) | mx_target_sig(b, X)), 9);
            pr_i++;
          } else {
            /* pruned: sign and full mantissa byte plus the coded exponent to verif */
            int64_t pin = r * (C - k) + pr_i;
            int pbyte_sec = c1 ? V1_PRUNED : V2_PRUNED;
            int code_sec = c1 ? V1_CODES : V2_CODES;
            verif[hv.off[pbyte_sec] + pin] = (uint8_t)((s << 7) | f);
            put_unary(verif + hv.off[code_sec], vpos, rank_v[e]);
            vpos += (uint64_t)rank_v[e] + 1;
            pr_i++;
          }
        }
        sbase = spos; vbase = vpos; kbase = kpos;
      }
      if (c1) memcpy(spec + hs.off[S1_RANK], perm_s, 256);
      else memcpy(spec + hs.off[S2_SHEXP], shexp, (size_t)(n / 32));
      if (format != ORC_FMT_C2T)
        memcpy(verif + (c1 ? hv.off[V1_RANK] : hv.off[V2_RANK]), perm_v, 256);
    }
  }
  free(keep); free(shexp); free(sbits); free(vbits); free(kbits);
  return status;
}

/* ------------------------------------------------------------------ decode */

/* Decode row r into out[C]: the draft when verif == NULL, else the exact
 * original.  Checks the per-block offsets and counts on the way. */
static int decode_row(const uint8_t* spec, const hdr_t* hs, const uint8_t* verif,
                      const hdr_t* hv, int64_t r, uint16_t* out) {
  const int64_t C = hs->C, B = hs->B, k = hs->k, nb = C / B;
  const int m = (int)hs->mant;
  int64_t kept_i = 0, pr_i = 0;
  if (hs->format == ORC_FMT_C1 || hs->format == ORC_FMT_C1S) {
    const int sbm = hs->format == ORC_FMT_C1S;
    const int64_t SB = ORC_SUPERBLOCK_BLOCKS, nsb = (nb + SB - 1) / SB;
    uint64_t sb_base = 0;
    const uint8_t* perm_s = spec + hs->off[S1_RANK];
    const uint8_t* bm = spec + hs->off[S1_BITMAP];
    const uint8_t* fields = spec + hs->off[S1_FIELDS];
    const uint8_t* codes = spec + hs->off[S1_CODES];
    uint64_t send = (uint64_t)hs->len[S1_CODES] * 8;
    uint64_t sbase = get_u64(spec + hs->off[S1_ROWBASE] + 8 * (sbm ? r * nsb : r)), spos = sbase;
    uint64_t vbase = 0, vpos = 0, vend = 0;
    if (verif) {
      vbase = get_u64(verif + hv->off[V1_ROWBASE] + 8 * r);
      vpos = vbase;
      vend = (uint64_t)hv->len[V1_CODES] * 8;
    }
    for (int64_t j = 0; j < C; j++) {
      if (j % B == 0) {
        int64_t blk = r * nb + j / B;
        if (sbm) {
          if ((j / B) % SB == 0) {
            sb_base = get_u64(spec + hs->off[S1_ROWBASE] + 8 * (r * nsb + (j / B) / SB));
            if (sb_base != spos) return ORC_ERR_CORRUPT;
          }
          if (get_u16(spec + hs->off[S1_BLKOFF] + 2 * blk) != spos - sb_base) return ORC_ERR_CORRUPT;
        } else if (get_u32(spec + hs->off[S1_BLKOFF] + 4 * blk) != spos - sbase) {
          return ORC_ERR_CORRUPT;
        }
        if (get_u16(spec + hs->off[S1_KEPTB] + 2 * blk) != (uint16_t)kept_i) return ORC_ERR_CORRUPT;
        if (verif && get_u32(verif + hv->off[V1_BLKOFF] + 4 * blk) != vpos - vbase)
          return ORC_ERR_CORRUPT;
      }
      if (get_bits(bm, (uint64_t)(r * C + j), 1)) {
        if (kept_i >= k) return ORC_ERR_CORRUPT;
        int64_t kin = r * k + kept_i;
        int field = (int)get_bits(fields, (uint64_t)kin * (1 + m), 1 + m);
        int rank = get_unary(codes, spos, send);
        if (rank < 0) return ORC_ERR_CORRUPT;
        spos += (uint64_t)rank + 1;
        int s = field >> m, ft = field & ((1 << m) - 1), e = perm_s[rank];
        uint16_t d = (uint16_t)((s << 15) | (e << 7) | (ft << (7 - m)));
        if (verif) {
          int fl = (int)get_bits(verif + hv->off[V1_LOWMANT], (uint64_t)kin * (7 - m), 7 - m);
          d |= (uint16_t)fl;
        }
        out[j] = d;
        kept_i++;
      } else {
        if (verif) {
          if (pr_i >= C - k) return ORC_ERR_CORRUPT;
          int byte = verif[hv->off[V1_PRUNED] + r * (C - k) + pr_i];
          int rank = get_unary(verif + hv->off[V1_CODES], vpos, vend);
          if (rank < 0) return ORC_ERR_CORRUPT;
          vpos += (uint64_t)rank + 1;
          int e = verif[hv->off[V1_RANK] + rank];
          out[j] = (uint16_t)(((byte >> 7) << 15) | (e << 7) | (byte & 0x7F));
        } else {
          out[j] = 0x0000; /* zero fill [R31] */
        }
        pr_i++;
      }
    }
    if (kept_i != k) return ORC_ERR_CORRUPT;
    if (r + 1 < hs->R && get_u64(spec + hs->off[S1_ROWBASE] + 8 * (sbm ? (r + 1) * nsb : r + 1)) != spos)
      return ORC_ERR_CORRUPT;
    if (verif && r + 1 < hs->R && get_u64(verif + hv->off[V1_ROWBASE] + 8 * (r + 1)) != vpos)
      return ORC_ERR_CORRUPT;
    return ORC_OK;
  }
  /* Cassandra-2 */
  const uint8_t* bm = spec + hs->off[S2_BITMAP];
  const uint8_t* shexp = spec + hs->off[S2_SHEXP];
  const uint8_t* fields = spec + hs->off[S2_FIELDS];
  const int c2t = hs->format == ORC_FMT_C2T;
  uint64_t kbase = 0, kpos = 0, kend = 0, vbase = 0, vpos = 0, vend = 0;
  if (verif && !c2t) {
    kbase = get_u64(verif + hv->off[V2_ROWBASE_K] + 8 * r);
    vbase = get_u64(verif + hv->off[V2_ROWBASE_P] + 8 * r);
    kpos = kbase; vpos = vbase;
    kend = (uint64_t)hv->len[V2_RESID] * 8;
    vend = (uint64_t)hv->len[V2_CODES] * 8;
  }
  for (int64_t j = 0; j < C; j++) {
    if (j % B == 0) {
      int64_t blk = r * nb + j / B;
      if (get_u16(spec + hs->off[S2_KEPTB] + 2 * blk) != (uint16_t)kept_i) return ORC_ERR_CORRUPT;
      if (verif && !c2t && (get_u32(verif + hv->off[V2_BLKOFF_K] + 4 * blk) != kpos - kbase ||
                            get_u32(verif + hv->off[V2_BLKOFF_P] + 4 * blk) != vpos - vbase))
        return ORC_ERR_CORRUPT;
    }
    /* format 3: the target's group exponent (at least 1 in a valid stream) */
    const int X = verif && c2t ? verif[hv->off[V3_GEXP] + (r * C + j) / 32] : 0;
    if (verif && c2t && X < 1) return ORC_ERR_CORRUPT;
    if (get_bits(bm, (uint64_t)(r * C + j), 1)) {
      if (kept_i >= k) return ORC_ERR_CORRUPT;
      int64_t kin = r * k + kept_i;
      int field = (int)get_bits(fields, (uint64_t)kin * (2 + m), 2 + m);
      int s = field >> (m + 1), a = field & ((1 << (m + 1)) - 1);
      int E = shexp[(r * C + j) / 32];
      if (!verif) {
        out[j] = mx_draft_bits(s, a, E, m);
      } else if (c2t) {
        /* t = the draft's a followed by the 7-m low bits; X equals E where
         * the group keeps anything */
        if (X != E) return ORC_ERR_CORRUPT;
        int low = (int)get_bits(verif + hv->off[V3_LOW], (uint64_t)kin * (7 - m), 7 - m);
        out[j] = mx_draft_bits(s, (a << (7 - m)) | low, X, 7);
      } else {
        int d = get_unary(verif + hv->off[V2_RESID], kpos, kend);
        if (d < 0) return ORC_ERR_CORRUPT;
        kpos += (uint64_t)d + 1;
        int wdt = 7 - m + d < 8 ? 7 - m + d : 8;
        if (kpos + (uint64_t)wdt > kend) return ORC_ERR_CORRUPT;
        int L = (int)get_bits(verif + hv->off[V2_RESID], kpos, wdt);
        kpos += (uint64_t)wdt;
        int M = wdt < 8 ? (a << wdt) | L : L;
        int e = M >= 128 ? E - d : 0;
        if (e < 0 || M > 255) return ORC_ERR_CORRUPT;
        out[j] = (uint16_t)((s << 15) | (e << 7) | (M & 0x7F));
      }
      kept_i++;
    } else {
      if (verif && c2t) {
        if (pr_i >= C - k) return ORC_ERR_CORRUPT;
        int v = (int)get_bits(verif + hv->off[V3_PRUNED], (uint64_t)(r * (C - k) + pr_i) * 9, 9);
        out[j] = mx_draft_bits(v >> 8, v & 0xFF, X, 7);
      } else if (verif) {
        if (pr_i >= C - k) return ORC_ERR_CORRUPT;
        int byte = verif[hv->off[V2_PRUNED] + r * (C - k) + pr_i];
        int rank = get_unary(verif + hv->off[V2_CODES], vpos, vend);
        if (rank < 0) return ORC_ERR_CORRUPT;
        vpos += (uint64_t)rank + 1;
        int e = verif[hv->off[V2_RANK] + rank];
        out[j] = (uint16_t)(((byte >> 7) << 15) | (e << 7) | (byte & 0x7F));
      } else {
        out[j] = 0x0000;
      }
      pr_i++;
    }
  }
  if (kept_i != k) return ORC_ERR_CORRUPT;
  return ORC_OK;
}

static int open_pair(const uint8_t* spec, int64_t spec_len, const uint8_t* verif,
                     int64_t verif_len, hdr_t* hs, hdr_t* hv) {
  int st = read_header(spec, spec_len, ORC_MAGIC_SPEC, hs);
  if (st) return st;
  if (verif) {
    st = read_header(verif, verif_len, ORC_MAGIC_VERIF, hv);
    if (st) return st;
    if (hv->format != hs->format || hv->mant != hs->mant || hv->R != hs->R ||
        hv->C != hs->C || hv->B != hs->B || hv->k != hs->k)
      return ORC_ERR_CORRUPT;
  }
  return ORC_OK;
}

int orc_draft_decode(const uint8_t* spec, int64_t spec_len, uint16_t* out) {
  hdr_t hs;
  int st = open_pair(spec, spec_len, NULL, 0, &hs, NULL);
  if (st) return st;
  for (int64_t r = 0; r < hs.R; r++) {
    st = decode_row(spec, &hs, NULL, NULL, r, out + r * hs.C);
    if (st) return st;
  }
  return ORC_OK;
}

int orc_reconstruct(const uint8_t* spec, int64_t spec_len, const uint8_t* verif,
                    int64_t verif_len, uint16_t* out) {
  hdr_t hs, hv;
  if (!verif) return ORC_ERR_INVALID;
  int st = open_pair(spec, spec_len, verif, verif_len, &hs, &hv);
  if (st) return st;
  for (int64_t r = 0; r < hs.R; r++) {
    st = decode_row(spec, &hs, verif, &hv, r, out + r * hs.C);
    if (st) return st;
  }
  return ORC_OK;
}

/* Draft product (verif == NULL) [R31: the draft runs full-size products on
 * the zero-filled weights] or verification product on the exact weights. */
int orc_product(const uint8_t* spec, int64_t spec_len, const uint8_t* verif,
                int64_t verif_len, const uint16_t* x, int64_t ntok, double* y,
                double* absy, int threads) {
  hdr_t hs, hv;
  int st = open_pair(spec, spec_len, verif, verif_len, &hs, &hv);
  if (st) return st;
  if (ntok < 0 || (ntok > 0 && (!x || !y))) return ORC_ERR_INVALID;
  const int64_t R = hs.R, C = hs.C;
  int bad = 0;
  (void)threads;
#pragma omp parallel for schedule(dynamic, 16) num_threads(threads > 0 ? threads : 1) reduction(| : bad)
  for (int64_t r = 0; r < R; r++) {
    uint16_t* row = (uint16_t*)malloc((size_t)C * sizeof(uint16_t));
    int s = row ? decode_row(spec, &hs, verif, verif ? &hv : NULL, r, row) : ORC_ERR_CAPACITY;
    if (s) { bad |= 1; free(row); continue; }
    for (int64_t t = 0; t < ntok; t++) {
      double acc = 0.0, aacc = 0.0;
      for (int64_t j = 0; j < C; j++) {
        double wv = bf16_to_double(row[j]);
        double xv = bf16_to_double(x[t * C + j]);
        acc += wv * xv;
        aacc += fabs(wv) * fabs(xv);
      }
      y[t * R + r] = acc;
      if (absy) absy[t * R + r] = aacc;
    }
    free(row);
  }
  return bad ? ORC_ERR_CORRUPT : ORC_OK;
}

/* The same product restricted to the listed rows: y[t][i] and absy[t][i] for
 * row rows[i] (used to check single outputs of very large tensors). */
int orc_product_rows(const uint8_t* spec, int64_t spec_len, const uint8_t* verif,
                     int64_t verif_len, const uint16_t* x, int64_t ntok, const int64_t* rows,
                     int64_t nrows, double* y, double* absy) {
  hdr_t hs, hv;
  int st = open_pair(spec, spec_len, verif, verif_len, &hs, &hv);
  if (st) return st;
  const int64_t C = hs.C;
  uint16_t* row = (uint16_t*)malloc((size_t)C * sizeof(uint16_t));
  if (!row) return ORC_ERR_CAPACITY;
  for (int64_t i = 0; i < nrows; i++) {
    if (rows[i] < 0 || rows[i] >= hs.R) { free(row); return ORC_ERR_INVALID; }
    st = decode_row(spec, &hs, verif, verif ? &hv : NULL, rows[i], row);
    if (st) { free(row); return st; }
    for (int64_t t = 0; t < ntok; t++) {
      double acc = 0.0, aacc = 0.0;
      for (int64_t j = 0; j < C; j++) {
        double wv = bf16_to_double(row[j]);
        double xv = bf16_to_double(x[t * C + j]);
        acc += wv * xv;
        aacc += fabs(wv) * fabs(xv);
      }
      y[t * nrows + i] = acc;
      absy[t * nrows + i] = aacc;
    }
  }
  free(row);
  return ORC_OK;
}

/* ---------------------------------------------------------------- KV cache */
/* [R31] the KV cache goes through the same value pruning, mantissa truncation
 * and exponent coding as the weights; [R33] (Cassandra review, section 3.3):
 * KV entries are produced during inference, so the encoder runs online, one
 * append at a time.  Group = one token's vector of one head; the rank tables
 * are those of the first append (a reading: the pages do not say how an
 * online encoder picks its table). */

static int64_t kv_part(int64_t* pos, int64_t bytes) {
  const int64_t o = *pos;
  *pos = align256(*pos + bytes + 16);
  return o;
}

int orc_kv_layout(int fmt, int64_t D, int64_t k, int m, int64_t T_max, int64_t code_cap,
                  int64_t vcode_cap, int64_t spec_off[5], int64_t verif_off[5],
                  int64_t* spec_bytes, int64_t* verif_bytes) {
  if ((fmt != ORC_FMT_C1 && fmt != ORC_FMT_C2) || D <= 0 || D % 32 || D > 65536 || k < 0 ||
      k > D || m < 0 || m > 7 || T_max < 0 || code_cap < 0 || vcode_cap < 0 ||
      code_cap >= ((int64_t)1 << 32) || vcode_cap >= ((int64_t)1 << 32))
    return ORC_ERR_INVALID;
  int64_t p = 0;
  spec_off[0] = kv_part(&p, 256);
  spec_off[1] = kv_part(&p, T_max * D / 8);
  if (fmt == ORC_FMT_C1) {
    spec_off[2] = kv_part(&p, 4 * T_max);
    spec_off[3] = kv_part(&p, (T_max * k * (1 + m) + 7) / 8);
    spec_off[4] = kv_part(&p, (code_cap + 7) / 8);
  } else {
    spec_off[2] = kv_part(&p, T_max * D / 32);               /* shared exponents */
    spec_off[3] = kv_part(&p, (T_max * k * (2 + m) + 7) / 8); /* sign + aligned significand */
    spec_off[4] = kv_part(&p, 0);
  }
  *spec_bytes = p;
  p = 0;
  verif_off[0] = kv_part(&p, 256);
  if (fmt == ORC_FMT_C1)
    verif_off[1] = kv_part(&p, (T_max * k * (7 - m) + 7) / 8);
  else
    verif_off[1] = kv_part(&p, (code_cap + 7) / 8);          /* kept residues */
  verif_off[2] = kv_part(&p, T_max * (D - k));
  verif_off[3] = kv_part(&p, (fmt == ORC_FMT_C1 ? 4 : 8) * T_max);
  verif_off[4] = kv_part(&p, (vcode_cap + 7) / 8);
  *verif_bytes = p;
  return ORC_OK;
}

int orc_kv_encode(int fmt, const uint16_t* vec, int64_t T, int64_t T0, int64_t D, int64_t k,
                  int m, int64_t T_max, int64_t code_cap, int64_t vcode_cap, uint8_t* spec,
                  uint8_t* verif, uint64_t tails[2]) {
  int64_t so[5], vo[5], sb, vb;
  int st = orc_kv_layout(fmt, D, k, m, T_max, code_cap, vcode_cap, so, vo, &sb, &vb);
  if (st) return st;
  if (T < 0 || T > T_max || (T > 0 && (T0 < 1 || T0 > T))) return ORC_ERR_INVALID;
  memset(spec, 0, (size_t)sb);
  memset(verif, 0, (size_t)vb);
  uint8_t* keep = (uint8_t*)malloc((size_t)(T * D + 1));
  if (!keep) return ORC_ERR_CAPACITY;
  orc_select(vec, T, D, k, keep);  /* pruning per token vector */
  uint64_t hk[256], hp[256];
  uint8_t perm_s[256], perm_v[256];
  int rank_s[256], rank_v[256];
  orc_histograms(vec, keep, T0 * D, hk, hp);  /* the first append's exponents */
  orc_rank_table(hk, perm_s);
  orc_rank_table(hp, perm_v);
  for (int r = 0; r < 256; r++) { rank_s[perm_s[r]] = r; rank_v[perm_v[r]] = r; }
  if (fmt == ORC_FMT_C1) memcpy(spec + so[0], perm_s, 256);
  memcpy(verif + vo[0], perm_v, 256);
  uint64_t stail = 0, vtail = 0;  /* C-2: stail counts residue bits */
  for (int64_t t = 0; t < T; t++) {
    if (fmt == ORC_FMT_C1) {
      put_u32(spec + so[2] + 4 * t, (uint32_t)stail);
      put_u32(verif + vo[3] + 4 * t, (uint32_t)vtail);
    } else {
      put_u32(verif + vo[3] + 8 * t, (uint32_t)stail);
      put_u32(verif + vo[3] + 8 * t + 4, (uint32_t)vtail);
      /* shared exponent of each 32 positions: the largest max(e,1) over the
       * kept values, 0 when none is kept [MX] */
      for (int64_t g = 0; g < D / 32; g++) {
        int E = 0;
        for (int64_t j = g * 32; j < g * 32 + 32; j++)
          if (keep[t * D + j] && mx_eff(vec[t * D + j]) > E) E = mx_eff(vec[t * D + j]);
        spec[so[2] + t * (D / 32) + g] = (uint8_t)E;
      }
    }
    int64_t kept_i = 0, pr_i = 0;
    for (int64_t j = 0; j < D; j++) {
      uint16_t b = vec[t * D + j];
      int s = bf_s(b), e = bf_e(b), f = bf_f(b);
      if (keep[t * D + j]) {
        int64_t kin = t * k + kept_i;
        put_bits(spec + so[1], (uint64_t)(t * D + j), 1, 1);
        if (fmt == ORC_FMT_C1) {
          put_bits(spec + so[3], (uint64_t)kin * (1 + m), (uint64_t)((s << m) | (f >> (7 - m))), 1 + m);
          if (stail + (uint64_t)rank_s[e] + 1 > (uint64_t)code_cap) { free(keep); return ORC_ERR_CAPACITY; }
          put_unary(spec + so[4], stail, rank_s[e]);
          stail += (uint64_t)rank_s[e] + 1;
          put_bits(verif + vo[1], (uint64_t)kin * (7 - m), (uint64_t)(f & ((1 << (7 - m)) - 1)), 7 - m);
        } else {
          const int E = spec[so[2] + t * (D / 32) + j / 32];
          const int d = E - mx_eff(b), M = mx_sig(b), shift = 7 - m + d;
          const int a = shift >= 8 ? 0 : M >> shift, wdt = shift < 8 ? shift : 8;
          put_bits(spec + so[3], (uint64_t)kin * (2 + m), (uint64_t)((s << (m + 1)) | a), 2 + m);
          if (stail + (uint64_t)d + 1 + (uint64_t)wdt > (uint64_t)code_cap) { free(keep); return ORC_ERR_CAPACITY; }
          put_unary(verif + vo[1], stail, d);
          stail += (uint64_t)d + 1;
          put_bits(verif + vo[1], stail, (uint64_t)(M & ((1 << wdt) - 1)), wdt);
          stail += (uint64_t)wdt;
        }
        kept_i++;
      } else {
        verif[vo[2] + t * (D - k) + pr_i] = (uint8_t)((s << 7) | f);
        if (vtail + (uint64_t)rank_v[e] + 1 > (uint64_t)vcode_cap) { free(keep); return ORC_ERR_CAPACITY; }
        put_unary(verif + vo[4], vtail, rank_v[e]);
        vtail += (uint64_t)rank_v[e] + 1;
        pr_i++;
      }
    }
  }
  tails[0] = stail;
  tails[1] = vtail;
  free(keep);
  return ORC_OK;
}

int orc_kv_decode(int fmt, const uint8_t* spec, const uint8_t* verif, int64_t T, int64_t D,
                  int64_t k, int m, int64_t T_max, int64_t code_cap, int64_t vcode_cap,
                  uint16_t* out) {
  int64_t so[5], vo[5], sb, vb;
  int st = orc_kv_layout(fmt, D, k, m, T_max, code_cap, vcode_cap, so, vo, &sb, &vb);
  if (st) return st;
  if (T < 0 || T > T_max) return ORC_ERR_INVALID;
  for (int64_t t = 0; t < T; t++) {
    uint64_t spos, vpos = 0;
    if (fmt == ORC_FMT_C1) {
      spos = get_u32(spec + so[2] + 4 * t);
      if (verif) vpos = get_u32(verif + vo[3] + 4 * t);
    } else {
      spos = verif ? get_u32(verif + vo[3] + 8 * t) : 0;
      if (verif) vpos = get_u32(verif + vo[3] + 8 * t + 4);
    }
    int64_t kept_i = 0, pr_i = 0;
    for (int64_t j = 0; j < D; j++) {
      if (get_bits(spec + so[1], (uint64_t)(t * D + j), 1)) {
        if (kept_i >= k) return ORC_ERR_CORRUPT;
        int64_t kin = t * k + kept_i;
        if (fmt == ORC_FMT_C1) {
          int field = (int)get_bits(spec + so[3], (uint64_t)kin * (1 + m), 1 + m);
          int rank = get_unary(spec + so[4], spos, (uint64_t)code_cap);
          if (rank < 0) return ORC_ERR_CORRUPT;
          spos += (uint64_t)rank + 1;
          int s = field >> m, ft = field & ((1 << m) - 1), e = spec[so[0] + rank];
          uint16_t d = (uint16_t)((s << 15) | (e << 7) | (ft << (7 - m)));
          if (verif) d |= (uint16_t)get_bits(verif + vo[1], (uint64_t)kin * (7 - m), 7 - m);
          out[t * D + j] = d;
        } else {
          int field = (int)get_bits(spec + so[3], (uint64_t)kin * (2 + m), 2 + m);
          int s = field >> (m + 1), a = field & ((2 << m) - 1);
          int E = spec[so[2] + t * (D / 32) + j / 32];
          if (!verif) {
            out[t * D + j] = mx_draft_bits(s, a, E, m);
          } else {
            int d = get_unary(verif + vo[1], spos, (uint64_t)code_cap);
            if (d < 0) return ORC_ERR_CORRUPT;
            spos += (uint64_t)d + 1;
            int wdt = 7 - m + d < 8 ? 7 - m + d : 8;
            int L = (int)get_bits(verif + vo[1], spos, wdt);
            spos += (uint64_t)wdt;
            int M = wdt < 8 ? ((a << wdt) | L) : L;
            int e = M >= 128 ? E - d : 0;
            out[t * D + j] = (uint16_t)((s << 15) | ((e & 0xFF) << 7) | (M & 0x7F));
          }
        }
        kept_i++;
      } else {
        if (verif) {
          int byte = verif[vo[2] + t * (D - k) + pr_i];
          int rank = get_unary(verif + vo[4], vpos, (uint64_t)vcode_cap);
          if (rank < 0) return ORC_ERR_CORRUPT;
          vpos += (uint64_t)rank + 1;
          int e = verif[vo[0] + rank];
          out[t * D + j] = (uint16_t)(((byte >> 7) << 15) | (e << 7) | (byte & 0x7F));
        } else {
          out[t * D + j] = 0x0000;
        }
        pr_i++;
      }
    }
    if (kept_i != k) return ORC_ERR_CORRUPT;
  }
  return ORC_OK;
}

/* Attention as defined: softmax of scaled dot products, then the weighted sum
 * of values; the draft runs it on the zero-filled KV, the target on the exact
 * KV (Cassandra review, sections 3.1 and 1). */
int orc_attention(const uint16_t* q, int64_t nq, const uint16_t* K, const uint16_t* V,
                  int64_t T, int64_t D, double scale, const int64_t* visible, double* out) {
  double* s = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
  if (!s) return ORC_ERR_CAPACITY;
  for (int64_t i = 0; i < nq; i++) {
    const int64_t n = visible ? visible[i] : T;
    if (n < 1 || n > T) { free(s); return ORC_ERR_INVALID; }
    double mx = -INFINITY;
    for (int64_t t = 0; t < n; t++) {
      double acc = 0.0;
      for (int64_t d = 0; d < D; d++)
        acc += bf16_to_double(q[i * D + d]) * bf16_to_double(K[t * D + d]);
      s[t] = scale * acc;
      if (s[t] > mx) mx = s[t];
    }
    double sum = 0.0;
    for (int64_t t = 0; t < n; t++) {
      s[t] = exp(s[t] - mx);
      sum += s[t];
    }
    for (int64_t d = 0; d < D; d++) {
      double acc = 0.0;
      for (int64_t t = 0; t < n; t++) acc += s[t] * bf16_to_double(V[t * D + d]);
      out[i * D + d] = acc / sum;
    }
  }
  free(s);
  return ORC_OK;
}

/* ------------------------------------------- comparison exponent codes */

/* [R32] also weighs Huffman codes against the unary code: Huffman codes are a
 * little shorter but are parsed serially, by bit or through a table of 2^N
 * entries (N = the longest code), while unary codes can be split anywhere by
 * counting ones.  These functions build both as prefix codes so the two can be
 * compared on the same exponent sequences. */

/* Length-limited Huffman code lengths by package-merge (Larmore and
 * Hirschberg's coin-collector formulation): at each of max_len levels the
 * list holds the leaves and the pairs formed from the previous level's list,
 * in weight order; a leaf's code length is the number of times it occurs in
 * the first 2n-2 items of the last list.  Order among equal weights: leaves
 * before packages, leaves by (count, symbol), packages in the order formed. */
typedef struct {
  uint64_t w;
  int leaf;           /* leaf index, or -1 for a package */
  uint16_t* mult;     /* occurrences of each leaf inside the item */
} pm_item;

int orc_huffman_lengths(const uint64_t hist[256], int max_len, uint8_t len[256]) {
  if (max_len < 1 || max_len > 32) return ORC_ERR_INVALID;
  memset(len, 0, 256);
  int sym[256], n = 0;
  for (int s = 0; s < 256; s++)
    if (hist[s]) sym[n++] = s;
  if (n == 0) return ORC_OK;
  if (n == 1) { len[sym[0]] = 1; return ORC_OK; }
  if (max_len < 32 && ((int64_t)1 << max_len) < n) return ORC_ERR_INVALID;
  /* leaves by (count, symbol) ascending: insertion sort */
  for (int i = 1; i < n; i++) {
    int s = sym[i], j = i - 1;
    while (j >= 0 && (hist[sym[j]] > hist[s] || (hist[sym[j]] == hist[s] && sym[j] > s))) {
      sym[j + 1] = sym[j];
      j--;
    }
    sym[j + 1] = s;
  }
  const int cap = 2 * n + 2;
  pm_item* cur = (pm_item*)calloc((size_t)cap, sizeof(pm_item));
  pm_item* nxt = (pm_item*)calloc((size_t)cap, sizeof(pm_item));
  uint16_t* pool_a = (uint16_t*)calloc((size_t)cap * n, sizeof(uint16_t));
  uint16_t* pool_b = (uint16_t*)calloc((size_t)cap * n, sizeof(uint16_t));
  if (!cur || !nxt || !pool_a || !pool_b) {
    free(cur); free(nxt); free(pool_a); free(pool_b);
    return ORC_ERR_CAPACITY;
  }
  for (int i = 0; i < cap; i++) { cur[i].mult = pool_a + (size_t)i * n; nxt[i].mult = pool_b + (size_t)i * n; }
  /* deepest level: the leaves alone */
  int ncur = n;
  for (int i = 0; i < n; i++) {
    cur[i].w = hist[sym[i]];
    cur[i].leaf = i;
    memset(cur[i].mult, 0, (size_t)n * sizeof(uint16_t));
    cur[i].mult[i] = 1;
  }
  for (int level = max_len - 1; level >= 1; level--) {
    /* packages: adjacent pairs of the current list */
    int npk = ncur / 2, li = 0, pi = 0, nn = 0;
    while (li < n || pi < npk) {
      int take_leaf;
      if (li >= n) take_leaf = 0;
      else if (pi >= npk) take_leaf = 1;
      else take_leaf = hist[sym[li]] <= cur[2 * pi].w + cur[2 * pi + 1].w;
      pm_item* it = &nxt[nn++];
      if (take_leaf) {
        it->w = hist[sym[li]];
        it->leaf = li;
        memset(it->mult, 0, (size_t)n * sizeof(uint16_t));
        it->mult[li] = 1;
        li++;
      } else {
        const pm_item* a = &cur[2 * pi];
        const pm_item* b = &cur[2 * pi + 1];
        it->w = a->w + b->w;
        it->leaf = -1;
        for (int i = 0; i < n; i++) it->mult[i] = (uint16_t)(a->mult[i] + b->mult[i]);
        pi++;
      }
    }
    pm_item* t = cur; cur = nxt; nxt = t;
    uint16_t* tp = pool_a; pool_a = pool_b; pool_b = tp;
    ncur = nn;
  }
  /* code lengths: occurrences in the first 2n-2 items */
  for (int i = 0; i < 2 * n - 2 && i < ncur; i++)
    for (int j = 0; j < n; j++) len[sym[j]] = (uint8_t)(len[sym[j]] + cur[i].mult[j]);
  free(cur); free(nxt); free(pool_a); free(pool_b);
  return ORC_OK;
}

/* Canonical code values from lengths: symbols ordered by (length, symbol),
 * each code the previous one plus one, shifted left when the length grows. */
int orc_canonical_codes(const uint8_t len[256], uint32_t code[256]) {
  memset(code, 0, 256 * sizeof(uint32_t));
  uint32_t c = 0;
  int prev = 0, first = 1;
  for (int l = 1; l <= 32; l++)
    for (int s = 0; s < 256; s++) {
      if (len[s] != l) continue;
      if (first) { c = 0; first = 0; }
      else c = (c + 1) << (l - prev);
      prev = l;
      code[s] = c;
    }
  return ORC_OK;
}

/* Cassandra-1's frequency-ranked unary code as a prefix code: rank r is r
 * zeros then a one (in stream order), i.e. length r+1 and value 1. */
int orc_unary_code(const uint64_t hist[256], uint8_t len[256], uint32_t code[256]) {
  uint8_t perm[256];
  orc_rank_table(hist, perm);
  for (int r = 0; r < 256; r++) {
    len[perm[r]] = (uint8_t)(r + 1 > 255 ? 255 : r + 1);
    code[perm[r]] = 1;
  }
  return ORC_OK;
}

/* Concatenate the codes of sym[0..n) (most significant code bit first, in
 * stream bit order); blkoff[b] = bit offset of symbol b*block.  The stream
 * must be zeroed.  *bits receives the total length. */
int orc_prefix_encode(const uint8_t* sym, int64_t n, int64_t block, const uint8_t len[256],
                      const uint32_t code[256], uint8_t* stream, int64_t cap_bytes,
                      uint32_t* blkoff, int64_t* bits) {
  if (n < 0 || block < 1) return ORC_ERR_INVALID;
  uint64_t pos = 0;
  for (int64_t i = 0; i < n; i++) {
    int l = len[sym[i]];
    if (l == 0 || l > 32) return ORC_ERR_INVALID;
    if (i % block == 0 && blkoff) blkoff[i / block] = (uint32_t)pos;
    for (int j = l - 1; j >= 0; j--) {
      if (stream) {
        if ((int64_t)(pos >> 3) >= cap_bytes) return ORC_ERR_CAPACITY;
        if ((code[sym[i]] >> j) & 1) stream[pos >> 3] |= (uint8_t)(1u << (pos & 7));
      }
      pos++;
    }
  }
  if (bits) *bits = (int64_t)pos;
  return ORC_OK;
}

/* Decode n symbols bit by bit: extend the code one bit at a time and stop at
 * the first (length, value) pair some symbol owns. */
int orc_prefix_decode(const uint8_t* stream, int64_t bytes, int64_t n, const uint8_t len[256],
                      const uint32_t code[256], uint8_t* out) {
  uint64_t pos = 0;
  for (int64_t i = 0; i < n; i++) {
    uint32_t c = 0;
    int found = -1;
    for (int l = 1; l <= 32 && found < 0; l++) {
      if ((int64_t)(pos >> 3) >= bytes) return ORC_ERR_CORRUPT;
      c = (c << 1) | ((stream[pos >> 3] >> (pos & 7)) & 1u);
      pos++;
      for (int s = 0; s < 256; s++)
        if (len[s] == l && code[s] == c) { found = s; break; }
    }
    if (found < 0) return ORC_ERR_CORRUPT;
    out[i] = (uint8_t)found;
  }
  return ORC_OK;
}
