/*
 * CPU oracle for the Cassandra bit-level weight format -- TEST INFRASTRUCTURE.
 *
 * A plain, slow, scalar C implementation of what the format and the draft /
 * verify products compute.  Only tests, the smoke check and the CPU-baseline
 * leg of the benchmark may call it; the HIP library never does, and the two
 * share no code.  Every function follows the method's steps in the order the
 * pages give them:
 *   pruning -> mantissa truncation -> exponent coding, producing a
 *   speculation stream and a verification stream
 *   (Cassandra review, marsggbo.github.io, section 3.1 "从 bit 里抠 draft model";
 *    exponent coding: section 3.2, Cassandra-1 unary code and Cassandra-2 MX).
 *
 * Byte layout of a stream (written out here independently of the library):
 *   [0,256)  header: u32 magic, u32 version(=1), u32 format, u32 mant_bits,
 *            i64 rows, i64 cols, i64 block, i64 keep, i64 total_bytes,
 *            u32 n_sections, u32 reserved, then 12 x {i64 offset, i64 bytes}.
 *   sections follow in a fixed order, each starting at a multiple of 256 B;
 *   padding bytes and pad bits are zero.  Bit i of a bit section is bit (i&7)
 *   of byte i>>3 (least significant bit first).
 *
 * Status codes match the library's public ones by value.
 */
#ifndef CASS_ORACLE_H
#define CASS_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_OK = 0, ORC_ERR_INVALID = 1, ORC_ERR_UNSUPPORTED = 2, ORC_ERR_OVERFLOW = 3,
       ORC_ERR_CORRUPT = 4, ORC_ERR_CAPACITY = 5 };
enum { ORC_FMT_C1 = 1, ORC_FMT_C2 = 2, ORC_FMT_C2T = 3, ORC_FMT_C1S = 4 };
/* Format 4, Cassandra-1 with superblock metadata (pith.science review,
 * Figure 11: superblock-based data management): the speculation stream's
 * row bases and u32 block offsets give way to a u64 code base per
 * superblock of ORC_SUPERBLOCK_BLOCKS blocks of a row (the last one of a row
 * may be shorter; superblock j of row r at entry r*ceil(nb/16)+j of section 2)
 * and u16 block offsets from their superblock's base (section 3).  Everything
 * else is Cassandra-1's.  Encoding fails with ORC_ERR_OVERFLOW when a block
 * starts 2^16 or more code bits after its superblock's base.  Both headers
 * hold ORC_SUPERBLOCK_BLOCKS in the u32 at byte 60 (0 in other formats). */
#define ORC_SUPERBLOCK_BLOCKS 16

#define ORC_MAGIC_SPEC  0x50535343u /* "CSSP" */
#define ORC_MAGIC_VERIF 0x46565343u /* "CSVF" */

/* --- individual steps, exposed so tests can pin them one by one --- */

/* Step 1, pruning: per row of C values keep exactly k, ordered by |w| (the 15
 * magnitude bits) descending, ties to the lower column.  keep[r*C+j] = 0/1. */
int orc_select(const uint16_t* w, int64_t R, int64_t C, int64_t k, uint8_t* keep);

/* Exponent histograms: hist_kept[e] over kept values, hist_pruned[e] over the rest. */
int orc_histograms(const uint16_t* w, const uint8_t* keep, int64_t n,
                   uint64_t hist_kept[256], uint64_t hist_pruned[256]);

/* Frequency ranking: perm[r] = symbol of rank r, symbols ordered by count
 * descending, ties (and absent symbols) by symbol ascending. */
void orc_rank_table(const uint64_t hist[256], uint8_t perm[256]);

/* Cassandra-2 with an MX-quantised target (format 3, the reading in which the
 * "slight loss" of Cassandra-2 reaches the target too): the target weights of
 * w[R][C].  Per group of 32 positions of a row, X = the largest max(e,1) over
 * all 32 values; each value keeps its sign and the top bits of its 8-bit
 * significand M (hidden bit included) aligned to X, t = M >> (X - max(e,1))
 * (0 when the shift reaches 8), i.e. the value t * 2^(X-134) written as a bf16
 * pattern (+0 when t = 0).  Chopping, never rounding, as the draft does. */
int orc_mx_target(const uint16_t* w, int64_t R, int64_t C, uint16_t* out);

/* --- Cassandra-1 (unary exponents, lossless) and Cassandra-2 (MX-32) --- */

/* Encode w[R][C] (bf16 bit patterns).  With spec == NULL (or verif == NULL)
 * only the sizes are returned.  Returns a status code. */
int orc_encode(const uint16_t* w, int64_t R, int64_t C, int64_t k, int m, int64_t B,
               int format, uint8_t* spec, int64_t spec_cap, uint8_t* verif,
               int64_t verif_cap, int64_t* spec_bytes, int64_t* verif_bytes);

/* Zero-filled draft weights from the speculation stream alone: out[R][C]. */
int orc_draft_decode(const uint8_t* spec, int64_t spec_len, uint16_t* out);

/* Exact original weights from both streams: out[R][C]. */
int orc_reconstruct(const uint8_t* spec, int64_t spec_len, const uint8_t* verif,
                    int64_t verif_len, uint16_t* out);

/* y[t][n] = sum_j f64(W'[n][j]) * f64(x[t][j]), j ascending, where W' is the
 * draft (verif == NULL) or the exact reconstruction.  absy[t][n] receives
 * sum_j |W'[n][j]| * |x[t][j]| (the tolerance scale).  x is bf16 [ntok][C]. */
int orc_product(const uint8_t* spec, int64_t spec_len, const uint8_t* verif,
                int64_t verif_len, const uint16_t* x, int64_t ntok, double* y,
                double* absy, int threads);

/* orc_product for the listed rows only: y[t][i], absy[t][i] belong to rows[i]. */
int orc_product_rows(const uint8_t* spec, int64_t spec_len, const uint8_t* verif,
                     int64_t verif_len, const uint16_t* x, int64_t ntok, const int64_t* rows,
                     int64_t nrows, double* y, double* absy);

/* --- comparison exponent codes (Cassandra review, section 3.2: Huffman
 * codes are a little shorter than the unary code but parse serially) --- */
/* Length-limited Huffman code lengths (package-merge); len = 0 for absent
 * symbols, 1 for a lone symbol. */
int orc_huffman_lengths(const uint64_t hist[256], int max_len, uint8_t len[256]);
/* Canonical code values for the lengths (order by length, then symbol). */
int orc_canonical_codes(const uint8_t len[256], uint32_t code[256]);
/* Cassandra-1's frequency-ranked unary code as (length, value) pairs. */
int orc_unary_code(const uint64_t hist[256], uint8_t len[256], uint32_t code[256]);
/* Concatenated codes, most significant bit first; block offsets in bits. */
int orc_prefix_encode(const uint8_t* sym, int64_t n, int64_t block, const uint8_t len[256],
                      const uint32_t code[256], uint8_t* stream, int64_t cap_bytes,
                      uint32_t* blkoff, int64_t* bits);
int orc_prefix_decode(const uint8_t* stream, int64_t bytes, int64_t n, const uint8_t len[256],
                      const uint32_t code[256], uint8_t* out);

/* Read header fields: out[0..7] = format, mant_bits, rows, cols, block, keep,
 * total_bytes, n_sections; sec_off/sec_len receive the 12 section entries. */
int orc_header(const uint8_t* buf, int64_t len, uint32_t expect_magic, int64_t out[8],
               int64_t sec_off[12], int64_t sec_len[12]);

/* --- KV cache (online compression, one stream = one (head, K|V) sequence) ---
 * Region layout of one stream (byte offsets from the region start; each part
 * 256-aligned and followed by >= 16 zero bytes):
 *   speculation region: perm[256] | bitmap (T_max*D bits, token t at bit t*D)
 *     | code offsets u32[T_max] (bit offset of token t's first code in the
 *     code area) | fields ((s<<m)|ft, 1+m bits, token t value i at bit
 *     (t*k+i)*(1+m)) | codes (code_cap bits)
 *   verification region: perm[256] | low mantissas (7-m bits at (t*k+i)*(7-m))
 *     | pruned bytes (token t pruned i at byte t*(D-k)+i) | code offsets
 *     u32[T_max] | codes (vcode_cap bits)
 * Cassandra-2 (fmt = ORC_FMT_C2; OCP MX shared exponent per 32 positions):
 *   speculation region: (256 unused bytes) | bitmap | shared exponents
 *     (u8 per 32 positions, token t group g at byte t*D/32+g) | fields
 *     ((s<<(m+1))|a, m+2 bits at (t*k+i)*(m+2)) | (empty)
 *   verification region: perm[256] of pruned exponents | kept residues
 *     (unary(d) then min(8, 7-m+d) low significand bits, code_cap bits) |
 *     pruned bytes | offsets u32[2*T_max] (token t: residue bit, pruned-code
 *     bit) | pruned codes (vcode_cap bits)
 * The rank tables come from the tokens of the first append (t < T0) and are
 * frozen afterwards.  tails[0] counts the speculation codes (C-1) or the
 * residue bits (C-2), tails[1] the pruned codes. */
int orc_kv_layout(int fmt, int64_t D, int64_t k, int m, int64_t T_max, int64_t code_cap,
                  int64_t vcode_cap, int64_t spec_off[5], int64_t verif_off[5],
                  int64_t* spec_bytes, int64_t* verif_bytes);
int orc_kv_encode(int fmt, const uint16_t* vec, int64_t T, int64_t T0, int64_t D, int64_t k,
                  int m, int64_t T_max, int64_t code_cap, int64_t vcode_cap, uint8_t* spec,
                  uint8_t* verif, uint64_t tails[2]);
/* Draft (verif == NULL) or exact vectors of the first T tokens: out[T][D]. */
int orc_kv_decode(int fmt, const uint8_t* spec, const uint8_t* verif, int64_t T, int64_t D,
                  int64_t k, int m, int64_t T_max, int64_t code_cap, int64_t vcode_cap,
                  uint16_t* out);

/* Softmax attention of nq queries over T tokens, fp64:
 * s_t = scale * sum_d q[d] K[t][d]; p = softmax over t < visible[i];
 * out[i][d] = sum_t p_t V[t][d].  q, K, V are bf16 patterns. */
int orc_attention(const uint16_t* q, int64_t nq, const uint16_t* K, const uint16_t* V,
                  int64_t T, int64_t D, double scale, const int64_t* visible, double* out);

#ifdef __cplusplus
}
#endif
#endif
