/*
 * libcassandra -- the Cassandra bit-level weight format on AMD Instinct MI355X
 * (gfx950): encoder, draft GEMV, verification GEMM and exact reconstruction.
 *
 * The method (Cassandra review, marsggbo.github.io, section 3.1): each bf16
 * tensor goes through unstructured value pruning (keep the most salient values
 * of a group), mantissa truncation of the kept values and exponent
 * compression, and is split into a speculation stream -- all the draft model
 * loads, zero-filled back to bf16 -- and a verification stream, which together
 * with the speculation stream rebuilds the original bits exactly.  Exponent
 * coding (same page, section 3.2): Cassandra-1 gives frequent exponents short
 * unary codes (decoding counts zeros up to the one), Cassandra-2 shares one
 * MX exponent per 32 values (OCP Microscaling spec, cited by the paper).
 *
 * Conventions for every call:
 *  - All tensor data lives in device memory owned by the caller; the library
 *    never allocates device memory and keeps no state besides its code object
 *    and a thread-local error string.
 *  - bf16 data is passed as its 16-bit patterns (uint16_t).  Products are fp32.
 *  - Matrices are row-major; a weight matrix W is [rows = out features][cols =
 *    in features]; the pruning group is one row.
 *  - Kernels run on the caller's stream; only cass_encode_plan synchronises it.
 *  - Argument errors are returned before anything is launched; a launch
 *    failure returns CASS_ERR_HIP.  cass_last_error() gives the detail.
 *  - Descriptors are checked against the shape's closed-form section sizes
 *    before any launch; the contents of device streams (row bases, block
 *    offsets, codes) are trusted.  Streams from an untrusted source are
 *    checked on the host with cass_tensor_validate first.
 *
 * Stream layout (both streams): a 256-byte header (u32 magic, u32 version=1,
 * u32 format, u32 mant_bits, i64 rows, cols, block, keep, total_bytes, u32
 * n_sections, u32 0, then 12 x {i64 offset, i64 bytes}) followed by the
 * sections, each starting on a multiple of 256 bytes and followed by at least
 * 16 zero bytes.  Bit sections are little-endian: bit i is bit (i & 31) of
 * 32-bit word i >> 5.
 *
 *  Cassandra-1 speculation sections: 0 rank table (256 B, exponent of rank r),
 *   1 keep bitmap (rows*cols bits), 2 row bases (u64 per row: first code bit
 *   of the row in section 6), 3 block offsets (u32 per block of `block`
 *   positions, code bits relative to the row base), 4 kept-before counts
 *   (u16 per block), 5 sign+top-m mantissa fields ((s<<m)|ft, 1+m bits per
 *   kept value, value i of row r at bit (r*keep+i)*(1+m)), 6 exponent codes
 *   (rank r -> r zero bits then a one bit; kept values in row-major order).
 *  Cassandra-1 verification sections: 0 rank table of pruned exponents,
 *   1 row bases, 2 block offsets (for section 5), 3 low mantissa bits of kept
 *   values (7-m bits each), 4 pruned values' (s<<7)|mantissa bytes, 5 pruned
 *   exponent codes.
 *  Cassandra-2 speculation sections: 0 keep bitmap, 1 shared exponent (u8 per
 *   32 positions: the largest max(e,1) over the kept values, 0 if none),
 *   2 kept-before counts, 3 fields ((s<<(m+1))|a, m+2 bits, a = the value's
 *   significand aligned to the shared exponent and cut to m+1 bits).
 *  Cassandra-2 verification sections: 0 pruned rank table, 1 residue row
 *   bases, 2 residue block offsets, 3 kept residues (unary(d) then the
 *   min(8, 7-m+d) bits the draft dropped, d = shared - own exponent),
 *   4 pruned bytes, 5 pruned-code row bases, 6 pruned-code block offsets,
 *   7 pruned exponent codes.
 *  Format 3, Cassandra-2 with an MX-quantised target (the reading of section
 *   3.2 in which Cassandra-2's slight precision loss reaches the target too):
 *   the target is not the original tensor but its MX-32 quantisation -- per
 *   group of 32 positions of a row, X = the largest max(e,1) over all 32
 *   values, and each value keeps its sign and t = its 8-bit significand
 *   (hidden bit included) shifted right by X - max(e,1) (0 from a shift of 8),
 *   i.e. it is truncated toward zero to a multiple of 2^(X-134) (zero -> +0).
 *   The speculation stream is the Cassandra-2 one (its field a is the top m+1
 *   bits of t).  Verification sections, all at fixed positions: 0 X (u8 per
 *   32 positions), 1 low 7-m bits of each kept value's t (value i of row r at
 *   bit (r*keep+i)*(7-m)), 2 pruned values' (s<<8)|t, 9 bits each (pruned
 *   value i of row r at bit (r*(cols-keep)+i)*9).  cass_reconstruct returns
 *   the quantised target and cass_verify_gemm multiplies with it.
 *  Format 4, Cassandra-1 with superblock metadata (pith.science review,
 *   Figure 11: superblock-based data management): a superblock is
 *   CASS_SUPERBLOCK_BLOCKS consecutive blocks of one row (the last of a row
 *   may be shorter).  Speculation sections as Cassandra-1's but 2 = u64 code
 *   base per superblock (superblock j of row r at entry r*ceil(nb/16)+j) and
 *   3 = u16 code offset per block from its superblock's base; the
 *   verification stream is Cassandra-1's.  Both headers hold 16 in the u32 at
 *   byte 60 (0 in the other formats).  Encoding returns CASS_ERR_OVERFLOW when
 *   a block starts 2^16 or more code bits after its superblock's base.  The
 *   draft GEMV, verification GEMM and decoders of format 4 are the per-thread
 *   stream readers (the balanced and staged kernels take format 1).
 */
#ifndef CASSANDRA_H
#define CASSANDRA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CASS_VERSION 1

enum cass_status {
  CASS_OK = 0,
  CASS_ERR_INVALID = 1,     /* bad argument, shape or descriptor */
  CASS_ERR_UNSUPPORTED = 2, /* valid but not implemented here (e.g. batch > 8) */
  CASS_ERR_OVERFLOW = 3,    /* a size or offset does not fit its field */
  CASS_ERR_CORRUPT = 4,     /* a stream fails validation */
  CASS_ERR_CAPACITY = 5,    /* a caller buffer is too small */
  CASS_ERR_HIP = 6          /* a HIP runtime call or launch failed */
};

enum cass_format { CASS_FMT_C1_UNARY = 1, CASS_FMT_C2_MX32 = 2, CASS_FMT_C2_MX_TARGET = 3,
                   CASS_FMT_C1_SUPERBLOCK = 4 };
#define CASS_SUPERBLOCK_BLOCKS 16

#define CASS_MAX_SECTIONS 12

/* Encoding parameters.  keep = values kept per row (the pages' keep ratio
 * times cols, chosen by the caller); mant_bits = mantissa bits kept, 0..7;
 * block = positions per offset block, a power of two >= 32 dividing cols. */
typedef struct cass_params {
  int32_t format;
  int32_t mant_bits;
  int64_t block;
  int64_t keep;
} cass_params;

/* Descriptor of an encoded tensor: a plain host struct pointing at the
 * caller's device buffers.  Filled by cass_encode_tensor or by
 * cass_tensor_describe from the two stream headers. */
typedef struct cass_tensor {
  int32_t format;
  int32_t mant_bits;
  int64_t rows, cols, block, keep;
  const void* spec;   /* device, spec_bytes long */
  int64_t spec_bytes;
  const void* verif;  /* device, or NULL when only the draft is needed */
  int64_t verif_bytes;
  int64_t spec_sec[CASS_MAX_SECTIONS];  /* byte offsets of the sections */
  int64_t verif_sec[CASS_MAX_SECTIONS];
} cass_tensor;

/* Result of the planning pass of the encoder (host struct). */
typedef struct cass_plan {
  int64_t rows, cols, ld;
  cass_params p;
  int64_t spec_bytes, verif_bytes;      /* buffer sizes cass_encode_tensor needs */
  int64_t spec_sec[CASS_MAX_SECTIONS], spec_len[CASS_MAX_SECTIONS];
  int64_t verif_sec[CASS_MAX_SECTIONS], verif_len[CASS_MAX_SECTIONS];
  uint64_t hist_kept[256], hist_pruned[256]; /* exponent histograms */
  uint8_t perm_spec[256], perm_verif[256];   /* rank -> exponent tables */
  uint64_t spec_code_bits, verif_code_bits, resid_bits;
  const void* ws;                       /* workspace the plan was made in */
  int64_t ws_bytes;
} cass_plan;

/* Workspace bytes cass_encode_plan needs for a rows x cols tensor
 * (Cassandra review, section 3.1: the offline weight transform).  Host only. */
int cass_encode_ws_bytes(int64_t rows, int64_t cols, const cass_params* p, int64_t* ws_bytes);

/* Planning pass of the encoder (Cassandra review, section 3.1, the first two
 * transform steps, and section 3.2, exponent statistics): per-row
 * top-`keep` selection by |w| with ties to the lower column, exponent
 * histograms of kept and pruned values, frequency-ranked tables (count
 * descending, exponent ascending), code lengths and offsets.  w: device
 * [rows][ld] bf16 patterns, ld >= cols elements.  ws: device workspace of
 * ws_bytes >= cass_encode_ws_bytes(); it holds intermediate results that
 * cass_encode_tensor reads, so it must stay untouched in between.
 * Synchronises `stream` twice (histograms, sizes).  rows may be 0. */
int cass_encode_plan(const uint16_t* w, int64_t rows, int64_t cols, int64_t ld,
                     const cass_params* p, void* ws, int64_t ws_bytes, hipStream_t stream,
                     cass_plan* plan);

/* Packing pass (Cassandra review, section 3.1: the split into speculation and
 * verification data; section 3.2: unary exponent codes or the shared MX
 * exponent): writes both streams, byte for byte the canonical encoding, to
 * the device buffers spec (>= plan->spec_bytes) and verif (>= plan->
 * verif_bytes), 256-byte aligned, and fills *out.  w, ld and ws must be those
 * given to the plan.  Asynchronous. */
int cass_encode_tensor(const uint16_t* w, int64_t ld, const cass_plan* plan, void* spec,
                       int64_t spec_cap, void* verif, int64_t verif_cap, hipStream_t stream,
                       cass_tensor* out);

/* Build a descriptor from host copies of the two 256-byte stream headers and
 * the device buffers holding the streams (verif may be NULL): the layout the
 * encoder writes (Cassandra review, section 3.1, two streams per tensor).
 * The header's section table must match the shape's closed-form sizes and
 * lie inside the buffers; else CASS_ERR_CORRUPT.  Host only. */
int cass_tensor_describe(const void* spec_header, const void* spec, int64_t spec_bytes,
                         const void* verif_header, const void* verif, int64_t verif_bytes,
                         cass_tensor* out);

/* Draft GEMV (section 3.1: the draft runs the full-size product on the
 * zero-filled speculation data): y[b][n] = sum_j Wdraft[n][j] * x[b][j] for
 * b < batch, accumulated in fp32.  x: device bf16 [batch][ldx], ldx >= cols;
 * y: device fp32 [batch][ldy], ldy >= rows.  batch 1..8.  Reads only the
 * speculation stream.  Asynchronous. */
int cass_draft_gemv(const cass_tensor* W, const uint16_t* x, int batch, int64_t ldx,
                    float* y, int64_t ldy, hipStream_t stream);

/* Verification GEMM for the k+1 drafted tokens (Cassandra review, section 1:
 * the target verifies the drafted tokens in parallel; section 3.1: it loads
 * both streams and reassembles the weights losslessly):
 * Y[t][n] = sum_j W[n][j] * X[t][j], t < ntok, W the exact original weights,
 * fp32 accumulation.  X: device bf16 [ntok][ldx]; Y: device fp32 [ntok][ldy].
 * ntok 1..16.  Needs W->verif.  Asynchronous. */
int cass_verify_gemm(const cass_tensor* W, const uint16_t* X, int ntok, int64_t ldx,
                     float* Y, int64_t ldy, hipStream_t stream);

/* Exact reconstruction of the original bf16 patterns from both streams
 * (Cassandra review, section 3.1: the target reassembles speculation and
 * verification data losslessly): out: device [rows][cols], 16-byte aligned.
 * Asynchronous. */
int cass_reconstruct(const cass_tensor* W, uint16_t* out, hipStream_t stream);

/* Zero-filled draft weights from the speculation stream alone (Cassandra
 * review, section 3.1: the draft loads only speculation data, zero-filled
 * back to standard floating point): out: device [rows][cols] bf16 patterns,
 * 16-byte aligned.  Asynchronous. */
int cass_draft_decode(const cass_tensor* W, uint16_t* out, hipStream_t stream);

/* Host-only structural validation of a stream pair held in host memory
 * (verif may be NULL), for streams of untrusted origin (the format of
 * Cassandra review, sections 3.1 and 3.2): header fields, section bounds,
 * bitmap counts, the kept-before counts and that every row base and block
 * offset lands on a code boundary.  Returns CASS_OK or CASS_ERR_CORRUPT.
 * Touches no GPU. */
int cass_tensor_validate(const void* spec, int64_t spec_bytes, const void* verif,
                         int64_t verif_bytes);

/* ------------------------------------------------------------- KV cache
 * Online compression of one layer's KV cache (Cassandra review, section 3.3:
 * KV entries are produced during inference, so the encoder runs online;
 * section 3.1: the KV cache gets the same pruning, truncation and exponent
 * coding as the weights).  The pruning group is one token's vector of one
 * head (head_dim values).  Each (head, K|V) pair is one append-only stream,
 * stream index 2*head + (0 for K, 1 for V), each with its own region of
 * spec_stream_bytes in `spec` and verif_stream_bytes in `verif`:
 *   speculation region: rank table (256 B) | keep bitmap (max_tokens *
 *     head_dim bits) | code offsets (u32 per token: bit offset of the token's
 *     first code) | fields ((s<<m)|ft, 1+m bits, token t value i at bit
 *     (t*keep+i)*(1+m)) | codes (code_cap_bits)
 *   verification region: rank table | low mantissas (7-m bits, same order) |
 *     pruned bytes (token t, pruned i at byte t*(head_dim-keep)+i) | code
 *     offsets | codes (vcode_cap_bits)
 * With format CASS_FMT_C2_MX32 (OCP MX: one shared exponent per 32
 * positions, here the largest max(e,1) over the kept values, 0 if none):
 *   speculation region: 256 unused bytes | keep bitmap | shared exponents
 *     (u8 per 32 positions, token t group g at byte t*head_dim/32+g) | fields
 *     ((s<<(m+1))|a, m+2 bits, a = the significand aligned to the shared
 *     exponent and cut to m+1 bits) | (empty)
 *   verification region: rank table of pruned exponents | kept residues
 *     (unary(d) then the min(8, 7-m+d) bits the draft dropped, d = shared -
 *     own exponent; code_cap_bits) | pruned bytes | offsets (u32 pair per
 *     token: first residue bit, first pruned-code bit) | pruned codes
 * Each part starts on a multiple of 256 bytes and is followed by >= 16 zero
 * bytes.  The rank tables are built on the device from the first append's
 * tokens and frozen afterwards.  `state` (device, CASS_KV_STATE_BYTES) holds
 * the token count, flags and the code tails of every stream. */
#define CASS_KV_STATE_BYTES 4096
enum { CASS_KV_FLAG_TABLES = 1, CASS_KV_FLAG_OVERFLOW = 2 };

typedef struct cass_kv_params {
  int32_t n_kv_heads;      /* 1..64 */
  int32_t head_dim;        /* multiple of 32, at most 256 */
  int32_t keep;            /* values kept per token vector, 0..head_dim */
  int32_t mant_bits;       /* 0..7 */
  int64_t max_tokens;
  int64_t code_cap_bits;   /* speculation code capacity per stream, < 2^32 */
  int64_t vcode_cap_bits;  /* verification code capacity per stream, < 2^32 */
  int32_t format;          /* CASS_FMT_C1_UNARY (0 means this) or CASS_FMT_C2_MX32 */
} cass_kv_params;

typedef struct cass_kv {
  cass_kv_params p;
  void* spec;               /* device, 2*n_kv_heads*spec_stream_bytes */
  void* verif;              /* device, 2*n_kv_heads*verif_stream_bytes */
  void* state;              /* device, CASS_KV_STATE_BYTES */
  int64_t spec_stream_bytes, verif_stream_bytes;
  int64_t spec_part[5], verif_part[5]; /* part offsets inside a stream region */
  int64_t tokens;           /* tokens appended so far (host copy, kept by the calls) */
} cass_kv;

/* Buffer sizes for a cache with these parameters (the online KV format of
 * Cassandra review, section 3.3; layout above).  Host only. */
int cass_kv_bytes(const cass_kv_params* p, int64_t* spec_bytes, int64_t* verif_bytes,
                  int64_t* state_bytes);
/* Fill *kv and zero the three device buffers of an empty cache (Cassandra
 * review, section 3.3).  Asynchronous. */
int cass_kv_init(cass_kv* kv, const cass_kv_params* p, void* spec, void* verif, void* state,
                 hipStream_t stream);
/* Workspace bytes cass_kv_append_encode needs for ntok tokens (section 3.3
 * of the Cassandra review: the online encoder).  Host only. */
int cass_kv_append_ws_bytes(const cass_kv* kv, int ntok, int64_t* ws_bytes);
/* Online encoder (Cassandra review, section 3.3: KV entries appear during
 * inference and are compressed as they are appended; section 3.1: the same
 * pruning, truncation and exponent coding as the weights).
 * Append ntok tokens: k, v device bf16 [ntok][n_kv_heads][head_dim].  The
 * first call also builds the rank tables from its tokens.  Pruning, splitting,
 * coding and packing all run on the device without a host synchronisation;
 * codes that would exceed a stream's capacity are not written and raise
 * CASS_KV_FLAG_OVERFLOW (see cass_kv_status).  Advances kv->tokens. */
int cass_kv_append_encode(cass_kv* kv, const uint16_t* k, const uint16_t* v, int ntok,
                          void* ws, int64_t ws_bytes, hipStream_t stream);
/* Drop the newest tokens: keep tokens [0, tokens) of the kv->tokens cached
 * (Cassandra review, section 1: drafted tokens that the target's parallel
 * verification rejects are discarded, and the draft's own keys and values of
 * the drafted tokens give way to the target's).  Every per-token part past
 * the kept tokens returns to zero and each code tail moves back, so the
 * regions hold exactly the bytes of appending the kept tokens (the rank
 * tables stay frozen; truncating to 0 makes the next append build them
 * again).  A stream closed by an overflow reopens when the codes of the
 * first dropped token had been written (else it stays closed, its tail at the
 * capacity); CASS_KV_FLAG_OVERFLOW stays set.  0 <= tokens <=
 * kv->tokens, else CASS_ERR_INVALID.  One launch, no host synchronisation;
 * sets kv->tokens. */
int cass_kv_truncate(cass_kv* kv, int64_t tokens, hipStream_t stream);
/* Token count and flags from the device state of the online encoder
 * (Cassandra review, section 3.3).  Synchronises the stream. */
int cass_kv_status(const cass_kv* kv, int64_t* tokens, uint32_t* flags, hipStream_t stream);
/* Decoded cache (Cassandra review, section 3.1: zero-filled draft data, or
 * the lossless reassembly of both streams): out device bf16 [2][n_kv_heads]
 * [tokens][head_dim] (K then V); exact != 0 rebuilds the original values,
 * else the zero-filled draft. */
int cass_kv_decode(const cass_kv* kv, int exact, uint16_t* out, hipStream_t stream);

/* Workspace bytes for an attention call over the current tokens (draft or
 * verification attention, Cassandra review, sections 1 and 3.3).  Host only. */
int cass_kv_attn_ws_bytes(const cass_kv* kv, int nq, int n_q_heads, int64_t* ws_bytes);
/* Draft attention of one query (Cassandra review, section 3.3: the KV cache
 * is compressed online and the draft reads only its speculation data,
 * zero-filled, as in section 3.1) (grouped-query: query head g reads KV head
 * g / (n_q_heads / n_kv_heads)) over all cached tokens, on the zero-filled
 * draft keys and values: out[g][d] = sum_t softmax_t(scale * q_g . K~_t) V~_t[d].
 * q: device bf16 [n_q_heads][head_dim]; out: device fp32 [n_q_heads][head_dim].
 * head_dim must be 128. */
int cass_kv_draft_attn(const cass_kv* kv, const uint16_t* q, int n_q_heads, float scale,
                       float* out, void* ws, int64_t ws_bytes, hipStream_t stream);
/* Verification attention for the nq = k+1 newest tokens (Cassandra review,
 * section 1: the drafted tokens are verified in one parallel pass) on the
 * exact keys and values: query i sees tokens 0 .. tokens-nq+i (causal over
 * the appended block).  q: [nq][n_q_heads][head_dim] bf16; out: fp32, same
 * shape.  nq <= 8, n_q_heads / n_kv_heads * nq <= 32, head_dim 128. */
int cass_kv_verify_attn(const cass_kv* kv, const uint16_t* q, int nq, int n_q_heads, float scale,
                        float* out, void* ws, int64_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * cass_kv_draft_attn with no workspace argument.  Its per-chunk partials go
 * to a fixed scratch array of CASS_KV_STATIC_SCRATCH_BYTES that the library
 * holds on each device it runs on (until the process ends); the call
 * allocates nothing.  The partials take n_kv_heads * ceil(tokens / 128) *
 * (n_q_heads / n_kv_heads) * 520 bytes (128K tokens of 32 query heads fit);
 * a larger call returns CASS_ERR_CAPACITY before launching anything.  Every
 * call on one device shares that device's scratch: calls that overlap in
 * time on one device (two streams, two threads) race and must be ordered by
 * the caller.  Same arguments and results as cass_kv_draft_attn. */
#define CASS_KV_STATIC_SCRATCH_BYTES (32ll << 20)
int cass_kv_draft_attn_static(const cass_kv* kv, const uint16_t* q, int n_q_heads, float scale,
                              float* out, hipStream_t stream);

/* ------------------------------------------- comparison exponent codecs
 * Cassandra review, section 3.2: the unary exponent code is preferred to a
 * Huffman code although Huffman codes are a little shorter, because a Huffman
 * stream parses serially (bit by bit, or through a table of 2^N entries for
 * N-bit codes) while unary codes decode in parallel.  These calls build both
 * codes for a sequence of exponent symbols (u8) and decode them three ways,
 * so the trade can be measured.  A code is a prefix code given by (length,
 * value) per symbol; a code's value is written most significant bit first, in
 * stream bit order (bit i of a stream is bit i & 31 of 32-bit word i >> 5).
 * A stream is the concatenation of the symbols' codes; blkoff[b] is the bit
 * offset of symbol b * block. */
typedef struct cass_prefix_code {
  int32_t max_len;     /* the longest length in len[] */
  uint8_t len[256];    /* code length of each symbol, 0..32 (0: no code) */
  uint32_t code[256];  /* code value (its low len bits) */
} cass_prefix_code;
enum { CASS_PREFIX_TABLE = 1, CASS_PREFIX_UNARY_SERIAL = 2, CASS_PREFIX_UNARY_PARALLEL = 3 };
/* Length-limited Huffman code for a symbol histogram (package-merge; among
 * equal weights leaves precede pairs, leaves ordered by (count, symbol)), with
 * canonical values (symbols ordered by (length, symbol), consecutive values,
 * shifted left as the length grows).  Absent symbols get no code; a lone
 * symbol gets a 1-bit code.  max_len in 1..32.  Host only. */
int cass_prefix_code_huffman(const uint64_t* hist, int max_len, cass_prefix_code* out);
/* Cassandra-1's frequency-ranked unary code (rank r: r zero bits then a one,
 * i.e. length r+1, value 1; ranks by count, ties to the smaller symbol);
 * ranks past 31 get no code.  Host only. */
int cass_prefix_code_unary(const uint64_t* hist, cass_prefix_code* out);
/* Total code bits of a histogram under a code (CASS_ERR_INVALID if a
 * present symbol has no code).  Host only. */
int cass_prefix_stream_bits(const cass_prefix_code* c, const uint64_t* hist, int64_t* bits);
/* Encode sym[0..n) (device) into stream (device, 16-byte aligned, a multiple
 * of 16 bytes, at least the code bits plus 16 zero bytes, below 2^29 bytes)
 * and blkoff (device, u32 per block; block a multiple of 16).  Every symbol
 * must have a code; blocks whose codes would not fit the buffer are left
 * unwritten.  Four launches, no host synchronisation. */
int cass_prefix_encode(const cass_prefix_code* c, const uint8_t* sym, int64_t n, int64_t block,
                       void* stream, int64_t stream_bytes, uint32_t* blkoff, hipStream_t stream_h);
/* Workspace of the parallel unary decoder for a stream of stream_bytes. */
int cass_prefix_decode_ws_bytes(int64_t stream_bytes, int64_t* ws_bytes);
/* Decode n symbols (n a multiple of 16) into out (device, 16-byte aligned):
 * CASS_PREFIX_TABLE -- one thread per block with a 2^max_len table in shared
 * memory (max_len <= 12, any prefix code); CASS_PREFIX_UNARY_SERIAL -- one
 * thread per block counting trailing zeros (unary codes); CASS_PREFIX_UNARY_
 * PARALLEL -- no block offsets (blkoff may be NULL): each word of the stream
 * on its own, code index from a prefix count of one bits (unary codes; ws
 * from cass_prefix_decode_ws_bytes).  Reads stay inside stream_bytes whatever
 * the stream holds. */
int cass_prefix_decode(const cass_prefix_code* c, const void* stream, int64_t stream_bytes,
                       const uint32_t* blkoff, int64_t n, int64_t block, int method, uint8_t* out,
                       void* ws, int64_t ws_bytes, hipStream_t stream_h);

/* Status code -> fixed English text, and the detail of the last error on
 * the calling thread ("" if none); plumbing, not part of the method. */
const char* cass_status_string(int status);
const char* cass_last_error(void);
/* CASS_VERSION of the loaded library. */
int cass_version(void);

/* Device bounds checks of the debug build (libcassandra_debug.so, compiled
 * with CASS_DEBUG; plumbing, not part of the method).  A failed check sets a
 * CASS_DBG_* bit and the kernel carries on; *flags receives the OR of the
 * bits raised since the previous call, which clears them.  Call after the
 * work has completed (host only).  Release builds set *flags to 0 and return
 * CASS_ERR_UNSUPPORTED. */
enum {
  CASS_DBG_STAGE = 1 << 0,  /* a staged copy would pass the end of its shared-memory region */
  CASS_DBG_ALIGN = 1 << 1,  /* a shared-memory DMA source or target off its 16-byte boundary */
  CASS_DBG_TILE = 1 << 2,   /* a decoded value written outside its tile row */
  CASS_DBG_WINDOW = 1 << 3  /* a bit position outside its staged section */
};
int cass_debug_flags(uint32_t* flags);

/* Code-path switches for tests and benchmarks, process-wide, 0 = default
 * (not part of the method; every path computes the same result):
 *   "gemv_parts"   parts per row of the balanced draft GEMV, power of two 1..64
 *   "gemv_path"    1: staged draft GEMV kernel, 2: direct kernel
 *   "gemv_sub"     lanes per block of the staged kernel
 *   "exact_path"   1: per-thread stream readers for verification/reconstruction
 *   "exact_blocks" blocks per stage of the staged exact decoder, 1 or 2
 *   "kv_exact_path" 1: per-thread decoders for Cassandra-1 verification
 *                  attention (default: split decode, matrix-core scores)
 *   "kv_append_path" 1: the five-launch append also for appends of up to 16
 *                  tokens (default there: one launch, one wave per stream)
 * Unknown names or values out of range give CASS_ERR_INVALID.  Not
 * synchronised with launches in flight on other threads. */
int cass_set_option(const char* name, int64_t value);

/* Measurement utility (not part of the method): reads `bytes` (a multiple of
 * 16) of the 16-byte aligned device buffer once with streaming loads, the
 * achievable-read ceiling of the GPU; out: device, CASS_STREAM_READ_BLOCKS
 * words (a fold of the data, so the loads are not dropped).  Asynchronous. */
#define CASS_STREAM_READ_BLOCKS 2048
int cass_stream_read(const void* buf, int64_t bytes, uint32_t* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif
