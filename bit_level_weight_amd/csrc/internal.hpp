// Internal declarations shared by the library's translation units.
// Stream layout: see include/cassandra.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cassandra.h"

namespace cass {

constexpr int kHeaderBytes = 256;
constexpr uint32_t kMagicSpec = 0x50535343u;   // "CSSP"
constexpr uint32_t kMagicVerif = 0x46565343u;  // "CSVF"

// Section indices of each stream.
enum SpecC1 { S1_RANK = 0, S1_BITMAP, S1_ROWBASE, S1_BLKOFF, S1_KEPTB, S1_FIELDS, S1_CODES, S1_COUNT };
enum VerifC1 { V1_RANK = 0, V1_ROWBASE, V1_BLKOFF, V1_LOWMANT, V1_PRUNED, V1_CODES, V1_COUNT };
enum SpecC2 { S2_BITMAP = 0, S2_SHEXP, S2_KEPTB, S2_FIELDS, S2_COUNT };
enum VerifC2 { V2_RANK = 0, V2_ROWBASE_K, V2_BLKOFF_K, V2_RESID, V2_PRUNED, V2_ROWBASE_P,
               V2_BLKOFF_P, V2_CODES, V2_COUNT };
// Format 3 (MX-quantised target): the speculation stream is Cassandra-2's.
enum VerifC3 { V3_GEXP = 0, V3_LOW, V3_PRUNED, V3_COUNT };

// Tables passed to kernels by value.
struct RankTables {
  uint8_t rank_kept[256];    // exponent -> rank, speculation codes (C-1)
  uint8_t rank_pruned[256];  // exponent -> rank, verification codes
};

struct HeaderBlob {
  uint8_t spec_hdr[kHeaderBytes];
  uint8_t verif_hdr[kHeaderBytes];
  uint8_t perm_spec[256];
  uint8_t perm_verif[256];
};

// Workspace carve-up of cass_encode_plan / cass_encode_tensor.
struct Workspace {
  uint32_t* bitmap;      // rows*cols/32 keep words
  uint8_t* shexp;        // rows*cols/32 shared exponents (C-2)
  unsigned long long* hist;  // [2][256]: kept, pruned
  uint32_t* blk_a;       // per block: C-1 spec code bits / C-2 residue bits
  uint32_t* blk_v;       // per block: pruned code bits
  uint32_t* blk_kept;    // per block: kept count
  uint32_t* off_a;       // per block: exclusive prefix of blk_a within the row
  uint32_t* off_v;
  uint16_t* keptb;       // per block: kept-before count
  unsigned long long* row_a;  // per row: totals, then (after scan) bases
  unsigned long long* row_v;
  unsigned long long* totals; // [2]
  int64_t bytes;
};

Workspace carve_workspace(void* base, int64_t rows, int64_t cols, int64_t block);

// Device views of the sections a kernel reads.
struct SpecViewC1 {
  const uint8_t* perm;       // rank -> exponent
  const uint32_t* bitmap;
  const unsigned long long* rowbase;
  const uint32_t* blkoff;
  const uint16_t* keptb;
  const uint32_t* fields;
  const uint32_t* codes;
  // 32-bit words from the start of each bit section to the end of the stream
  // buffer: bulk copies never read past these.
  int64_t bitmap_limit, fields_limit, codes_limit;
  int64_t blkoff_limit;  // the same for the block offsets (words)
  int64_t keptb_limit;   // and for the kept-before counts (16-bit entries)
  // format 4 (superblock metadata): code base per superblock of 2^sb_log
  // blocks and 16-bit block offsets from it; sb_log < 0 for format 1
  const unsigned long long* sbbase;
  const uint16_t* blkoff16;
  int sb_log;
  int64_t nsb;           // superblocks per row
  int64_t sbbase_limit;  // u64 entries from the bases to the end of the stream buffer
};

// First code bit of block bi (of row `row`, nb blocks per row).
__device__ __forceinline__ uint64_t c1_code_start(const SpecViewC1& v, int64_t row, int64_t bi,
                                                   int64_t nb) {
  if (v.sb_log < 0) return v.rowbase[row] + v.blkoff[bi];
  return v.sbbase[row * v.nsb + ((bi - row * nb) >> v.sb_log)] + v.blkoff16[bi];
}

__host__ __device__ __forceinline__ bool is_c1_format(int f) {
  return f == CASS_FMT_C1_UNARY || f == CASS_FMT_C1_SUPERBLOCK;
}
struct VerifViewC1 {
  const uint8_t* perm;
  const unsigned long long* rowbase;
  const uint32_t* blkoff;
  const uint32_t* lowmant;
  const uint8_t* pruned;
  const uint32_t* codes;
  // 32-bit words from the start of each bit section to the end of the stream
  // buffer (whole 16-byte units): bulk copies never read past these.
  int64_t lowmant_limit, pruned_limit, codes_limit;
};
struct SpecViewC2 {
  const uint32_t* bitmap;
  const uint8_t* shexp;
  const uint16_t* keptb;
  const uint32_t* fields;
  int64_t bitmap_limit, shexp_limit, fields_limit;  // as in SpecViewC1 (shexp: bytes/4)
  int64_t keptb_limit;  // (16-bit entries)
};
struct VerifViewC2 {
  const uint8_t* perm;
  const unsigned long long* rowbase_k;
  const uint32_t* blkoff_k;
  const uint32_t* resid;
  const uint8_t* pruned;
  const unsigned long long* rowbase_p;
  const uint32_t* blkoff_p;
  const uint32_t* codes;
};

struct VerifViewC3 {
  const uint8_t* gexp;    // X per 32 positions
  const uint32_t* low;    // kept values' low 7-m bits of t
  const uint32_t* pruned; // pruned values' (s<<8)|t, 9 bits
};

struct Shape {
  int64_t rows, cols, block, keep;
  int mant;
  int64_t ld;  // row stride of the bf16 input (encoder only; elements)
};

// Internal code-path switches, set through cass_set_option (tests and
// benchmarking select the fallback kernels with them).  0 is the default.
enum Option {
  OPT_GEMV_PARTS = 0,  // parts per row of the balanced GEMV (power of two 1..64)
  OPT_GEMV_PATH,       // 1: staged kernel, 2: direct kernel
  OPT_GEMV_SUB,        // lanes per block of the staged kernel's sub-split
  OPT_EXACT_PATH,      // 1: per-thread stream readers for verify/reconstruct
  OPT_EXACT_BLOCKS,    // blocks per stage of the staged exact decoder (1 or 2)
  OPT_KV_EXACT_PATH,   // 1: per-thread decoders for Cassandra-1 verification attention
  OPT_KV_APPEND_PATH,  // 1: the five-launch append for any token count
  OPT_COUNT
};
int option(Option o);

// ---- launchers (return hipSuccess or the launch error) ----
hipError_t launch_fill_zero(void* p, int64_t bytes, hipStream_t s);
hipError_t launch_select(const uint16_t* w, const Shape& sh, uint32_t* bitmap, hipStream_t s);
hipError_t launch_histograms(const uint16_t* w, const Shape& sh, int format, const Workspace& ws,
                             hipStream_t s);
hipError_t launch_block_bits(const uint16_t* w, const Shape& sh, int format, const Workspace& ws,
                             const RankTables& rt, hipStream_t s);
hipError_t launch_row_scan(const Shape& sh, const Workspace& ws, hipStream_t s);
// Largest code offset of a block from its superblock's first block (into
// ws.totals[2]; the row scan must have run).
hipError_t launch_superblock_span(const Shape& sh, const Workspace& ws, int sblocks, hipStream_t s);
hipError_t launch_rows_scan(const Shape& sh, const Workspace& ws, hipStream_t s);
hipError_t launch_write_headers(const HeaderBlob& hb, uint8_t* spec, int64_t spec_rank_off,
                                uint8_t* verif, int64_t verif_rank_off, hipStream_t s);
hipError_t launch_pack(const uint16_t* w, const Shape& sh, int format, const Workspace& ws,
                       const RankTables& rt, uint8_t* spec, const int64_t* spec_sec,
                       uint8_t* verif, const int64_t* verif_sec, hipStream_t s);

// Draft GEMV.  The staged kernels copy each tile's compressed bytes to LDS;
// the direct kernels read every stream word from global memory and serve
// shapes whose tiles do not fit in LDS.
hipError_t launch_draft_gemv_c1(const SpecViewC1& v, const Shape& sh, const uint16_t* x,
                                int batch, int64_t ldx, float* y, int64_t ldy, hipStream_t s);
hipError_t launch_draft_gemv_c2(const SpecViewC2& v, const Shape& sh, const uint16_t* x,
                                int batch, int64_t ldx, float* y, int64_t ldy, hipStream_t s);
hipError_t launch_draft_gemv_c1_direct(const SpecViewC1& v, const Shape& sh, const uint16_t* x,
                                       int batch, int64_t ldx, float* y, int64_t ldy,
                                       hipStream_t s);
hipError_t launch_draft_gemv_c2_direct(const SpecViewC2& v, const Shape& sh, const uint16_t* x,
                                       int batch, int64_t ldx, float* y, int64_t ldy,
                                       hipStream_t s);
int64_t draft_gemv_direct_lds_bytes(const Shape& sh, int batch);
// Balanced kernel (Cassandra-1): equal kept-value parts per lane.
bool draft_gemv_bal_fits(const Shape& sh, int batch, int64_t code_limit_words, int64_t nsb);
bool draft_gemv_bal_c2_fits(const Shape& sh, int batch);
hipError_t launch_draft_gemv_c2_bal(const SpecViewC2& v, const Shape& sh, const uint16_t* x,
                                    int batch, int64_t ldx, float* y, int64_t ldy,
                                    hipStream_t s);
hipError_t launch_draft_gemv_c1_bal(const SpecViewC1& v, const Shape& sh, const uint16_t* x,
                                    int batch, int64_t ldx, float* y, int64_t ldy,
                                    hipStream_t s);
bool draft_gemv_staged_fits(const Shape& sh, int batch, int format, int64_t code_limit_words);
hipError_t launch_decode_c1(const SpecViewC1& sv, const VerifViewC1* vv, const Shape& sh,
                            uint16_t* out, hipStream_t s);
hipError_t launch_decode_c2(const SpecViewC2& sv, const VerifViewC2* vv, const Shape& sh,
                            uint16_t* out, hipStream_t s);
hipError_t launch_verify_gemm_c1(const SpecViewC1& sv, const VerifViewC1& vv, const Shape& sh,
                                 const uint16_t* X, int ntok, int64_t ldx, float* Y,
                                 int64_t ldy, hipStream_t s);
// Staged exact decoders for Cassandra-1 (verification GEMM, reconstruction).
bool exact_staged_fits(const Shape& sh, const SpecViewC1& sv, const VerifViewC1& vv);
hipError_t launch_verify_gemm_c1_staged(const SpecViewC1& sv, const VerifViewC1& vv,
                                        const Shape& sh, const uint16_t* X, int ntok,
                                        int64_t ldx, float* Y, int64_t ldy, hipStream_t s);
hipError_t launch_reconstruct_c1_staged(const SpecViewC1& sv, const VerifViewC1& vv,
                                        const Shape& sh, uint16_t* out, hipStream_t s);
hipError_t launch_draft_decode_c1_staged(const SpecViewC1& sv, const Shape& sh, uint16_t* out,
                                         hipStream_t s);
hipError_t launch_verify_gemm_c2(const SpecViewC2& sv, const VerifViewC2& vv, const Shape& sh,
                                 const uint16_t* X, int ntok, int64_t ldx, float* Y,
                                 int64_t ldy, hipStream_t s);
hipError_t launch_decode_c3(const SpecViewC2& sv, const VerifViewC3& vv, const Shape& sh,
                            uint16_t* out, hipStream_t s);
hipError_t launch_verify_gemm_c3(const SpecViewC2& sv, const VerifViewC3& vv, const Shape& sh,
                                 const uint16_t* X, int ntok, int64_t ldx, float* Y,
                                 int64_t ldy, hipStream_t s);

int device_cu_count();

// Debug build (CASS_DEBUG): device bounds checks.  Each translation unit has
// its own flag words (one per lane, so the atomic is a vector one) and
// registers a reader that returns and clears them; CASS_DCHECK compiles to
// nothing in release builds.
void debug_register(uint32_t (*read_and_clear)());
#ifdef CASS_DEBUG
namespace {
__device__ uint32_t g_debug_bits[64];
uint32_t debug_read_and_clear() {
  uint32_t h[64] = {}, z[64] = {};
  if (hipMemcpyFromSymbol(h, HIP_SYMBOL(g_debug_bits), sizeof h) != hipSuccess) return 0x80000000u;
  if (hipMemcpyToSymbol(HIP_SYMBOL(g_debug_bits), z, sizeof z) != hipSuccess) return 0x80000000u;
  uint32_t v = 0;
  for (int i = 0; i < 64; ++i) v |= h[i];
  return v;
}
struct DebugRegistrar {
  DebugRegistrar() { debug_register(&debug_read_and_clear); }
};
DebugRegistrar g_debug_registrar;
}  // namespace
#define CASS_DCHECK(cond, bit)                                                 \
  do {                                                                         \
    if (!(cond)) atomicOr(&g_debug_bits[threadIdx.x & 63], (uint32_t)(bit));   \
  } while (0)
#else
#define CASS_DCHECK(cond, bit) \
  do {                         \
  } while (0)
#endif

// Sets the calling thread's error text (cass_last_error) and returns status.
int report(int status, const char* fmt, ...);
void clear_error();

}  // namespace cass
