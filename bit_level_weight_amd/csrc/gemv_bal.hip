// Fused draft GEMV, balanced variant (the default path for Cassandra-1):
//   y[b][n] = sum over kept j of Wdraft[n][j] * x[b][j], fp32 accumulation.
//
// Method: Cassandra review (marsggbo.github.io), section 3.1 -- the draft runs
// the full-size product on the zero-filled speculation data, so only kept
// values contribute and only speculation bytes are read; sections 3.2 and 3.3
// -- a unary exponent code is decoded by counting the zeros up to its one, and
// the keep bitmap is de-sparsified, here by the SIMD lanes.
//
// Work split.  The k kept values of a row are cut into P parts of equal size
// (P a power of two, at most 64).  One lane decodes one part, and the P lanes
// of a row sit next to each other in a wave, so every lane of a wave runs the
// same number of steps and the row's partial sums combine with a fixed
// shuffle butterfly (deterministic).  A wave copies the compressed bytes of
// its 64/P rows -- bitmap words, sign/mantissa fields, exponent codes and the
// per-block kept counts and code offsets -- from HBM into its own LDS region
// with 16-byte loads, each byte once, and decodes from there.  x is staged
// once per workgroup.
//
// Decode.  A lane first finds where its part starts: the block from the
// kept-before counts of the estimated block and its neighbours, the bit inside
// the block and the start of its code by binary search over popcounts.  Then
// it takes U values per group from three windows read at its bit positions
// (two LDS words and a funnel shift each): 64 keep bits, 32 code bits and 32
// field bits.  Per value: position = find-first-set of the keep window, rank
// = count-trailing-zeros of the code window, field = bit-field extract, weight
// = one LDS table entry indexed by (rank, field), a bf16 pattern (exact for
// m <= 7) multiplied with x's bf16 by one dot-product instruction.  A group
// whose windows do not hold U values for every lane of the wave runs as two
// half groups; only a half that still falls short (codes of 32 bits or more,
// long runs of pruned positions) is decoded one value at a time by the
// general step.  The part's last group is masked.
#include <stdlib.h>
#include <string.h>

#include <algorithm>

#include "internal.hpp"
#include "staged_decode.hpp"

namespace cass {

namespace {

constexpr int kBalThreads = 256;
constexpr int kBalWaves = kBalThreads / 64;
constexpr int kRanks = 32;     // ranks of the (rank, field) -> weight table
constexpr int kSlack = 8;      // LDS words after each staged section (window look-ahead)
constexpr int kMaxFw = 6;      // field widths the table path serves (table <= 8 KB)
constexpr int64_t kBalMaxLds = 150 * 1024;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct BalGeom {
  int P, logP, rpw;     // parts per row, log2(P), rows per wave round (64 / P)
  int nb_top;           // largest power of two <= blocks per row
  float nb_per_k;       // blocks per row / kept per row (block estimate of a value)
  int64_t nrounds;      // wave rounds: ceil(rows / rpw)
  int lut_off;          // LDS byte offsets (x at 0)
  int wave_off, wave_bytes;
  int kb_off, bo_off, bm_off, f_off, c_off;  // inside a wave region
  int sb_off;           // inside a wave region: superblock code bases (format 4)
  int perm_off;         // inside a wave region: the wave's copy of the rank table (C-1)
  int c_cap;            // code words a wave region holds
  int lds_bytes;
  uint32_t xstride;     // LDS bytes between the batch rows of x
  uint32_t word_bits;   // 27: width of a word index in a bit position (a kernel
                        // argument, so the extract stays one instruction)
};

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Bit index of the set bit of rank n (0-based) in the 256-bit little-endian
// word array q, or ~0 when q holds n or fewer set bits: binary search over
// popcounts of halves, quarters and words, then a select inside the word.
__device__ __forceinline__ uint32_t select256(const uint32_t (&q)[8], int n) {
  const int c4 = __builtin_popcount(q[0]) + __builtin_popcount(q[1]) + __builtin_popcount(q[2]) +
                 __builtin_popcount(q[3]);
  const bool h = n >= c4;
  n -= h ? c4 : 0;
  const uint32_t a0 = h ? q[4] : q[0], a1 = h ? q[5] : q[1], a2 = h ? q[6] : q[2],
                 a3 = h ? q[7] : q[3];
  const int c2 = __builtin_popcount(a0) + __builtin_popcount(a1);
  const bool hq = n >= c2;
  n -= hq ? c2 : 0;
  const uint32_t b0 = hq ? a2 : a0, b1 = hq ? a3 : a1;
  const int c1 = __builtin_popcount(b0);
  const bool hw = n >= c1;
  n -= hw ? c1 : 0;
  const uint32_t wd = hw ? b1 : b0;
  if (n >= __builtin_popcount(wd)) return ~0u;
  return (h ? 128u : 0u) + (hq ? 64u : 0u) + (hw ? 32u : 0u) + (uint32_t)select_bit(wd, n + 1);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(4))) const unsigned long long const_u64;

// Issues the copy of n 16-byte chunks from global memory to LDS by LDS DMA:
// one instruction per 64 chunks, lane i's chunk landing at dst + 16 i (the
// LDS address is the wave's, so dst must be uniform).  Nontemporal: each
// byte is read once.  Completion is awaited by wait_dma.
__device__ __forceinline__ void dma_run(const u32x4* src, u32x4* dst, int n, int lane) {
  CASS_DCHECK((((uintptr_t)src | (uintptr_t)dst) & 15) == 0, CASS_DBG_ALIGN);
  for (int base = 0; base < n; base += 64)
    if (base + lane < n)
      __builtin_amdgcn_global_load_lds((const void*)(src + base + lane), (lds_void*)(dst + base),
                                       16, 0, 2 /* nt */);
}

// Waits for every global load and LDS DMA of the wave (vmcnt 0), then makes
// the LDS contents visible to all its lanes.
__device__ __forceinline__ void wait_dma() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  wave_sync();
}

typedef __attribute__((address_space(3))) const uint16_t lds_u16;
typedef __attribute__((address_space(3))) const uint8_t lds_u8;

// LDS byte address of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(lds_u8*)p;
}

// x element at LDS byte address a (bf16 pattern -> fp32).
__device__ __forceinline__ float x_at_addr(uint32_t a) {
  return __uint_as_float((uint32_t)(*(lds_u16*)(uintptr_t)a) << 16);
}

// One value, any sparsity and any code length: the next kept position at or
// after bp, its field at fp and its code at cp (codes from `cw`, LDS or
// global memory).  x element j of batch row bb is at byte xs + 2*j + bb*xstride.
template <int BATCH>
__device__ __forceinline__ void c1_step(const uint32_t* bm_l, uint32_t& bp, const uint32_t* f_l,
                                        uint32_t& fp, const uint32_t* cw, uint32_t& cp,
                                        uint32_t rowbit, int64_t row_len, const uint32_t* lut,
                                        const uint8_t* perm, int m, const uint8_t* xs,
                                        uint32_t xstride, float* acc) {
  const int fw = 1 + m;
  uint32_t w = window32(bm_l, bp);
  // a valid part always has its next value inside the row (rowbit + C); the
  // bound only keeps a corrupt stream from spinning
  for (uint32_t lim = rowbit + (uint32_t)row_len; w == 0u && bp < lim;) {
    bp += 32u;
    w = window32(bm_l, bp);
  }
  const uint32_t pos = bp + (uint32_t)__builtin_ctz(w);
  bp = pos + 1u;
  const uint32_t f = window32(f_l, fp) & ((1u << fw) - 1u);
  fp += (uint32_t)fw;
  const int r = unary_at(cw, cp);
  uint32_t bits;
  if (r < kRanks)
    bits = lut[((uint32_t)r << fw) | f] << 16;
  else
    bits = ((f >> m) << 31) | ((uint32_t)perm[r] << 23) | ((f & ((1u << m) - 1u)) << (23 - m));
  const float wv = __uint_as_float(bits);
  const uint32_t xa = 2u * (pos - rowbit);
#pragma unroll
  for (int bb = 0; bb < BATCH; ++bb)
    acc[bb] = __builtin_fmaf(wv, x_at(xs, xa + bb * xstride), acc[bb]);
}

// The raw LDS words behind a group's three windows: three bitmap words at
// bp, two field words at fp, two code words at cp.  They are read one group
// ahead, together with the current group's table and x reads, so a group
// waits for LDS once.
struct Raw {
  uint32_t q0, q1, q2, f0, f1, c0, c1;
};

typedef __attribute__((address_space(3))) const uint32_t lds_u32;

// LDS word holding bit `pos` of a stream staged at LDS byte address `base`:
// word index by bit-field extract, then one shift-and-add.  `wb` = 27 comes
// from a kernel argument; with a literal width the extract is rewritten into
// a shift and a mask (three instructions instead of two).
__device__ __forceinline__ lds_u32* word_at(uint32_t base, uint32_t pos, uint32_t wb) {
  return (lds_u32*)(uintptr_t)(base + (__builtin_amdgcn_ubfe(pos, 5u, wb) << 2));
}

__device__ __forceinline__ Raw load_raw(uint32_t bm_b, uint32_t f_b, uint32_t c_b, uint32_t bp,
                                        uint32_t fp, uint32_t cp, uint32_t wb) {
  lds_u32* qb = word_at(bm_b, bp, wb);
  lds_u32* qf = word_at(f_b, fp, wb);
  lds_u32* qc = word_at(c_b, cp, wb);
  return Raw{qb[0], qb[1], qb[2], qf[0], qf[1], qc[0], qc[1]};
}

typedef __attribute__((address_space(3))) const float lds_f32;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// acc + w * x for a bf16 weight and a bf16 x, each zero-extended to 32 bits
// (the high halves multiply to zero): one dot-product instruction in place of
// a conversion and a fused multiply-add.  A product of two bf16 values is
// exact in fp32.
__device__ __forceinline__ float fma_bf16(uint32_t w, uint32_t x, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                         __builtin_bit_cast(bf16x2_t, x), acc, false);
}

// U values from the windows in `w` (read at bp, fp, cp), each window holding
// at least U values: 64 keep bits, 32 field bits, 32 code bits.  Three phases:
// positions, ranks and fields for all U values (VALU only); every table and x
// read of the group plus the next group's window words (LDS only); the U
// products.  With MASKED, slots u >= t add nothing (the part's last group).
// With ADVANCE (the default when not MASKED) the positions advance past the U
// slots and `w` receives the next group's words; a masked group advances
// correctly only for lanes whose t is U (the others have no values left).
//   lutb  LDS byte address of the (rank, field) -> bf16 table (u32 entries)
//   xorg  LDS byte address of x for staged bitmap bit 0
template <int BATCH, int U, bool MASKED, bool ADVANCE = !MASKED>
__device__ __forceinline__ void c1_group(Raw& w, uint32_t& bp, uint32_t& fp, uint32_t& cp,
                                         uint32_t bm_b, uint32_t f_b, uint32_t c_b,
                                         uint32_t xorg, uint32_t lutb,
                                         int fw, uint32_t xstride, uint32_t wb, int t, float* acc) {
  const uint32_t sb = bp & 31u;
  const uint32_t lo0 = __builtin_amdgcn_alignbit(w.q1, w.q0, sb);
  // (MASKED: the windows may hold only t values; a set bit 63 keeps the
  // positions of slots u >= t inside the window, and a set code bit 31 their
  // ranks inside the table)
  const uint32_t hi0 = __builtin_amdgcn_alignbit(w.q2, w.q1, sb) | (MASKED ? 0x80000000u : 0u);
  const uint32_t wf = __builtin_amdgcn_alignbit(w.f1, w.f0, fp & 31u);
  const uint32_t wc0 = __builtin_amdgcn_alignbit(w.c1, w.c0, cp & 31u);
  // phase 1: addresses
  uint32_t la[U], xa[U];
  uint32_t lo = lo0, wc = wc0, p = 0;
  const uint32_t xlo = xorg + 2u * bp, xhi = xlo + 64u;
  uint32_t xs = xlo;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    // the window holds U keep bits: lo runs out at most once
    const bool z = lo == 0u;
    lo = z ? hi0 : lo;
    xs = z ? xhi : xs;
    p = (uint32_t)__builtin_ctz(lo);
    lo &= lo - 1u;
    // code = r zeros, then a one
    const uint32_t r = (uint32_t)__builtin_ctz(MASKED ? wc | 0x80000000u : wc);
    wc = (wc >> r) >> 1;
    const uint32_t f = __builtin_amdgcn_ubfe(wf, (uint32_t)(u * fw), (uint32_t)fw);
    la[u] = lutb + 4u * ((r << fw) | f);
    xa[u] = xs + 2u * p;
  }
  if (ADVANCE) {
    bp += ((xs - xlo) >> 1) + p + 1u;
    fp += (uint32_t)(U * fw);
    // bits the U codes took: the window was shifted right by that many
    const uint32_t c0 = (uint32_t)__builtin_clz(wc0);
    cp += (wc ? (uint32_t)__builtin_clz(wc) : 32u) - c0;
  }
  __builtin_amdgcn_sched_barrier(0);
  // phase 2: every LDS read of the group
  uint32_t wv[U], xv[BATCH][U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    wv[u] = *(lds_u32*)(uintptr_t)la[u];
#pragma unroll
    for (int bb = 0; bb < BATCH; ++bb) xv[bb][u] = *(lds_u16*)(uintptr_t)(xa[u] + bb * xstride);
  }
  if (ADVANCE) w = load_raw(bm_b, f_b, c_b, bp, fp, cp, wb);
  __builtin_amdgcn_sched_barrier(0);
  // phase 3: products
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int bb = 0; bb < BATCH; ++bb) {
      const float a = fma_bf16(wv[u], xv[bb][u], acc[bb]);
      acc[bb] = (MASKED && u >= t) ? acc[bb] : a;
    }
  }
}

// Where one lane's part stands: bit positions in the staged words.
struct Part {
  uint32_t bp, fp, cp, rowbit;
  int n;
  int64_t cabs;  // absolute code bit of the part's first value
};

// SB: format 4 -- a u64 code base per superblock of 16 blocks and u16 block
// offsets from it, in place of the u64 row base and u32 block offsets.
template <int BATCH, int U, bool SB>
__global__ void __launch_bounds__(kBalThreads) k_gemv_c1_bal(SpecViewC1 v, Shape sh, BalGeom g,
                                                             const uint16_t* __restrict__ x,
                                                             int64_t ldx, float* __restrict__ y,
                                                             int64_t ldy) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int64_t R = sh.rows, C = sh.cols, k = sh.keep;
  const int B = (int)sh.block, nb = (int)(C / B), nwb = B / 32;
  const int m = sh.mant, fw = 1 + m;
  const uint32_t fmask = (1u << fw) - 1u;
  // (wave index made visibly uniform so that per-round values and the row
  // bases of the first round come through scalar registers and loads)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t* lut = reinterpret_cast<uint32_t*>(smem + g.lut_off);  // bf16 patterns
  uint8_t* reg = smem + g.wave_off + wave * g.wave_bytes;
  uint16_t* kb_l = reinterpret_cast<uint16_t*>(reg + g.kb_off);
  uint32_t* bo_l = reinterpret_cast<uint32_t*>(reg + g.bo_off);
  uint16_t* bo16_l = reinterpret_cast<uint16_t*>(reg + g.bo_off);
  unsigned long long* sb_l = reinterpret_cast<unsigned long long*>(reg + g.sb_off);
  const int64_t nsb = SB ? v.nsb : 0;
  uint32_t* bm_l = reinterpret_cast<uint32_t*>(reg + g.bm_off);
  uint32_t* f_l = reinterpret_cast<uint32_t*>(reg + g.f_off);
  uint32_t* c_l = reinterpret_cast<uint32_t*>(reg + g.c_off);

  const int rl = lane >> g.logP, part = lane & (g.P - 1);
  const int n_min = (int)(k >> g.logP);  // each part has n_min or n_min + 1 values
  const int n_max = (int)((k + g.P - 1) >> g.logP);
  const int G = n_min / U;               // fast groups every part can take
  const int n_tail = n_max - G * U;      // values after them (upper bound)
  const int64_t wpr = C / 32;            // bitmap words per row
  const int64_t nwaves = (int64_t)gridDim.x * kBalWaves;
  const int nlut = kRanks << fw;

  // ---- one round's staging.  Every section of the round is copied to the
  // wave's LDS region by LDS DMA (64 chunks of 16 bytes per instruction), all
  // in flight at once; only the codes wait for the row bases.
  struct Plan {
    int64_t row0;
    int rows_here;
    int kb_sh, bo_sh, sb_sh;      // entries before the round's first one in the staged kb / bo / sb
    int64_t bm_a0, f_a0, c_a0;    // first staged word of bitmap, fields and codes
    bool c_in_lds;
  };
  auto plan = [&](int64_t round) {
    Plan pl;
    pl.row0 = round * g.rpw;
    pl.rows_here = (int)((R - pl.row0 < g.rpw) ? R - pl.row0 : g.rpw);
    pl.kb_sh = (int)((pl.row0 * nb) & 7);
    pl.bo_sh = (int)((pl.row0 * nb) & (SB ? 7 : 3));
    pl.sb_sh = SB ? (int)((pl.row0 * nsb) & 1) : 0;
    pl.bm_a0 = (pl.row0 * wpr) & ~(int64_t)3;
    pl.f_a0 = ((pl.row0 * k * fw) >> 5) & ~(int64_t)3;
    pl.c_a0 = 0;
    pl.c_in_lds = false;
    return pl;
  };
  // block metadata, bitmap words and fields (no dependence on loaded data)
  auto stage_fixed = [&](const Plan& pl) {
    const int64_t e0 = pl.row0 * nb, e1 = e0 + (int64_t)pl.rows_here * nb;
    const int64_t kb1 = std::min<int64_t>((e1 + 7) & ~(int64_t)7, v.keptb_limit);
    CASS_DCHECK(((kb1 - (e0 - pl.kb_sh)) >> 3) * 16 <= g.bo_off - g.kb_off, CASS_DBG_STAGE);
    dma_run(reinterpret_cast<const u32x4*>(v.keptb + (e0 - pl.kb_sh)),
            reinterpret_cast<u32x4*>(kb_l), (int)((kb1 - (e0 - pl.kb_sh)) >> 3), lane);
    if (SB) {
      // u16 block offsets (eight per chunk) and u64 superblock bases (two per chunk)
      const int64_t o1 = std::min<int64_t>((e1 + 7) & ~(int64_t)7, 2 * v.blkoff_limit);
      CASS_DCHECK(((o1 - (e0 - pl.bo_sh)) >> 3) * 16 <= g.sb_off - g.bo_off, CASS_DBG_STAGE);
      dma_run(reinterpret_cast<const u32x4*>(v.blkoff16 + (e0 - pl.bo_sh)),
              reinterpret_cast<u32x4*>(bo16_l), (int)((o1 - (e0 - pl.bo_sh)) >> 3), lane);
      const int64_t s0 = pl.row0 * nsb, s1 = (pl.row0 + pl.rows_here) * nsb;
      const int64_t q1 = std::min<int64_t>((s1 + 1) & ~(int64_t)1, v.sbbase_limit);
      CASS_DCHECK(((q1 - (s0 - pl.sb_sh)) >> 1) * 16 <= g.bm_off - g.sb_off, CASS_DBG_STAGE);
      dma_run(reinterpret_cast<const u32x4*>(v.sbbase + (s0 - pl.sb_sh)),
              reinterpret_cast<u32x4*>(sb_l), (int)((q1 - (s0 - pl.sb_sh)) >> 1), lane);
    } else {
      const int64_t bo1 = std::min<int64_t>((e1 + 3) & ~(int64_t)3, v.blkoff_limit);
      CASS_DCHECK(((bo1 - (e0 - pl.bo_sh)) >> 2) * 16 <= g.sb_off - g.bo_off, CASS_DBG_STAGE);
      dma_run(reinterpret_cast<const u32x4*>(v.blkoff + (e0 - pl.bo_sh)),
              reinterpret_cast<u32x4*>(bo_l), (int)((bo1 - (e0 - pl.bo_sh)) >> 2), lane);
    }
    const int64_t bm1 = std::min<int64_t>(((pl.row0 + pl.rows_here) * wpr + 3) & ~(int64_t)3,
                                          v.bitmap_limit);
    CASS_DCHECK(((bm1 - pl.bm_a0) >> 2) * 16 <= g.f_off - g.bm_off, CASS_DBG_STAGE);
    dma_run(reinterpret_cast<const u32x4*>(v.bitmap + pl.bm_a0), reinterpret_cast<u32x4*>(bm_l),
            (int)((bm1 - pl.bm_a0) >> 2), lane);
    const int64_t fb1 = (pl.row0 + pl.rows_here) * k * fw;
    const int64_t f1 = std::min<int64_t>((((fb1 + 31) >> 5) + 3) & ~(int64_t)3, v.fields_limit);
    CASS_DCHECK(((f1 - pl.f_a0) >> 2) * 16 <= g.c_off - g.f_off, CASS_DBG_STAGE);
    dma_run(reinterpret_cast<const u32x4*>(v.fields + pl.f_a0), reinterpret_cast<u32x4*>(f_l),
            (int)((f1 - pl.f_a0) >> 2), lane);
  };
  // the codes of the round's rows, bits [cb0, cb1)
  auto stage_codes = [&](Plan& pl, int64_t cb0, int64_t cb1) {
    pl.c_a0 = (cb0 >> 5) & ~(int64_t)3;
    const int64_t c1 = std::min<int64_t>((((cb1 + 31) >> 5) + 3) & ~(int64_t)3, v.codes_limit);
    const int n = (int)((c1 - pl.c_a0) >> 2);
    pl.c_in_lds = n * 4 <= g.c_cap;
    CASS_DCHECK(!pl.c_in_lds || n * 16 <= g.perm_off - g.c_off, CASS_DBG_STAGE);
    if (pl.c_in_lds)
      dma_run(reinterpret_cast<const u32x4*>(v.codes + pl.c_a0), reinterpret_cast<u32x4*>(c_l), n,
              lane);
  };
  auto load_bounds = [&](int64_t round, int64_t& cb0, int64_t& cb1, int64_t& rowcb) {
    const int64_t r0 = round * g.rpw, r1 = r0 + g.rpw;
    // the round's two bounds through the scalar cache (the table is read-only
    // here), so that the codes' copy waits for nothing else
    // (format 4: a row's first code bit is its first superblock's base)
    const const_u64* rb = (const const_u64*)(SB ? v.sbbase : v.rowbase);
    const int64_t rs = SB ? nsb : 1;
    cb0 = (int64_t)rb[r0 * rs];
    cb1 = r1 < R ? (int64_t)rb[r1 * rs] : v.codes_limit * 32;
    rowcb = r0 + rl < R ? (int64_t)(SB ? v.sbbase : v.rowbase)[(r0 + rl) * rs] : 0;
  };

  // Where this lane's part of the round starts.  The block holding its first
  // value: the kept counts of the estimated block and its neighbours, read at
  // once (the estimate k / nb values per block is almost always within one
  // block; otherwise a stepping search).  The bit inside the block: binary
  // search over popcounts of the block's words.  The code: the same select
  // over the code ones, from the block's code offset.  Per-lane offsets are
  // 32-bit (bit positions in the staged regions, kept indices in a row); the
  // round's bases are uniform.
  auto locate = [&](const Plan& pl, int64_t rowcb) {
    Part pt;
    const uint32_t uk = (uint32_t)k;
    const uint32_t i0 = ((uint32_t)part * uk) >> g.logP;
    pt.n = rl < pl.rows_here ? (int)((((uint32_t)part + 1u) * uk) >> g.logP) - (int)i0 : 0;
    pt.rowbit = (uint32_t)((pl.row0 * wpr - pl.bm_a0) * 32) + (uint32_t)rl * (uint32_t)C;
    pt.bp = pt.rowbit;
    pt.fp = 0;
    pt.cp = 0;
    pt.cabs = 0;
    if (pt.n <= 0) return pt;
    const uint16_t* kbr = kb_l + pl.kb_sh + rl * nb;
    // kept before block j, for any j (0 before the row, k after it)
    auto kb_at = [&](int j) -> int { return j <= 0 ? 0 : (j >= nb ? (int)k : (int)kbr[j]); };
    int e = (int)((float)i0 * g.nb_per_k);
    e = e < 0 ? 0 : (e >= nb ? nb - 1 : e);
    const int km = kb_at(e - 1), k0 = kb_at(e), k1 = kb_at(e + 1), k2 = kb_at(e + 2);
    const int ii = (int)i0;
    int b = e - 1 + (k0 <= ii ? 1 : 0) + (k1 <= ii ? 1 : 0);
    int kbb = b == e - 1 ? km : (b == e ? k0 : k1);
    if (!(km <= ii && ii < k2)) {
      // (rare) the estimate is two or more blocks off
      b = e;
      for (int it = 0; it < nb; ++it) {
        const int lo = kb_at(b), hi = kb_at(b + 1);
        if (lo > ii && b > 0) --b;
        else if (hi <= ii && b + 1 < nb) ++b;
        else break;
      }
      kbb = kb_at(b);
    }
    const int skip = ii - kbb;
    const uint32_t* bw = bm_l + (pt.rowbit >> 5) + b * nwb;
    uint32_t inblk;
    if (nwb == 8) {
      uint32_t q[8];
#pragma unroll
      for (int w = 0; w < 8; ++w) q[w] = bw[w];
      inblk = select256(q, skip);
      inblk = inblk == ~0u ? 0u : inblk;  // (corrupt streams only: stay inside the block)
    } else {
      int wi = 0, rem = skip;
      uint32_t wd = bw[0];
      for (;;) {
        const int c = __builtin_popcount(wd);
        if (rem < c || wi == nwb - 1) break;  // (the second test: corrupt streams only)
        rem -= c;
        wd = bw[++wi];
      }
      inblk = (uint32_t)(wi * 32 + select_bit(wd, rem + 1));
    }
    pt.bp = pt.rowbit + (uint32_t)(b * B) + inblk;
    pt.fp = (uint32_t)(pl.row0 * k * fw - pl.f_a0 * 32) + ((uint32_t)rl * uk + i0) * (uint32_t)fw;
    // the codes: the block's code offset, then `skip` codes on
    // the block's first code bit, from the row's first
    const uint32_t bo =
        SB ? (uint32_t)(sb_l[pl.sb_sh + rl * nsb + (b >> v.sb_log)] - (unsigned long long)rowcb) +
                 bo16_l[pl.bo_sh + rl * nb + b]
           : bo_l[pl.bo_sh + rl * nb + b];
    pt.cabs = rowcb + bo;
    if (pl.c_in_lds) {
      const uint32_t cpos = (uint32_t)(rowcb - pl.c_a0 * 32) + bo;
      pt.cp = cpos;
      if (skip > 0) {
        // the skip-th one bit at or after cpos, among the next 256 - (cpos & 31) bits
        uint32_t q[8];
        const uint32_t* qc = c_l + (cpos >> 5);
#pragma unroll
        for (int w = 0; w < 8; ++w) q[w] = qc[w];
        q[0] &= ~0u << (cpos & 31u);
        const uint32_t idx = select256(q, skip - 1);
        pt.cp = idx != ~0u ? (cpos & ~31u) + idx + 1u : skip_codes(c_l, cpos, skip);
      }
    } else {
      pt.cp = skip_codes(v.codes + (pt.cabs >> 5), (uint32_t)(pt.cabs & 31), skip);
    }
    return pt;
  };

  // ---- first round, x and the (rank, field) -> bf16 table.  Every copy of
  // the first round is in flight at once: the rank table, the sections, the
  // codes (whose range needs only the two row bases, scalar loads) and x.
  int64_t round = (int64_t)blockIdx.x * kBalWaves + wave;
  const uint8_t* perm_l = reg + g.perm_off;
  dma_run(reinterpret_cast<const u32x4*>(v.perm), reinterpret_cast<u32x4*>(reg + g.perm_off), 16,
          lane);
  const bool first = round < g.nrounds;
  Plan pl{};
  int64_t cb0 = 0, cb1 = 0, rowcb = 0;
  if (first) {
    pl = plan(round);
    stage_fixed(pl);
  }
  const bool x_dma = (C & 7) == 0 && ((uintptr_t)x & 15) == 0 && (ldx & 7) == 0;
  for (int bb = 0; bb < BATCH; ++bb) {
    uint16_t* xr = reinterpret_cast<uint16_t*>(smem + bb * g.xstride);
    const uint16_t* xg = x + bb * ldx;
    if (x_dma) {
      // the workgroup's waves take interleaved runs of 64 chunks
      const int nx = (int)(C >> 3);
      for (int base = wave * 64; base < nx; base += kBalThreads)
        dma_run(reinterpret_cast<const u32x4*>(xg) + base, reinterpret_cast<u32x4*>(xr) + base,
                nx - base < 64 ? nx - base : 64, lane);
    } else {
      for (int64_t j = threadIdx.x; j < C; j += kBalThreads) xr[j] = xg[j];
    }
    // zeros after the row: masked slots of a part's last group may read there
    if (threadIdx.x < 128) xr[C + threadIdx.x] = 0;
  }
  // (after every copy that does not need them: a scalar-load wait covers all
  // scalar loads in flight)
  if (first) {
    load_bounds(round, cb0, cb1, rowcb);
    stage_codes(pl, cb0, cb1);
  }
  wait_dma();  // the rank table, this wave's sections and codes, its x chunks
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = threadIdx.x + kBalThreads * j;
    if (i < nlut) {
      const uint32_t f = (uint32_t)i & fmask;
      // (m <= 7: the fp32 pattern's low 16 bits are zero, so the value is a bf16)
      lut[i] = (((f >> m) << 31) | ((uint32_t)perm_l[i >> fw] << 23) |
                ((f & ((1u << m) - 1u)) << (23 - m))) >> 16;
    }
  }
  Part pt{};
  if (first) pt = locate(pl, rowcb);
  __syncthreads();  // x (every wave's chunks) and the table are in LDS
  if (!first) return;

  for (;;) {
    const int64_t next = round + nwaves;
    const bool more = next < g.nrounds;
    // the next round's row bases load while this round decodes
    int64_t ncb0 = 0, ncb1 = 0, nrowcb = 0;
    if (more) load_bounds(next, ncb0, ncb1, nrowcb);

    const bool active = rl < pl.rows_here;
    const int n = pt.n;
    uint32_t bp = pt.bp, fp = pt.fp, cp = pt.cp;
    const uint32_t rowbit = pt.rowbit;
    float acc[BATCH];
#pragma unroll
    for (int bb = 0; bb < BATCH; ++bb) acc[bb] = 0.f;

    // rounds where every lane has a part and the codes sit in LDS take the
    // grouped path; others (last partial round, tiny k, codes over the LDS
    // share) decode one value at a time
    const bool grouped = pl.c_in_lds && pl.rows_here == g.rpw && n_min > 0;
    if (grouped) {
      const uint32_t xorg = lds_addr(smem) - 2u * rowbit;  // x address of staged bit 0
      const uint32_t lutb = lds_addr(reinterpret_cast<const uint8_t*>(lut));
      const uint32_t bm_b = lds_addr(reinterpret_cast<const uint8_t*>(bm_l));
      const uint32_t f_b = lds_addr(reinterpret_cast<const uint8_t*>(f_l));
      const uint32_t c_b = lds_addr(reinterpret_cast<const uint8_t*>(c_l));
      Raw w = load_raw(bm_b, f_b, c_b, bp, fp, cp, g.word_bits);
      // full groups: runs of fast groups; a group whose windows fall short
      // for some lane goes value by value
      int gi = 0;
      auto fits = [&](int need) {
        const uint32_t sb = bp & 31u;
        const int have = __builtin_popcount(__builtin_amdgcn_alignbit(w.q1, w.q0, sb)) +
                         __builtin_popcount(__builtin_amdgcn_alignbit(w.q2, w.q1, sb));
        const int ncode = __builtin_popcount(__builtin_amdgcn_alignbit(w.c1, w.c0, cp & 31u));
        return __all(min(have, ncode) >= need);
      };
      while (gi < G) {
        // two groups per iteration, so the window words of the next group
        // alternate between two register sets instead of being copied back
        for (; gi + 1 < G; gi += 2) {
          if (!fits(U)) break;
          c1_group<BATCH, U, false>(w, bp, fp, cp, bm_b, f_b, c_b, xorg, lutb, fw, g.xstride, g.word_bits, U,
                                    acc);
          if (!fits(U)) { ++gi; break; }
          c1_group<BATCH, U, false>(w, bp, fp, cp, bm_b, f_b, c_b, xorg, lutb, fw, g.xstride, g.word_bits, U,
                                    acc);
        }
        if (gi + 1 == G && fits(U)) {
          c1_group<BATCH, U, false>(w, bp, fp, cp, bm_b, f_b, c_b, xorg, lutb, fw, g.xstride, g.word_bits, U,
                                    acc);
          ++gi;
        }
        if (gi < G) {
          // some lane's windows hold fewer than U values: the group as two halves
          // (windows short of U/2 values are far rarer), value by value only if
          // a half falls short too (codes of 32+ bits, long runs of pruned values)
          constexpr int H = U / 2;
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const uint32_t sbh = bp & 31u;
            const int hv = __builtin_popcount(__builtin_amdgcn_alignbit(w.q1, w.q0, sbh)) +
                           __builtin_popcount(__builtin_amdgcn_alignbit(w.q2, w.q1, sbh));
            const int hc = __builtin_popcount(__builtin_amdgcn_alignbit(w.c1, w.c0, cp & 31u));
            if (__all(min(hv, hc) >= H)) {
              c1_group<BATCH, H, false>(w, bp, fp, cp, bm_b, f_b, c_b, xorg, lutb, fw, g.xstride,
                                        g.word_bits, H, acc);
            } else {
              for (int u = 0; u < H; ++u)
                c1_step<BATCH>(bm_l, bp, f_l, fp, c_l, cp, rowbit, C, lut, perm_l, m, smem,
                               g.xstride, acc);
              w = load_raw(bm_b, f_b, c_b, bp, fp, cp, g.word_bits);
            }
          }
          ++gi;
        }
      }
      // the part's last t = n - G*U <= U values
      if (n_tail > 0) {
        const int t = n - G * U;
        const uint32_t sb = bp & 31u;
        const int have = __builtin_popcount(__builtin_amdgcn_alignbit(w.q1, w.q0, sb)) +
                         __builtin_popcount(__builtin_amdgcn_alignbit(w.q2, w.q1, sb));
        const int ncode = __builtin_popcount(__builtin_amdgcn_alignbit(w.c1, w.c0, cp & 31u));
        if (__all(min(have, ncode) >= t)) {
          c1_group<BATCH, U, true>(w, bp, fp, cp, bm_b, f_b, c_b, xorg, lutb, fw, g.xstride, g.word_bits, t,
                                   acc);
        } else {
          // in two halves, as for a full group that falls short
          constexpr int H = U / 2;
          const int t1 = t < H ? t : H, t2 = t - t1;
          if (__all(min(have, ncode) >= t1)) {
            c1_group<BATCH, H, true, true>(w, bp, fp, cp, bm_b, f_b, c_b, xorg, lutb, fw,
                                           g.xstride, g.word_bits, t1, acc);
            const uint32_t sb2 = bp & 31u;
            const int have2 = __builtin_popcount(__builtin_amdgcn_alignbit(w.q1, w.q0, sb2)) +
                              __builtin_popcount(__builtin_amdgcn_alignbit(w.q2, w.q1, sb2));
            const int ncode2 = __builtin_popcount(__builtin_amdgcn_alignbit(w.c1, w.c0, cp & 31u));
            if (__all(min(have2, ncode2) >= t2)) {
              c1_group<BATCH, H, true>(w, bp, fp, cp, bm_b, f_b, c_b, xorg, lutb, fw, g.xstride,
                                       g.word_bits, t2, acc);
            } else {
              for (int u = 0; u < H; ++u)
                if (u < t2)
                  c1_step<BATCH>(bm_l, bp, f_l, fp, c_l, cp, rowbit, C, lut, perm_l, m, smem,
                                 g.xstride, acc);
            }
          } else {
            for (int u = 0; u < U; ++u)
              if (u < t)
                c1_step<BATCH>(bm_l, bp, f_l, fp, c_l, cp, rowbit, C, lut, perm_l, m, smem,
                               g.xstride, acc);
          }
        }
      }
    } else if (pl.c_in_lds) {
      for (int i = 0; i < n_max; ++i)
        if (i < n)
          c1_step<BATCH>(bm_l, bp, f_l, fp, c_l, cp, rowbit, C, lut, perm_l, m, smem, g.xstride,
                         acc);
    } else {
      // codes straight from global memory (a round whose codes exceed the LDS share)
      const uint32_t* cg = v.codes + (pt.cabs >> 5);
      uint32_t cpg = cp;
      for (int i = 0; i < n_max; ++i)
        if (i < n)
          c1_step<BATCH>(bm_l, bp, f_l, fp, cg, cpg, rowbit, C, lut, perm_l, m, smem, g.xstride,
                         acc);
    }

    if (n == 0) {
#pragma unroll
      for (int bb = 0; bb < BATCH; ++bb) acc[bb] = 0.f;
    }
    for (int o = g.P >> 1; o >= 1; o >>= 1) {
#pragma unroll
      for (int bb = 0; bb < BATCH; ++bb) acc[bb] += __shfl_xor(acc[bb], o, 64);
    }
    if (active && part == 0) {
#pragma unroll
      for (int bb = 0; bb < BATCH; ++bb) y[bb * ldy + pl.row0 + rl] = acc[bb];
    }
    if (!more) break;
    wave_sync();  // every lane is done with the staged words before they are replaced
    pl = plan(next);
    stage_fixed(pl);
    stage_codes(pl, ncb0, ncb1);
    wait_dma();
    pt = locate(pl, nrowcb);
    round = next;
  }
}


// ---- Cassandra-2: no exponent codes; the exponent of a kept value is the
// shared exponent of its 32-position group (one byte per bitmap word).  A
// value is ldexp(+-a, E - 127 - m) for its (m+2)-bit field (sign, aligned
// significand a): a table gives +-a as fp32, v_ldexp_f32 the scaling (exact,
// subnormal results included).  Same work split, staging and three-phase
// groups as the Cassandra-1 kernel; a part's start needs no code search.
// (Method: Cassandra review, section 3.2, Cassandra-2; OCP MX specification.)

struct C2Raw {
  uint32_t q0, q1, q2, f0, f1;
};
__device__ __forceinline__ C2Raw c2raw(const uint32_t* bm_l, const uint32_t* f_l, uint32_t bp,
                                       uint32_t fp) {
  const uint32_t* qb = bm_l + (bp >> 5);
  const uint32_t* qf = f_l + (fp >> 5);
  return C2Raw{qb[0], qb[1], qb[2], qf[0], qf[1]};
}

typedef __attribute__((address_space(3))) const uint8_t lds_u8v;

// Kept positions in the 64-bit keep window of w at bp.
__device__ __forceinline__ int c2_have(const C2Raw& w, uint32_t bp) {
  const uint32_t sb = bp & 31u;
  return __builtin_popcount(__builtin_amdgcn_alignbit(w.q1, w.q0, sb)) +
         __builtin_popcount(__builtin_amdgcn_alignbit(w.q2, w.q1, sb));
}

// U values from the windows in w.  MASKED: slots u >= t add nothing (the
// part's last group; bit 63 of the keep window set keeps their reads in range).
// ADVANCE (the default when not MASKED): the positions move past the U slots
// and w receives the next windows (for a masked group, right only for lanes
// whose t is U).
//   eorg  LDS byte address of the shared exponent of staged bitmap word 0
template <int BATCH, int U, bool MASKED, bool ADVANCE = !MASKED>
__device__ __forceinline__ void c2_group(C2Raw& w, uint32_t& bp, uint32_t& fp,
                                         const uint32_t* bm_l, const uint32_t* f_l,
                                         uint32_t xorg, uint32_t eorg, uint32_t lutb, int fw,
                                         int ebias, uint32_t xstride, int t, float* acc) {
  const uint32_t sbit = bp & 31u;
  const uint32_t lo0 = __builtin_amdgcn_alignbit(w.q1, w.q0, sbit);
  const uint32_t hi0 = __builtin_amdgcn_alignbit(w.q2, w.q1, sbit) | (MASKED ? 0x80000000u : 0u);
  const uint32_t wf = __builtin_amdgcn_alignbit(w.f1, w.f0, fp & 31u);
  uint32_t la[U], xa[U], ea[U];
  uint32_t lo = lo0, p = 0, base = bp;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const bool z = lo == 0u;
    lo = z ? hi0 : lo;
    base = z ? bp + 32u : base;
    p = (uint32_t)__builtin_ctz(lo);
    lo &= lo - 1u;
    const uint32_t pos = base + p;  // staged bitmap bit
    const uint32_t f = __builtin_amdgcn_ubfe(wf, (uint32_t)(u * fw), (uint32_t)fw);
    la[u] = lutb + 4u * f;
    xa[u] = xorg + 2u * pos;
    ea[u] = eorg + (pos >> 5);
  }
  if (ADVANCE) {
    bp = base + p + 1u;
    fp += (uint32_t)(U * fw);
  }
  __builtin_amdgcn_sched_barrier(0);
  float lv[U], xv[BATCH][U];
  int ev[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    lv[u] = *(lds_f32*)(uintptr_t)la[u];
    ev[u] = *(lds_u8v*)(uintptr_t)ea[u];
#pragma unroll
    for (int bb = 0; bb < BATCH; ++bb) xv[bb][u] = x_at_addr(xa[u] + bb * xstride);
  }
  if (ADVANCE) w = c2raw(bm_l, f_l, bp, fp);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float wv = __builtin_amdgcn_ldexpf(lv[u], ev[u] - ebias);
#pragma unroll
    for (int bb = 0; bb < BATCH; ++bb) {
      const float a = __builtin_fmaf(wv, xv[bb][u], acc[bb]);
      acc[bb] = (MASKED && u >= t) ? acc[bb] : a;
    }
  }
}

// One value at any sparsity: the next kept position at or after bp.
template <int BATCH>
__device__ __forceinline__ void c2_step(const uint32_t* bm_l, uint32_t& bp, const uint32_t* f_l,
                                        uint32_t& fp, uint32_t rowbit, int64_t row_len,
                                        const float* lut, const uint8_t* eb0, int fw, int ebias,
                                        const uint8_t* xs, uint32_t xstride, float* acc) {
  uint32_t w = window32(bm_l, bp);
  for (uint32_t lim = rowbit + (uint32_t)row_len; w == 0u && bp < lim;) {
    bp += 32u;
    w = window32(bm_l, bp);
  }
  const uint32_t pos = bp + (uint32_t)__builtin_ctz(w);
  bp = pos + 1u;
  const uint32_t f = window32(f_l, fp) & ((1u << fw) - 1u);
  fp += (uint32_t)fw;
  const float wv = __builtin_amdgcn_ldexpf(lut[f], (int)eb0[pos >> 5] - ebias);
  const uint32_t xa = 2u * (pos - rowbit);
#pragma unroll
  for (int bb = 0; bb < BATCH; ++bb)
    acc[bb] = __builtin_fmaf(wv, x_at(xs, xa + bb * xstride), acc[bb]);
}

template <int BATCH, int U>
__global__ void __launch_bounds__(kBalThreads) k_gemv_c2_bal(SpecViewC2 v, Shape sh, BalGeom g,
                                                             const uint16_t* __restrict__ x,
                                                             int64_t ldx, float* __restrict__ y,
                                                             int64_t ldy) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int64_t R = sh.rows, C = sh.cols, k = sh.keep;
  const int B = (int)sh.block, nb = (int)(C / B), nwb = B / 32;
  const int m = sh.mant, fw = 2 + m;
  const int ebias = 127 + m;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  float* lut = reinterpret_cast<float*>(smem + g.lut_off);
  uint8_t* reg = smem + g.wave_off + wave * g.wave_bytes;
  uint16_t* kb_l = reinterpret_cast<uint16_t*>(reg + g.kb_off);
  uint32_t* bm_l = reinterpret_cast<uint32_t*>(reg + g.bm_off);
  uint32_t* f_l = reinterpret_cast<uint32_t*>(reg + g.f_off);
  uint8_t* e_l = reg + g.c_off;  // shared exponents (one byte per bitmap word)

  const int rl = lane >> g.logP, part = lane & (g.P - 1);
  const int n_min = (int)(k >> g.logP);
  const int n_max = (int)((k + g.P - 1) >> g.logP);
  const int G = n_min / U;
  const int n_tail = n_max - G * U;
  const int64_t wpr = C / 32;
  const int64_t nwaves = (int64_t)gridDim.x * kBalWaves;

  struct Plan {
    int64_t row0;
    int rows_here, kb_sh;
    int64_t bm_a0, f_a0, e_a0;
  };
  auto plan = [&](int64_t round) {
    Plan pl;
    pl.row0 = round * g.rpw;
    pl.rows_here = (int)((R - pl.row0 < g.rpw) ? R - pl.row0 : g.rpw);
    pl.kb_sh = (int)((pl.row0 * nb) & 7);
    pl.bm_a0 = (pl.row0 * wpr) & ~(int64_t)3;
    pl.f_a0 = ((pl.row0 * k * fw) >> 5) & ~(int64_t)3;
    pl.e_a0 = (pl.row0 * wpr) & ~(int64_t)15;
    return pl;
  };
  auto stage = [&](const Plan& pl) {
    const int64_t e0 = pl.row0 * nb, e1 = e0 + (int64_t)pl.rows_here * nb;
    const int64_t kb1 = std::min<int64_t>((e1 + 7) & ~(int64_t)7, v.keptb_limit);
    dma_run(reinterpret_cast<const u32x4*>(v.keptb + (e0 - pl.kb_sh)),
            reinterpret_cast<u32x4*>(kb_l), (int)((kb1 - (e0 - pl.kb_sh)) >> 3), lane);
    const int64_t w1 = (pl.row0 + pl.rows_here) * wpr;
    const int64_t bm1 = std::min<int64_t>((w1 + 3) & ~(int64_t)3, v.bitmap_limit);
    dma_run(reinterpret_cast<const u32x4*>(v.bitmap + pl.bm_a0), reinterpret_cast<u32x4*>(bm_l),
            (int)((bm1 - pl.bm_a0) >> 2), lane);
    const int64_t fb1 = (pl.row0 + pl.rows_here) * k * fw;
    const int64_t f1 = std::min<int64_t>((((fb1 + 31) >> 5) + 3) & ~(int64_t)3, v.fields_limit);
    dma_run(reinterpret_cast<const u32x4*>(v.fields + pl.f_a0), reinterpret_cast<u32x4*>(f_l),
            (int)((f1 - pl.f_a0) >> 2), lane);
    const int64_t e1b = std::min<int64_t>((w1 + 15) & ~(int64_t)15, v.shexp_limit * 4);
    dma_run(reinterpret_cast<const u32x4*>(v.shexp + pl.e_a0), reinterpret_cast<u32x4*>(e_l),
            (int)((e1b - pl.e_a0) >> 4), lane);
  };
  // Where this lane's part starts: as in the Cassandra-1 kernel (the block
  // from the kept counts of the estimated block and its neighbours in one
  // round trip, the bit by binary search over popcounts); no code search.
  auto locate = [&](const Plan& pl) {
    Part pt;
    const uint32_t uk = (uint32_t)k;
    const uint32_t i0 = ((uint32_t)part * uk) >> g.logP;
    pt.n = rl < pl.rows_here ? (int)((((uint32_t)part + 1u) * uk) >> g.logP) - (int)i0 : 0;
    pt.rowbit = (uint32_t)((pl.row0 * wpr - pl.bm_a0) * 32) + (uint32_t)rl * (uint32_t)C;
    pt.bp = pt.rowbit;
    pt.fp = 0;
    pt.cp = 0;
    pt.cabs = 0;
    if (pt.n <= 0) return pt;
    const uint16_t* kbr = kb_l + pl.kb_sh + rl * nb;
    auto kb_at = [&](int j) -> int { return j <= 0 ? 0 : (j >= nb ? (int)k : (int)kbr[j]); };
    int e = (int)((float)i0 * g.nb_per_k);
    e = e < 0 ? 0 : (e >= nb ? nb - 1 : e);
    const int km = kb_at(e - 1), k0 = kb_at(e), k1 = kb_at(e + 1), k2 = kb_at(e + 2);
    const int ii = (int)i0;
    int b = e - 1 + (k0 <= ii ? 1 : 0) + (k1 <= ii ? 1 : 0);
    int kbb = b == e - 1 ? km : (b == e ? k0 : k1);
    if (!(km <= ii && ii < k2)) {
      b = e;
      for (int it = 0; it < nb; ++it) {
        const int lo = kb_at(b), hi = kb_at(b + 1);
        if (lo > ii && b > 0) --b;
        else if (hi <= ii && b + 1 < nb) ++b;
        else break;
      }
      kbb = kb_at(b);
    }
    const int skip = ii - kbb;
    const uint32_t* bw = bm_l + (pt.rowbit >> 5) + b * nwb;
    uint32_t inblk;
    if (nwb == 8) {
      uint32_t q[8];
#pragma unroll
      for (int w = 0; w < 8; ++w) q[w] = bw[w];
      inblk = select256(q, skip);
      inblk = inblk == ~0u ? 0u : inblk;  // (corrupt streams only: stay inside the block)
    } else {
      int wi = 0, rem = skip;
      uint32_t wd = bw[0];
      for (;;) {
        const int c = __builtin_popcount(wd);
        if (rem < c || wi == nwb - 1) break;  // (the second test: corrupt streams only)
        rem -= c;
        wd = bw[++wi];
      }
      inblk = (uint32_t)(wi * 32 + select_bit(wd, rem + 1));
    }
    pt.bp = pt.rowbit + (uint32_t)(b * B) + inblk;
    pt.fp = (uint32_t)(pl.row0 * k * fw - pl.f_a0 * 32) + ((uint32_t)rl * uk + i0) * (uint32_t)fw;
    return pt;
  };

  // ---- first round, x and the +-significand table
  int64_t round = (int64_t)blockIdx.x * kBalWaves + wave;
  const bool first = round < g.nrounds;
  Plan pl{};
  if (first) {
    pl = plan(round);
    stage(pl);
  }
  const bool x_dma = (C & 7) == 0 && ((uintptr_t)x & 15) == 0 && (ldx & 7) == 0;
  for (int bb = 0; bb < BATCH; ++bb) {
    uint16_t* xr = reinterpret_cast<uint16_t*>(smem + bb * g.xstride);
    const uint16_t* xg = x + bb * ldx;
    if (x_dma) {
      const int nx = (int)(C >> 3);
      for (int base = wave * 64; base < nx; base += kBalThreads)
        dma_run(reinterpret_cast<const u32x4*>(xg) + base, reinterpret_cast<u32x4*>(xr) + base,
                nx - base < 64 ? nx - base : 64, lane);
    } else {
      for (int64_t j = threadIdx.x; j < C; j += kBalThreads) xr[j] = xg[j];
    }
    if (threadIdx.x < 128) xr[C + threadIdx.x] = 0;
  }
  for (int i = threadIdx.x; i < (1 << fw); i += kBalThreads) {
    const float a = (float)(i & ((1 << (m + 1)) - 1));
    lut[i] = (i >> (m + 1)) ? -a : a;
  }
  wait_dma();
  Part pt{};
  if (first) pt = locate(pl);
  __syncthreads();  // x (every wave's chunks) and the table are in LDS
  if (!first) return;

  for (;;) {
    const int64_t next = round + nwaves;
    const bool more = next < g.nrounds;
    const bool active = rl < pl.rows_here;
    const int n = pt.n;
    uint32_t bp = pt.bp, fp = pt.fp;
    const uint32_t rowbit = pt.rowbit;
    const uint8_t* eb0 = e_l + (pl.bm_a0 - pl.e_a0);  // exponent of staged bitmap word 0
    float acc[BATCH];
#pragma unroll
    for (int bb = 0; bb < BATCH; ++bb) acc[bb] = 0.f;

    if (pl.rows_here == g.rpw && n_min > 0) {
      const uint32_t xorg = lds_addr(smem) - 2u * rowbit;
      const uint32_t eorg = lds_addr(eb0);
      const uint32_t lutb = lds_addr(reinterpret_cast<const uint8_t*>(lut));
      C2Raw w = c2raw(bm_l, f_l, bp, fp);
      int gi = 0;
      while (gi < G) {
        // two groups per iteration, as in the Cassandra-1 kernel
        for (; gi + 1 < G; gi += 2) {
          if (!__all(c2_have(w, bp) >= U)) break;
          c2_group<BATCH, U, false>(w, bp, fp, bm_l, f_l, xorg, eorg, lutb, fw, ebias,
                                    g.xstride, U, acc);
          if (!__all(c2_have(w, bp) >= U)) { ++gi; break; }
          c2_group<BATCH, U, false>(w, bp, fp, bm_l, f_l, xorg, eorg, lutb, fw, ebias,
                                    g.xstride, U, acc);
        }
        if (gi + 1 == G && __all(c2_have(w, bp) >= U)) {
          c2_group<BATCH, U, false>(w, bp, fp, bm_l, f_l, xorg, eorg, lutb, fw, ebias,
                                    g.xstride, U, acc);
          ++gi;
        }
        if (gi < G) {
          // some lane's keep window holds fewer than U positions: the group as
          // two parts on the fast path, value by value only if a part falls short
          constexpr int H1 = U / 2, H2 = U - U / 2;
          if (__all(c2_have(w, bp) >= H1)) {
            c2_group<BATCH, H1, false>(w, bp, fp, bm_l, f_l, xorg, eorg, lutb, fw, ebias,
                                       g.xstride, H1, acc);
          } else {
            for (int u = 0; u < H1; ++u)
              c2_step<BATCH>(bm_l, bp, f_l, fp, rowbit, C, lut, eb0, fw, ebias, smem, g.xstride,
                             acc);
            w = c2raw(bm_l, f_l, bp, fp);
          }
          if (__all(c2_have(w, bp) >= H2)) {
            c2_group<BATCH, H2, false>(w, bp, fp, bm_l, f_l, xorg, eorg, lutb, fw, ebias,
                                       g.xstride, H2, acc);
          } else {
            for (int u = 0; u < H2; ++u)
              c2_step<BATCH>(bm_l, bp, f_l, fp, rowbit, C, lut, eb0, fw, ebias, smem, g.xstride,
                             acc);
            w = c2raw(bm_l, f_l, bp, fp);
          }
          ++gi;
        }
      }
      if (n_tail > 0) {
        const int t = n - G * U;
        const uint32_t sb = bp & 31u;
        const int have = __builtin_popcount(__builtin_amdgcn_alignbit(w.q1, w.q0, sb)) +
                         __builtin_popcount(__builtin_amdgcn_alignbit(w.q2, w.q1, sb));
        if (__all(have >= t)) {
          c2_group<BATCH, U, true>(w, bp, fp, bm_l, f_l, xorg, eorg, lutb, fw, ebias, g.xstride,
                                   t, acc);
        } else {
          constexpr int H1 = U / 2, H2 = U - U / 2;
          const int t1 = t < H1 ? t : H1, t2 = t - t1;
          if (__all(have >= t1)) {
            c2_group<BATCH, H1, true, true>(w, bp, fp, bm_l, f_l, xorg, eorg, lutb, fw, ebias,
                                            g.xstride, t1, acc);
            if (__all(c2_have(w, bp) >= t2)) {
              c2_group<BATCH, H2, true>(w, bp, fp, bm_l, f_l, xorg, eorg, lutb, fw, ebias,
                                        g.xstride, t2, acc);
            } else {
              for (int u = 0; u < H2; ++u)
                if (u < t2)
                  c2_step<BATCH>(bm_l, bp, f_l, fp, rowbit, C, lut, eb0, fw, ebias, smem,
                                 g.xstride, acc);
            }
          } else {
            for (int u = 0; u < U; ++u)
              if (u < t)
                c2_step<BATCH>(bm_l, bp, f_l, fp, rowbit, C, lut, eb0, fw, ebias, smem, g.xstride,
                               acc);
          }
        }
      }
    } else {
      for (int i = 0; i < n_max; ++i)
        if (i < n)
          c2_step<BATCH>(bm_l, bp, f_l, fp, rowbit, C, lut, eb0, fw, ebias, smem, g.xstride,
                         acc);
    }

    if (n == 0) {
#pragma unroll
      for (int bb = 0; bb < BATCH; ++bb) acc[bb] = 0.f;
    }
    for (int o = g.P >> 1; o >= 1; o >>= 1) {
#pragma unroll
      for (int bb = 0; bb < BATCH; ++bb) acc[bb] += __shfl_xor(acc[bb], o, 64);
    }
    if (active && part == 0) {
#pragma unroll
      for (int bb = 0; bb < BATCH; ++bb) y[bb * ldy + pl.row0 + rl] = acc[bb];
    }
    if (!more) break;
    wave_sync();  // every lane is done with the staged words before they are replaced
    pl = plan(next);
    stage(pl);
    wait_dma();
    pt = locate(pl);
    round = next;
  }
}

int a16(int64_t v) { return (int)((v + 15) / 16 * 16); }

int pick_u(const Shape& sh) {
  const int fw = 1 + sh.mant;
  const double q = sh.cols > 0 ? (double)sh.keep / (double)sh.cols : 0.0;
  // P(a 64-bit keep window holds fewer than U bits) stays near 1e-4 or below
  if (fw <= 4 && q >= 0.28) return 8;
  if (fw <= 5 && q >= 0.23) return 6;
  return 4;
}

// LDS plan; lds_bytes > kBalMaxLds means "does not fit".
BalGeom make_bal_geom(const Shape& sh, int batch, int64_t code_limit_words, int64_t nsb) {
  BalGeom g = {};
  const int64_t R = sh.rows, C = sh.cols, k = sh.keep, nb = C / sh.block;
  const int fw = 1 + sh.mant;
  // parts per row: 32 (two rows per wave round) keeps about six waves per SIMD
  // resident within LDS; very tall matrices take 16 (more values per part,
  // fewer part starts); parts keep at least 16 values
  int P = R >= 16384 ? 16 : 32;
  while (P > 1 && k / P < 16) P /= 2;
  if (const int p = option(OPT_GEMV_PARTS); p >= 1 && p <= 64 && (p & (p - 1)) == 0) P = p;
  g.P = P;
  g.logP = __builtin_ctz(P);
  g.rpw = 64 / P;
  g.nb_top = 1;
  while (2 * g.nb_top < nb) g.nb_top *= 2;
  g.nrounds = (R + g.rpw - 1) / g.rpw;
  g.nb_per_k = k > 0 ? (float)nb / (float)k : 0.f;
  g.xstride = (uint32_t)a16(2 * C + 256);
  g.word_bits = 27;
  int64_t pos = (int64_t)batch * g.xstride;
  g.lut_off = (int)pos;
  pos += a16((int64_t)(kRanks << fw) * 4);
  g.wave_off = (int)pos;
  int64_t w = 0;
  // staged runs start up to one chunk early and end up to one chunk late
  g.kb_off = (int)w;
  w += a16((int64_t)g.rpw * nb * 2 + 32);
  g.bo_off = (int)w;
  // (format 4, nsb > 0: u16 offsets in this region, then the superblock bases)
  w += nsb > 0 ? a16((int64_t)g.rpw * nb * 2 + 32) : a16(((int64_t)g.rpw * nb + 8) * 4);
  g.sb_off = (int)w;
  if (nsb > 0) w += a16(((int64_t)g.rpw * nsb + 4) * 8);
  g.bm_off = (int)w;
  w += a16((g.rpw * C / 32 + 4 + kSlack) * 4);
  g.f_off = (int)w;
  w += a16(((g.rpw * k * fw + 31) / 32 + 8 + kSlack) * 4);
  g.c_off = (int)w;
  const int64_t avg = R > 0 ? code_limit_words * g.rpw / R : 0;
  int64_t cap = 2 * avg + 64;
  if (cap > 4096) cap = 4096;
  g.c_cap = (int)cap;
  w += a16((cap + 4 + kSlack) * 4);
  g.perm_off = (int)w;
  w += 256;
  g.wave_bytes = (int)w;
  pos += (int64_t)kBalWaves * w;
  g.lds_bytes = (fw > kMaxFw || pos > kBalMaxLds) ? (int)(kBalMaxLds + 1) : (int)pos;
  return g;
}

template <int BATCH, int U>
hipError_t launch_bal(const SpecViewC1& v, const Shape& sh, const BalGeom& g, const uint16_t* x,
                      int64_t ldx, float* y, int64_t ldy, hipStream_t s) {
  auto kern = v.sb_log >= 0 ? k_gemv_c1_bal<BATCH, U, true> : k_gemv_c1_bal<BATCH, U, false>;
  if (g.lds_bytes > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, g.lds_bytes);
    if (e != hipSuccess) return e;
  }
  // every workgroup resident at once (as many per CU as registers and LDS allow)
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void*)kern, kBalThreads,
                                                   (size_t)g.lds_bytes) != hipSuccess || occ < 1)
    occ = 1;
  int64_t grid = (int64_t)device_cu_count() * occ;
  const int64_t need = (g.nrounds + kBalWaves - 1) / kBalWaves;
  if (grid > need) grid = need;
  if (grid < 1) grid = 1;
  kern<<<(unsigned)grid, kBalThreads, (size_t)g.lds_bytes, s>>>(v, sh, g, x, ldx, y, ldy);
  return hipGetLastError();
}

template <int BATCH>
hipError_t launch_bal_u(const SpecViewC1& v, const Shape& sh, const BalGeom& g, int U,
                        const uint16_t* x, int64_t ldx, float* y, int64_t ldy, hipStream_t s) {
  switch (U) {
    case 8: return launch_bal<BATCH, 8>(v, sh, g, x, ldx, y, ldy, s);
    case 6: return launch_bal<BATCH, 6>(v, sh, g, x, ldx, y, ldy, s);
    default: return launch_bal<BATCH, 4>(v, sh, g, x, ldx, y, ldy, s);
  }
}


// LDS plan for Cassandra-2 (the code region holds the shared exponents).
BalGeom make_bal_geom_c2(const Shape& sh, int batch) {
  BalGeom g = {};
  const int64_t R = sh.rows, C = sh.cols, k = sh.keep, nb = C / sh.block;
  const int fw = 2 + sh.mant;
  int P = R >= 16384 ? 16 : 32;
  while (P > 1 && k / P < 16) P /= 2;
  if (const int p = option(OPT_GEMV_PARTS); p >= 1 && p <= 64 && (p & (p - 1)) == 0) P = p;
  g.P = P;
  g.logP = __builtin_ctz(P);
  g.rpw = 64 / P;
  g.nrounds = (R + g.rpw - 1) / g.rpw;
  g.nb_per_k = k > 0 ? (float)nb / (float)k : 0.f;
  g.xstride = (uint32_t)a16(2 * C + 256);
  int64_t pos = (int64_t)batch * g.xstride;
  g.lut_off = (int)pos;
  pos += a16((int64_t)(1 << fw) * 4);
  g.wave_off = (int)pos;
  int64_t w = 0;
  g.kb_off = (int)w;
  w += a16((int64_t)g.rpw * nb * 2 + 32);
  g.bm_off = (int)w;
  w += a16((g.rpw * C / 32 + 4 + kSlack) * 4);
  g.f_off = (int)w;
  w += a16(((g.rpw * k * fw + 31) / 32 + 8 + kSlack) * 4);
  g.c_off = (int)w;
  w += a16(g.rpw * C / 32 + 32);  // exponents: one byte per word, a chunk either side
  g.wave_bytes = (int)w;
  pos += (int64_t)kBalWaves * w;
  g.lds_bytes = (fw > 9 || pos > kBalMaxLds) ? (int)(kBalMaxLds + 1) : (int)pos;
  return g;
}

template <int BATCH, int U>
hipError_t launch_bal_c2(const SpecViewC2& v, const Shape& sh, const BalGeom& g,
                         const uint16_t* x, int64_t ldx, float* y, int64_t ldy, hipStream_t s) {
  auto kern = k_gemv_c2_bal<BATCH, U>;
  if (g.lds_bytes > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, g.lds_bytes);
    if (e != hipSuccess) return e;
  }
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void*)kern, kBalThreads,
                                                   (size_t)g.lds_bytes) != hipSuccess || occ < 1)
    occ = 1;
  int64_t grid = (int64_t)device_cu_count() * occ;
  const int64_t need = (g.nrounds + kBalWaves - 1) / kBalWaves;
  if (grid > need) grid = need;
  if (grid < 1) grid = 1;
  kern<<<(unsigned)grid, kBalThreads, (size_t)g.lds_bytes, s>>>(v, sh, g, x, ldx, y, ldy);
  return hipGetLastError();
}

template <int BATCH>
hipError_t launch_bal_c2_u(const SpecViewC2& v, const Shape& sh, const BalGeom& g,
                           const uint16_t* x, int64_t ldx, float* y, int64_t ldy,
                           hipStream_t s) {
  // values per group: as many fields as a 32-bit window holds, at most 8
  const int fw = 2 + sh.mant;
  const int u = std::min(8, 32 / fw);
  switch (u) {
    case 8: return launch_bal_c2<BATCH, 8>(v, sh, g, x, ldx, y, ldy, s);
    case 6: return launch_bal_c2<BATCH, 6>(v, sh, g, x, ldx, y, ldy, s);
    case 5: return launch_bal_c2<BATCH, 5>(v, sh, g, x, ldx, y, ldy, s);
    case 4: return launch_bal_c2<BATCH, 4>(v, sh, g, x, ldx, y, ldy, s);
    default: return launch_bal_c2<BATCH, 3>(v, sh, g, x, ldx, y, ldy, s);
  }
}
}  // namespace

bool draft_gemv_bal_fits(const Shape& sh, int batch, int64_t code_limit_words, int64_t nsb) {
  return make_bal_geom(sh, batch, code_limit_words, nsb).lds_bytes <= kBalMaxLds;
}

hipError_t launch_draft_gemv_c1_bal(const SpecViewC1& v, const Shape& sh, const uint16_t* x,
                                    int batch, int64_t ldx, float* y, int64_t ldy,
                                    hipStream_t s) {
  if (sh.rows == 0) return hipSuccess;
  const BalGeom g = make_bal_geom(sh, batch, v.codes_limit, v.sb_log >= 0 ? v.nsb : 0);
  if (g.lds_bytes > kBalMaxLds) return hipErrorInvalidValue;
  const int U = pick_u(sh);
  switch (batch) {
    case 1: return launch_bal_u<1>(v, sh, g, U, x, ldx, y, ldy, s);
    case 2: return launch_bal_u<2>(v, sh, g, U, x, ldx, y, ldy, s);
    case 3: return launch_bal_u<3>(v, sh, g, U, x, ldx, y, ldy, s);
    case 4: return launch_bal_u<4>(v, sh, g, U, x, ldx, y, ldy, s);
    case 5: return launch_bal_u<5>(v, sh, g, U, x, ldx, y, ldy, s);
    case 6: return launch_bal_u<6>(v, sh, g, U, x, ldx, y, ldy, s);
    case 7: return launch_bal_u<7>(v, sh, g, U, x, ldx, y, ldy, s);
    case 8: return launch_bal_u<8>(v, sh, g, U, x, ldx, y, ldy, s);
    default: return hipErrorInvalidValue;
  }
}

bool draft_gemv_bal_c2_fits(const Shape& sh, int batch) {
  return make_bal_geom_c2(sh, batch).lds_bytes <= kBalMaxLds;
}

hipError_t launch_draft_gemv_c2_bal(const SpecViewC2& v, const Shape& sh, const uint16_t* x,
                                    int batch, int64_t ldx, float* y, int64_t ldy,
                                    hipStream_t s) {
  if (sh.rows == 0) return hipSuccess;
  const BalGeom g = make_bal_geom_c2(sh, batch);
  if (g.lds_bytes > kBalMaxLds) return hipErrorInvalidValue;
  switch (batch) {
    case 1: return launch_bal_c2_u<1>(v, sh, g, x, ldx, y, ldy, s);
    case 2: return launch_bal_c2_u<2>(v, sh, g, x, ldx, y, ldy, s);
    case 3: return launch_bal_c2_u<3>(v, sh, g, x, ldx, y, ldy, s);
    case 4: return launch_bal_c2_u<4>(v, sh, g, x, ldx, y, ldy, s);
    case 5: return launch_bal_c2_u<5>(v, sh, g, x, ldx, y, ldy, s);
    case 6: return launch_bal_c2_u<6>(v, sh, g, x, ldx, y, ldy, s);
    case 7: return launch_bal_c2_u<7>(v, sh, g, x, ldx, y, ldy, s);
    case 8: return launch_bal_c2_u<8>(v, sh, g, x, ldx, y, ldy, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace cass
