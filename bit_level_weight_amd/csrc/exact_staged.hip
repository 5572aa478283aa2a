// Verification GEMM and exact reconstruction for Cassandra-1, decoded from
// streams staged in LDS.
//
// Method: Cassandra review (marsggbo.github.io), section 1 -- the target
// model checks the drafted tokens in one parallel pass; section 3.1 -- it
// loads both streams and reassembles the original weights losslessly;
// section 3.2 -- a unary exponent code is decoded by counting the zeros up to
// its one; section 3.3 -- the keep bitmap is de-sparsified.
//
// Work split.  A workgroup takes 16 rows; its waves take their columns in
// stages of Wb blocks, in turn (neighbouring stages run side by side), and the
// verification GEMM adds the waves' products in wave order (no atomics: the
// result is the same on every run).  A stage copies, for every row, the row's
// range of each section -- bitmap, fields, low mantissas, pruned bytes and
// both code sections -- into LDS by LDS DMA: per section every row gets a slot
// as long as the longest of the 16 runs (packed back to back instead when the
// slots do not fit), and every instruction moves 64 chunks of 16 bytes, so a
// stage takes a handful of instructions, all in flight at once.  The next
// stage's block words and this stage's X columns load while it decodes.
//
// Decode.  Four lanes serve each row.  The row's kept values of the stage are
// cut into four equal parts, one per lane, and so are its pruned values, so
// all lanes run the same number of steps.  A lane finds where its part starts
// (block from the kept-before counts, word and bit by popcounts and a select,
// code start by skipping codes) and then decodes U values per group from LDS
// windows in three phases -- positions, ranks and fields (VALU only); every
// table read of the group plus the next group's window words (LDS only);
// the values, written to their columns of a 16 x (Wb*B) bf16 tile.  The
// verification GEMM multiplies the tile with the matching columns of X on the
// matrix cores (v_mfma_f32_16x16x32_bf16, tokens padded to 16); the
// reconstruction copies the tile rows to the output.
#include <stdlib.h>

#include <algorithm>

#include "internal.hpp"
#include "staged_decode.hpp"

namespace cass {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) const uint8_t lds_u8c;
typedef __attribute__((address_space(3))) const uint16_t lds_u16c;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) const uint32_t lds_u32c;

constexpr int kRows = 16;   // rows per wave
constexpr int kMaxWaves = 8;  // waves per workgroup: the same 16 rows, column ranges side by side
constexpr int kSec = 6;     // bitmap, fields, low mantissas, pruned bytes, spec codes, verif codes
constexpr int kPU = 6;      // pruned values per group (6 codes nearly always fit 32 bits)
constexpr int kXPre = 8;    // X column steps of a stage loaded before its decode

struct XGeom {
  int Wb;                    // blocks per stage
  int TS;                    // u16 per tile row (Wb*B + 2)
  int64_t nstage;
  int nsplit;                // waves per workgroup; wave w takes stages w, w + nsplit, ...
  int perm_off, klut_off, plut_off, wave_off, wave_bytes;  // shared tables, wave regions
  int meta_off, dummy_off, tile_off;                       // inside a wave region
  int fix_off, fix_cap, cod_off, cod_cap, lds_bytes;
  uint32_t wbits;            // 27, the width of a bit position's word index (see word_ptr)
};

__device__ __forceinline__ void wsync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint32_t u32(int64_t v) { return (uint32_t)v; }

__device__ __forceinline__ uint32_t lds_addr_of(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(lds_u8c*)p;
}
__device__ __forceinline__ uint32_t ldh(uint32_t a) { return *(lds_u16c*)(uintptr_t)a; }
__device__ __forceinline__ void sth(uint32_t a, uint32_t v) { *(lds_u16*)(uintptr_t)a = (uint16_t)v; }

__device__ __forceinline__ void wait_all() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  wsync();
}

// 32 bits of the LDS bit stream at byte address base, bit offset pos.
__device__ __forceinline__ uint32_t lwin(uint32_t base, uint32_t pos) {
  const lds_u32c* q = (const lds_u32c*)(uintptr_t)(base + ((pos >> 5) << 2));
  return __builtin_amdgcn_alignbit(q[1], q[0], pos & 31u);
}

// Unary code at LDS bit pos (up to 256 bits); advances pos.
__device__ __forceinline__ int lunary(uint32_t base, uint32_t& pos) {
  uint32_t win = lwin(base, pos);
  int r = 0;
  for (int it = 0; it < 8 && win == 0u; ++it) {
    pos += 32;
    r += 32;
    win = lwin(base, pos);
  }
  if (win == 0u) {
    pos += 32;
    return 255;
  }
  const int t = __builtin_ctz(win);
  pos += (uint32_t)t + 1u;
  return r + t;
}

// Inclusive sum over each row of 16 lanes (DPP row shifts, zero fill).
__device__ __forceinline__ int scan16(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  return v;
}

// Maximum over each row of 16 lanes (every row of the wave holds the same 16
// values here, so this is also the wave's maximum).
__device__ __forceinline__ int max16(int v) {
  v = max(v, __shfl_xor(v, 1, 64));
  v = max(v, __shfl_xor(v, 2, 64));
  v = max(v, __shfl_xor(v, 4, 64));
  v = max(v, __shfl_xor(v, 8, 64));
  return v;
}

// ---- groups
// Window words of a kept group: bitmap (3 words at bp), fields (2 at fp),
// low mantissas (2 at lp), spec codes (2 at cp).  Bit positions are LDS bit
// offsets from the start of shared memory.
struct KRaw {
  uint32_t q0, q1, q2, f0, f1, l0, l1, c0, c1;
};
// The LDS word holding bit `pos` of the staged words at byte address sb: the
// word index by bit-field extract, then one shift-and-add.  `wb` = 27 comes
// from a kernel argument (with a literal width the extract becomes a shift
// and a mask).  Reads index the returned pointer, so the offsets of the next
// words go into the reads' offset fields instead of separate adds.
__device__ __forceinline__ const lds_u32c* word_ptr(uint32_t sb, uint32_t pos, uint32_t wb) {
  return (const lds_u32c*)(uintptr_t)(sb + (__builtin_amdgcn_ubfe(pos, 5u, wb) << 2));
}

__device__ __forceinline__ KRaw kraw(uint32_t sb, uint32_t bp, uint32_t fp, uint32_t lp,
                                     uint32_t cp, uint32_t wb) {
  const lds_u32c *q = word_ptr(sb, bp, wb), *f = word_ptr(sb, fp, wb);
  const lds_u32c *l = word_ptr(sb, lp, wb), *c = word_ptr(sb, cp, wb);
  return KRaw{q[0], q[1], q[2], f[0], f[1], l[0], l[1], c[0], c[1]};
}

// Pruned group: bitmap (3 words at bp, inverted on use), pruned bytes (3 at
// yp), verification codes (2 at cp).
struct PRaw {
  uint32_t q0, q1, q2, y0, y1, y2, c0, c1;
};
__device__ __forceinline__ PRaw praw(uint32_t sb, uint32_t bp, uint32_t yp, uint32_t cp,
                                     uint32_t wb) {
  const lds_u32c *q = word_ptr(sb, bp, wb), *y = word_ptr(sb, yp, wb);
  const lds_u32c* c = word_ptr(sb, cp, wb);
  return PRaw{q[0], q[1], q[2], y[0], y[1], y[2], c[0], c[1]};
}

// Whether the windows in w hold t values: t keep (or pruned) positions in the
// 64-bit window at bp and t codes in the 32-bit window at cp.
__device__ __forceinline__ bool ok1_kept(const KRaw& w, uint32_t bp, uint32_t cp, int t) {
  const uint32_t sbit = bp & 31u;
  const int have = __builtin_popcount(__builtin_amdgcn_alignbit(w.q1, w.q0, sbit)) +
                   __builtin_popcount(__builtin_amdgcn_alignbit(w.q2, w.q1, sbit));
  const int ncode = __builtin_popcount(__builtin_amdgcn_alignbit(w.c1, w.c0, cp & 31u));
  return min(have, ncode) >= t;
}
__device__ __forceinline__ bool ok1_pruned(const PRaw& w, uint32_t bp, uint32_t cp, int t) {
  const uint32_t sbit = bp & 31u;
  const int have = __builtin_popcount(~__builtin_amdgcn_alignbit(w.q1, w.q0, sbit)) +
                   __builtin_popcount(~__builtin_amdgcn_alignbit(w.q2, w.q1, sbit));
  const int ncode = __builtin_popcount(__builtin_amdgcn_alignbit(w.c1, w.c0, cp & 31u));
  return min(have, ncode) >= t;
}

// U kept values.  With MASKED, slots u >= t write to the lane's dummy slot (a
// set bit 63 of the keep window and a set code bit 31 keep their positions
// and ranks in range), and only lanes with t == U move on: a lane with fewer
// has finished its part.
//   torg   LDS byte address of the lane's tile row minus 2 * the bitmap bit of
//          its column 0 (a value at bitmap bit b goes to torg + 2 b)
//   lw     shift of the mantissa field's low end (7 - m); lwid the width of the
//          low-mantissa field read (7 - m, or 0 for the zero-filled draft)
template <int U, bool KLUT, bool MASKED>
__device__ __forceinline__ void kept_group(KRaw& w, uint32_t& bp, uint32_t& fp, uint32_t& lp,
                                           uint32_t& cp, uint32_t sb, uint32_t torg,
                                           uint32_t klutb, uint32_t dummy, int fw, int lw,
                                           int lwid, int m, int t, uint32_t wb) {
  const uint32_t sbit = bp & 31u;
  const uint32_t lo0 = __builtin_amdgcn_alignbit(w.q1, w.q0, sbit);
  const uint32_t hi0 = __builtin_amdgcn_alignbit(w.q2, w.q1, sbit) | (MASKED ? 0x80000000u : 0u);
  const uint32_t wf = __builtin_amdgcn_alignbit(w.f1, w.f0, fp & 31u);
  const uint32_t wl = __builtin_amdgcn_alignbit(w.l1, w.l0, lp & 31u);
  const uint32_t wc0 = __builtin_amdgcn_alignbit(w.c1, w.c0, cp & 31u);
  // phase 1: table addresses and tile addresses
  uint32_t la[U], ta[U], low[U], fv[U];
  uint32_t lo = lo0, wc = wc0, p = 0, base = bp;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    // the window holds U keep bits: lo runs out at most once
    const bool z = lo == 0u;
    lo = z ? hi0 : lo;
    base = z ? bp + 32u : base;
    p = (uint32_t)__builtin_ctz(lo);
    lo &= lo - 1u;
    const uint32_t r = (uint32_t)__builtin_ctz(MASKED ? wc | 0x80000000u : wc);
    wc = (wc >> r) >> 1;
    const uint32_t f = __builtin_amdgcn_ubfe(wf, (uint32_t)(u * fw), (uint32_t)fw);
    low[u] = __builtin_amdgcn_ubfe(wl, (uint32_t)(u * lwid), (uint32_t)lwid);
    fv[u] = f;
    la[u] = KLUT ? klutb + 2u * ((r << fw) | f) : klutb + 2u * r;
    const uint32_t a = torg + 2u * (base + p);
    ta[u] = (MASKED && u >= t) ? dummy : a;
  }
  {
    const bool go = !MASKED || t == U;
    bp = go ? base + p + 1u : bp;
    fp = go ? fp + (uint32_t)(U * fw) : fp;
    lp = go ? lp + (uint32_t)(U * lwid) : lp;
    // bits the U codes took: the window was shifted right by that many
    const uint32_t c0 = (uint32_t)__builtin_clz(wc0);
    const uint32_t cn = cp + (wc ? (uint32_t)__builtin_clz(wc) : 32u) - c0;
    cp = go ? cn : cp;
  }
  __builtin_amdgcn_sched_barrier(0);
  // phase 2: every table read of the group and the next group's words
  uint32_t hv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) hv[u] = ldh(la[u]);
  w = kraw(sb, bp, fp, lp, cp, wb);
  __builtin_amdgcn_sched_barrier(0);
  // phase 3: the values
#pragma unroll
  for (int u = 0; u < U; ++u) {
    uint32_t v;
    if (KLUT) {
      v = hv[u] | low[u];
    } else {
      const uint32_t f = fv[u];
      v = ((f >> m) << 15) | hv[u] | ((f & ((1u << m) - 1u)) << lw) | low[u];
    }
    sth(ta[u], v);
  }
}

// U <= kPU pruned values (positions: zero bits of the bitmap); MASKED as for
// the kept groups.  W32: the 32 positions at bp hold U pruned values for every
// lane (pruned values are the dense ones), so the window never moves on to
// its second word.
template <int U, bool MASKED, bool W32 = false>
__device__ __forceinline__ void pruned_group(PRaw& w, uint32_t& bp, uint32_t& yp, uint32_t& cp,
                                             uint32_t sb, uint32_t torg, uint32_t plutb,
                                             uint32_t dummy, int t, uint32_t wb) {
  static_assert(U <= 8, "pruned bytes come from two 32-bit windows");
  static_assert(!(W32 && MASKED), "the 32-bit window serves full groups");
  const uint32_t sbit = bp & 31u;
  const uint32_t lo0 = ~__builtin_amdgcn_alignbit(w.q1, w.q0, sbit);
  const uint32_t hi0 = W32 ? 0u : ~__builtin_amdgcn_alignbit(w.q2, w.q1, sbit) | (MASKED ? 0x80000000u : 0u);
  const uint32_t ysh = yp & 31u;
  const uint32_t ylo = __builtin_amdgcn_alignbit(w.y1, w.y0, ysh);
  const uint32_t yhi = __builtin_amdgcn_alignbit(w.y2, w.y1, ysh);
  const uint32_t wc0 = __builtin_amdgcn_alignbit(w.c1, w.c0, cp & 31u);
  uint32_t la[U], ta[U], mt[U];
  uint32_t lo = lo0, wc = wc0, p = 0, base = bp;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (!W32) {
      const bool z = lo == 0u;
      lo = z ? hi0 : lo;
      base = z ? bp + 32u : base;
    }
    p = (uint32_t)__builtin_ctz(lo);
    lo &= lo - 1u;
    const uint32_t r = (uint32_t)__builtin_ctz(MASKED ? wc | 0x80000000u : wc);
    wc = (wc >> r) >> 1;
    const uint32_t yw = u < 4 ? ylo : yhi;  // (u is a constant: no select)
    const uint32_t sh = (uint32_t)(8 * (u & 3));
    const uint32_t sgn = __builtin_amdgcn_ubfe(yw, sh + 7u, 1u);
    mt[u] = __builtin_amdgcn_ubfe(yw, sh, 7u);
    la[u] = plutb + 2u * ((r << 1) | sgn);
    const uint32_t a = torg + 2u * (base + p);
    ta[u] = (MASKED && u >= t) ? dummy : a;
  }
  {
    const bool go = !MASKED || t == U;
    bp = go ? base + p + 1u : bp;
    yp = go ? yp + (uint32_t)(8 * U) : yp;
    const uint32_t c0 = (uint32_t)__builtin_clz(wc0);
    const uint32_t cn = cp + (wc ? (uint32_t)__builtin_clz(wc) : 32u) - c0;
    cp = go ? cn : cp;
  }
  __builtin_amdgcn_sched_barrier(0);
  uint32_t hv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) hv[u] = ldh(la[u]);
  w = praw(sb, bp, yp, cp, wb);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < U; ++u) sth(ta[u], hv[u] | mt[u]);
}

// One kept value, any code length (codes from LDS, or from global memory at
// cg when it is set).
__device__ __forceinline__ void kept_step(uint32_t sb, uint32_t& bp, uint32_t bp_end,
                                          uint32_t& fp, uint32_t& lp, uint32_t& cp,
                                          const uint32_t* cg, uint32_t torg, const uint8_t* ps,
                                          int fw, int lw, int lwid, int m) {
  uint32_t w = lwin(sb, bp);
  // a valid part has its next value inside the row's stage; the bound only
  // keeps a corrupt stream from spinning
  for (; w == 0u && bp < bp_end;) {
    bp += 32u;
    w = lwin(sb, bp);
  }
  const uint32_t pos = bp + (uint32_t)__builtin_ctz(w);
  CASS_DCHECK(pos < bp_end, CASS_DBG_TILE);
  bp = pos + 1u;
  const uint32_t f = lwin(sb, fp) & ((1u << fw) - 1u);
  fp += (uint32_t)fw;
  const uint32_t low = lwid ? (lwin(sb, lp) & ((1u << lwid) - 1u)) : 0u;
  lp += (uint32_t)lwid;
  const int r = cg ? unary_at(cg, cp) : lunary(sb, cp);
  const uint32_t e = ps[r];
  sth(torg + 2u * pos, ((f >> m) << 15) | (e << 7) | ((f & ((1u << m) - 1u)) << lw) | low);
}

__device__ __forceinline__ void pruned_step(uint32_t sb, uint32_t& bp, uint32_t bp_end,
                                            uint32_t& yp, uint32_t& cp, const uint32_t* cg,
                                            uint32_t torg, const uint8_t* pv) {
  uint32_t w = ~lwin(sb, bp);
  for (; w == 0u && bp < bp_end;) {
    bp += 32u;
    w = ~lwin(sb, bp);
  }
  const uint32_t pos = bp + (uint32_t)__builtin_ctz(w);
  CASS_DCHECK(pos < bp_end, CASS_DBG_TILE);
  bp = pos + 1u;
  const uint32_t byte = lwin(sb, yp) & 0xFFu;
  yp += 8u;
  const int r = cg ? unary_at(cg, cp) : lunary(sb, cp);
  const uint32_t e = pv[r];
  sth(torg + 2u * pos, ((byte >> 7) << 15) | (e << 7) | (byte & 0x7Fu));
}

// Bit offset, inside the nwb words at LDS byte address wa, of the
// (skip+1)-th set bit (zero bit when INV); the count lies inside them.
template <bool INV>
__device__ __forceinline__ uint32_t find_in_block(uint32_t wa, int nwb, int skip) {
  int rem = skip, wsel = nwb - 1;
  uint32_t wd = 0;
  const lds_u32c* q = (const lds_u32c*)(uintptr_t)wa;
  if (nwb <= 8) {
    uint32_t wv[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) wv[w] = w < nwb ? (INV ? ~q[w] : q[w]) : 0u;
    bool found = false;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int c = __builtin_popcount(wv[w]);
      const bool here = !found && w < nwb && rem < c;
      wsel = here ? w : wsel;
      wd = here ? wv[w] : wd;
      rem -= (!found && !here) ? c : 0;
      found = found || here;
    }
  } else {
    int wi = 0;
    wd = INV ? ~q[0] : q[0];
    for (;;) {
      const int c = __builtin_popcount(wd);
      if (rem < c || wi == nwb - 1) break;  // (the second test: corrupt streams only)
      rem -= c;
      ++wi;
      wd = INV ? ~q[wi] : q[wi];
    }
    wsel = wi;
  }
  return (uint32_t)(wsel * 32 + select_bit(wd, rem + 1));
}

// MODE 0: verification GEMM into Y; 1: reconstruction; 2: zero-filled draft
// (speculation stream only: vv is not read)
template <int MODE, int KU, bool KLUT>
__global__ void __launch_bounds__(64 * kMaxWaves) k_exact_staged(SpecViewC1 sv, VerifViewC1 vv, Shape sh,
                                                     XGeom g, const uint16_t* __restrict__ X,
                                                     int ntok, int64_t ldx,
                                                     float* __restrict__ Y, int64_t ldy,
                                                     uint16_t* __restrict__ out) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t R = sh.rows, C = sh.cols, k = sh.keep, B = sh.block, nb = C / B;
  const int m = sh.mant, fw = 1 + m, lw = 7 - m;
  const int nwb = (int)(B / 32);
  const int lwid = MODE == 2 ? 0 : lw;
  const uint32_t sb = lds_addr_of(smem);
  const uint32_t* sm32 = reinterpret_cast<const uint32_t*>(smem);

  // this wave's region: 16 rows of its own
  const int wbase = g.wave_off + wave * g.wave_bytes;
  uint8_t* wsm = smem + wbase;
  const uint32_t klutb = sb + g.klut_off, plutb = sb + g.plut_off;
  const uint32_t dummy = sb + wbase + g.dummy_off + 4u * lane;
  const uint32_t tileb = sb + wbase + g.tile_off;

  const int r = lane & 15, j = lane >> 4;
  const int xn = lane & 15, xkq = lane >> 4;  // MFMA operand lane: token / row n, k slice
  // the workgroup's waves share its 16 rows and take their stages in turn; the
  // verification GEMM sums the waves' products in wave order
  const int64_t row0 = (int64_t)blockIdx.x * kRows;
  if (row0 >= R) return;
  const int64_t row = row0 + r;
  const bool row_ok = row < R;
  const int64_t rowc = row_ok ? row : R - 1;  // clamped for loads
  const uint32_t rowk = u32(rowc) * u32(k), rowpk = u32(rowc) * u32(C - k);  // mod 2^32
  // stages interleaved over the waves (wave w takes w, w + nsplit, ...), so
  // neighbouring blocks of a row, which share the 128-byte lines at their
  // boundary, are read at about the same time and the second read hits in L2
  const int64_t st0 = wave, sstep = g.nsplit;
  // format 4 (sv.sb_log >= 0): a row's first code bit is its first superblock's
  // base, and a block's code offset from it is (superblock base - that) + the
  // block's 16-bit offset
  const bool sbm = sv.sb_log >= 0;
  const unsigned long long* rb0 = sbm ? sv.sbbase : sv.rowbase;
  const int64_t rstride = sbm ? sv.nsb : 1;
  const int64_t rbs = (int64_t)rb0[rowc * rstride];
  const int64_t rbv = MODE == 2 ? 0 : (int64_t)vv.rowbase[rowc];
  const int64_t rbs_next =
      rowc + 1 < R ? (int64_t)rb0[(rowc + 1) * rstride] : sv.codes_limit * 32;
  const int64_t rbv_next =
      MODE == 2 ? 0 : (rowc + 1 < R ? (int64_t)vv.rowbase[rowc + 1] : vv.codes_limit * 32);
  const uint8_t* sec_base[kSec] = {
      reinterpret_cast<const uint8_t*>(sv.bitmap), reinterpret_cast<const uint8_t*>(sv.fields),
      reinterpret_cast<const uint8_t*>(vv.lowmant), vv.pruned,
      reinterpret_cast<const uint8_t*>(sv.codes), reinterpret_cast<const uint8_t*>(vv.codes)};
  const int64_t sec_lim[kSec] = {sv.bitmap_limit / 4, sv.fields_limit / 4,
                                 vv.lowmant_limit / 4, vv.pruned_limit / 4,
                                 sv.codes_limit / 4,   vv.codes_limit / 4};  // in chunks
  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};

  // kept-before and code offsets at a stage's block boundaries (i = 0..Wb),
  // loaded one stage ahead as plain words (indices clamped, so the loads are
  // unconditional and nothing waits for them until the next stage)
  struct MetaRaw {
    uint32_t kb[3], bs[3], bv[3], o16[3];  // (format 4: bs the superblock base's low word)
  };
  // (one branch on the format around all the loads, and no arithmetic on the
  // loaded words until they are stored: a branch or a use after a load makes
  // the compiler wait for the loads in flight)
  auto load_meta = [&](int64_t stg) {
    MetaRaw mr;
    const int64_t bf = stg * g.Wb;
    int64_t bb[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) bb[i] = rowc * nb + std::min<int64_t>(bf + i, nb - 1);
    if (sbm) {
      const uint32_t* sb32 = reinterpret_cast<const uint32_t*>(sv.sbbase);
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        mr.kb[i] = sv.keptb[bb[i]];
        mr.bs[i] = sb32[2 * (rowc * sv.nsb + ((bb[i] - rowc * nb) >> sv.sb_log))];
        mr.o16[i] = sv.blkoff16[bb[i]];
        mr.bv[i] = MODE == 2 ? 0u : vv.blkoff[bb[i]];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        mr.kb[i] = sv.keptb[bb[i]];
        mr.bs[i] = sv.blkoff[bb[i]];
        mr.o16[i] = 0u;
        mr.bv[i] = MODE == 2 ? 0u : vv.blkoff[bb[i]];
      }
    }
    return mr;
  };
  // the current stage's words sit in shared memory: written at the end of the
  // previous stage (so their loads have had the whole decode to land)
  uint32_t* meta_s = reinterpret_cast<uint32_t*>(wsm + g.meta_off);  // [16][9]
  auto put_meta = [&](const MetaRaw& mr) {
    if (j == 0) {
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        meta_s[r * 9 + i] = mr.kb[i];
        // format 4: a block's code offset from the row's first code bit is
        // (superblock base - row base) + its 16-bit offset, taken mod 2^32
        meta_s[r * 9 + 3 + i] = sbm ? mr.bs[i] - u32(rbs) + mr.o16[i] : mr.bs[i];
        meta_s[r * 9 + 6 + i] = mr.bv[i];
      }
    }
  };
  // (the row bases and the first stage's words are loaded before the tables
  // are built, so the three global round trips overlap)
  MetaRaw mr0{};
  if (st0 < g.nstage) mr0 = load_meta(st0);

  // rank tables: bytes for the one-value steps, bf16 templates for the groups
  uint8_t* ps = smem + g.perm_off;
  uint8_t* pv = ps + 256;
  uint16_t* klut = reinterpret_cast<uint16_t*>(smem + g.klut_off);
  uint16_t* plut = reinterpret_cast<uint16_t*>(smem + g.plut_off);
  // (tables shared by the workgroup's waves)
  for (int i = threadIdx.x; i < 256; i += blockDim.x) {
    ps[i] = sv.perm[i];
    pv[i] = MODE == 2 ? 0 : vv.perm[i];
  }
  if (KLUT) {
    for (int i = threadIdx.x; i < (32 << fw); i += blockDim.x) {
      const uint32_t f = (uint32_t)i & ((1u << fw) - 1u);
      klut[i] = (uint16_t)(((f >> m) << 15) | ((uint32_t)sv.perm[i >> fw] << 7) |
                           ((f & ((1u << m) - 1u)) << lw));
    }
  } else if (threadIdx.x < 32) {
    klut[threadIdx.x] = (uint16_t)((uint32_t)sv.perm[threadIdx.x] << 7);
  }
  if (MODE != 2 && threadIdx.x < 64)
    plut[lane] = (uint16_t)(((uint32_t)(lane & 1) << 15) | ((uint32_t)vv.perm[lane >> 1] << 7));
  __syncthreads();  // the tables
  if (st0 < g.nstage) put_meta(mr0);
  wsync();

  for (int64_t st = st0; st < g.nstage; st += sstep) {
    const int64_t bf = st * g.Wb;
    const int64_t be = std::min<int64_t>(bf + g.Wb, nb);
    const int nbs = (int)(be - bf);  // 1 or 2
    int64_t kbv[3], bos[3], bov[3];
    {
      MetaRaw mr;
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        mr.kb[i] = meta_s[r * 9 + i];
        mr.bs[i] = meta_s[r * 9 + 3 + i];
        mr.bv[i] = meta_s[r * 9 + 6 + i];
      }
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        if (i > nbs) {
          kbv[i] = kbv[i - 1];
          bos[i] = bos[i - 1];
          bov[i] = bov[i - 1];
        } else if (bf + i < nb) {
          kbv[i] = mr.kb[i];
          bos[i] = rbs + mr.bs[i];
          bov[i] = rbv + mr.bv[i];
        } else {
          kbv[i] = k;
          bos[i] = rbs_next;
          bov[i] = rbv_next;
        }
      }
    }
    const int64_t kbe = nbs > 1 ? kbv[2] : kbv[1];
    const int64_t bose = nbs > 1 ? bos[2] : bos[1];
    const int64_t bove = nbs > 1 ? bov[2] : bov[1];
    int64_t lo[kSec], hi[kSec];
    lo[0] = (rowc * nb + bf) * B;
    hi[0] = (rowc * nb + be) * B;
    lo[1] = (rowc * k + kbv[0]) * fw;
    hi[1] = (rowc * k + kbe) * fw;
    lo[2] = (rowc * k + kbv[0]) * lw;
    hi[2] = (rowc * k + kbe) * lw;
    lo[3] = (rowc * (C - k) + bf * B - kbv[0]) * 8;
    hi[3] = (rowc * (C - k) + be * B - kbe) * 8;
    lo[4] = bos[0];
    hi[4] = bose;
    lo[5] = bov[0];
    hi[5] = bove;

    // ---- staging.  Per section, each row's run of 16-byte chunks.  Usually
    // every row gets a slot of S chunks, S the longest run of the 16 (row r's
    // run at slot offset r*S): a DMA lane then finds its row by one division
    // and takes the row's first chunk and run length from the row's lane.  When
    // the slots do not fit the region (rows with very different runs), the 16
    // runs are packed back to back instead, and a lane finds its row through
    // the runs' prefix sums.
    int64_t bias[kSec];
    int n_l[kSec];        // this lane's row: run length in chunks
    int c0_l[kSec];       // and first source chunk (sections hold fewer than 2^30 chunks)
    int S[kSec];          // longest run of the 16 rows (uniform)
#pragma unroll
    for (int sec = 0; sec < kSec; ++sec) {
      const int64_t c0 = lo[sec] >> 7;
      int64_t c1 = (hi[sec] + 127) >> 7;
      if (c1 > sec_lim[sec]) c1 = sec_lim[sec];
      // (the draft stages the speculation sections only)
      const bool used = MODE != 2 || sec == 0 || sec == 1 || sec == 4;
      n_l[sec] = (used && row_ok && hi[sec] > lo[sec] && c1 > c0) ? (int)(c1 - c0) : 0;
      c0_l[sec] = (int)c0;
      S[sec] = __builtin_amdgcn_readfirstlane(max16(n_l[sec]));
    }
    // (all six sections share the fixed and code regions, which are adjacent)
    int smax = 0, stot = 0;
#pragma unroll
    for (int sec = 0; sec < kSec; ++sec) {
      smax = max(smax, S[sec]);
      stot += S[sec];
    }
    const int ucap = g.fix_cap + 64 + g.cod_cap;  // (cod_off = fix_off + fix_cap + 64)
    const bool uni = smax <= 64 && kRows * 16 * stot <= ucap;
    bool overflow = false;  // codes over the region: read from global memory
    {
      int foff = 0, coff = 0, uoff = 0;
#pragma unroll
      for (int sec = 0; sec < kSec; ++sec) {
        const bool fixed = sec < 4;
        if (uni) {
          const int Ss = S[sec], tot = kRows * Ss;
          const int off = wbase + g.fix_off + uoff;
          uoff += 16 * tot;
          CASS_DCHECK(uoff <= ucap, CASS_DBG_STAGE);
          bias[sec] = (int64_t)(off + 16 * Ss * r) * 8 - (int64_t)c0_l[sec] * 128;
          if (Ss > 0) {
            // row of slot s = floor((s + 1/2) / S), exact in fp32 for s < 1024
            // and S <= 64 even with a reciprocal one ulp off
            const float rs = __builtin_amdgcn_rcpf((float)Ss), hs = 0.5f * rs;
            for (int base = 0; base < tot; base += 64) {
              const int s = base + lane;
              const int d = (int)__builtin_fmaf((float)s, rs, hs);
              const int q = s - d * Ss;
              // lanes 0..15 hold rows 0..15
              const int cd = __builtin_amdgcn_ds_bpermute(d << 2, c0_l[sec]);
              const int nd = __builtin_amdgcn_ds_bpermute(d << 2, n_l[sec]);
              if (s < tot && q < nd) {
                CASS_DCHECK(d < kRows, CASS_DBG_STAGE);
                __builtin_amdgcn_global_load_lds(
                    (const void*)(sec_base[sec] + 16 * (int64_t)(cd + q)),
                    (lds_void*)(smem + off + 16 * base), 16, 0, 0);
              }
            }
          }
          continue;
        }
        // packed runs
        const int off = wbase + (fixed ? g.fix_off + foff : g.cod_off + coff);
        const int n = n_l[sec];
        const int incl = scan16(n);
        const int pre = incl - n;
        const int N = __builtin_amdgcn_readlane(incl, 15);
        if (fixed) {
          foff += 16 * N;
          CASS_DCHECK(foff <= g.fix_cap, CASS_DBG_STAGE);
        } else {
          if (coff + 16 * N > g.cod_cap) overflow = true;
          coff += 16 * N;
        }
        bias[sec] = (int64_t)(off + 16 * pre) * 8 - (int64_t)c0_l[sec] * 128;
        if (N > 0 && (fixed || !overflow)) {
          const int dl = c0_l[sec] - pre;  // first source chunk - first packed chunk
          // the section's row table in scalars (lanes 0..15 hold rows 0..15)
          // the section's row table in scalars (lanes 0..15 hold rows 0..15)
          int inc[16], dd[16];
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            inc[q] = __builtin_amdgcn_readlane(incl, q);
            dd[q] = __builtin_amdgcn_readlane(dl, q);
          }
          for (int base = 0; base < N; base += 64) {
            const int c = base + lane;
            if (c < N) {
              // row of packed chunk c: past every row whose run ends at or before it
              int d = dd[0];
#pragma unroll
              for (int q = 0; q < 15; ++q) d = inc[q] <= c ? dd[q + 1] : d;
              __builtin_amdgcn_global_load_lds(
                  (const void*)(sec_base[sec] + 16 * (int64_t)(c + d)),
                  (lds_void*)(smem + off + 16 * base), 16, 0, 0);
            }
          }
        }
      }
    }
    // (both layouts copy with the default, allocating cache policy: a row's
    // run for one block covers part of a 128-byte line whose rest the next
    // stage reads)
    wait_all();
    const bool more = st + sstep < g.nstage;

    MetaRaw mr_next{};
    // X for the stage's first kXPre column steps
    const int nks = nbs * (int)B / 32;
    const int64_t xcol0 = bf * B;
    auto x_frag = [&](int ks) {
      v8s v = v8s{0, 0, 0, 0, 0, 0, 0, 0};
      if (xn < ntok && ks < nks) {
        const uint16_t* xp = X + (int64_t)xn * ldx + xcol0 + ks * 32 + 8 * xkq;
        v = v8s{(short)xp[0], (short)xp[1], (short)xp[2], (short)xp[3],
                (short)xp[4], (short)xp[5], (short)xp[6], (short)xp[7]};
      }
      return v;
    };
    v8s xq[kXPre];
    // ---- decode: kept values, then pruned values, into the tile
    // (LDS bit positions are taken mod 2^32 in 32-bit arithmetic: a 64-bit
    // product truncated afterwards leaves a don't-care high half that the
    // compiler may place in a register with a load still in flight)
    const uint32_t bm_row = u32(bias[0]) + (u32(rowc) * u32(nb) + u32(bf)) * u32(B);  // bitmap bit of column 0
    const uint32_t torg = tileb + 2u * (uint32_t)(r * g.TS) - 2u * bm_row;
    const uint32_t bm_end = bm_row + (uint32_t)(nbs * B);
    if (MODE == 2) {
      // zero-filled draft: clear the stage's columns of every row, then the
      // kept pass writes its values over them
      if (row_ok)
        for (int w = j; w < nbs * (int)B / 2; w += 4)
          *(__attribute__((address_space(3))) uint32_t*)(uintptr_t)(tileb + 4u * (uint32_t)(r * (g.TS / 2) + w)) = 0u;
      wsync();
    }
    {
      const int64_t K = kbe - kbv[0];
      const int64_t i0 = (K * j) >> 2;
      const int n = row_ok ? (int)(((K * (j + 1)) >> 2) - i0) : 0;
      const int64_t kidx = kbv[0] + i0;  // row-relative kept index of the part's first value
      uint32_t bp = bm_row, fp = 0, lp = 0, cp = 0;
      const uint32_t* cg = nullptr;
      if (n > 0) {
        const int bi = (nbs > 1 && kidx >= kbv[1]) ? 1 : 0;
        const int skip = (int)(kidx - kbv[bi]);
        const uint32_t blk = bm_row + (uint32_t)(bi * B);
        bp = blk + find_in_block<false>(sb + (blk >> 3), nwb, skip);
        const uint32_t kabs = rowk + u32(kidx);
        fp = u32(bias[1]) + kabs * (uint32_t)fw;
        lp = u32(bias[2]) + kabs * (uint32_t)lw;
        if (!overflow) {
          cp = skip_codes8(sm32, u32(bias[4]) + u32(bos[bi]), skip);
        } else {
          cg = sv.codes + (bos[bi] >> 5);
          cp = skip_codes(cg, (uint32_t)(bos[bi] & 31), skip);
        }
      }
      // the next stage's words and this stage's X: issued here, after the
      // part start, so they land while the groups decode (a 32-bit multiply-
      // add in the part start is selected as a 64-bit one whose don't-care
      // high half may share a register with a load in flight, which would
      // make it wait for the load)
      if (more) mr_next = load_meta(st + sstep);
#pragma unroll
      for (int q = 0; q < kXPre; ++q) xq[q] = MODE == 0 ? x_frag(q) : v8s{0, 0, 0, 0, 0, 0, 0, 0};
      int nmax = n;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) nmax = max(nmax, __shfl_xor(nmax, o, 64));
      if (!overflow) {
        KRaw w = kraw(sb, bp, fp, lp, cp, g.wbits);
        for (int done = 0; done < nmax; done += KU) {
          const int t = min(max(n - done, 0), KU);
          const uint32_t sbit = bp & 31u;
          const int have = __builtin_popcount(__builtin_amdgcn_alignbit(w.q1, w.q0, sbit)) +
                           __builtin_popcount(__builtin_amdgcn_alignbit(w.q2, w.q1, sbit));
          const int ncode = __builtin_popcount(__builtin_amdgcn_alignbit(w.c1, w.c0, cp & 31u));
          const bool ok = min(have, ncode) >= t;
          if (__all(t == KU && ok)) {
            kept_group<KU, KLUT, false>(w, bp, fp, lp, cp, sb, torg, klutb, dummy, fw, lw, lwid, m,
                                        KU, g.wbits);
          } else if (__all(ok)) {
            // some part ends inside this group
            kept_group<KU, KLUT, true>(w, bp, fp, lp, cp, sb, torg, klutb, dummy, fw, lw, lwid, m,
                                       t, g.wbits);
          } else {
            // some lane's windows hold fewer than its t values: the group in two
            // halves on the fast path (a lane whose first half is short of its
            // slots has no second half), value by value only if a half falls short
            constexpr int H1 = KU / 2, H2 = KU - KU / 2;
            const int t1 = t < H1 ? t : H1, t2 = t - t1;
            if (__all(ok1_kept(w, bp, cp, t1))) {
              kept_group<H1, KLUT, true>(w, bp, fp, lp, cp, sb, torg, klutb, dummy, fw, lw, lwid,
                                         m, t1, g.wbits);
              if (__all(ok1_kept(w, bp, cp, t2))) {
                kept_group<H2, KLUT, true>(w, bp, fp, lp, cp, sb, torg, klutb, dummy, fw, lw,
                                           lwid, m, t2, g.wbits);
              } else {
                for (int u = 0; u < H2; ++u)
                  if (u < t2)
                    kept_step(sb, bp, bm_end, fp, lp, cp, nullptr, torg, ps, fw, lw, lwid, m);
                w = kraw(sb, bp, fp, lp, cp, g.wbits);
              }
            } else {
              for (int u = 0; u < KU; ++u)
                if (u < t) kept_step(sb, bp, bm_end, fp, lp, cp, nullptr, torg, ps, fw, lw, lwid, m);
              w = kraw(sb, bp, fp, lp, cp, g.wbits);
            }
          }
        }
      } else {
        for (int i = 0; i < nmax; ++i)
          if (i < n) kept_step(sb, bp, bm_end, fp, lp, cp, cg, torg, ps, fw, lw, lwid, m);
      }
    }
    if (MODE != 2) {
      const int64_t P = (int64_t)nbs * B - (kbe - kbv[0]);
      const int64_t i0 = (P * j) >> 2;
      const int n = row_ok ? (int)(((P * (j + 1)) >> 2) - i0) : 0;
      const int64_t pidx = bf * B - kbv[0] + i0;  // row-relative pruned index
      uint32_t bp = bm_row, yp = 0, cp = 0;
      const uint32_t* cg = nullptr;
      if (n > 0) {
        const int64_t pb1 = (bf + 1) * B - kbv[1];
        const int bi = (nbs > 1 && pidx >= pb1) ? 1 : 0;
        const int skip = (int)(pidx - (bi ? pb1 : bf * B - kbv[0]));
        const uint32_t blk = bm_row + (uint32_t)(bi * B);
        bp = blk + find_in_block<true>(sb + (blk >> 3), nwb, skip);
        yp = u32(bias[3]) + (rowpk + u32(pidx)) * 8u;
        if (!overflow) {
          cp = skip_codes8(sm32, u32(bias[5]) + u32(bov[bi]), skip);
        } else {
          cg = vv.codes + (bov[bi] >> 5);
          cp = skip_codes(cg, (uint32_t)(bov[bi] & 31), skip);
        }
      }
      int nmax = n;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) nmax = max(nmax, __shfl_xor(nmax, o, 64));
      if (!overflow) {
        int done = 0;
        PRaw w = praw(sb, bp, yp, cp, g.wbits);
        for (; done < nmax; done += kPU) {
          const int t = min(max(n - done, 0), kPU);
          const uint32_t sbit = bp & 31u;
          const int have = __builtin_popcount(~__builtin_amdgcn_alignbit(w.q1, w.q0, sbit)) +
                           __builtin_popcount(~__builtin_amdgcn_alignbit(w.q2, w.q1, sbit));
          const int ncode = __builtin_popcount(__builtin_amdgcn_alignbit(w.c1, w.c0, cp & 31u));
          const bool ok = min(have, ncode) >= t;
          const int have32 = __builtin_popcount(~__builtin_amdgcn_alignbit(w.q1, w.q0, sbit));
          if (__all(t == kPU && ncode >= kPU && have32 >= kPU)) {
            pruned_group<kPU, false, true>(w, bp, yp, cp, sb, torg, plutb, dummy, kPU, g.wbits);
            // a second full group at once when it also fits the 32-bit windows
            // (fewer trips through the loop's tests and branches)
            const int t2 = min(max(n - done - kPU, 0), kPU);
            const uint32_t sb2 = bp & 31u;
            const int nc2 = __builtin_popcount(__builtin_amdgcn_alignbit(w.c1, w.c0, cp & 31u));
            const int h2 = __builtin_popcount(~__builtin_amdgcn_alignbit(w.q1, w.q0, sb2));
            if (__all(t2 == kPU && nc2 >= kPU && h2 >= kPU)) {
              pruned_group<kPU, false, true>(w, bp, yp, cp, sb, torg, plutb, dummy, kPU, g.wbits);
              done += kPU;
            }
          } else if (__all(t == kPU && ok)) {
            pruned_group<kPU, false>(w, bp, yp, cp, sb, torg, plutb, dummy, kPU, g.wbits);
          } else if (__all(ok)) {
            pruned_group<kPU, true>(w, bp, yp, cp, sb, torg, plutb, dummy, t, g.wbits);
          } else {
            // in two halves, as for the kept values
            constexpr int H1 = kPU / 2, H2 = kPU - kPU / 2;
            const int t1 = t < H1 ? t : H1, t2 = t - t1;
            if (__all(ok1_pruned(w, bp, cp, t1))) {
              pruned_group<H1, true>(w, bp, yp, cp, sb, torg, plutb, dummy, t1, g.wbits);
              if (__all(ok1_pruned(w, bp, cp, t2))) {
                pruned_group<H2, true>(w, bp, yp, cp, sb, torg, plutb, dummy, t2, g.wbits);
              } else {
                for (int u = 0; u < H2; ++u)
                  if (u < t2) pruned_step(sb, bp, bm_end, yp, cp, nullptr, torg, pv);
                w = praw(sb, bp, yp, cp, g.wbits);
              }
            } else {
              for (int u = 0; u < kPU; ++u)
                if (u < t) pruned_step(sb, bp, bm_end, yp, cp, nullptr, torg, pv);
              w = praw(sb, bp, yp, cp, g.wbits);
            }
          }
        }
      } else {
        for (int i = 0; i < nmax; ++i)
          if (i < n) pruned_step(sb, bp, bm_end, yp, cp, cg, torg, pv);
      }
    }
    wsync();  // the tile is complete

    if (MODE == 0) {
      // v_mfma_f32_16x16x32_bf16: lane (n, kq) feeds tile row n and token n,
      // columns 8kq..8kq+7 of each 32-column step
      auto step = [&](int ks, const v8s& bop) {
        const uint32_t ta = tileb + 2u * (uint32_t)(xn * g.TS + ks * 32 + 8 * xkq);
        const lds_u32c* tp = (const lds_u32c*)(uintptr_t)ta;
        const uint32_t a0 = tp[0], a1 = tp[1], a2 = tp[2], a3 = tp[3];
        const v8s aop = v8s{(short)(a0 & 0xFFFF), (short)(a0 >> 16), (short)(a1 & 0xFFFF),
                            (short)(a1 >> 16), (short)(a2 & 0xFFFF), (short)(a2 >> 16),
                            (short)(a3 & 0xFFFF), (short)(a3 >> 16)};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, aop),
                                                      __builtin_bit_cast(v8bf, bop), acc, 0, 0, 0);
      };
#pragma unroll
      for (int q = 0; q < kXPre; ++q)
        if (q < nks) step(q, xq[q]);
      for (int ks = kXPre; ks < nks; ++ks) step(ks, x_frag(ks));
    } else {
      const int cpr = nbs * (int)B / 8;  // 16-byte chunks per tile row
      for (int c = lane; c < kRows * cpr; c += 64) {
        const int rr = c / cpr, cc = c - rr * cpr;
        if (row0 + rr < R) {
          const uint32_t ta = tileb + 2u * (uint32_t)(rr * g.TS + cc * 8);
          const lds_u32c* tp = (const lds_u32c*)(uintptr_t)ta;
          const u32x4 v = u32x4{tp[0], tp[1], tp[2], tp[3]};
          *reinterpret_cast<u32x4*>(out + (row0 + rr) * C + bf * B + cc * 8) = v;
        }
      }
    }
    wsync();  // every lane is done with the tile, the staged runs and the stage's words
    if (more) put_meta(mr_next);
    wsync();
  }

  if (MODE == 0) {
    // the waves' partial products through shared memory (each wave's tile
    // region), summed in wave order: the result does not depend on timing
    float* part = reinterpret_cast<float*>(smem + g.wave_off + g.tile_off);
    const int pstride = g.wave_bytes / 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) part[wave * pstride + 64 * e + lane] = acc[e];
    __syncthreads();
    if (wave == 0) {
      float sum[4] = {0.f, 0.f, 0.f, 0.f};
      for (int w = 0; w < g.nsplit; ++w) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sum[e] += part[w * pstride + 64 * e + lane];
      }
      // D[i][j]: this lane holds rows 4 kq + e of the 16, token n
      const int n = lane & 15, kq = lane >> 4;
      if (n < ntok) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t rr = row0 + 4 * kq + e;
          if (rr < R) Y[(int64_t)n * ldy + rr] = sum[e];
        }
      }
    }
  }
}

int a16(int64_t v) { return (int)((v + 15) / 16 * 16); }

constexpr int64_t kMaxLds = 150 * 1024;

XGeom make_xgeom(const Shape& sh, const SpecViewC1& sv, const VerifViewC1& vv) {
  XGeom g = {};
  const int64_t B = sh.block, nb = sh.cols / B;
  const int fw = 1 + sh.mant;
  g.Wb = B >= 256 ? 1 : 2;
  if (const int w = option(OPT_EXACT_BLOCKS); w >= 1 && w <= 2) g.Wb = w;
  g.TS = (int)(g.Wb * B + 2);
  g.nstage = (nb + g.Wb - 1) / g.Wb;
  g.wbits = 27;
  const int64_t pos = (int64_t)g.Wb * B;  // positions per row per stage
  // fixed-width sections: 1 + 8 bits per position, plus chunk rounding
  const int64_t fix_row = (9 * pos + 127) / 128 * 16 + 7 * 16;
  // codes: twice the tensor's average code bits per position, at least 4
  const double tot = (double)(sv.codes_limit + vv.codes_limit) * 32.0;
  const double avg = sh.rows * sh.cols > 0 ? tot / ((double)sh.rows * (double)sh.cols) : 4.0;
  const double cbits = std::max(4.0, 2.0 * avg + 0.5);
  const int64_t cod_row = ((int64_t)(pos * cbits / 128.0) + 4) * 16;
  int64_t o = 0;
  g.perm_off = (int)o;
  o += 512;
  g.klut_off = (int)o;
  o += a16(fw <= 5 ? (int64_t)(32 << fw) * 2 : 64);
  g.plut_off = (int)o;
  o += 128;
  g.wave_off = (int)o;
  int64_t w = 0;  // one wave's region
  g.meta_off = (int)w;
  w += kRows * 9 * 4;
  g.dummy_off = (int)w;
  w += 256;
  g.tile_off = (int)w;
  w += a16((int64_t)kRows * g.TS * 2);
  g.fix_off = (int)w;
  g.fix_cap = (int)(kRows * fix_row);
  w += g.fix_cap + 64;  // window look-ahead
  g.cod_off = (int)w;
  g.cod_cap = (int)std::min<int64_t>(kRows * cod_row, 24 * 1024);
  w += g.cod_cap + 64;
  g.wave_bytes = (int)a16(w);
  // waves per workgroup: as many as shared memory holds, at most kMaxWaves and
  // at most one per stage; they take the row's stages in turn
  int64_t W = std::min<int64_t>(kMaxWaves, g.nstage);
  while (W > 1 && o + W * g.wave_bytes > kMaxLds) --W;
  if (W < 1) W = 1;
  g.nsplit = (int)W;
  g.lds_bytes = (int)(o + (int64_t)g.nsplit * g.wave_bytes);
  return g;
}

template <int MODE, int KU, bool KLUT>
hipError_t launch_staged_t(const SpecViewC1& sv, const VerifViewC1& vv, const Shape& sh,
                           XGeom g, const uint16_t* X, int ntok, int64_t ldx, float* Y,
                           int64_t ldy, uint16_t* out, hipStream_t s) {
  auto kern = k_exact_staged<MODE, KU, KLUT>;
  if (g.lds_bytes > kMaxLds) return hipErrorInvalidValue;
  if (g.lds_bytes > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, g.lds_bytes);
    if (e != hipSuccess) return e;
  }
  // one workgroup per 16 rows; its g.nsplit waves take the stages in turn, so
  // every output element is written once, by one wave
  const int64_t gx = (sh.rows + kRows - 1) / kRows;
  kern<<<dim3((unsigned)gx), 64 * g.nsplit, (size_t)g.lds_bytes, s>>>(sv, vv, sh, g, X, ntok, ldx,
                                                                    Y, ldy, out);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_staged(const SpecViewC1& sv, const VerifViewC1& vv, const Shape& sh,
                         const uint16_t* X, int ntok, int64_t ldx, float* Y, int64_t ldy,
                         uint16_t* out, hipStream_t s) {
  const XGeom g = make_xgeom(sh, sv, vv);
  if (sh.mant == 3)
    return launch_staged_t<MODE, 8, true>(sv, vv, sh, g, X, ntok, ldx, Y, ldy, out, s);
  if (sh.mant <= 4)
    return launch_staged_t<MODE, 4, true>(sv, vv, sh, g, X, ntok, ldx, Y, ldy, out, s);
  return launch_staged_t<MODE, 4, false>(sv, vv, sh, g, X, ntok, ldx, Y, ldy, out, s);
}

}  // namespace

bool exact_staged_fits(const Shape& sh, const SpecViewC1& sv, const VerifViewC1& vv) {
  if (sh.block < 32 || sh.block % 32) return false;
  // staged chunk indices are 32-bit: every section under 2^30 chunks of 16 bytes
  const int64_t lim = (int64_t)1 << 32;  // in 32-bit words
  if (sv.bitmap_limit >= lim || sv.fields_limit >= lim || sv.codes_limit >= lim ||
      vv.lowmant_limit >= lim || vv.pruned_limit >= lim || vv.codes_limit >= lim)
    return false;
  return make_xgeom(sh, sv, vv).lds_bytes <= kMaxLds;
}

hipError_t launch_verify_gemm_c1_staged(const SpecViewC1& sv, const VerifViewC1& vv,
                                        const Shape& sh, const uint16_t* X, int ntok,
                                        int64_t ldx, float* Y, int64_t ldy, hipStream_t s) {
  if (sh.rows == 0 || ntok == 0) return hipSuccess;
  return launch_staged<0>(sv, vv, sh, X, ntok, ldx, Y, ldy, nullptr, s);
}

hipError_t launch_reconstruct_c1_staged(const SpecViewC1& sv, const VerifViewC1& vv,
                                        const Shape& sh, uint16_t* out, hipStream_t s) {
  if (sh.rows == 0) return hipSuccess;
  return launch_staged<1>(sv, vv, sh, nullptr, 0, 0, nullptr, 0, out, s);
}

hipError_t launch_draft_decode_c1_staged(const SpecViewC1& sv, const Shape& sh, uint16_t* out,
                                         hipStream_t s) {
  if (sh.rows == 0) return hipSuccess;
  const VerifViewC1 none = {};
  return launch_staged<2>(sv, none, sh, nullptr, 0, 0, nullptr, 0, out, s);
}

}  // namespace cass
