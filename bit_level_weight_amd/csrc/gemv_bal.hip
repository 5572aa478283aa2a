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
// Decode.  A lane first finds where its part starts: binary search over the
// row's kept-before counts, popcounts inside the block, a select inside the
// word, and a select over the code ones.  Then it takes U values per group
// from three windows read at its bit positions (two LDS words and a funnel
// shift each): 64 keep bits, 32 code bits and 32 field bits.  Per value:
// position = find-first-set of the keep window, rank = count-trailing-zeros
// of the code window, field = bit-field extract, weight = one LDS table entry
// indexed by (rank, field).  A group whose windows do not hold U values for
// every lane of the wave (rare at the shipped keep ratios) is decoded one
// value at a time by the general step, which also serves the last few values
// of each part and codes of 32 bits or more.
#include <stdlib.h>
#include <string.h>

#include <algorithm>

#include "internal.hpp"
#include "staged_decode.hpp"

namespace cass {

namespace {

constexpr int kBalThreads = 256;
constexpr int kBalWaves = kBalThreads / 64;
constexpr int kRanks = 32;     // ranks of the (rank, field) -> fp32 table
constexpr int kSlack = 8;      // LDS words after each staged section (window look-ahead)
constexpr int kMaxFw = 6;      // field widths the table path serves (table <= 8 KB)
constexpr int64_t kBalMaxLds = 150 * 1024;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct BalGeom {
  int P, logP, rpw;     // parts per row, log2(P), rows per wave round (64 / P)
  int nb_top;           // largest power of two <= blocks per row
  int64_t nrounds;      // wave rounds: ceil(rows / rpw)
  int lut_off;          // LDS byte offsets (x at 0)
  int wave_off, wave_bytes;
  int kb_off, bo_off, bm_off, f_off, c_off;  // inside a wave region
  int c_cap;            // code words a wave region holds
  int lds_bytes;
  uint32_t xstride;     // LDS bytes between the batch rows of x
};

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One wave copies words [w0, w1) of src (16-byte aligned section base) to dst
// with 16-byte loads.  The copy starts at w0 rounded down to 4 words, which is
// returned, and never reads at or past word `limit` (a multiple of 4).
__device__ __forceinline__ int64_t wave_stage(uint32_t* dst, const uint32_t* src, int64_t w0,
                                              int64_t w1, int64_t limit, int lane) {
  const int64_t a0 = w0 & ~(int64_t)3;
  int64_t a1 = (w1 + 3) & ~(int64_t)3;
  if (a1 > limit) a1 = limit;
  const int64_t n4 = (a1 - a0) >> 2;
  const u32x4* s4 = reinterpret_cast<const u32x4*>(src + a0);
  u32x4* d4 = reinterpret_cast<u32x4*>(dst);
  for (int64_t i = lane; i < n4; i += 64) d4[i] = __builtin_nontemporal_load(s4 + i);
  return a0;
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
                                        uint32_t rowbit, int64_t row_len, const float* lut,
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
    bits = __float_as_uint(lut[((uint32_t)r << fw) | f]);
  else
    bits = ((f >> m) << 31) | ((uint32_t)perm[r] << 23) | ((f & ((1u << m) - 1u)) << (23 - m));
  const float wv = __uint_as_float(bits);
  const uint32_t xa = 2u * (pos - rowbit);
#pragma unroll
  for (int bb = 0; bb < BATCH; ++bb)
    acc[bb] = __builtin_fmaf(wv, x_at(xs, xa + bb * xstride), acc[bb]);
}

// U values from the windows at (bp, fp, cp): lo0/hi0 the 64 keep bits at bp,
// wf the 32 field bits at fp, wc0 the 32 code bits at cp, each holding at
// least U values.  With MASKED, slots u >= t add nothing (the part's last
// group); otherwise the positions advance past the U values.
template <int BATCH, int U, bool MASKED>
__device__ __forceinline__ void c1_group(uint32_t lo0, uint32_t hi0, uint32_t wf, uint32_t wc0,
                                         uint32_t& bp, uint32_t& fp, uint32_t& cp,
                                         uint32_t xorg, const float* lut, int fw,
                                         uint32_t xstride, int t, float* acc) {
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
    const uint32_t r = (uint32_t)__builtin_ctz(wc);  // code = r zeros, then a one
    wc = (wc >> r) >> 1;
    const uint32_t f = __builtin_amdgcn_ubfe(wf, (uint32_t)(u * fw), (uint32_t)fw);
    float wv = lut[(r << fw) | f];
    if (MASKED) wv = u < t ? wv : 0.f;
    const uint32_t xa = xs + 2u * p;
#pragma unroll
    for (int bb = 0; bb < BATCH; ++bb)
      acc[bb] = __builtin_fmaf(wv, x_at_addr(xa + bb * xstride), acc[bb]);
  }
  if (!MASKED) {
    bp += ((xs - xlo) >> 1) + p + 1u;
    fp += (uint32_t)(U * fw);
    // bits the U codes took: the window was shifted right by that many
    const uint32_t c0 = (uint32_t)__builtin_clz(wc0);
    cp += (wc ? (uint32_t)__builtin_clz(wc) : 32u) - c0;
  }
}

template <int BATCH, int U>
__global__ void __launch_bounds__(kBalThreads) k_gemv_c1_bal(SpecViewC1 v, Shape sh, BalGeom g,
                                                             const uint16_t* __restrict__ x,
                                                             int64_t ldx, float* __restrict__ y,
                                                             int64_t ldy) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int64_t R = sh.rows, C = sh.cols, k = sh.keep;
  const int B = (int)sh.block, nb = (int)(C / B), nwb = B / 32;
  const int m = sh.mant, fw = 1 + m;
  const uint32_t fmask = (1u << fw) - 1u;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // x (bf16 patterns) and the (rank, field) -> fp32 table, once per workgroup
  for (int bb = 0; bb < BATCH; ++bb) {
    uint16_t* xr = reinterpret_cast<uint16_t*>(smem + bb * g.xstride);
    for (int64_t j = threadIdx.x; j < C; j += kBalThreads) xr[j] = x[bb * ldx + j];
    // zeros after the row: masked slots of a part's last group may read there
    if (threadIdx.x < 128) xr[C + threadIdx.x] = 0;
  }
  float* lut = reinterpret_cast<float*>(smem + g.lut_off);
  for (int i = threadIdx.x; i < (kRanks << fw); i += kBalThreads) {
    const uint32_t r = (uint32_t)i >> fw, f = (uint32_t)i & fmask;
    lut[i] = __uint_as_float(((f >> m) << 31) | ((uint32_t)v.perm[r] << 23) |
                             ((f & ((1u << m) - 1u)) << (23 - m)));
  }
  __syncthreads();

  uint8_t* reg = smem + g.wave_off + wave * g.wave_bytes;
  uint16_t* kb_l = reinterpret_cast<uint16_t*>(reg + g.kb_off);
  uint32_t* bo_l = reinterpret_cast<uint32_t*>(reg + g.bo_off);
  uint32_t* bm_l = reinterpret_cast<uint32_t*>(reg + g.bm_off);
  uint32_t* f_l = reinterpret_cast<uint32_t*>(reg + g.f_off);
  uint32_t* c_l = reinterpret_cast<uint32_t*>(reg + g.c_off);

  const int rl = lane >> g.logP, part = lane & (g.P - 1);
  const int n_min = (int)(k >> g.logP);  // each part has n_min or n_min + 1 values
  const int n_max = (int)((k + g.P - 1) >> g.logP);
  const int G = n_min / U;               // fast groups every part can take
  const int n_tail = n_max - G * U;      // single steps after them (upper bound)
  const int64_t wpr = C / 32;            // bitmap words per row
  const int64_t nwaves = (int64_t)gridDim.x * kBalWaves;

  for (int64_t round = (int64_t)blockIdx.x * kBalWaves + wave; round < g.nrounds;
       round += nwaves) {
    const int64_t row0 = round * g.rpw;
    const int rows_here = (int)((R - row0 < g.rpw) ? R - row0 : g.rpw);
    // ---- stage this round's rows
    const int64_t bm_a0 = wave_stage(bm_l, v.bitmap, row0 * wpr, (row0 + rows_here) * wpr,
                                     v.bitmap_limit, lane);
    const int64_t fb0 = row0 * k * fw, fb1 = (row0 + rows_here) * k * fw;
    const int64_t f_a0 = wave_stage(f_l, v.fields, fb0 >> 5, (fb1 + 31) >> 5, v.fields_limit,
                                    lane);
    const int64_t cb0 = (int64_t)v.rowbase[row0];
    const int64_t cb1 = (row0 + rows_here < R) ? (int64_t)v.rowbase[row0 + rows_here]
                                                : v.codes_limit * 32;
    const int64_t cw0 = (cb0 >> 5) & ~(int64_t)3;
    int64_t cw1 = (((cb1 + 31) >> 5) + 3) & ~(int64_t)3;
    if (cw1 > v.codes_limit) cw1 = v.codes_limit;
    const bool c_in_lds = cw1 - cw0 <= g.c_cap;
    if (c_in_lds) wave_stage(c_l, v.codes, cb0 >> 5, (cb1 + 31) >> 5, v.codes_limit, lane);
    for (int i = lane; i < rows_here * nb; i += 64) {
      kb_l[i] = v.keptb[row0 * nb + i];
      bo_l[i] = v.blkoff[row0 * nb + i];
    }
    wave_sync();

    // ---- where this lane's part starts
    const int64_t row = row0 + rl;
    const bool active = rl < rows_here;
    const int i0 = (int)(((int64_t)part * k) >> g.logP);
    const int n = active ? (int)((((int64_t)part + 1) * k) >> g.logP) - i0 : 0;
    const uint32_t rowbit = (uint32_t)((row0 * wpr - bm_a0) * 32 + (int64_t)rl * C);
    uint32_t bp = 0, fp = 0, cp = 0;
    int64_t cabs = 0;  // absolute code bit of the part's first value
    if (n > 0) {
      const uint16_t* kbr = kb_l + rl * nb;
      int b = 0;
      for (int s = g.nb_top; s >= 1; s >>= 1)
        if (b + s < nb && kbr[b + s] <= i0) b += s;
      const int skip = i0 - kbr[b];
      int rem = skip;
      const uint32_t* bw = bm_l + (rowbit >> 5) + b * nwb;
      int wi = 0;
      uint32_t wd = bw[0];
      for (;;) {
        const int c = __builtin_popcount(wd);
        if (rem < c || wi == nwb - 1) break;  // (the second test: corrupt streams only)
        rem -= c;
        wd = bw[++wi];
      }
      bp = rowbit + (uint32_t)(b * B + wi * 32 + select_bit(wd, rem + 1));
      fp = (uint32_t)((row * k + i0) * fw - f_a0 * 32);
      cabs = (int64_t)v.rowbase[row] + bo_l[rl * nb + b];
      if (c_in_lds) {
        cp = skip_codes(c_l, (uint32_t)(cabs - cw0 * 32), skip);
      } else {
        cp = skip_codes(v.codes + (cabs >> 5), (uint32_t)(cabs & 31), skip);
      }
    }

    float acc[BATCH];
#pragma unroll
    for (int bb = 0; bb < BATCH; ++bb) acc[bb] = 0.f;

    // rounds where every lane has a part and the codes sit in LDS take the
    // grouped path; others (last partial round, tiny k, codes over the LDS
    // share) decode one value at a time
    const bool grouped = c_in_lds && rows_here == g.rpw && n_min > 0;
    if (grouped) {
      const uint32_t xorg = lds_addr(smem) - 2u * rowbit;  // x address of staged bit 0
      for (int gi = 0; gi <= G; ++gi) {
        // gi == G: the part's last t = n - G*U <= U values, slots u >= t masked
        const int t = gi < G ? U : n - G * U;
        if (gi == G && n_tail == 0) break;
        const uint32_t* qb = bm_l + (bp >> 5);
        const uint32_t sb = bp & 31u;
        const uint32_t q0 = qb[0], q1 = qb[1], q2 = qb[2];
        const uint32_t lo0 = __builtin_amdgcn_alignbit(q1, q0, sb);
        const uint32_t hi0 = __builtin_amdgcn_alignbit(q2, q1, sb);
        const uint32_t wf = window32(f_l, fp);
        const uint32_t wc0 = window32(c_l, cp);
        const int have = __builtin_popcount(lo0) + __builtin_popcount(hi0);
        const bool ok = min(have, __builtin_popcount(wc0)) >= U;
        if (__all(ok)) {
          if (gi < G)
            c1_group<BATCH, U, false>(lo0, hi0, wf, wc0, bp, fp, cp, xorg, lut, fw, g.xstride,
                                      U, acc);
          else
            c1_group<BATCH, U, true>(lo0, hi0, wf, wc0, bp, fp, cp, xorg, lut, fw, g.xstride,
                                     t, acc);
        } else {
          for (int u = 0; u < t; ++u)
            c1_step<BATCH>(bm_l, bp, f_l, fp, c_l, cp, rowbit, C, lut, v.perm, m, smem, g.xstride,
                           acc);
        }
      }
    } else if (c_in_lds) {
      for (int i = 0; i < n_max; ++i)
        if (i < n)
          c1_step<BATCH>(bm_l, bp, f_l, fp, c_l, cp, rowbit, C, lut, v.perm, m, smem, g.xstride,
                         acc);
    } else {
      // codes straight from global memory (a round whose codes exceed the LDS share)
      const uint32_t* cg = v.codes + (cabs >> 5);
      uint32_t cpg = cp;
      for (int i = 0; i < n_max; ++i)
        if (i < n)
          c1_step<BATCH>(bm_l, bp, f_l, fp, cg, cpg, rowbit, C, lut, v.perm, m, smem, g.xstride,
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
      for (int bb = 0; bb < BATCH; ++bb) y[bb * ldy + row] = acc[bb];
    }
    wave_sync();  // every lane is done with the staged words before the next round
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
BalGeom make_bal_geom(const Shape& sh, int batch, int64_t code_limit_words) {
  BalGeom g = {};
  const int64_t R = sh.rows, C = sh.cols, k = sh.keep, nb = C / sh.block;
  const int fw = 1 + sh.mant;
  // parts per row: 32 (two rows per wave round) keeps about six waves per SIMD
  // resident within LDS; very tall matrices take 16 (more values per part,
  // fewer part starts); parts keep at least 16 values
  int P = R >= 16384 ? 16 : 32;
  while (P > 1 && k / P < 16) P /= 2;
  if (const char* e = getenv("CASS_GEMV_PARTS")) {
    const int p = atoi(e);
    if (p >= 1 && p <= 64 && (p & (p - 1)) == 0) P = p;
  }
  g.P = P;
  g.logP = __builtin_ctz(P);
  g.rpw = 64 / P;
  g.nb_top = 1;
  while (2 * g.nb_top < nb) g.nb_top *= 2;
  g.nrounds = (R + g.rpw - 1) / g.rpw;
  g.xstride = (uint32_t)a16(2 * C + 256);
  int64_t pos = (int64_t)batch * g.xstride;
  g.lut_off = (int)pos;
  pos += a16((int64_t)(kRanks << fw) * 4);
  g.wave_off = (int)pos;
  int64_t w = 0;
  g.kb_off = (int)w;
  w += a16((int64_t)g.rpw * nb * 2);
  g.bo_off = (int)w;
  w += a16((int64_t)g.rpw * nb * 4);
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
  g.wave_bytes = (int)w;
  pos += (int64_t)kBalWaves * w;
  g.lds_bytes = (fw > kMaxFw || pos > kBalMaxLds) ? (int)(kBalMaxLds + 1) : (int)pos;
  return g;
}

template <int BATCH, int U>
hipError_t launch_bal(const SpecViewC1& v, const Shape& sh, const BalGeom& g, const uint16_t* x,
                      int64_t ldx, float* y, int64_t ldy, hipStream_t s) {
  auto kern = k_gemv_c1_bal<BATCH, U>;
  if (g.lds_bytes > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, g.lds_bytes);
    if (e != hipSuccess) return e;
  }
  const int per_cu = std::max(1, std::min(8, (160 * 1024) / std::max(g.lds_bytes, 1)));
  int64_t grid = (g.nrounds + kBalWaves - 1) / kBalWaves;
  const int64_t cap = (int64_t)device_cu_count() * per_cu;
  if (grid > cap) grid = cap;
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

}  // namespace

bool draft_gemv_bal_fits(const Shape& sh, int batch, int64_t code_limit_words) {
  return make_bal_geom(sh, batch, code_limit_words).lds_bytes <= kBalMaxLds;
}

hipError_t launch_draft_gemv_c1_bal(const SpecViewC1& v, const Shape& sh, const uint16_t* x,
                                    int batch, int64_t ldx, float* y, int64_t ldy,
                                    hipStream_t s) {
  if (sh.rows == 0) return hipSuccess;
  const BalGeom g = make_bal_geom(sh, batch, v.codes_limit);
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

}  // namespace cass
