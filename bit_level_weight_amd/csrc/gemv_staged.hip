// Fused draft GEMV, staged variant (the default path):
//   y[b][n] = sum over kept j of Wdraft[n][j] * x[b][j], fp32 accumulation.
//
// Method: Cassandra review (marsggbo.github.io), section 3.1 -- the draft
// model runs the full-size product on the zero-filled speculation data, so only
// kept values contribute and only speculation bytes are read; section 3.3 --
// the decoder's bit-level work is de-sparsification (here: find-first-set over
// the keep bitmap) and unary decoding (here: count-trailing-zeros over the code
// bits), done by the SIMD lanes instead of a dedicated decoder.
//
// Work split: a workgroup owns a tile of whole rows.  Per tile it first copies
// the tile's bitmap words, sign/mantissa fields and exponent codes from HBM to
// LDS with coalesced 16-byte non-temporal loads (each compressed byte is read
// from HBM once), then each lane decodes one (row, block of 256 positions) from
// LDS: it walks the block's bitmap bits, takes the (1+m)-bit field and the
// unary rank of each kept value, turns (rank, field) into the fp32 weight with
// one LDS table lookup, and multiplies it with x (staged once per workgroup).
// Block partials of a row are summed in a fixed order (deterministic).
#include <stdlib.h>
#include <string.h>

#include <algorithm>

#include "internal.hpp"
#include "staged_decode.hpp"

namespace cass {

namespace {

constexpr int kThreads = 256;
constexpr int kLutRanks = 32;     // ranks of the (rank, field) -> fp32 bits table
constexpr int kSlackWords = 8;    // LDS words after each staged buffer (reader look-ahead)
constexpr int64_t kMaxLds = 150 * 1024;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct StagedGeom {
  int rows_per_tile;
  int64_t ntiles;
  int off_lut, off_part, off_bm, off_f, off_c;  // LDS byte offsets (x at 0)
  int lds_bytes;
  int bm_cap, f_cap, c_cap;  // words
  int rmax;                  // ranks covered by the table
  int sub;                   // bitmap words decoded per lane (C-1)
  uint32_t xstride;          // LDS bytes per batch row of x (padded layout)
};

// Copy words [w0, w1) of src (16-byte aligned section base) into dst with
// 16-byte loads; the copy starts at w0 rounded down to 4 words, which is
// returned, and never reads at or past word `limit` (a multiple of 4).
__device__ __forceinline__ int64_t stage_words(uint32_t* dst, const uint32_t* src, int64_t w0,
                                               int64_t w1, int64_t limit) {
  const int64_t a0 = w0 & ~(int64_t)3;
  int64_t a1 = (w1 + 3) & ~(int64_t)3;
  if (a1 > limit) a1 = limit;
  const int64_t n4 = (a1 - a0) >> 2;
  const u32x4* s4 = reinterpret_cast<const u32x4*>(src + a0);
  u32x4* d4 = reinterpret_cast<u32x4*>(dst);
  for (int64_t i = threadIdx.x; i < n4; i += kThreads) d4[i] = __builtin_nontemporal_load(s4 + i);
  return a0;
}

// x into LDS in the padded layout of x_lds_off, batch rows xstride bytes apart.
template <int BATCH>
__device__ __forceinline__ void stage_x(const uint16_t* __restrict__ x, int64_t ldx, int64_t C,
                                        uint8_t* xs, uint32_t xstride) {
  for (int bb = 0; bb < BATCH; ++bb)
    for (int64_t j = threadIdx.x; j < C; j += kThreads)
      *reinterpret_cast<uint16_t*>(xs + bb * xstride + x_lds_off((uint32_t)j)) = x[bb * ldx + j];
}

// Sum the nb partials of each row of the tile: one wave per (row, batch)
// pair, lanes read consecutive partials (no LDS bank conflicts) and a fixed
// butterfly combines them, so the result does not depend on timing.
template <int BATCH>
__device__ __forceinline__ void reduce_rows(const float* part, int rows_here, int64_t nb,
                                            int64_t row0, float* __restrict__ y, int64_t ldy) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = wave; i < rows_here * BATCH; i += kThreads / 64) {
    const int r = i / BATCH, bb = i % BATCH;
    float s = 0.f;
    for (int64_t b = lane; b < nb; b += 64) s += part[((int64_t)r * nb + b) * BATCH + bb];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
    if (lane == 0) y[bb * ldy + row0 + r] = s;
  }
}

template <int BATCH>
__global__ void __launch_bounds__(kThreads) k_gemv_c1_staged(SpecViewC1 v, Shape sh, StagedGeom g,
                                                             const uint16_t* __restrict__ x,
                                                             int64_t ldx, float* __restrict__ y,
                                                             int64_t ldy) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int64_t C = sh.cols, B = sh.block, nb = C / B, k = sh.keep;
  const int m = sh.mant, fw = 1 + m;
  uint8_t* xsb = smem;
  uint32_t* lut = reinterpret_cast<uint32_t*>(smem + g.off_lut);
  float* part = reinterpret_cast<float*>(smem + g.off_part);
  uint32_t* bm_l = reinterpret_cast<uint32_t*>(smem + g.off_bm);
  uint32_t* f_l = reinterpret_cast<uint32_t*>(smem + g.off_f);
  uint32_t* c_l = reinterpret_cast<uint32_t*>(smem + g.off_c);

  stage_x<BATCH>(x, ldx, C, xsb, g.xstride);
  const int lut_n = g.rmax << fw;
  for (int i = threadIdx.x; i < lut_n; i += kThreads) {
    const uint32_t r = (uint32_t)i >> fw, f = (uint32_t)i & ((1u << fw) - 1u);
    lut[i] = ((f >> m) << 31) | ((uint32_t)v.perm[r] << 23) | ((f & ((1u << m) - 1u)) << (23 - m));
  }

  for (int64_t tile = blockIdx.x; tile < g.ntiles; tile += gridDim.x) {
    const int64_t row0 = tile * g.rows_per_tile;
    const int rows_here =
        (int)((sh.rows - row0 < g.rows_per_tile) ? sh.rows - row0 : g.rows_per_tile);
    // stage the tile's compressed bytes
    const int64_t bm_a0 = stage_words(bm_l, v.bitmap, row0 * (C / 32),
                                      (row0 + rows_here) * (C / 32), v.bitmap_limit);
    const int64_t fb0 = row0 * k * fw, fb1 = (row0 + rows_here) * k * fw;
    const int64_t f_a0 = stage_words(f_l, v.fields, fb0 >> 5, (fb1 + 31) >> 5, v.fields_limit);
    const int64_t cb0 = (int64_t)v.rowbase[row0];
    const int64_t cb1 = (row0 + rows_here < sh.rows) ? (int64_t)v.rowbase[row0 + rows_here]
                                                      : v.codes_limit * 32;
    const int64_t cw0 = (cb0 >> 5) & ~(int64_t)3;
    int64_t cw1 = (((cb1 + 31) >> 5) + 3) & ~(int64_t)3;
    if (cw1 > v.codes_limit) cw1 = v.codes_limit;
    const bool codes_in_lds = (cw1 - cw0) <= g.c_cap;
    int64_t c_a0 = 0;
    if (codes_in_lds) c_a0 = stage_words(c_l, v.codes, cb0 >> 5, (cb1 + 31) >> 5, v.codes_limit);
    __syncthreads();

    // one lane per `sub` bitmap words (a part of a block): lanes_pb lanes per block
    const int nwb = (int)(B / 32);
    const int lanes_pb = nwb / g.sub;
    const int64_t lpr = nb * lanes_pb;  // lanes per row
    for (int64_t p = threadIdx.x; p < (int64_t)rows_here * lpr; p += kThreads) {
      const int64_t row = row0 + p / lpr, q = p % lpr;
      const int64_t b = q / lanes_pb;
      const int j = (int)(q % lanes_pb);
      const int64_t bi = row * nb + b;
      float acc[BATCH];
#pragma unroll
      for (int bb = 0; bb < BATCH; ++bb) acc[bb] = 0.f;
      const uint32_t* bw0 = bm_l + (bi * nwb - bm_a0);
      int kbs = 0;  // kept values of the block before this part
      for (int w = 0; w < j * g.sub; ++w) kbs += __builtin_popcount(bw0[w]);
      const uint32_t kb = v.keptb[bi] + (uint32_t)kbs;
      const uint64_t epos = v.rowbase[row] + v.blkoff[bi];
      const uint32_t fp = (uint32_t)(((uint64_t)row * k + kb) * (uint64_t)fw - (uint64_t)f_a0 * 32);
      const uint32_t e0 = (uint32_t)(b * B + j * g.sub * 32);  // first x element of the part
      const uint32_t* pw = bw0 + j * g.sub;
      // codes from LDS, or straight from global memory when the tile's codes
      // did not fit the LDS buffer (two instances, so each reads its own space)
      if (codes_in_lds) {
        const uint32_t cp = skip_codes(c_l, (uint32_t)(epos - (uint64_t)c_a0 * 32), kbs);
        bool fast = g.sub == 2 || g.sub == 4;  // and no empty word before the part's last
        for (int w = 0; w + 1 < g.sub; ++w) fast = fast && pw[w] != 0u;
        float accf[BATCH];
#pragma unroll
        for (int bb = 0; bb < BATCH; ++bb) accf[bb] = 0.f;
        if (fast) {
          fast = g.sub == 2
                     ? c1_part_regs<BATCH, 2>(pw, f_l, fp, c_l, cp, xsb, x_lds_off(e0), g.xstride,
                                              lut, m, accf)
                     : c1_part_regs<BATCH, 4>(pw, f_l, fp, c_l, cp, xsb, x_lds_off(e0), g.xstride,
                                              lut, m, accf);
        }
        if (fast) {
#pragma unroll
          for (int bb = 0; bb < BATCH; ++bb) acc[bb] = accf[bb];
        } else {
          c1_block<BATCH>(pw, g.sub, f_l, fp, c_l, cp, xsb, e0, g.xstride, lut, g.rmax, m, v.perm,
                          acc);
        }
      } else {
        const uint32_t* cg = v.codes + (epos >> 5);
        const uint32_t cp = skip_codes(cg, (uint32_t)(epos & 31), kbs);
        c1_block<BATCH>(pw, g.sub, f_l, fp, cg, cp, xsb, e0, g.xstride, lut, g.rmax, m, v.perm,
                        acc);
      }
#pragma unroll
      for (int bb = 0; bb < BATCH; ++bb) part[p * BATCH + bb] = acc[bb];
    }
    __syncthreads();
    reduce_rows<BATCH>(part, rows_here, lpr, row0, y, ldy);
    __syncthreads();
  }
}

// Cassandra-2: a kept value is sign * a * 2^(E - 127 - m) with E the shared
// exponent of its 32 positions (OCP MX: one shared 8-bit exponent per 32).
template <int BATCH>
__global__ void __launch_bounds__(kThreads) k_gemv_c2_staged(SpecViewC2 v, Shape sh, StagedGeom g,
                                                             const uint16_t* __restrict__ x,
                                                             int64_t ldx, float* __restrict__ y,
                                                             int64_t ldy) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int64_t C = sh.cols, B = sh.block, nb = C / B, k = sh.keep;
  const int m = sh.mant, fw = 2 + m;
  uint8_t* xsb = smem;
  float* part = reinterpret_cast<float*>(smem + g.off_part);
  uint32_t* bm_l = reinterpret_cast<uint32_t*>(smem + g.off_bm);
  uint32_t* f_l = reinterpret_cast<uint32_t*>(smem + g.off_f);
  uint32_t* e_l = reinterpret_cast<uint32_t*>(smem + g.off_c);
  const uint32_t amask = (2u << m) - 1u;

  stage_x<BATCH>(x, ldx, C, xsb, g.xstride);

  for (int64_t tile = blockIdx.x; tile < g.ntiles; tile += gridDim.x) {
    const int64_t row0 = tile * g.rows_per_tile;
    const int rows_here =
        (int)((sh.rows - row0 < g.rows_per_tile) ? sh.rows - row0 : g.rows_per_tile);
    const int64_t g0 = row0 * (C / 32), g1 = (row0 + rows_here) * (C / 32);
    const int64_t bm_a0 = stage_words(bm_l, v.bitmap, g0, g1, v.bitmap_limit);
    const int64_t e_a0 = stage_words(e_l, reinterpret_cast<const uint32_t*>(v.shexp), g0 >> 2,
                                     (g1 + 3) >> 2, v.shexp_limit);
    const int64_t fb0 = row0 * k * fw, fb1 = (row0 + rows_here) * k * fw;
    const int64_t f_a0 = stage_words(f_l, v.fields, fb0 >> 5, (fb1 + 31) >> 5, v.fields_limit);
    __syncthreads();
    const uint8_t* se_l = reinterpret_cast<const uint8_t*>(e_l) - e_a0 * 4;

    for (int64_t p = threadIdx.x; p < (int64_t)rows_here * nb; p += kThreads) {
      const int64_t row = row0 + p / nb, b = p % nb;
      const int64_t bi = row * nb + b;
      float acc[BATCH];
#pragma unroll
      for (int bb = 0; bb < BATCH; ++bb) acc[bb] = 0.f;
      const uint32_t kb = v.keptb[bi];
      uint32_t fp = (uint32_t)(((uint64_t)row * k + kb) * (uint64_t)fw - (uint64_t)f_a0 * 32);
      const uint32_t* bmw = bm_l + (bi * (B / 32) - bm_a0);
      const uint8_t* se = se_l + bi * (B / 32);
      // one bitmap word at a time: the shared exponent is per 32 positions
      for (int wi = 0; wi < (int)(B / 32); ++wi) {
        uint32_t bw = bmw[wi];
        if (!bw) continue;
        // 2^(E-127-m) as an fp32 (normal for E-m >= 1, subnormal below)
        const int em = (int)se[wi] - m;
        const float scale = __uint_as_float(em >= 1 ? ((uint32_t)em << 23) : (1u << (em + 22)));
        const uint32_t xw = x_lds_off((uint32_t)(b * B + wi * 32));
        while (bw) {
          const int pb = __builtin_ctz(bw);
          bw &= bw - 1u;
          const uint32_t f = window32(f_l, fp);
          fp += (uint32_t)fw;
          const float mag = (float)(f & amask) * scale;
          const float wv = __uint_as_float(__float_as_uint(mag) | (((f >> (m + 1)) & 1u) << 31));
#pragma unroll
          for (int bb = 0; bb < BATCH; ++bb)
            acc[bb] = __builtin_fmaf(wv, x_at(xsb, xw + 2u * (uint32_t)pb + bb * g.xstride), acc[bb]);
        }
      }
#pragma unroll
      for (int bb = 0; bb < BATCH; ++bb) part[p * BATCH + bb] = acc[bb];
    }
    __syncthreads();
    reduce_rows<BATCH>(part, rows_here, nb, row0, y, ldy);
    __syncthreads();
  }
}

int align16(int64_t v) { return (int)((v + 15) / 16 * 16); }

// LDS plan of the staged kernels; lds_bytes > kMaxLds means "does not fit".
StagedGeom make_geom(const Shape& sh, int batch, int format, int64_t code_limit_words) {
  StagedGeom g = {};
  const int64_t C = sh.cols, nb = C / sh.block;
  const int nwb = (int)(sh.block / 32);
  const int fw = format == CASS_FMT_C1_UNARY ? 1 + sh.mant : 2 + sh.mant;
  // Words of bitmap per lane: the largest power of two (at most a block) that
  // still gives about four waves per SIMD; fewer words per lane means more
  // lanes but more idle lanes (kept counts per part vary more).
  g.sub = nwb < 4 ? nwb : 4;
  if (format == CASS_FMT_C1_UNARY) {
    const int64_t want_lanes = (int64_t)device_cu_count() * 4 * 4 * 64;
    while (g.sub > 1 && sh.rows * nb * (nwb / g.sub) < want_lanes) g.sub /= 2;
    if (const int s = option(OPT_GEMV_SUB); s >= 1 && s <= nwb && (nwb % s) == 0) g.sub = s;
  }
  const int64_t lpr = nb * (nwb / g.sub);  // lanes per row
  g.rows_per_tile = (int)(lpr >= kThreads ? 1 : kThreads / lpr);
  if (sh.rows > 0 && g.rows_per_tile > sh.rows) g.rows_per_tile = (int)sh.rows;
  if (g.rows_per_tile < 1) g.rows_per_tile = 1;
  const int T = g.rows_per_tile;
  g.ntiles = (sh.rows + T - 1) / T;
  g.rmax = kLutRanks;  // the fast loop decodes ranks 0..31 from one 32-bit window
  g.xstride = (uint32_t)align16(2 * C + 4 * (C / 32));
  int64_t pos = (int64_t)batch * g.xstride;
  g.off_lut = (int)pos;
  if (format == CASS_FMT_C1_UNARY) pos += align16((int64_t)(g.rmax << fw) * 4);
  g.off_part = (int)pos;
  pos += align16((int64_t)T * lpr * batch * 4);
  g.bm_cap = (int)(T * C / 32 + kSlackWords);
  g.off_bm = (int)pos;
  pos += align16((int64_t)g.bm_cap * 4);
  const int64_t f_words = ((int64_t)T * sh.keep * fw + 31) / 32 + 2 + kSlackWords;
  g.f_cap = (int)f_words;
  g.off_f = (int)pos;
  pos += align16(f_words * 4);
  if (format == CASS_FMT_C1_UNARY) {
    // codes: twice the average per tile (the tile falls back to global reads beyond)
    const int64_t avg = sh.rows > 0 ? code_limit_words / sh.rows : 0;
    int64_t cap = 2 * avg * T + 64;
    if (cap > 8192) cap = 8192;
    g.c_cap = (int)cap;
    g.off_c = (int)pos;
    pos += align16((cap + kSlackWords) * 4);
  } else {
    g.c_cap = (int)(T * C / 32 / 4 + 2 + kSlackWords);  // shared exponents, bytes/4
    g.off_c = (int)pos;
    pos += align16((int64_t)g.c_cap * 4);
  }
  g.lds_bytes = pos > kMaxLds ? (int)(kMaxLds + 1) : (int)pos;
  return g;
}

template <typename Kern, typename View>
hipError_t launch_staged(Kern kern, const View& v, const Shape& sh, const StagedGeom& g,
                         const uint16_t* x, int64_t ldx, float* y, int64_t ldy, hipStream_t s) {
  if (g.lds_bytes > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, g.lds_bytes);
    if (e != hipSuccess) return e;
  }
  const int per_cu = g.lds_bytes > 0 ? std::max(1, (160 * 1024) / g.lds_bytes) : 8;
  int64_t grid = g.ntiles;
  const int64_t cap = (int64_t)device_cu_count() * std::min(per_cu, 8);
  if (grid > cap) grid = cap;
  kern<<<(unsigned)grid, kThreads, (size_t)g.lds_bytes, s>>>(v, sh, g, x, ldx, y, ldy);
  return hipGetLastError();
}

// gemv_path 2 selects the direct kernels (the tests cover that path on shapes
// the staged kernels accept).
bool force_direct() { return option(OPT_GEMV_PATH) == 2; }

}  // namespace

bool draft_gemv_staged_fits(const Shape& sh, int batch, int format, int64_t code_limit_words) {
  return make_geom(sh, batch, format, code_limit_words).lds_bytes <= kMaxLds;
}

#define CASS_BATCH_CASES(KERN, VIEW)                                                        \
  switch (batch) {                                                                          \
    case 1: return launch_staged(KERN<1>, VIEW, sh, g, x, ldx, y, ldy, s);                  \
    case 2: return launch_staged(KERN<2>, VIEW, sh, g, x, ldx, y, ldy, s);                  \
    case 3: return launch_staged(KERN<3>, VIEW, sh, g, x, ldx, y, ldy, s);                  \
    case 4: return launch_staged(KERN<4>, VIEW, sh, g, x, ldx, y, ldy, s);                  \
    case 5: return launch_staged(KERN<5>, VIEW, sh, g, x, ldx, y, ldy, s);                  \
    case 6: return launch_staged(KERN<6>, VIEW, sh, g, x, ldx, y, ldy, s);                  \
    case 7: return launch_staged(KERN<7>, VIEW, sh, g, x, ldx, y, ldy, s);                  \
    case 8: return launch_staged(KERN<8>, VIEW, sh, g, x, ldx, y, ldy, s);                  \
    default: return hipErrorInvalidValue;                                                   \
  }

hipError_t launch_draft_gemv_c1(const SpecViewC1& v, const Shape& sh, const uint16_t* x,
                                int batch, int64_t ldx, float* y, int64_t ldy, hipStream_t s) {
  if (sh.rows == 0) return hipSuccess;
  const bool want_staged = option(OPT_GEMV_PATH) == 1;
  const bool sb = v.sb_log >= 0;  // format 4: the balanced kernel or the direct one
  if (!force_direct() && !want_staged &&
      draft_gemv_bal_fits(sh, batch, v.codes_limit, sb ? v.nsb : 0))
    return launch_draft_gemv_c1_bal(v, sh, x, batch, ldx, y, ldy, s);
  const StagedGeom g = make_geom(sh, batch, CASS_FMT_C1_UNARY, v.codes_limit);
  if (sb || g.lds_bytes > kMaxLds || force_direct())
    return launch_draft_gemv_c1_direct(v, sh, x, batch, ldx, y, ldy, s);
  CASS_BATCH_CASES(k_gemv_c1_staged, v)
}

hipError_t launch_draft_gemv_c2(const SpecViewC2& v, const Shape& sh, const uint16_t* x,
                                int batch, int64_t ldx, float* y, int64_t ldy, hipStream_t s) {
  if (sh.rows == 0) return hipSuccess;
  const bool want_staged = option(OPT_GEMV_PATH) == 1;
  if (!force_direct() && !want_staged && draft_gemv_bal_c2_fits(sh, batch))
    return launch_draft_gemv_c2_bal(v, sh, x, batch, ldx, y, ldy, s);
  const StagedGeom g = make_geom(sh, batch, CASS_FMT_C2_MX32, 0);
  if (g.lds_bytes > kMaxLds || force_direct())
    return launch_draft_gemv_c2_direct(v, sh, x, batch, ldx, y, ldy, s);
  CASS_BATCH_CASES(k_gemv_c2_staged, v)
}

#undef CASS_BATCH_CASES

}  // namespace cass
