// Fused draft GEMV, direct variant: every stream word is read from global
// memory by the lane that decodes it (no LDS staging of the compressed bytes).
// Serves shapes whose tiles do not fit the staged kernels' LDS plan.
//
// Fused draft GEMV: decode the speculation stream and multiply in one pass,
// y[b][n] = sum over kept j of Wdraft[n][j] * x[b][j], fp32 accumulation.
//
// Method: Cassandra review (marsggbo.github.io), section 3.1 -- the draft
// model runs the full-size product on the zero-filled speculation data, so only
// the kept values contribute and only speculation bytes are read; section 3.3
// -- de-sparsification and unary decoding are the bit-level work a decoder
// must do (done here per lane: bitmap bits are walked with find-first-set,
// unary codes are decoded with count-trailing-zeros).
//
// Work split: one lane per (row, block of `block` positions).  A workgroup
// owns a tile of whole rows, so the per-block partial sums of a row are
// reduced in LDS in a fixed order (deterministic result).  x is staged in LDS
// once per workgroup as bf16; the workgroup then walks row tiles.
#include "bits.hpp"
#include "internal.hpp"

namespace cass {

namespace {

constexpr int kThreads = 256;

struct GemvGeom {
  int rows_per_tile;
  int64_t ntiles;
  int64_t x_lds_elems;  // batch * cols, rounded up to 8
};

template <int BATCH>
__device__ __forceinline__ void stage_x(const uint16_t* __restrict__ x, int64_t ldx, int64_t C,
                                        uint16_t* xs) {
  for (int bb = 0; bb < BATCH; ++bb)
    for (int64_t j = threadIdx.x; j < C; j += kThreads) xs[bb * C + j] = x[bb * ldx + j];
}

template <int BATCH>
__device__ __forceinline__ void reduce_tile(const float* part, int rows_here, int64_t nb,
                                            int64_t row0, float* __restrict__ y, int64_t ldy) {
  for (int i = threadIdx.x; i < rows_here * BATCH; i += kThreads) {
    const int r = i / BATCH, bb = i % BATCH;
    float s = 0.f;
    for (int64_t b = 0; b < nb; ++b) s += part[((int64_t)r * nb + b) * BATCH + bb];
    y[bb * ldy + row0 + r] = s;
  }
}

template <int BATCH>
__global__ void __launch_bounds__(kThreads) k_draft_gemv_c1(SpecViewC1 v, Shape sh, GemvGeom g,
                                                            const uint16_t* __restrict__ x,
                                                            int64_t ldx, float* __restrict__ y,
                                                            int64_t ldy) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int64_t C = sh.cols, B = sh.block, nb = C / B;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  uint32_t* ebits = reinterpret_cast<uint32_t*>(smem + g.x_lds_elems * 2);
  float* part = reinterpret_cast<float*>(ebits + 256);

  stage_x<BATCH>(x, ldx, C, xs);
  // rank -> fp32 exponent field
  ebits[threadIdx.x] = (uint32_t)v.perm[threadIdx.x] << 23;
  __syncthreads();

  const int m = sh.mant;
  const uint32_t mmask = (1u << m) - 1u;
  const int fshift = 23 - m;
  const int64_t pairs = (int64_t)g.rows_per_tile * nb;

  for (int64_t tile = blockIdx.x; tile < g.ntiles; tile += gridDim.x) {
    const int64_t row0 = tile * g.rows_per_tile;
    const int rows_here = (int)((sh.rows - row0 < g.rows_per_tile) ? sh.rows - row0 : g.rows_per_tile);
    for (int64_t p = threadIdx.x; p < (int64_t)rows_here * nb; p += kThreads) {
      const int64_t row = row0 + p / nb, b = p % nb;
      const int64_t bi = row * nb + b;
      float acc[BATCH];
#pragma unroll
      for (int bb = 0; bb < BATCH; ++bb) acc[bb] = 0.f;
      const uint32_t kb = v.keptb[bi];
      BitReader fr, er;
      fr.init(v.fields, ((uint64_t)row * sh.keep + kb) * (uint64_t)(1 + m));
      er.init(v.codes, c1_code_start(v, row, bi, nb));
      const uint32_t* bmp = v.bitmap + bi * (B / 32);
      const uint16_t* xb = xs + b * B;
      for (int64_t wi = 0; wi < B / 32; ++wi) {
        uint32_t bw = __builtin_nontemporal_load(bmp + wi);
        while (bw) {
          const int pbit = __builtin_ctz(bw);
          bw &= bw - 1u;
          const uint32_t f = fr.take(1 + m);
          const int r = er.unary();
          const uint32_t bits = ((f >> m) << 31) | ebits[r] | ((f & mmask) << fshift);
          const float wv = __uint_as_float(bits);
          const int col = (int)(wi * 32 + pbit);
#pragma unroll
          for (int bb = 0; bb < BATCH; ++bb)
            acc[bb] = __builtin_fmaf(wv, bf16_bits_to_float(xb[bb * C + col]), acc[bb]);
        }
      }
#pragma unroll
      for (int bb = 0; bb < BATCH; ++bb) part[p * BATCH + bb] = acc[bb];
    }
    __syncthreads();
    reduce_tile<BATCH>(part, rows_here, nb, row0, y, ldy);
    __syncthreads();
  }
}

template <int BATCH>
__global__ void __launch_bounds__(kThreads) k_draft_gemv_c2(SpecViewC2 v, Shape sh, GemvGeom g,
                                                            const uint16_t* __restrict__ x,
                                                            int64_t ldx, float* __restrict__ y,
                                                            int64_t ldy) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int64_t C = sh.cols, B = sh.block, nb = C / B;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* part = reinterpret_cast<float*>(smem + g.x_lds_elems * 2 + 1024);

  stage_x<BATCH>(x, ldx, C, xs);
  __syncthreads();

  const int m = sh.mant;
  const uint32_t amask = (2u << m) - 1u;
  for (int64_t tile = blockIdx.x; tile < g.ntiles; tile += gridDim.x) {
    const int64_t row0 = tile * g.rows_per_tile;
    const int rows_here = (int)((sh.rows - row0 < g.rows_per_tile) ? sh.rows - row0 : g.rows_per_tile);
    for (int64_t p = threadIdx.x; p < (int64_t)rows_here * nb; p += kThreads) {
      const int64_t row = row0 + p / nb, b = p % nb;
      const int64_t bi = row * nb + b;
      float acc[BATCH];
#pragma unroll
      for (int bb = 0; bb < BATCH; ++bb) acc[bb] = 0.f;
      const uint32_t kb = v.keptb[bi];
      BitReader fr;
      fr.init(v.fields, ((uint64_t)row * sh.keep + kb) * (uint64_t)(2 + m));
      const uint32_t* bmp = v.bitmap + bi * (B / 32);
      const uint8_t* se = v.shexp + bi * (B / 32);
      const uint16_t* xb = xs + b * B;
      for (int64_t wi = 0; wi < B / 32; ++wi) {
        uint32_t bw = __builtin_nontemporal_load(bmp + wi);
        if (!bw) continue;
        // 2^(E-127-m) as an fp32 (normal for E-m >= 1, subnormal below)
        const int em = (int)se[wi] - m;
        const float scale = __uint_as_float(em >= 1 ? ((uint32_t)em << 23) : (1u << (em + 22)));
        while (bw) {
          const int pbit = __builtin_ctz(bw);
          bw &= bw - 1u;
          const uint32_t f = fr.take(2 + m);
          const float mag = (float)(f & amask) * scale;
          const float wv = __uint_as_float(__float_as_uint(mag) | ((f >> (m + 1)) << 31));
          const int col = (int)(wi * 32 + pbit);
#pragma unroll
          for (int bb = 0; bb < BATCH; ++bb)
            acc[bb] = __builtin_fmaf(wv, bf16_bits_to_float(xb[bb * C + col]), acc[bb]);
        }
      }
#pragma unroll
      for (int bb = 0; bb < BATCH; ++bb) part[p * BATCH + bb] = acc[bb];
    }
    __syncthreads();
    reduce_tile<BATCH>(part, rows_here, nb, row0, y, ldy);
    __syncthreads();
  }
}

int64_t lds_bytes(const GemvGeom& g, const Shape& sh, int batch) {
  return g.x_lds_elems * 2 + 1024 + (int64_t)g.rows_per_tile * (sh.cols / sh.block) * batch * 4;
}

GemvGeom make_geom(const Shape& sh, int batch) {
  GemvGeom g;
  const int64_t nb = sh.cols / sh.block;
  g.rows_per_tile = (int)(nb >= kThreads ? 1 : kThreads / nb);
  g.ntiles = (sh.rows + g.rows_per_tile - 1) / g.rows_per_tile;
  g.x_lds_elems = (batch * sh.cols + 7) / 8 * 8;
  return g;
}

template <typename Kern, typename View>
hipError_t launch_gemv(Kern kern, const View& v, const Shape& sh, const GemvGeom& g, int batch,
                       const uint16_t* x, int64_t ldx, float* y, int64_t ldy, hipStream_t s) {
  const int64_t lds = lds_bytes(g, sh, batch);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  int64_t grid = g.ntiles;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  if (grid > cap) grid = cap;
  kern<<<(unsigned)grid, kThreads, (size_t)lds, s>>>(v, sh, g, x, ldx, y, ldy);
  return hipGetLastError();
}

}  // namespace

int64_t draft_gemv_direct_lds_bytes(const Shape& sh, int batch) {
  return lds_bytes(make_geom(sh, batch), sh, batch);
}

hipError_t launch_draft_gemv_c1_direct(const SpecViewC1& v, const Shape& sh, const uint16_t* x,
                                       int batch, int64_t ldx, float* y, int64_t ldy,
                                       hipStream_t s) {
  if (sh.rows == 0) return hipSuccess;
  const GemvGeom g = make_geom(sh, batch);
  switch (batch) {
    case 1: return launch_gemv(k_draft_gemv_c1<1>, v, sh, g, batch, x, ldx, y, ldy, s);
    case 2: return launch_gemv(k_draft_gemv_c1<2>, v, sh, g, batch, x, ldx, y, ldy, s);
    case 3: return launch_gemv(k_draft_gemv_c1<3>, v, sh, g, batch, x, ldx, y, ldy, s);
    case 4: return launch_gemv(k_draft_gemv_c1<4>, v, sh, g, batch, x, ldx, y, ldy, s);
    case 5: return launch_gemv(k_draft_gemv_c1<5>, v, sh, g, batch, x, ldx, y, ldy, s);
    case 6: return launch_gemv(k_draft_gemv_c1<6>, v, sh, g, batch, x, ldx, y, ldy, s);
    case 7: return launch_gemv(k_draft_gemv_c1<7>, v, sh, g, batch, x, ldx, y, ldy, s);
    case 8: return launch_gemv(k_draft_gemv_c1<8>, v, sh, g, batch, x, ldx, y, ldy, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_draft_gemv_c2_direct(const SpecViewC2& v, const Shape& sh, const uint16_t* x,
                                       int batch, int64_t ldx, float* y, int64_t ldy,
                                       hipStream_t s) {
  if (sh.rows == 0) return hipSuccess;
  const GemvGeom g = make_geom(sh, batch);
  switch (batch) {
    case 1: return launch_gemv(k_draft_gemv_c2<1>, v, sh, g, batch, x, ldx, y, ldy, s);
    case 2: return launch_gemv(k_draft_gemv_c2<2>, v, sh, g, batch, x, ldx, y, ldy, s);
    case 3: return launch_gemv(k_draft_gemv_c2<3>, v, sh, g, batch, x, ldx, y, ldy, s);
    case 4: return launch_gemv(k_draft_gemv_c2<4>, v, sh, g, batch, x, ldx, y, ldy, s);
    case 5: return launch_gemv(k_draft_gemv_c2<5>, v, sh, g, batch, x, ldx, y, ldy, s);
    case 6: return launch_gemv(k_draft_gemv_c2<6>, v, sh, g, batch, x, ldx, y, ldy, s);
    case 7: return launch_gemv(k_draft_gemv_c2<7>, v, sh, g, batch, x, ldx, y, ldy, s);
    case 8: return launch_gemv(k_draft_gemv_c2<8>, v, sh, g, batch, x, ldx, y, ldy, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace cass
