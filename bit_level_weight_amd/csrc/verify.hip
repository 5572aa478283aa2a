// Verification GEMM for the k+1 drafted tokens: Y[t][n] = sum_j W[n][j] X[t][j]
// with W rebuilt exactly from both streams inside the kernel (format 3: the
// MX-quantised target rebuilt from them).
//
// Method: Cassandra review (marsggbo.github.io), section 1 -- the target
// model checks the drafted tokens in one parallel pass; section 3.1 -- it
// loads both streams and reassembles the original weights losslessly.
//
// Work split: one wave per (64 rows, range of blocks).  Each lane decodes one
// row, 32 positions at a time, into an LDS tile of 64 x 32 bf16; the wave then
// multiplies the tile with the matching 32 columns of X on the matrix cores
// (v_mfma_f32_16x16x32_bf16, tokens padded to 16).  Partial sums over block
// ranges are combined with fp32 atomics on Y, which the launcher zeroes first.
#include "decoders.hpp"

namespace cass {

namespace {

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ const uint8_t* spec_perm_of(const SpecViewC1& s) { return s.perm; }
__device__ __forceinline__ const uint8_t* spec_perm_of(const SpecViewC2&) { return nullptr; }
__device__ __forceinline__ const uint8_t* verif_perm_of(const VerifViewC1& v) { return v.perm; }
__device__ __forceinline__ const uint8_t* verif_perm_of(const VerifViewC2& v) { return v.perm; }
__device__ __forceinline__ const uint8_t* verif_perm_of(const VerifViewC3&) { return nullptr; }

constexpr int kTileStride = 17;  // u32 per LDS tile row (16 used + 1 pad against bank conflicts)

__global__ void __launch_bounds__(256) k_zero_rows(float* Y, int ntok, int64_t rows, int64_t ldy) {
  const int64_t n = (int64_t)ntok * rows;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    Y[(i / rows) * ldy + (i % rows)] = 0.f;
}

template <typename Dec, typename SV, typename VV>
__global__ void __launch_bounds__(64) k_verify(SV sv, VV vv, Shape sh,
                                               const uint16_t* __restrict__ X, int ntok,
                                               int64_t ldx, float* __restrict__ Y, int64_t ldy,
                                               int64_t blocks_per_split) {
  __shared__ uint32_t tile[64 * kTileStride];
  __shared__ uint8_t ps[256], pv[256];
  const int lane = threadIdx.x;
  const uint8_t* gps = spec_perm_of(sv);
  const uint8_t* gpv = verif_perm_of(vv);
  for (int i = lane; i < 256; i += 64) {  // rank tables to shared memory
    ps[i] = gps ? gps[i] : 0;
    pv[i] = gpv ? gpv[i] : 0;
  }
  __syncthreads();
  const int64_t nb = sh.cols / sh.block;
  const int64_t row0 = (int64_t)blockIdx.x * 64;
  const int64_t row = row0 + lane;
  const bool row_ok = row < sh.rows;
  const int64_t b0 = (int64_t)blockIdx.y * blocks_per_split;
  const int64_t b1 = (b0 + blocks_per_split < nb) ? b0 + blocks_per_split : nb;
  const int n = lane & 15;  // token column of the B operand / D
  const int kq = lane >> 4; // which 4-wide k slice this lane feeds
  v4f acc[4];
#pragma unroll
  for (int rg = 0; rg < 4; ++rg) acc[rg] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int64_t b = b0; b < b1; ++b) {
    Dec d;
    if (row_ok) d.init(sv, vv, sh, row, b, ps, pv);
    for (int64_t wi = 0; wi < sh.block / 32; ++wi) {
      if (row_ok) {
        const uint32_t bw = sv.bitmap[(row * nb + b) * (sh.block / 32) + wi];
        // the word's kept positions, then its pruned ones (two loops, no
        // per-position branch), straight into this lane's tile row
        uint16_t* trow = reinterpret_cast<uint16_t*>(tile + lane * kTileStride);
        for (uint32_t km = bw; km; km &= km - 1u) trow[__builtin_ctz(km)] = (uint16_t)d.kept((int)wi);
        for (uint32_t pm = ~bw; pm; pm &= pm - 1u) trow[__builtin_ctz(pm)] = (uint16_t)d.pruned((int)wi);
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) tile[lane * kTileStride + j] = 0u;
      }
      __syncthreads();
      const int64_t col0 = b * sh.block + wi * 32;
      // v_mfma_f32_16x16x32_bf16: lane (n, kq) feeds tile row n of each 16-row
      // group and token n, columns 8kq..8kq+7 of the word's 32
      {
        v8s bop = v8s{0, 0, 0, 0, 0, 0, 0, 0};
        if (n < ntok) {
          const uint16_t* xp = X + (int64_t)n * ldx + col0 + 8 * kq;
          bop = v8s{(short)xp[0], (short)xp[1], (short)xp[2], (short)xp[3],
                    (short)xp[4], (short)xp[5], (short)xp[6], (short)xp[7]};
        }
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const uint32_t* tp = tile + (rg * 16 + n) * kTileStride + 4 * kq;
          const uint32_t a0 = tp[0], a1 = tp[1], a2 = tp[2], a3 = tp[3];
          const v8s aop = v8s{(short)(a0 & 0xFFFF), (short)(a0 >> 16), (short)(a1 & 0xFFFF),
                              (short)(a1 >> 16), (short)(a2 & 0xFFFF), (short)(a2 >> 16),
                              (short)(a3 & 0xFFFF), (short)(a3 >> 16)};
          acc[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, aop),
                                                            __builtin_bit_cast(v8bf, bop), acc[rg],
                                                            0, 0, 0);
        }
      }
      __syncthreads();
    }
  }
  // D[i][j]: lane holds rows 4*kq + e of each 16-row group, token n
  if (n < ntok) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t r = row0 + rg * 16 + 4 * kq + e;
        if (r < sh.rows) atomicAdd(Y + (int64_t)n * ldy + r, acc[rg][e]);
      }
    }
  }
}

template <typename Dec, typename SV, typename VV>
hipError_t launch_verify(const SV& sv, const VV& vv, const Shape& sh, const uint16_t* X, int ntok,
                         int64_t ldx, float* Y, int64_t ldy, hipStream_t s) {
  if (sh.rows == 0 || ntok == 0) return hipSuccess;
  {
    int64_t g = ((int64_t)ntok * sh.rows + 255) / 256;
    if (g > 4096) g = 4096;
    k_zero_rows<<<(unsigned)g, 256, 0, s>>>(Y, ntok, sh.rows, ldy);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t nb = sh.cols / sh.block;
  const int64_t gx = (sh.rows + 63) / 64;
  const int64_t want_waves = (int64_t)device_cu_count() * 32;
  int64_t nsplit = (want_waves + gx - 1) / gx;
  if (nsplit > nb) nsplit = nb;
  if (nsplit < 1) nsplit = 1;
  const int64_t bps = (nb + nsplit - 1) / nsplit;
  nsplit = (nb + bps - 1) / bps;
  k_verify<Dec, SV, VV><<<dim3((unsigned)gx, (unsigned)nsplit), 64, 0, s>>>(sv, vv, sh, X, ntok,
                                                                           ldx, Y, ldy, bps);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_verify_gemm_c1(const SpecViewC1& sv, const VerifViewC1& vv, const Shape& sh,
                                 const uint16_t* X, int ntok, int64_t ldx, float* Y, int64_t ldy,
                                 hipStream_t s) {
  return launch_verify<ExactC1>(sv, vv, sh, X, ntok, ldx, Y, ldy, s);
}

hipError_t launch_verify_gemm_c2(const SpecViewC2& sv, const VerifViewC2& vv, const Shape& sh,
                                 const uint16_t* X, int ntok, int64_t ldx, float* Y, int64_t ldy,
                                 hipStream_t s) {
  return launch_verify<ExactC2>(sv, vv, sh, X, ntok, ldx, Y, ldy, s);
}

hipError_t launch_verify_gemm_c3(const SpecViewC2& sv, const VerifViewC3& vv, const Shape& sh,
                                 const uint16_t* X, int ntok, int64_t ldx, float* Y, int64_t ldy,
                                 hipStream_t s) {
  return launch_verify<TargetC3>(sv, vv, sh, X, ntok, ldx, Y, ldy, s);
}

}  // namespace cass
