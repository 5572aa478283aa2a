// Whole-tensor decoders: exact reconstruction (both streams), the zero-filled
// draft (speculation stream only), and the MX-quantised target of format 3.
//
// Method: Cassandra review (marsggbo.github.io), section 3.1 -- the draft
// loads only speculation data and zero-fills it back to standard floating
// point; the target loads both streams and reassembles the original
// losslessly.
#include "decoders.hpp"

namespace cass {

namespace {

// The rank tables (rank -> exponent) of both streams, copied to shared memory
// once per workgroup.
__device__ __forceinline__ void load_tables(uint8_t* ps, uint8_t* pv, const uint8_t* gs,
                                            const uint8_t* gv) {
  for (int i = threadIdx.x; i < 256; i += blockDim.x) {
    ps[i] = gs ? gs[i] : 0;
    pv[i] = gv ? gv[i] : 0;
  }
  __syncthreads();
}

// Decode one block into out[pos0 .. pos0+B), one bitmap word (32 positions)
// at a time: the word's kept positions, then its pruned positions, into this
// thread's 64-byte slot of shared memory, then four 16-byte stores.
template <typename Dec>
__device__ __forceinline__ void decode_block_to(Dec& d, const uint32_t* __restrict__ bitmap,
                                                int64_t pos0, int64_t B, uint16_t* slot,
                                                uint16_t* __restrict__ out) {
  for (int64_t wi = 0; wi < B / 32; ++wi) {
    const uint32_t bw = bitmap[pos0 / 32 + wi];
    for (uint32_t km = bw; km; km &= km - 1u) slot[__builtin_ctz(km)] = (uint16_t)d.kept((int)wi);
    for (uint32_t pm = ~bw; pm; pm &= pm - 1u) slot[__builtin_ctz(pm)] = (uint16_t)d.pruned((int)wi);
    const uint4* sl = reinterpret_cast<const uint4*>(slot);
    uint4* o = reinterpret_cast<uint4*>(out + pos0 + wi * 32);
    o[0] = sl[0];
    o[1] = sl[1];
    o[2] = sl[2];
    o[3] = sl[3];
  }
}

__global__ void __launch_bounds__(256) k_exact_c1(SpecViewC1 sv, VerifViewC1 vv, Shape sh,
                                                  uint16_t* __restrict__ out) {
  __shared__ uint8_t ps[256], pv[256];
  __shared__ __align__(16) uint16_t slots[256 * 32];
  load_tables(ps, pv, sv.perm, vv.perm);
  const int64_t nb = sh.cols / sh.block, nblk = sh.rows * nb;
  for (int64_t bi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; bi < nblk;
       bi += (int64_t)gridDim.x * blockDim.x) {
    ExactC1 d;
    d.init(sv, vv, sh, bi / nb, bi % nb, ps, pv);
    decode_block_to(d, sv.bitmap, bi * sh.block, sh.block, slots + threadIdx.x * 32, out);
  }
}

__global__ void __launch_bounds__(256) k_draft_c1(SpecViewC1 sv, Shape sh,
                                                  uint16_t* __restrict__ out) {
  __shared__ uint8_t ps[256], pv[256];
  __shared__ __align__(16) uint16_t slots[256 * 32];
  load_tables(ps, pv, sv.perm, nullptr);
  const int64_t nb = sh.cols / sh.block, nblk = sh.rows * nb;
  for (int64_t bi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; bi < nblk;
       bi += (int64_t)gridDim.x * blockDim.x) {
    DraftC1 d;
    d.init(sv, sh, bi / nb, bi % nb, ps);
    decode_block_to(d, sv.bitmap, bi * sh.block, sh.block, slots + threadIdx.x * 32, out);
  }
}

__global__ void __launch_bounds__(256) k_exact_c2(SpecViewC2 sv, VerifViewC2 vv, Shape sh,
                                                  uint16_t* __restrict__ out) {
  __shared__ uint8_t ps[256], pv[256];
  __shared__ __align__(16) uint16_t slots[256 * 32];
  load_tables(ps, pv, nullptr, vv.perm);
  const int64_t nb = sh.cols / sh.block, nblk = sh.rows * nb;
  for (int64_t bi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; bi < nblk;
       bi += (int64_t)gridDim.x * blockDim.x) {
    ExactC2 d;
    d.init(sv, vv, sh, bi / nb, bi % nb, ps, pv);
    decode_block_to(d, sv.bitmap, bi * sh.block, sh.block, slots + threadIdx.x * 32, out);
  }
}

__global__ void __launch_bounds__(256) k_draft_c2(SpecViewC2 sv, Shape sh,
                                                  uint16_t* __restrict__ out) {
  __shared__ __align__(16) uint16_t slots[256 * 32];
  const int64_t nb = sh.cols / sh.block, nblk = sh.rows * nb;
  for (int64_t bi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; bi < nblk;
       bi += (int64_t)gridDim.x * blockDim.x) {
    DraftC2 d;
    d.init(sv, sh, bi / nb, bi % nb);
    decode_block_to(d, sv.bitmap, bi * sh.block, sh.block, slots + threadIdx.x * 32, out);
  }
}

__global__ void __launch_bounds__(256) k_target_c3(SpecViewC2 sv, VerifViewC3 vv, Shape sh,
                                                   uint16_t* __restrict__ out) {
  __shared__ __align__(16) uint16_t slots[256 * 32];
  const int64_t nb = sh.cols / sh.block, nblk = sh.rows * nb;
  for (int64_t bi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; bi < nblk;
       bi += (int64_t)gridDim.x * blockDim.x) {
    TargetC3 d;
    d.init(sv, vv, sh, bi / nb, bi % nb, nullptr, nullptr);
    decode_block_to(d, sv.bitmap, bi * sh.block, sh.block, slots + threadIdx.x * 32, out);
  }
}

unsigned grid_blocks(int64_t nblk) {
  int64_t g = (nblk + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  if (g > cap) g = cap;
  return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_decode_c1(const SpecViewC1& sv, const VerifViewC1* vv, const Shape& sh,
                            uint16_t* out, hipStream_t s) {
  const int64_t nblk = sh.rows * (sh.cols / sh.block);
  if (nblk == 0) return hipSuccess;
  if (vv) k_exact_c1<<<grid_blocks(nblk), 256, 0, s>>>(sv, *vv, sh, out);
  else k_draft_c1<<<grid_blocks(nblk), 256, 0, s>>>(sv, sh, out);
  return hipGetLastError();
}

hipError_t launch_decode_c2(const SpecViewC2& sv, const VerifViewC2* vv, const Shape& sh,
                            uint16_t* out, hipStream_t s) {
  const int64_t nblk = sh.rows * (sh.cols / sh.block);
  if (nblk == 0) return hipSuccess;
  if (vv) k_exact_c2<<<grid_blocks(nblk), 256, 0, s>>>(sv, *vv, sh, out);
  else k_draft_c2<<<grid_blocks(nblk), 256, 0, s>>>(sv, sh, out);
  return hipGetLastError();
}

hipError_t launch_decode_c3(const SpecViewC2& sv, const VerifViewC3& vv, const Shape& sh,
                            uint16_t* out, hipStream_t s) {
  const int64_t nblk = sh.rows * (sh.cols / sh.block);
  if (nblk == 0) return hipSuccess;
  k_target_c3<<<grid_blocks(nblk), 256, 0, s>>>(sv, vv, sh, out);
  return hipGetLastError();
}

}  // namespace cass
