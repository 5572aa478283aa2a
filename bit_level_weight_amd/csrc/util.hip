// Measurement utility: a plain streaming read of a device buffer, the
// achievable-read ceiling that the compressed-stream kernels are compared to.
// Every 16-byte chunk is loaded once (non-temporal, four loads in flight per
// thread) and folded into an XOR so the loads cannot be dropped; one word per
// workgroup is written.
#include "internal.hpp"

namespace cass {

namespace {

constexpr int kReadThreads = 256;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kReadThreads) k_stream_read(const u32x4* __restrict__ p,
                                                              int64_t n16,
                                                              uint32_t* __restrict__ out) {
  __shared__ uint32_t part[kReadThreads / 64];
  const int64_t stride = (int64_t)gridDim.x * kReadThreads;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    const u32x4 b = __builtin_nontemporal_load(p + i + stride);
    const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
    const u32x4 e = a ^ b ^ c ^ d;
    acc ^= e.x ^ e.y ^ e.z ^ e.w;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t v = 0;
    for (int w = 0; w < kReadThreads / 64; ++w) v ^= part[w];
    out[blockIdx.x] = v;
  }
}

}  // namespace

}  // namespace cass

using namespace cass;

extern "C" int cass_stream_read(const void* buf, int64_t bytes, uint32_t* out, hipStream_t stream) {
  if (!buf || !out || bytes < 0 || (bytes % 16) || ((uintptr_t)buf % 16))
    return report(CASS_ERR_INVALID,
                  "stream read needs a 16-byte aligned buffer of whole 16-byte chunks");
  clear_error();
  if (bytes == 0) return CASS_OK;
  k_stream_read<<<CASS_STREAM_READ_BLOCKS, kReadThreads, 0, stream>>>((const u32x4*)buf,
                                                                     bytes / 16, out);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? CASS_OK
                         : report(CASS_ERR_HIP, "stream read launch: %s", hipGetErrorString(e));
}
