// Device-side bit-stream helpers: little-endian bit order (bit i of a section
// is bit (i & 31) of 32-bit word i >> 5).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cass {

// Sequential reader of a bit section.  Keeps between 33 and 64 valid bits in
// a 64-bit buffer (any take() of up to 32 bits is a shift and a mask) plus the
// next 32-bit word already requested: a refill uses that word and issues the
// load of the one after, so the memory latency overlaps the decoding of the
// 32 bits in between.  It may fetch up to three words past the last bit it
// returns; every section is followed by >= 16 bytes of padding, so those
// reads stay inside the stream.
struct BitReader {
  const uint32_t* p;  // next word to request
  uint64_t buf;
  int n;              // valid bits in buf
  uint32_t nxt;       // word p[-1], requested ahead

  __device__ __forceinline__ void init(const uint32_t* base, uint64_t pos) {
    p = base + (pos >> 5);
    const int s = (int)(pos & 31);
    const uint32_t w0 = __builtin_nontemporal_load(p);
    const uint32_t w1 = __builtin_nontemporal_load(p + 1);
    nxt = __builtin_nontemporal_load(p + 2);
    p += 3;
    buf = (uint64_t)(w0 >> s) | ((uint64_t)w1 << (32 - s));
    n = 64 - s;
  }
  __device__ __forceinline__ void refill() {
    if (n <= 32) {
      buf |= (uint64_t)nxt << n;
      n += 32;
      nxt = __builtin_nontemporal_load(p);
      ++p;
    }
  }
  // width in 0..32
  __device__ __forceinline__ uint32_t take(int width) {
    const uint32_t v = (uint32_t)(buf & ((width >= 32) ? 0xFFFFFFFFull : ((1ull << width) - 1)));
    buf >>= width;
    n -= width;
    refill();
    return v;
  }
  // One unary code: the number of zero bits before the next one bit.  Codes
  // are at most 256 bits long; the loop is bounded by that.
  __device__ __forceinline__ int unary() {
    int r = 0;
    for (int it = 0; it < 8; ++it) {
      const uint32_t lo = (uint32_t)buf;
      if (lo != 0u) {
        const int t = __builtin_ctz(lo);
        buf >>= (t + 1);
        n -= t + 1;
        refill();
        return r + t;
      }
      r += 32;
      buf >>= 32;
      n -= 32;
      refill();
    }
    return 255;
  }
};

// Bounded variant of unary() for validation-style decoders: gives -1 after
// `limit` zero bits without a one.
__device__ __forceinline__ int unary_bounded(BitReader& br, int limit) {
  int r = 0;
  while (r <= limit) {
    const uint32_t lo = (uint32_t)br.buf;
    if (lo != 0u) {
      const int t = __builtin_ctz(lo);
      br.buf >>= (t + 1);
      br.n -= t + 1;
      br.refill();
      return (r + t <= limit) ? r + t : -1;
    }
    r += 32;
    br.buf >>= 32;
    br.n -= 32;
    br.refill();
  }
  return -1;
}

// Sequential writer into a zero-filled bit section shared with other threads:
// complete 32-bit words are merged with atomicOr (order independent, so the
// result does not depend on thread scheduling).
struct BitWriter {
  uint32_t* base;
  uint64_t word;  // index of the word being filled
  uint64_t acc;
  int nacc;       // bits of acc in use, including the offset inside the first word

  __device__ __forceinline__ void init(uint32_t* b, uint64_t pos) {
    base = b;
    word = pos >> 5;
    acc = 0;
    nacc = (int)(pos & 31);
  }
  __device__ __forceinline__ void flush_full() {
    while (nacc >= 32) {
      const uint32_t v = (uint32_t)acc;
      if (v) atomicOr(base + word, v);
      ++word;
      acc >>= 32;
      nacc -= 32;
    }
  }
  // width in 0..32
  __device__ __forceinline__ void put(uint32_t v, int width) {
    acc |= (uint64_t)v << nacc;
    nacc += width;
    flush_full();
  }
  __device__ __forceinline__ void put_unary(int r) {
    while (r >= 32) {
      nacc += 32;
      flush_full();
      r -= 32;
    }
    put(1u << r, r + 1);
  }
  __device__ __forceinline__ void finish() {
    if (nacc > 0) {
      const uint32_t v = (uint32_t)acc;
      if (v) atomicOr(base + word, v);
    }
  }
};

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) {
  return __uint_as_float(b << 16);
}

}  // namespace cass
