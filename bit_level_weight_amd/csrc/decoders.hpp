// Per-lane block decoders shared by the reconstruction, draft-decode and
// verification kernels.  A decoder walks one block of `block` positions of
// one row: kept() gives the block's kept values in position order, pruned()
// its pruned values, so a caller takes each bitmap word's kept positions and
// then its pruned positions in two loops (no per-position branch).  Every stream, the
// pruned bytes included, is read through a buffered BitReader; the rank
// tables (rank -> exponent) are passed in from shared memory, so a value
// costs no scattered global loads.
//
// Method: Cassandra review (marsggbo.github.io), section 3.1 -- the draft
// zero-fills the speculation data back to bf16; the target reassembles both
// streams losslessly.  Section 3.2 -- unary exponent codes are decoded by
// counting zeros up to the one; Cassandra-2 values share one exponent per 32
// positions (OCP MX specification).
#pragma once

#include "bits.hpp"
#include "internal.hpp"

namespace cass {

// Cassandra-1, both streams -> exact original bf16 patterns.
struct ExactC1 {
  BitReader fr, er, lr, vr, pr;
  const uint8_t* perm_s;  // shared memory
  const uint8_t* perm_v;  // shared memory
  int m;

  __device__ __forceinline__ void init(const SpecViewC1& sv, const VerifViewC1& vv,
                                       const Shape& sh, int64_t row, int64_t b,
                                       const uint8_t* ps, const uint8_t* pv) {
    const int64_t nb = sh.cols / sh.block;
    const int64_t bi = row * nb + b;
    m = sh.mant;
    const uint32_t kb = sv.keptb[bi];
    const uint64_t kin0 = (uint64_t)row * sh.keep + kb;
    fr.init(sv.fields, kin0 * (uint64_t)(1 + m));
    er.init(sv.codes, c1_code_start(sv, row, bi, nb));
    lr.init(vv.lowmant, kin0 * (uint64_t)(7 - m));
    vr.init(vv.codes, vv.rowbase[row] + vv.blkoff[bi]);
    const uint64_t pidx = (uint64_t)row * (sh.cols - sh.keep) + (uint64_t)(b * sh.block) - kb;
    pr.init(reinterpret_cast<const uint32_t*>(vv.pruned), pidx * 8u);
    perm_s = ps;
    perm_v = pv;
  }
  // the next kept value of the block (kept values come in position order)
  __device__ __forceinline__ uint32_t kept(int /*word*/) {
    const uint32_t f = fr.take(1 + m);
    const int r = er.unary();
    const uint32_t low = lr.take(7 - m);
    const uint32_t e = perm_s[r];
    return ((f >> m) << 15) | (e << 7) | ((f & ((1u << m) - 1)) << (7 - m)) | low;
  }
  // the next pruned value of the block (word: its bitmap word in the block)
  __device__ __forceinline__ uint32_t pruned(int /*word*/) {
    const uint32_t byte = pr.take(8);
    const uint32_t e = perm_v[vr.unary()];
    return ((byte >> 7) << 15) | (e << 7) | (byte & 0x7F);
  }
  static constexpr bool kHasPruned = true;
};

// Cassandra-1 speculation stream -> zero-filled draft.
struct DraftC1 {
  BitReader fr, er;
  const uint8_t* perm_s;
  int m;
  __device__ __forceinline__ void init(const SpecViewC1& sv, const Shape& sh, int64_t row,
                                       int64_t b, const uint8_t* ps) {
    const int64_t nb = sh.cols / sh.block;
    const int64_t bi = row * nb + b;
    m = sh.mant;
    const uint32_t kb = sv.keptb[bi];
    fr.init(sv.fields, ((uint64_t)row * sh.keep + kb) * (uint64_t)(1 + m));
    er.init(sv.codes, c1_code_start(sv, row, bi, nb));
    perm_s = ps;
  }
  __device__ __forceinline__ uint32_t kept(int /*word*/) {
    const uint32_t f = fr.take(1 + m);
    const uint32_t e = perm_s[er.unary()];
    return ((f >> m) << 15) | (e << 7) | ((f & ((1u << m) - 1)) << (7 - m));
  }
  __device__ __forceinline__ uint32_t pruned(int /*word*/) { return 0u; }  // zero-filled
  static constexpr bool kHasPruned = false;
};

// bf16 pattern of sign * a * 2^(E-127-m): normalise the (m+1)-bit significand.
__device__ __forceinline__ uint32_t mx_value_bits(uint32_t s, uint32_t a, int E, int m) {
  if (a == 0) return 0u;
  const int p = 31 - __builtin_clz(a);
  const int e = E - m + p;
  if (e >= 1) return (s << 15) | ((uint32_t)e << 7) | ((a << (7 - p)) & 0x7F);
  return (s << 15) | (a << (E - m + 6));
}

// Cassandra-2 speculation stream -> zero-filled (MX-truncated) draft.
struct DraftC2 {
  BitReader fr;
  const uint8_t* shexp;
  int64_t g0;
  int m, cur_word, E;
  __device__ __forceinline__ void init(const SpecViewC2& sv, const Shape& sh, int64_t row,
                                       int64_t b) {
    const int64_t nb = sh.cols / sh.block;
    const int64_t bi = row * nb + b;
    m = sh.mant;
    const uint32_t kb = sv.keptb[bi];
    fr.init(sv.fields, ((uint64_t)row * sh.keep + kb) * (uint64_t)(2 + m));
    shexp = sv.shexp;
    g0 = bi * sh.block / 32;
    cur_word = -1;
    E = 0;
  }
  __device__ __forceinline__ uint32_t kept(int word) {
    if (word != cur_word) {  // one shared exponent per 32 positions
      E = shexp[g0 + word];
      cur_word = word;
    }
    const uint32_t f = fr.take(2 + m);
    return mx_value_bits(f >> (m + 1), f & ((2u << m) - 1), E, m);
  }
  __device__ __forceinline__ uint32_t pruned(int /*word*/) { return 0u; }  // zero-filled
  static constexpr bool kHasPruned = false;
};

// Cassandra-2, both streams -> exact original bf16 patterns.
struct ExactC2 {
  BitReader fr, kr, vr, pr;
  const uint8_t* shexp;
  const uint8_t* perm_v;  // shared memory
  int64_t g0;
  int m, cur_word, E;
  __device__ __forceinline__ void init(const SpecViewC2& sv, const VerifViewC2& vv,
                                       const Shape& sh, int64_t row, int64_t b,
                                       const uint8_t* /*ps*/, const uint8_t* pv) {
    const int64_t nb = sh.cols / sh.block;
    const int64_t bi = row * nb + b;
    m = sh.mant;
    const uint32_t kb = sv.keptb[bi];
    fr.init(sv.fields, ((uint64_t)row * sh.keep + kb) * (uint64_t)(2 + m));
    kr.init(vv.resid, vv.rowbase_k[row] + vv.blkoff_k[bi]);
    vr.init(vv.codes, vv.rowbase_p[row] + vv.blkoff_p[bi]);
    const uint64_t pidx = (uint64_t)row * (sh.cols - sh.keep) + (uint64_t)(b * sh.block) - kb;
    pr.init(reinterpret_cast<const uint32_t*>(vv.pruned), pidx * 8u);
    shexp = sv.shexp;
    perm_v = pv;
    g0 = bi * sh.block / 32;
    cur_word = -1;
    E = 0;
  }
  __device__ __forceinline__ uint32_t kept(int word) {
    if (word != cur_word) {  // one shared exponent per 32 positions
      E = shexp[g0 + word];
      cur_word = word;
    }
    const uint32_t f = fr.take(2 + m);
    const uint32_t s = f >> (m + 1), a = f & ((2u << m) - 1);
    const int d = kr.unary();
    const int wd = (7 - m + d < 8) ? 7 - m + d : 8;
    const uint32_t L = kr.take(wd);
    const uint32_t M = (wd < 8) ? ((a << wd) | L) : L;
    const uint32_t e = (M >= 128u) ? (uint32_t)(E - d) : 0u;
    return (s << 15) | ((e & 0xFF) << 7) | (M & 0x7F);
  }
  __device__ __forceinline__ uint32_t pruned(int /*word*/) {
    const uint32_t byte = pr.take(8);
    const uint32_t e = perm_v[vr.unary()];
    return ((byte >> 7) << 15) | (e << 7) | (byte & 0x7F);
  }
  static constexpr bool kHasPruned = true;
};

// Format 3: Cassandra-2 speculation stream plus the fixed-width verification
// sections -> the MX-quantised target (sign * t * 2^(X-134) per value, X the
// group exponent of its 32 positions).
struct TargetC3 {
  BitReader fr, lr, pr;
  const uint8_t* gexp;
  int64_t g0;
  int m, cur_word, X;
  __device__ __forceinline__ void init(const SpecViewC2& sv, const VerifViewC3& vv,
                                       const Shape& sh, int64_t row, int64_t b,
                                       const uint8_t* /*ps*/, const uint8_t* /*pv*/) {
    const int64_t nb = sh.cols / sh.block;
    const int64_t bi = row * nb + b;
    m = sh.mant;
    const uint32_t kb = sv.keptb[bi];
    const uint64_t kin0 = (uint64_t)row * sh.keep + kb;
    fr.init(sv.fields, kin0 * (uint64_t)(2 + m));
    lr.init(vv.low, kin0 * (uint64_t)(7 - m));
    const uint64_t pidx = (uint64_t)row * (sh.cols - sh.keep) + (uint64_t)(b * sh.block) - kb;
    pr.init(vv.pruned, pidx * 9u);
    gexp = vv.gexp;
    g0 = bi * sh.block / 32;
    cur_word = -1;
    X = 0;
  }
  __device__ __forceinline__ void group(int word) {
    if (word != cur_word) {
      X = gexp[g0 + word];
      cur_word = word;
    }
  }
  __device__ __forceinline__ uint32_t kept(int word) {
    group(word);
    const uint32_t f = fr.take(2 + m);
    const uint32_t t = ((f & ((2u << m) - 1)) << (7 - m)) | lr.take(7 - m);
    return mx_value_bits(f >> (m + 1), t, X, 7);
  }
  __device__ __forceinline__ uint32_t pruned(int word) {
    group(word);
    const uint32_t v = pr.take(9);
    return mx_value_bits(v >> 8, v & 0xFF, X, 7);
  }
  static constexpr bool kHasPruned = true;
};

}  // namespace cass
