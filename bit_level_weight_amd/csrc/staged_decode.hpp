// Per-lane decoding helpers of the staged draft GEMV, over words already
// copied to LDS.
//
// Streams are read statelessly: the next field or code is taken from the
// 32-bit window that starts at the current bit position (two adjacent words
// and one funnel shift), so a lane keeps one bit counter per stream.
//
// Method: Cassandra review (marsggbo.github.io), section 3.2 -- a unary code is
// decoded by counting the zeros up to the one (here count-trailing-zeros of
// the window); section 3.3 -- de-sparsification of the kept values (here
// find-first-set over the keep bitmap).
#pragma once

#include "bits.hpp"

namespace cass {

// 32 bits of a word stream starting at bit `pos`.
__device__ __forceinline__ uint32_t window32(const uint32_t* w, uint32_t pos) {
  const uint32_t* q = w + (pos >> 5);
  return __builtin_amdgcn_alignbit(q[1], q[0], pos & 31);
}

// Unary code at bit `pos` of w.  Returns the rank and advances pos past the
// code (a code of 32 bits or more takes the slow path).
__device__ __forceinline__ int unary_at(const uint32_t* w, uint32_t& pos) {
  uint32_t win = window32(w, pos);
  int r = 0;
  if (__builtin_expect(win == 0u, 0)) {
    for (int it = 0; it < 7 && win == 0u; ++it) {
      pos += 32;
      r += 32;
      win = window32(w, pos);
    }
    if (win == 0u) {
      pos += 32;
      return 255;
    }
  }
  const int t = __builtin_ctz(win);
  pos += (uint32_t)t + 1u;
  return r + t;
}

// Bit index (0..31) of the n-th set bit of w, n >= 1 and n <= popcount(w).
__device__ __forceinline__ int select_bit(uint32_t w, int n) {
  int pos = 0;
  int c = __builtin_popcount(w & 0xFFFFu);
  if (c < n) { n -= c; w >>= 16; pos += 16; }
  c = __builtin_popcount(w & 0xFFu);
  if (c < n) { n -= c; w >>= 8; pos += 8; }
  c = __builtin_popcount(w & 0xFu);
  if (c < n) { n -= c; w >>= 4; pos += 4; }
  c = __builtin_popcount(w & 0x3u);
  if (c < n) { n -= c; w >>= 2; pos += 2; }
  c = (int)(w & 1u);
  if (c < n) pos += 1;
  return pos;
}

// Bit position just after the n-th unary code that starts at `pos` (each
// code ends with its only one bit, so this is a select over one bits).
// A code is at most 256 bits, so a valid stream ends the loop within
// 8n + 1 windows; the cap only keeps a corrupt stream from spinning.
__device__ __forceinline__ uint32_t skip_codes(const uint32_t* w, uint32_t pos, int n) {
  for (int it = 8 * n + 1; n > 0 && it > 0; --it) {
    const uint32_t win = window32(w, pos);
    const int c = __builtin_popcount(win);
    if (c >= n) return pos + (uint32_t)select_bit(win, n) + 1u;
    n -= c;
    pos += 32;
  }
  return pos;
}

// skip_codes with the first 256 bits read at once (nine words, one LDS round
// trip); longer skips continue word by word.
__device__ __forceinline__ uint32_t skip_codes8(const uint32_t* w, uint32_t pos, int n) {
  if (n <= 0) return pos;
  const uint32_t* q = w + (pos >> 5);
  const uint32_t sh = pos & 31u;
  uint32_t qv[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) qv[i] = q[i];
  int rem = n, sel = -1;
  uint32_t wsel = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t win = __builtin_amdgcn_alignbit(qv[i + 1], qv[i], sh);
    const int c = __builtin_popcount(win);
    const bool here = sel < 0 && rem <= c;
    sel = here ? i : sel;
    wsel = here ? win : wsel;
    rem -= (sel < 0) ? c : 0;
  }
  if (sel < 0) return skip_codes(w, pos + 256u, rem);
  return pos + 32u * (uint32_t)sel + (uint32_t)select_bit(wsel, rem) + 1u;
}

// Byte offset of x element e in LDS: two bf16 of padding after every 32
// elements (one bitmap word), so lanes working on different parts of a row
// hit different banks.  Consecutive words of positions are 68 bytes apart.
__device__ __forceinline__ uint32_t x_lds_off(uint32_t e) { return 2u * e + 4u * (e >> 5); }
constexpr uint32_t kXWordBytes = 68;

__device__ __forceinline__ float x_at(const uint8_t* xs, uint32_t off) {
  return bf16_bits_to_float(*reinterpret_cast<const uint16_t*>(xs + off));
}

// Hot loop for parts of exactly SUB bitmap words with no empty word before
// the last.  The words sit in registers and shift down on a word advance, so
// per kept value the loop reads the field window, the code window and x from
// LDS plus one (rank, field) -> fp32 table entry, with no data-dependent
// branch.  The table covers ranks 0..31; a code of 32 bits or more (not met
// for kept exponents in practice) makes the function return false, and the
// caller decodes the part again with c1_block.  Until then the reader steps
// through that code's zero bits, so it stays inside the part's codes.
//   xoff      LDS byte offset of x for the part's first position
//   xbstride  bytes between the batch rows of x in LDS
template <int BATCH, int SUB>
__device__ __forceinline__ bool c1_part_regs(const uint32_t* bmw, const uint32_t* fw_l,
                                             uint32_t fp, const uint32_t* cw_l, uint32_t cp,
                                             const uint8_t* xs, uint32_t xoff,
                                             uint32_t xbstride, const uint32_t* lut, int m,
                                             float* acc) {
  static_assert(SUB == 2 || SUB == 4, "two or four words per lane");
  const int fw = 1 + m;
  const uint32_t fmask = (1u << fw) - 1u;
  // the part's bitmap words, shifted down as they are used up
  uint32_t w0 = bmw[0], w1 = bmw[1], w2 = 0u, w3 = 0u;
  if (SUB == 4) {
    w2 = bmw[2];
    w3 = bmw[3];
  }
  const int cnt = __builtin_popcount(w0) + __builtin_popcount(w1) +
                  (SUB == 4 ? __builtin_popcount(w2) + __builtin_popcount(w3) : 0);
  uint32_t wbase = xoff;  // x byte offset of the current word's first position
  uint32_t zflag = 0xFFFFFFFFu;
  for (int i = 0; i < cnt; ++i) {
    const bool adv = w0 == 0u;
    w0 = adv ? w1 : w0;
    if (SUB == 4) {
      w1 = adv ? w2 : w1;
      w2 = adv ? w3 : w2;
      w3 = adv ? 0u : w3;
    } else {
      w1 = adv ? 0u : w1;
    }
    wbase += adv ? kXWordBytes : 0u;
    const uint32_t pb = (uint32_t)__builtin_ctz(w0);
    w0 &= w0 - 1u;
    const uint32_t f = window32(fw_l, fp) & fmask;
    fp += (uint32_t)fw;
    const uint32_t win = window32(cw_l, cp);
    zflag = zflag < win ? zflag : win;  // becomes 0 on a code of 32+ bits
    const uint32_t r = (uint32_t)__builtin_ctz(win | 0x80000000u);
    cp += r + 1u;
    const float wv = __uint_as_float(lut[(r << fw) | f]);
    const uint32_t xa = wbase + 2u * pb;
#pragma unroll
    for (int bb = 0; bb < BATCH; ++bb)
      acc[bb] = __builtin_fmaf(wv, x_at(xs, xa + bb * xbstride), acc[bb]);
  }
  return zflag != 0u;
}

// General decode of `nwords` bitmap words of one row, Cassandra-1 (any word
// count, empty words and codes of any length): acc[b] += W[j] * x[b][j].
//   e0  x element of the first position
template <int BATCH>
__device__ __forceinline__ void c1_block(const uint32_t* bmw, int nwords, const uint32_t* fw_l,
                                         uint32_t fp, const uint32_t* cw_l, uint32_t cp,
                                         const uint8_t* xs, uint32_t e0, uint32_t xbstride,
                                         const uint32_t* lut, int rmax, int m,
                                         const uint8_t* perm, float* acc) {
  const int fw = 1 + m;
  const uint32_t fmask = (1u << fw) - 1u;
  for (int wi = 0; wi < nwords; ++wi) {
    uint32_t cur = bmw[wi];
    while (cur) {
      const int pb = __builtin_ctz(cur);
      cur &= cur - 1u;
      const uint32_t f = window32(fw_l, fp) & fmask;
      fp += (uint32_t)fw;
      const int r = unary_at(cw_l, cp);
      uint32_t bits;
      if (r < rmax)
        bits = lut[((uint32_t)r << fw) | f];
      else
        bits = ((f >> m) << 31) | ((uint32_t)perm[r] << 23) | ((f & ((1u << m) - 1u)) << (23 - m));
      const float wv = __uint_as_float(bits);
      const uint32_t xa = x_lds_off(e0 + (uint32_t)(wi * 32 + pb));
#pragma unroll
      for (int bb = 0; bb < BATCH; ++bb)
        acc[bb] = __builtin_fmaf(wv, x_at(xs, xa + bb * xbstride), acc[bb]);
    }
  }
}

}  // namespace cass
