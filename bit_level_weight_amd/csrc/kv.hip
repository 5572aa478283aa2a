// KV cache: online append-encode, decode, and draft / verification attention
// on the compressed cache.
//
// Method: Cassandra review (marsggbo.github.io), section 3.1 -- the KV cache
// goes through the same pruning, mantissa truncation and exponent coding as
// the weights, split into speculation and verification data; section 3.3 --
// KV entries are produced during inference, so the encoder runs online;
// section 1 -- the draft guesses tokens and the target verifies them in one
// parallel pass.  Attention is the usual scaled-dot-product softmax.
//
// Stream layout: see include/cassandra.h.  Streams are indexed 2*head + kind
// (kind 0 = keys, 1 = values); a vector is one token of one head of one kind.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "bits.hpp"
#include "decoders.hpp"
#include "internal.hpp"
#include "staged_decode.hpp"

namespace cass {

namespace {

constexpr int kWaves = 4;  // waves per workgroup in the per-vector kernels

struct KvDev {
  uint8_t* spec;
  uint8_t* verif;
  unsigned long long* state;  // [0] tokens, [1] flags, [2+2s] spec tail, [3+2s] verif tail
  int64_t sstride, vstride;   // bytes per stream region
  int64_t so[5], vo[5];       // part offsets inside a region
  int H, D, k, m;
  int64_t T_max, ccap, vcap;
  int fmt;                    // CASS_FMT_C1_UNARY or CASS_FMT_C2_MX32
};

// Append workspace (per call, nvec = ntok * 2H vectors).
struct AppendWs {
  uint32_t* bm;     // nvec * D/32 keep words
  uint32_t* lens;   // nvec * 2: speculation / verification code bits
  uint32_t* start;  // nvec * 2: first code bit (0xFFFFFFFF: not written)
  uint32_t* hist;   // 2H * 512 exponent counts (first append)
};

__device__ __forceinline__ int key_of(uint16_t b) { return b & 0x7FFF; }

__device__ __forceinline__ const uint16_t* vec_ptr(const uint16_t* kk, const uint16_t* vv,
                                                    int64_t t, int h, int kind, int H, int D) {
  return (kind ? vv : kk) + (t * H + h) * (int64_t)D;
}

// ---- append, step 1: top-k of each vector (one wave per vector) ----
// Keep bits of vector x of stream s into bm[0 .. D/32) (lane 0 writes), and on
// the first append its exponents into the stream's histograms.  keys: the
// wave's shared-memory copy of the vector (D entries), which the later steps
// of the fused append read instead of x.
//
// The kept values are the k largest keys |x| (15 bits), ties to the lower
// index.  T, the k-th largest key, is found bit by bit from the top: a bit
// stays set when at least k keys are >= the prefix with it (one ballot per
// 64 keys per bit).  Then every key > T is kept, and of the keys equal to T
// the first k - #(keys > T) in index order.
constexpr int kSelChunks = 4;  // head_dim <= 256

// A vector's values for vec_select_loaded: lane l holds elements l, l + 64, ...
__device__ __forceinline__ void vec_load(const KvDev& kv, const uint16_t* x,
                                         uint16_t (&xin)[kSelChunks], int lane) {
  const int D = kv.D, nc = (D + 63) / 64;
#pragma unroll
  for (int c = 0; c < kSelChunks; ++c) {
    const int j = c * 64 + lane;
    xin[c] = (c < nc && j < D) ? x[j] : (uint16_t)0;
  }
}

__device__ __forceinline__ void vec_select_loaded(const KvDev& kv, const uint16_t (&xin)[kSelChunks],
                                                  int s, int first, const AppendWs& ws,
                                                  uint16_t* keys, uint32_t* bm, int lane) {
  const int D = kv.D, nc = (D + 63) / 64;
  int key[kSelChunks];
#pragma unroll
  for (int c = 0; c < kSelChunks; ++c) {
    const int j = c * 64 + lane;
    const bool in = c < nc && j < D;
    const uint16_t b = xin[c];
    if (in) keys[j] = b;
    key[c] = in ? key_of(b) : -1;  // -1: no value, below every candidate
  }
  int T = 0;
  for (int bit = 14; bit >= 0; --bit) {
    const int cand = T | (1 << bit);
    int cnt = 0;
#pragma unroll
    for (int c = 0; c < kSelChunks; ++c)
      if (c < nc) cnt += __builtin_popcountll(__ballot(key[c] >= cand));
    T = cnt >= kv.k ? cand : T;
  }
  int gt = 0;
#pragma unroll
  for (int c = 0; c < kSelChunks; ++c)
    if (c < nc) gt += __builtin_popcountll(__ballot(key[c] > T));
  const int need = kv.k - gt;  // keys equal to T that are kept
  const unsigned long long below = (1ull << lane) - 1ull;
  int ties = 0;
#pragma unroll
  for (int c = 0; c < kSelChunks; ++c) {
    if (c >= nc) break;
    const unsigned long long tm = __ballot(key[c] == T);
    const int trank = ties + __builtin_popcountll(tm & below);
    const bool keep = key[c] > T || (key[c] == T && trank < need);
    ties += __builtin_popcountll(tm);
    const int j = c * 64 + lane;
    if (first && j < D) {
      const int e = (keys[j] >> 7) & 0xFF;
      atomicAdd(ws.hist + s * 512 + (keep ? 0 : 256) + e, 1u);
    }
    const unsigned long long mask = __ballot(keep);
    if (lane == 0) {
      const int w0 = c * 2;
      if (w0 < D / 32) bm[w0] = (uint32_t)mask;
      if (w0 + 1 < D / 32) bm[w0 + 1] = (uint32_t)(mask >> 32);
    }
  }
}

__device__ __forceinline__ void vec_select(const KvDev& kv, const uint16_t* x, int s, int first,
                                           const AppendWs& ws, uint16_t* keys, uint32_t* bm,
                                           int lane) {
  uint16_t xin[kSelChunks];
  vec_load(kv, x, xin, lane);
  vec_select_loaded(kv, xin, s, first, ws, keys, bm, lane);
}

__global__ void __launch_bounds__(64 * kWaves) k_kv_select(KvDev kv, const uint16_t* kk,
                                                           const uint16_t* vv, int ntok, int first,
                                                           AppendWs ws) {
  __shared__ uint16_t keys[kWaves][256];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t nvec = (int64_t)ntok * 2 * kv.H;
  const int64_t vi = (int64_t)blockIdx.x * kWaves + wv;
  if (vi >= nvec) return;
  const int kind = (int)(vi & 1);
  const int64_t th = vi >> 1;
  const int h = (int)(th % kv.H);
  const int64_t t = th / kv.H;
  vec_select(kv, vec_ptr(kk, vv, t, h, kind, kv.H, kv.D), 2 * h + kind, first, ws, keys[wv],
             ws.bm + vi * (kv.D / 32), lane);
}

// ---- append, step 2 (first append only): rank tables from the histograms ----
__global__ void __launch_bounds__(256) k_kv_ranks(KvDev kv, AppendWs ws) {
  __shared__ uint32_t cnt[512];
  const int s = blockIdx.x;
  const int t = threadIdx.x;
  cnt[t] = ws.hist[s * 512 + t];
  cnt[256 + t] = ws.hist[s * 512 + 256 + t];
  __syncthreads();
  for (int which = 0; which < 2; ++which) {
    if (which == 0 && kv.fmt != CASS_FMT_C1_UNARY) continue;  // C-2 codes pruned exponents only
    const uint32_t* c = cnt + which * 256;
    int rank = 0;  // count descending, symbol ascending
    for (int u = 0; u < 256; ++u) rank += (c[u] > c[t]) || (c[u] == c[t] && u < t);
    uint8_t* perm = which ? kv.verif + s * kv.vstride + kv.vo[0] : kv.spec + s * kv.sstride + kv.so[0];
    perm[rank] = (uint8_t)t;
  }
  if (s == 0 && t == 0) kv.state[1] |= (unsigned long long)CASS_KV_FLAG_TABLES;
}

// Wave-private inverse rank tables (symbol -> rank) of stream s.
__device__ __forceinline__ void load_ranks(const KvDev& kv, int s, uint8_t* rs, uint8_t* rv,
                                           int lane) {
  const uint8_t* ps = kv.spec + s * kv.sstride + kv.so[0];
  const uint8_t* pv = kv.verif + s * kv.vstride + kv.vo[0];
  for (int r = lane; r < 256; r += 64) {
    rs[ps[r]] = (uint8_t)r;
    rv[pv[r]] = (uint8_t)r;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ bool kept_bit(const uint32_t* bm, int j) {
  return (bm[j >> 5] >> (j & 31)) & 1u;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

// Shared exponent of the lane's 32 positions (lanes 0-31 and 32-63 each hold
// one group): the largest max(e,1) over the group's kept values, 0 if none.
__device__ __forceinline__ int group_shexp(bool kept, int e) {
  int E = kept ? (e > 0 ? e : 1) : 0;
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) {
    const int u = __shfl_xor(E, o, 64);
    E = u > E ? u : E;
  }
  return E;
}

// ---- append, step 3: code bits of each vector ----
// Speculation (C-1) or residue (C-2) code bits, and pruned-code bits, of
// vector x with keep bits bm (rs / rv: the stream's inverse rank tables);
// the same in every lane.
__device__ __forceinline__ void vec_lengths(const KvDev& kv, const uint16_t* x, const uint32_t* bm,
                                            const uint8_t* rs, const uint8_t* rv, int lane,
                                            uint32_t& a_out, uint32_t& b_out) {
  uint32_t a = 0, b = 0;
  if (kv.fmt == CASS_FMT_C1_UNARY) {
    for (int j = lane; j < kv.D; j += 64) {
      const int e = (x[j] >> 7) & 0xFF;
      if (kept_bit(bm, j)) a += rs[e] + 1u;
      else b += rv[e] + 1u;
    }
  } else {
    // Cassandra-2: a kept value's residue is unary(d) and min(8, 7-m+d) bits
    for (int c0 = 0; c0 < kv.D; c0 += 64) {
      const int j = c0 + lane;
      const bool in = j < kv.D;
      const int e = in ? (x[j] >> 7) & 0xFF : 0;
      const bool kept = in && kept_bit(bm, j);
      const int d = group_shexp(kept, e) - (e > 0 ? e : 1);
      const int w = 7 - kv.m + d < 8 ? 7 - kv.m + d : 8;
      if (kept) a += (uint32_t)(d + 1 + w);
      else if (in) b += rv[e] + 1u;
    }
  }
  a_out = wave_sum(a);
  b_out = wave_sum(b);
}

__global__ void __launch_bounds__(64 * kWaves) k_kv_lengths(KvDev kv, const uint16_t* kk,
                                                            const uint16_t* vv, int ntok,
                                                            AppendWs ws) {
  __shared__ uint8_t rs[kWaves][256], rv[kWaves][256];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t nvec = (int64_t)ntok * 2 * kv.H;
  const int64_t vi = (int64_t)blockIdx.x * kWaves + wv;
  if (vi >= nvec) return;
  const int kind = (int)(vi & 1);
  const int h = (int)((vi >> 1) % kv.H);
  const int64_t t = (vi >> 1) / kv.H;
  const int s = 2 * h + kind;
  load_ranks(kv, s, rs[wv], rv[wv], lane);
  uint32_t a, b;
  vec_lengths(kv, vec_ptr(kk, vv, t, h, kind, kv.H, kv.D), ws.bm + vi * (kv.D / 32), rs[wv], rv[wv],
              lane, a, b);
  if (lane == 0) {
    ws.lens[2 * vi] = a;
    ws.lens[2 * vi + 1] = b;
  }
}

// ---- append, step 4: per stream, code positions of the new tokens ----
__global__ void __launch_bounds__(256) k_kv_scan(KvDev kv, int ntok, int64_t t0, AppendWs ws) {
  __shared__ unsigned long long tmp[256];
  __shared__ unsigned long long carry_s[2];
  const int s = blockIdx.x;
  const int h = s >> 1, kind = s & 1;
  const int t = threadIdx.x;
  unsigned long long base[2] = {kv.state[2 + 2 * s], kv.state[3 + 2 * s]};
  const unsigned long long cap[2] = {(unsigned long long)kv.ccap, (unsigned long long)kv.vcap};
  // token offsets: C-1 spec code / pruned code; C-2 a (residue, pruned code) pair
  const bool c1 = kv.fmt == CASS_FMT_C1_UNARY;
  uint32_t* vofs = (uint32_t*)(kv.verif + s * kv.vstride + kv.vo[3]);
  uint32_t* offs[2] = {c1 ? (uint32_t*)(kv.spec + s * kv.sstride + kv.so[2]) : vofs,
                       c1 ? vofs : vofs + 1};
  const int ostride = c1 ? 1 : 2;
  for (int which = 0; which < 2; ++which) {
    unsigned long long carry = base[which];
    bool over = false;
    for (int c0 = 0; c0 < ntok; c0 += 256) {
      const int i = c0 + t;
      const int64_t vi = ((int64_t)i * kv.H + h) * 2 + kind;
      const unsigned long long len = (i < ntok) ? ws.lens[2 * vi + which] : 0ull;
      tmp[t] = len;
      __syncthreads();
      for (int d = 1; d < 256; d <<= 1) {
        const unsigned long long add = (t >= d) ? tmp[t - d] : 0ull;
        __syncthreads();
        tmp[t] += add;
        __syncthreads();
      }
      const unsigned long long st = carry + tmp[t] - len;
      if (i < ntok) {
        const bool fits = st + len <= cap[which];
        ws.start[2 * vi + which] = fits ? (uint32_t)st : 0xFFFFFFFFu;
        offs[which][(t0 + i) * ostride] = fits ? (uint32_t)st : 0xFFFFFFFFu;
        if (!fits) over = true;
      }
      if (t == 255) carry_s[which] = carry + tmp[255];
      __syncthreads();
      carry = carry_s[which];
      __syncthreads();
    }
    const int any_over = __syncthreads_or(over ? 1 : 0);
    if (t == 0) {
      // on overflow the stream is closed: its tail moves to the capacity, so
      // later appends cannot write over the codes that did fit
      if (any_over) atomicOr(kv.state + 1, (unsigned long long)CASS_KV_FLAG_OVERFLOW);
      kv.state[2 + 2 * s + which] = any_over ? cap[which] : carry;
    }
  }
  if (s == 0 && t == 0) kv.state[0] += (unsigned long long)ntok;
}

__device__ __forceinline__ void or_bits(uint8_t* sec, uint64_t pos, uint32_t v, int width) {
  // v holds width <= 9 bits; touches at most two 32-bit words
  if (width == 0 || v == 0) return;
  uint32_t* w = reinterpret_cast<uint32_t*>(sec) + (pos >> 5);
  const int sh = (int)(pos & 31);
  atomicOr(w, v << sh);
  if (sh + width > 32) atomicOr(w + 1, v >> (32 - sh));
}

// ---- append, step 5: pack (one wave per vector) ----
// Vector x (keep bits bm) as token tok of stream s; its codes start at bits
// sstart / vstart of the code sections (0xFFFFFFFF: not written).
__device__ __forceinline__ void vec_pack(const KvDev& kv, const uint16_t* x, const uint32_t* bm,
                                         const uint8_t* rsw, const uint8_t* rvw, int s,
                                         int64_t tok, uint32_t sstart, uint32_t vstart, int lane) {
  uint8_t* sr = kv.spec + s * kv.sstride;
  uint8_t* vr = kv.verif + s * kv.vstride;
  const int D = kv.D, k = kv.k, m = kv.m;
  if (lane < D / 32) reinterpret_cast<uint32_t*>(sr + kv.so[1])[tok * (D / 32) + lane] = bm[lane];
  uint32_t kept_carry = 0, scode_carry = 0, vcode_carry = 0;
  if (kv.fmt != CASS_FMT_C1_UNARY) {
    // Cassandra-2: shared exponents, aligned significands, residues
    for (int c0 = 0; c0 < D; c0 += 64) {
      const int j = c0 + lane;
      const bool in = j < D;
      const uint16_t b = in ? x[j] : 0;
      const bool kept = in && kept_bit(bm, j);
      const int sgn = b >> 15, e = (b >> 7) & 0xFF, f = b & 0x7F;
      const int eff = e > 0 ? e : 1, M = ((e > 0) << 7) | f;
      const int E = group_shexp(kept, e);
      const int d = E - eff, shift = 7 - m + d;
      const int a = shift >= 8 ? 0 : M >> shift, w = shift < 8 ? shift : 8;
      const unsigned long long km = __ballot(kept);
      const unsigned long long pm = __ballot(in && !kept);
      const uint32_t kidx = kept_carry + (uint32_t)__builtin_popcountll(km & ((1ull << lane) - 1ull));
      const uint32_t pidx = (uint32_t)(c0 - kept_carry) +
                            (uint32_t)__builtin_popcountll(pm & ((1ull << lane) - 1ull));
      const uint32_t rlen = kept ? (uint32_t)(d + 1 + w) : 0u;
      const uint32_t vlen = (in && !kept) ? rvw[e] + 1u : 0u;
      const uint32_t rin = wave_incl_scan(rlen, lane), vin = wave_incl_scan(vlen, lane);
      if (in && (j & 31) == 0) (sr + kv.so[2])[tok * (D / 32) + j / 32] = (uint8_t)E;
      if (kept) {
        const uint64_t kin = (uint64_t)tok * k + kidx;
        or_bits(sr + kv.so[3], kin * (uint64_t)(2 + m), (uint32_t)((sgn << (m + 1)) | a), 2 + m);
        if (sstart != 0xFFFFFFFFu) {
          const uint64_t pos = (uint64_t)sstart + scode_carry + rin - rlen;
          or_bits(vr + kv.vo[1], pos + (uint64_t)d, 1u, 1);  // unary(d): its one bit
          or_bits(vr + kv.vo[1], pos + (uint64_t)d + 1u, (uint32_t)(M & ((1 << w) - 1)), w);
        }
      } else if (in) {
        (vr + kv.vo[2])[tok * (D - k) + pidx] = (uint8_t)((sgn << 7) | f);
        if (vstart != 0xFFFFFFFFu) {
          const uint64_t endbit = (uint64_t)vstart + vcode_carry + vin - 1u;
          or_bits(vr + kv.vo[4], endbit, 1u, 1);
        }
      }
      kept_carry += (uint32_t)__builtin_popcountll(km);
      scode_carry += __shfl(rin, 63, 64);
      vcode_carry += __shfl(vin, 63, 64);
    }
    return;
  }
  for (int c0 = 0; c0 < D; c0 += 64) {
    const int j = c0 + lane;
    const bool in = j < D;
    const uint16_t b = in ? x[j] : 0;
    const bool kept = in && kept_bit(bm, j);
    const int sgn = b >> 15, e = (b >> 7) & 0xFF, f = b & 0x7F;
    const unsigned long long km = __ballot(kept);
    const unsigned long long pm = __ballot(in && !kept);
    const uint32_t kidx = kept_carry + (uint32_t)__builtin_popcountll(km & ((1ull << lane) - 1ull));
    const uint32_t pidx = (uint32_t)(c0 - kept_carry) +
                          (uint32_t)__builtin_popcountll(pm & ((1ull << lane) - 1ull));
    const uint32_t slen = kept ? rsw[e] + 1u : 0u;
    const uint32_t vlen = (in && !kept) ? rvw[e] + 1u : 0u;
    const uint32_t sin = wave_incl_scan(slen, lane), vin = wave_incl_scan(vlen, lane);
    if (kept) {
      const uint64_t kin = (uint64_t)tok * k + kidx;
      or_bits(sr + kv.so[3], kin * (uint64_t)(1 + m), (uint32_t)((sgn << m) | (f >> (7 - m))), 1 + m);
      or_bits(vr + kv.vo[1], kin * (uint64_t)(7 - m), (uint32_t)(f & ((1 << (7 - m)) - 1)), 7 - m);
      if (sstart != 0xFFFFFFFFu) {  // the code's one bit ends it
        const uint64_t endbit = (uint64_t)sstart + scode_carry + sin - 1u;
        or_bits(sr + kv.so[4], endbit, 1u, 1);
      }
    } else if (in) {
      (vr + kv.vo[2])[tok * (D - k) + pidx] = (uint8_t)((sgn << 7) | f);
      if (vstart != 0xFFFFFFFFu) {
        const uint64_t endbit = (uint64_t)vstart + vcode_carry + vin - 1u;
        or_bits(vr + kv.vo[4], endbit, 1u, 1);
      }
    }
    kept_carry += (uint32_t)__builtin_popcountll(km);
    scode_carry += __shfl(sin, 63, 64);
    vcode_carry += __shfl(vin, 63, 64);
  }
}

__global__ void __launch_bounds__(64 * kWaves) k_kv_pack(KvDev kv, const uint16_t* kk,
                                                         const uint16_t* vv, int ntok, int64_t t0,
                                                         AppendWs ws) {
  __shared__ uint8_t rs[kWaves][256], rv[kWaves][256];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t nvec = (int64_t)ntok * 2 * kv.H;
  const int64_t vi = (int64_t)blockIdx.x * kWaves + wv;
  if (vi >= nvec) return;
  const int kind = (int)(vi & 1);
  const int h = (int)((vi >> 1) % kv.H);
  const int64_t i = (vi >> 1) / kv.H;
  const int s = 2 * h + kind;
  load_ranks(kv, s, rs[wv], rv[wv], lane);
  vec_pack(kv, vec_ptr(kk, vv, i, h, kind, kv.H, kv.D), ws.bm + vi * (kv.D / 32), rs[wv], rv[wv], s,
           t0 + i, ws.start[2 * vi], ws.start[2 * vi + 1], lane);
}

// ---- a few tokens in one launch: a workgroup per stream and a wave per token
// (the rank tables are frozen).  The waves select and measure their tokens side
// by side, take their code starts from the tokens' lengths in order through
// shared memory, and pack side by side (every multi-bit write is an atomic or
// into zeroed words, so neighbouring tokens may share a word).  The same bytes,
// tails and flags as the five-launch path.
constexpr int kFusedMaxTokens = 16;

__global__ void __launch_bounds__(64 * kFusedMaxTokens) k_kv_append_few(KvDev kv, const uint16_t* kk,
                                                                     const uint16_t* vv, int ntok,
                                                                     int64_t t0, AppendWs ws) {
  __shared__ uint16_t keys[kFusedMaxTokens][256];
  __shared__ uint32_t bm[kFusedMaxTokens][8];
  __shared__ uint8_t rs[256], rv[256];
  __shared__ uint32_t lens[kFusedMaxTokens][2];
  const int s = blockIdx.x, h = s >> 1, kind = s & 1;
  const int lane = threadIdx.x & 63, i = threadIdx.x >> 6;  // wave i takes token t0 + i
  // the token's vector is loaded before the rank tables, so the two loads
  // overlap
  uint16_t xin[kSelChunks];
  vec_load(kv, vec_ptr(kk, vv, i, h, kind, kv.H, kv.D), xin, lane);
  {
    const uint8_t* ps = kv.spec + s * kv.sstride + kv.so[0];
    const uint8_t* pv = kv.verif + s * kv.vstride + kv.vo[0];
    for (int r = threadIdx.x; r < 256; r += blockDim.x) {
      rs[ps[r]] = (uint8_t)r;
      rv[pv[r]] = (uint8_t)r;
    }
  }
  __syncthreads();  // the rank tables
  const bool c1 = kv.fmt == CASS_FMT_C1_UNARY;
  const unsigned long long tail0[2] = {kv.state[2 + 2 * s], kv.state[3 + 2 * s]};
  const unsigned long long cap[2] = {(unsigned long long)kv.ccap, (unsigned long long)kv.vcap};
  uint32_t* vofs = reinterpret_cast<uint32_t*>(kv.verif + s * kv.vstride + kv.vo[3]);
  uint32_t* offs[2] = {c1 ? reinterpret_cast<uint32_t*>(kv.spec + s * kv.sstride + kv.so[2]) : vofs,
                       c1 ? vofs : vofs + 1};
  const int ostride = c1 ? 1 : 2;
  // each wave selects its token's kept values and measures its two code runs
  vec_select_loaded(kv, xin, s, 0, ws, keys[i], bm[i], lane);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // (the vector is read from global memory once: the later steps take the
  // shared-memory copy)
  uint32_t len[2];
  vec_lengths(kv, keys[i], bm[i], rs, rv, lane, len[0], len[1]);
  if (lane == 0) {
    lens[i][0] = len[0];
    lens[i][1] = len[1];
  }
  __syncthreads();  // every token's lengths
  // a token's codes start after the stream's tail and the earlier tokens'
  // codes; a token that does not fit gets no code start, and then no later
  // one fits either (the tail only grows), so the stream overflows exactly
  // when its last token ends past the cap
  unsigned long long before[2] = {tail0[0], tail0[1]}, end[2] = {tail0[0], tail0[1]};
  for (int t = 0; t < ntok; ++t) {
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      before[which] += t < i ? lens[t][which] : 0u;
      end[which] += lens[t][which];
    }
  }
  uint32_t start[2];
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    start[which] = before[which] + len[which] <= cap[which] ? (uint32_t)before[which] : 0xFFFFFFFFu;
    if (lane == 0) offs[which][(t0 + i) * ostride] = start[which];
  }
  vec_pack(kv, keys[i], bm[i], rs, rv, s, t0 + i, start[0], start[1], lane);
  if (threadIdx.x == 0) {
    // on overflow the stream is closed, as in the five-launch path
    const bool over0 = end[0] > cap[0], over1 = end[1] > cap[1];
    if (over0 || over1) atomicOr(kv.state + 1, (unsigned long long)CASS_KV_FLAG_OVERFLOW);
    kv.state[2 + 2 * s] = over0 ? cap[0] : end[0];
    kv.state[3 + 2 * s] = over1 ? cap[1] : end[1];
    if (s == 0) kv.state[0] += (unsigned long long)ntok;
  }
}

// ---- truncation: drop the newest tokens of every stream ----
// Bits [b0, b1) of a bit section set to zero (one thread per word).
__device__ void clear_bits(uint8_t* sec, uint64_t b0, uint64_t b1, int tid, int nthr) {
  if (b1 <= b0) return;
  uint32_t* w = reinterpret_cast<uint32_t*>(sec);
  for (uint64_t i = (b0 >> 5) + tid; i <= (b1 - 1) >> 5; i += nthr) {
    const uint64_t lo = i * 32 > b0 ? i * 32 : b0, hi = i * 32 + 32 < b1 ? i * 32 + 32 : b1;
    const uint32_t width = (uint32_t)(hi - lo), sh = (uint32_t)(lo - i * 32);
    const uint32_t mask = width == 32 ? 0xFFFFFFFFu : ((1u << width) - 1u) << sh;
    w[i] &= ~mask;
  }
}

__device__ void clear_bytes(uint8_t* sec, int64_t b0, int64_t b1, int tid, int nthr) {
  for (int64_t i = b0 + tid; i < b1; i += nthr) sec[i] = 0;
}

// One workgroup per stream.  Keeps tokens [0, t_new) of the t_old cached:
// every per-token part past t_new goes back to zero and each code tail moves
// back to the first code bit of token t_new, so the stream holds exactly the
// bytes of t_new appended tokens (a stream closed by an overflow stays closed
// if token t_new's codes were not written).
__global__ void __launch_bounds__(256) k_kv_truncate(KvDev kv, int64_t t_new, int64_t t_old) {
  const int s = blockIdx.x, tid = threadIdx.x, nthr = blockDim.x;
  uint8_t* sr = kv.spec + s * kv.sstride;
  uint8_t* vr = kv.verif + s * kv.vstride;
  const int64_t D = kv.D, k = kv.k, m = kv.m;
  const bool c1 = kv.fmt == CASS_FMT_C1_UNARY;
  // first code bit of token t_new: C-1 speculation codes / pruned codes;
  // C-2 kept residues / pruned codes
  const uint32_t* vofs = reinterpret_cast<const uint32_t*>(vr + kv.vo[3]);
  const uint32_t first[2] = {c1 ? reinterpret_cast<const uint32_t*>(sr + kv.so[2])[t_new]
                                 : vofs[2 * t_new],
                             c1 ? vofs[t_new] : vofs[2 * t_new + 1]};
  uint8_t* code_sec[2] = {c1 ? sr + kv.so[4] : vr + kv.vo[1], vr + kv.vo[4]};
  __shared__ unsigned long long tail_s[2];
  if (tid < 2) tail_s[tid] = kv.state[2 + 2 * s + tid];
  __syncthreads();
  for (int which = 0; which < 2; ++which) {
    if (first[which] == 0xFFFFFFFFu) continue;  // closed before t_new: nothing written since
    clear_bits(code_sec[which], first[which], tail_s[which], tid, nthr);
  }
  // fixed-size per-token parts
  clear_bytes(sr + kv.so[1], t_new * D / 8, t_old * D / 8, tid, nthr);  // keep bitmap
  if (c1) {
    clear_bytes(sr + kv.so[2], 4 * t_new, 4 * t_old, tid, nthr);        // code offsets
    clear_bits(sr + kv.so[3], (uint64_t)(t_new * k * (1 + m)), (uint64_t)(t_old * k * (1 + m)),
               tid, nthr);                                               // sign + top mantissa
    clear_bits(vr + kv.vo[1], (uint64_t)(t_new * k * (7 - m)), (uint64_t)(t_old * k * (7 - m)),
               tid, nthr);                                               // low mantissa
  } else {
    clear_bytes(sr + kv.so[2], t_new * D / 32, t_old * D / 32, tid, nthr);  // shared exponents
    clear_bits(sr + kv.so[3], (uint64_t)(t_new * k * (2 + m)), (uint64_t)(t_old * k * (2 + m)),
               tid, nthr);                                               // sign + significand
  }
  clear_bytes(vr + kv.vo[2], t_new * (D - k), t_old * (D - k), tid, nthr);  // pruned bytes
  clear_bytes(vr + kv.vo[3], (c1 ? 4 : 8) * t_new, (c1 ? 4 : 8) * t_old, tid, nthr);  // offsets
  __syncthreads();
  if (tid < 2 && first[tid] != 0xFFFFFFFFu) kv.state[2 + 2 * s + tid] = first[tid];
  if (s == 0 && tid == 0) kv.state[0] = (unsigned long long)t_new;
}

// ---- per-lane decoder of one cached vector (token tok of stream s) ----
// kept(w) gives the vector's kept values in position order (w: the bitmap
// word the value sits in), pruned() its pruned values (exact decoding only);
// callers walk the keep-bitmap words with two loops, kept positions then
// pruned positions.  FMT: Cassandra-1 (unary exponent codes) or Cassandra-2
// (shared exponent per 32 positions, residues for the exact values).
template <bool EXACT, int FMT>
struct KvVec {
  BitReader fr, cr, lr, vcr, pr;
  // staged draft decode: field and code bit positions in shared-memory words
  const uint32_t* fw_l;
  const uint32_t* cw_l;
  uint32_t fpos, cpos;
  const uint8_t* perm_s;
  const uint8_t* perm_v;
  const uint8_t* shexp;
  const uint32_t* bm;
  int m;
  __device__ __forceinline__ void init(const KvDev& kv, int s, int64_t tok) {
    const uint8_t* sr = kv.spec + s * kv.sstride;
    const uint8_t* vr = kv.verif + s * kv.vstride;
    m = kv.m;
    bm = reinterpret_cast<const uint32_t*>(sr + kv.so[1]) + tok * (kv.D / 32);
    // a token whose codes did not fit (overflow flag) reads code bit 0 instead:
    // its values are meaningless but every read stays inside the region
    if (FMT == CASS_FMT_C1_UNARY) {
      perm_s = sr + kv.so[0];
      fr.init(reinterpret_cast<const uint32_t*>(sr + kv.so[3]), (uint64_t)tok * kv.k * (1 + m));
      const uint32_t off = reinterpret_cast<const uint32_t*>(sr + kv.so[2])[tok];
      cr.init(reinterpret_cast<const uint32_t*>(sr + kv.so[4]), off == 0xFFFFFFFFu ? 0u : off);
    } else {
      shexp = sr + kv.so[2] + tok * (kv.D / 32);
      fr.init(reinterpret_cast<const uint32_t*>(sr + kv.so[3]), (uint64_t)tok * kv.k * (2 + m));
    }
    if (EXACT) {
      perm_v = vr + kv.vo[0];
      pr.init(reinterpret_cast<const uint32_t*>(vr + kv.vo[2]), (uint64_t)tok * (kv.D - kv.k) * 8u);
      const uint32_t* ofs = reinterpret_cast<const uint32_t*>(vr + kv.vo[3]);
      uint32_t poff;
      if (FMT == CASS_FMT_C1_UNARY) {
        lr.init(reinterpret_cast<const uint32_t*>(vr + kv.vo[1]), (uint64_t)tok * kv.k * (7 - m));
        poff = ofs[tok];
      } else {
        const uint32_t roff = ofs[2 * tok];
        lr.init(reinterpret_cast<const uint32_t*>(vr + kv.vo[1]), roff == 0xFFFFFFFFu ? 0u : roff);
        poff = ofs[2 * tok + 1];
      }
      vcr.init(reinterpret_cast<const uint32_t*>(vr + kv.vo[4]), poff == 0xFFFFFFFFu ? 0u : poff);
    }
  }
  // Draft decode from copies of the chunk's speculation sections in shared
  // memory (see StagedSpec): bitmap words, fields from bit fbit of fl, shared
  // exponents (C-2) and, when cl is set, codes from bit cbit of cl.  Without
  // cl the codes are read from global memory as in init.
  __device__ __forceinline__ void init_staged(const KvDev& kv, int s, int64_t tok,
                                              const uint32_t* bml, const uint32_t* fl,
                                              uint64_t fbit, const uint8_t* shl,
                                              const uint32_t* cl, uint64_t cbit) {
    const uint8_t* sr = kv.spec + s * kv.sstride;
    m = kv.m;
    bm = bml;
    fr.init(fl, fbit);
    fw_l = fl;
    fpos = (uint32_t)fbit;
    cw_l = cl;
    cpos = (uint32_t)cbit;
    if (FMT == CASS_FMT_C1_UNARY) {
      perm_s = sr + kv.so[0];
      if (cl) {
        cr.init(cl, cbit);
      } else {
        const uint32_t off = reinterpret_cast<const uint32_t*>(sr + kv.so[2])[tok];
        cr.init(reinterpret_cast<const uint32_t*>(sr + kv.so[4]), off == 0xFFFFFFFFu ? 0u : off);
      }
    } else {
      shexp = shl;
    }
  }
  // read the rank tables from (shared-memory) copies instead
  __device__ __forceinline__ void use_tables(const uint8_t* ps, const uint8_t* pv) {
    perm_s = ps;
    perm_v = pv;
  }
  __device__ __forceinline__ uint32_t kept(int w) {
    if (FMT == CASS_FMT_C1_UNARY) {
      const uint32_t f = fr.take(1 + m);
      const uint32_t e = perm_s[cr.unary()];
      uint32_t bits = ((f >> m) << 15) | (e << 7) | ((f & ((1u << m) - 1u)) << (7 - m));
      if (EXACT) bits |= lr.take(7 - m);
      return bits;
    }
    const int E = shexp[w];
    const uint32_t f = fr.take(2 + m);
    const uint32_t sg = f >> (m + 1), a = f & ((2u << m) - 1u);
    if (!EXACT) return mx_value_bits(sg, a, E, m);
    const int d = lr.unary();
    const int wd = (7 - m + d < 8) ? 7 - m + d : 8;
    const uint32_t L = lr.take(wd);
    const uint32_t M = (wd < 8) ? ((a << wd) | L) : L;
    const uint32_t e = (M >= 128u) ? (uint32_t)(E - d) : 0u;
    return (sg << 15) | ((e & 0xFF) << 7) | (M & 0x7F);
  }
  __device__ __forceinline__ uint32_t pruned() {
    const uint32_t byte = pr.take(8);
    const uint32_t e = perm_v[vcr.unary()];
    return ((byte >> 7) << 15) | (e << 7) | (byte & 0x7F);
  }
  // Draft decode (Cassandra-1) of the vector's k kept values in groups of 8:
  // positions, fields and ranks of a group first (shift registers over the
  // D = 128 keep bits, bit readers), then every rank-table read of the group
  // at once, then use(d, bits) per value, so a group waits on shared memory
  // once instead of once per value.  Needs every keep word non-empty (the
  // caller checks; each word then holds the next values when the current one
  // runs out).
  template <typename F>
  __device__ __forceinline__ void kept_grouped(int k, F&& use) {
    uint32_t w0 = bm[0], w1 = bm[1], w2 = bm[2], w3 = bm[3];
    uint32_t base = 0;
    for (int i0 = 0; i0 < k; i0 += 8) {
      uint32_t dd[8], ff[8], rr[8], ee[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (i0 + u < k) {
          const bool adv = w0 == 0u;
          w0 = adv ? w1 : w0;
          w1 = adv ? w2 : w1;
          w2 = adv ? w3 : w2;
          w3 = adv ? 0u : w3;
          base += adv ? 32u : 0u;
          // (the mask keeps a corrupt vector's positions inside the row)
          dd[u] = (base + (uint32_t)__builtin_ctz(w0)) & 127u;
          w0 &= w0 - 1u;
          ff[u] = fr.take(1 + m);
          rr[u] = (uint32_t)cr.unary();
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + u < k) ee[u] = perm_s[rr[u]];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (i0 + u < k) {
          const uint32_t f = ff[u];
          use(dd[u], ((f >> m) << 15) | (ee[u] << 7) | ((f & ((1u << m) - 1u)) << (7 - m)));
        }
      }
    }
  }
  // One group of ng <= 8 values of kept_windows.  FULL: ng is 8, and the
  // group is straight-line code (a per-value test of u < ng, though uniform,
  // becomes a branch per value and splits the group into small blocks).
  template <bool FULL, typename F>
  __device__ __forceinline__ void windows_group(int ng, uint32_t& w0, uint32_t& w1, uint32_t& w2,
                                                uint32_t& w3, uint32_t& base, F&& use) {
    const uint32_t fw = 1u + (uint32_t)m, fmask = (1u << fw) - 1u;
    const uint32_t wf = window32(fw_l, fpos);
    const uint32_t wc0 = window32(cw_l, cpos);
    uint32_t dd[8], ff[8], rr[8], ee[8];
    if (__all(__builtin_popcount(wc0) >= (FULL ? 8 : ng))) {
      uint32_t wc = wc0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (FULL || u < ng) {
          const bool adv = w0 == 0u;
          w0 = adv ? w1 : w0;
          w1 = adv ? w2 : w1;
          w2 = adv ? w3 : w2;
          w3 = adv ? 0u : w3;
          base += adv ? 32u : 0u;
          dd[u] = (base + (uint32_t)__builtin_ctz(w0)) & 127u;
          w0 &= w0 - 1u;
          ff[u] = __builtin_amdgcn_ubfe(wf, (uint32_t)u * fw, fw);
          const uint32_t r = (uint32_t)__builtin_ctz(wc);
          rr[u] = r;
          wc = (wc >> r) >> 1;
        }
      }
      // bits the codes took: the window was shifted right by that many
      cpos += (wc ? (uint32_t)__builtin_clz(wc) : 32u) - (uint32_t)__builtin_clz(wc0);
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (FULL || u < ng) {
          const bool adv = w0 == 0u;
          w0 = adv ? w1 : w0;
          w1 = adv ? w2 : w1;
          w2 = adv ? w3 : w2;
          w3 = adv ? 0u : w3;
          base += adv ? 32u : 0u;
          dd[u] = (base + (uint32_t)__builtin_ctz(w0)) & 127u;
          w0 &= w0 - 1u;
          ff[u] = window32(fw_l, fpos + (uint32_t)u * fw) & fmask;
          // a code of any length (at most 256 bits; the bound keeps a
          // corrupt stream from running on)
          uint32_t r = 0, wv = window32(cw_l, cpos);
          for (int it = 0; it < 8 && wv == 0u; ++it) {
            r += 32u;
            cpos += 32u;
            wv = window32(cw_l, cpos);
          }
          const uint32_t t = (uint32_t)__builtin_ctz(wv | (wv ? 0u : 0x80000000u));
          r += t;
          cpos += t + 1u;
          rr[u] = r < 256u ? r : 255u;
        }
      }
    }
    fpos += (uint32_t)(FULL ? 8 : ng) * fw;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (FULL || u < ng) ee[u] = perm_s[rr[u]];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (FULL || u < ng) {
        const uint32_t f = ff[u];
        use(dd[u], ((f >> m) << 15) | (ee[u] << 7) | ((f & ((1u << m) - 1u)) << (7 - m)));
      }
    }
  }
  // The same, Cassandra-1 with the token's fields and codes staged (fw_l,
  // cw_l): 32-bit field and code windows read from shared memory (two words
  // and a funnel shift each), a rank as the zeros before the window's next
  // one, eight values per window.  A group whose code window holds fewer ones
  // than its values for some lane is decoded value by value.  Needs 1 + m <= 4
  // and every keep word non-empty (the caller checks).
  template <typename F>
  __device__ __forceinline__ void kept_windows(int k, F&& use) {
    uint32_t w0 = bm[0], w1 = bm[1], w2 = bm[2], w3 = bm[3];
    uint32_t base = 0;
    int i0 = 0;
    for (; i0 + 8 <= k; i0 += 8) windows_group<true>(8, w0, w1, w2, w3, base, use);
    if (i0 < k) windows_group<false>(k - i0, w0, w1, w2, w3, base, use);
  }
  // Cassandra-2 draft decode of the k kept values from the staged fields: four
  // (sign, significand) fields per 32-bit window (fields of up to 8 bits), the
  // shared exponent of a value's 32-position group from the token's four
  // exponent bytes (one word).  Needs every keep word non-empty.
  template <bool FULL, typename F>
  __device__ __forceinline__ void windows_group_c2(int ng, uint32_t& w0, uint32_t& w1,
                                                   uint32_t& w2, uint32_t& w3, uint32_t& base,
                                                   uint32_t e4, F&& use) {
    const uint32_t fw = 2u + (uint32_t)m;
    const uint32_t wf = window32(fw_l, fpos);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (FULL || u < ng) {
        const bool adv = w0 == 0u;
        w0 = adv ? w1 : w0;
        w1 = adv ? w2 : w1;
        w2 = adv ? w3 : w2;
        w3 = adv ? 0u : w3;
        base += adv ? 32u : 0u;
        const uint32_t d = (base + (uint32_t)__builtin_ctz(w0)) & 127u;
        w0 &= w0 - 1u;
        const uint32_t f = __builtin_amdgcn_ubfe(wf, (uint32_t)u * fw, fw);
        const int E = (int)((e4 >> (8u * ((base >> 5) & 3u))) & 0xFFu);
        use(d, mx_value_bits(f >> (m + 1), f & ((2u << m) - 1u), E, m));
      }
    }
    fpos += (uint32_t)(FULL ? 4 : ng) * fw;
  }
  template <typename F>
  __device__ __forceinline__ void kept_windows_c2(int k, F&& use) {
    uint32_t w0 = bm[0], w1 = bm[1], w2 = bm[2], w3 = bm[3];
    const uint32_t e4 = *reinterpret_cast<const uint32_t*>(shexp);
    uint32_t base = 0;
    int i0 = 0;
    // (full groups as straight-line code, the last partial group by value)
    for (; i0 + 4 <= k; i0 += 4) windows_group_c2<true>(4, w0, w1, w2, w3, base, e4, use);
    if (i0 < k) windows_group_c2<false>(k - i0, w0, w1, w2, w3, base, e4, use);
  }
  // the kept values into their positions of o[0..D) (the rest left as they are)
  __device__ __forceinline__ void kept_into(int D, uint16_t* o, int stride = 1) {
    for (int w = 0; w < D / 32; ++w)
      for (uint32_t km = bm[w]; km; km &= km - 1u)
        o[(w * 32 + __builtin_ctz(km)) * stride] = (uint16_t)kept(w);
  }
  // all D positions into o[0..D)
  __device__ __forceinline__ void all(int D, uint16_t* o) {
    for (int w = 0; w < D / 32; ++w) {
      const uint32_t word = bm[w];
      if (!EXACT)
        for (int b = 0; b < 32; ++b) o[w * 32 + b] = 0;
      for (uint32_t km = word; km; km &= km - 1u) o[w * 32 + __builtin_ctz(km)] = (uint16_t)kept(w);
      if (EXACT)
        for (uint32_t pm = ~word; pm; pm &= pm - 1u) o[w * 32 + __builtin_ctz(pm)] = (uint16_t)pruned();
    }
  }
};

// ---- decode the whole cache (tests, checks) ----
template <bool EXACT, int FMT>
__global__ void __launch_bounds__(256) k_kv_decode(KvDev kv, int64_t T, uint16_t* out) {
  const int64_t n = (int64_t)2 * kv.H * T;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t tok = idx % T;
    const int s = (int)(idx / T);  // out is [kind][head][T][D]
    const int kind = s / kv.H, h = s % kv.H;
    KvVec<EXACT, FMT> dec;
    dec.init(kv, 2 * h + kind, tok);
    dec.all(kv.D, out + idx * kv.D);
  }
}

// ---- attention: one workgroup per (KV head, chunk of 128 tokens) ----
constexpr int kChunk = 128;  // tokens per workgroup, one per thread
constexpr int kDim = 128;
constexpr int kVStride = kDim + 2;  // bf16 per LDS row of the value tile (bank spread)
// draft attention with at most 4 query rows: the value tile transposed,
// [dim][token] with 16-byte rows (P·V on the matrix cores reads 8 tokens of a
// dimension at once; rows 68 words apart spread a 16-lane read over the banks)
constexpr int kVTStride = kChunk + 8;
__host__ __device__ constexpr int vt_elems(bool transposed) {
  return transposed ? kDim * kVTStride : kChunk * kVStride;
}

typedef short xv4s __attribute__((ext_vector_type(4)));
typedef short xv8s __attribute__((ext_vector_type(8)));
typedef __bf16 xv8bf __attribute__((ext_vector_type(8)));
typedef float xv4f __attribute__((ext_vector_type(4)));

// bf16 bits of x rounded to nearest even (x finite).
__device__ __forceinline__ uint32_t x1_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
constexpr int kMaxRows = 32;
constexpr int kMaxChunksMerge = 8192;  // chunk partials one merge takes (512K tokens in 64-token chunks)

struct AttnArgs {
  const uint16_t* q;  // [nq][Hq][D]
  int nq, Hq, G;      // G = Hq / H query heads per KV head
  float scale;
  int64_t T;          // tokens in the cache
  int nchunks;
  float* part;        // chunk numerators [H][nchunks][rows][D]
  float* ml;          // chunk (row maximum, sum of p) [H][rows][nchunks][2]
  int fcap, ccap;     // draft: shared-memory words per stream for fields and codes
};

// Draft attention: the chunk's speculation sections of K and V, copied to
// shared memory before the decode.  Per stream: keep words [kChunk][D/32],
// fields (fcap words from the 16-byte boundary at or before the chunk's first
// field bit), codes (C-1: ccap words from the 16-byte boundary at or before
// the first token's first code bit) or shared exponents (C-2: [kChunk][D/32]
// bytes).

__host__ __device__ __forceinline__ int staged_words(int fcap, int ccap, int fmt) {
  return kChunk * (kDim / 32) + fcap + (fmt == CASS_FMT_C1_UNARY ? ccap : kChunk);
}

typedef __attribute__((address_space(3))) void lds_void;

// LDS DMA of up to n words from word a0 (a multiple of 4) of src, never past
// word lim, to dst (16-byte aligned): 64 chunks of 16 bytes per instruction,
// the waves' runs interleaved; the last 0-3 words of a run that ends inside a
// chunk by plain loads.  Completion: vmcnt(0) in every wave, then a barrier.
__device__ __forceinline__ void dma_words(uint32_t* dst, const uint32_t* src, int64_t a0, int n,
                                          int64_t lim, int tid, int nthr) {
  const int l64 = tid & 63, w64 = tid >> 6;
  CASS_DCHECK((((uintptr_t)(src + a0) | (uintptr_t)dst) & 15) == 0, CASS_DBG_ALIGN);
  int64_t a1 = a0 + n < lim ? a0 + n : lim;
  if (a1 < a0) a1 = a0;
  const int nw = (int)(a1 - a0), nch = nw >> 2;
  for (int base = w64 * 64; base < nch; base += nthr)
    if (base + l64 < nch)
      __builtin_amdgcn_global_load_lds((const void*)(src + a0 + 4 * (base + l64)),
                                       (lds_void*)(dst + 4 * base), 16, 0, 0);
  if (tid < (nw & 3)) dst[4 * nch + tid] = src[a0 + 4 * nch + tid];
}

// MAXR: a bound on the query rows (nq * G) the launch serves.  Shared
// memory: queries [128][MAXR] fp32 (a key position's entries side by side),
// scores [MAXR][kChunk] fp32, value tile [kChunk][130] bf16 (about 37 KB for
// one query of four heads), then for the draft the staged sections.
template <bool EXACT, int MAXR, int FMT>
__global__ void __launch_bounds__(2 * kChunk) k_kv_attn(KvDev kv, AttnArgs a) {
  // threads 0..kChunk-1: one token's key and its scores; threads kChunk..:
  // the same token's value row into the tile (the two decodes run side by side)
  extern __shared__ __align__(16) uint8_t smem[];
  float* qf = reinterpret_cast<float*>(smem);                // [128][MAXR]
  float* sc = qf + MAXR * kDim;                              // [MAXR][kChunk]
  uint16_t* vt = reinterpret_cast<uint16_t*>(sc + MAXR * kChunk);  // [kChunk][130]
  __shared__ float red[MAXR][kChunk / 64];
  __shared__ float lsum[MAXR][kChunk / 64];  // (up to 4 rows) per-wave sums of p
  __shared__ __align__(16) uint8_t tabs[4][256];  // rank tables: K spec, K verif, V spec, V verif
  const int h = blockIdx.x, c = blockIdx.y;
  const int rows = a.nq * a.G;
  const int tid = threadIdx.x;
  if (EXACT) {
    for (int i = tid; i < 4 * 256; i += 2 * kChunk) {
      const int s = 2 * h + (i >> 9), which = (i >> 8) & 1;
      const uint8_t* src = which ? kv.verif + s * kv.vstride + kv.vo[0] : kv.spec + s * kv.sstride + kv.so[0];
      tabs[i >> 8][i & 255] = src[i & 255];
    }
  } else if ((tid >> 6) == 1) {
    // the four rank tables by LDS DMA: 16 chunks each
    const int l = tid & 63;
    const int s = 2 * h + (l >> 5), which = (l >> 4) & 1;
    const uint8_t* src = which ? kv.verif + s * kv.vstride + kv.vo[0] : kv.spec + s * kv.sstride + kv.so[0];
    __builtin_amdgcn_global_load_lds((const void*)(src + 16 * (l & 15)), (lds_void*)&tabs[0][0], 16, 0,
                                     0);
  }
  // draft: stage the chunk's speculation sections of K and V.  Order of the
  // loads: the query, every fixed-width copy, the two code offsets, then the
  // code copies (which need the offsets); the query is stored last.  The
  // chain is an offset then its codes, with everything else in flight.
  const int64_t t0 = (int64_t)c * kChunk;
  const int fwid = FMT == CASS_FMT_C1_UNARY ? 1 + kv.m : 2 + kv.m;
  const int sw = staged_words(a.fcap, a.ccap, FMT);
  constexpr bool VTR = !EXACT && MAXR == 4;  // transposed value tile, P·V on the matrix cores
  uint32_t* stg = reinterpret_cast<uint32_t*>(vt + vt_elems(VTR));
  // (staged runs start at the 16-byte boundary at or before their first word)
  const int64_t fw0 = ((t0 * kv.k * fwid) >> 5) & ~(int64_t)3;  // first staged field word
  int64_t cw0[2] = {0, 0};                                      // first staged code word per stream
  // (through the scalar cache: the offsets are read-only here, and a scalar
  // wait does not wait for the vector loads and copies in flight)
  typedef __attribute__((address_space(4))) const uint32_t const_u32;
  // query rows of this KV head: row r = qi * G + g  (query qi, head h*G + g);
  // rows past `rows` stay zero
  constexpr int kQPer = MAXR * kDim / (2 * kChunk);
  static_assert(MAXR * kDim % (2 * kChunk) == 0, "query elements split evenly over the threads");
  uint16_t qv[kQPer];
#pragma unroll
  for (int i = 0; i < kQPer; ++i) {
    const int idx = tid + i * 2 * kChunk;
    const int r = idx / kDim, d = idx % kDim;
    const int rc = r < rows ? r : 0;  // (unconditional loads: no branch to wait at)
    const int qi = rc / a.G, g = rc % a.G;
    qv[i] = a.q[((int64_t)qi * a.Hq + h * a.G + g) * kDim + d];
  }
  if (!EXACT) {
    // every copy by LDS DMA, all in flight at once
    for (int j = 0; j < 2; ++j) {
      const uint8_t* sr = kv.spec + (2 * h + j) * kv.sstride;
      uint32_t* base = stg + j * sw;
      dma_words(base, reinterpret_cast<const uint32_t*>(sr + kv.so[1]), t0 * (kDim / 32),
                kChunk * (kDim / 32), kv.T_max * (kDim / 32), tid, 2 * kChunk);
      dma_words(base + kChunk * (kDim / 32), reinterpret_cast<const uint32_t*>(sr + kv.so[3]), fw0,
                a.fcap, (kv.T_max * kv.k * fwid + 31) / 32, tid, 2 * kChunk);
      if (FMT != CASS_FMT_C1_UNARY) {
        // shared exponents: D/32 = 4 bytes, one word, per token
        dma_words(base + kChunk * (kDim / 32) + a.fcap,
                  reinterpret_cast<const uint32_t*>(sr + kv.so[2]), t0, kChunk, kv.T_max, tid,
                  2 * kChunk);
      }
    }
    if (FMT == CASS_FMT_C1_UNARY) {
      // (the offsets after the fixed-width copies: a scalar wait covers every
      // scalar load in flight, kernel arguments included)
      uint32_t o0[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        o0[j] = ((const_u32*)(kv.spec + (2 * h + j) * kv.sstride + kv.so[2]))[t0];
      for (int j = 0; j < 2; ++j) {
        const uint8_t* sr = kv.spec + (2 * h + j) * kv.sstride;
        uint32_t* rest = stg + j * sw + kChunk * (kDim / 32) + a.fcap;
        cw0[j] = o0[j] == 0xFFFFFFFFu ? 0 : (int64_t)((o0[j] >> 5) & ~3u);
        dma_words(rest, reinterpret_cast<const uint32_t*>(sr + kv.so[4]), cw0[j], a.ccap,
                  (kv.ccap + 31) / 32, tid, 2 * kChunk);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kQPer; ++i) {
    const int idx = tid + i * 2 * kChunk;
    qf[(idx % kDim) * MAXR + idx / kDim] = idx / kDim < rows ? bf16_bits_to_float(qv[i]) : 0.f;
  }
  if (!EXACT) {
    // the draft value tile starts zero-filled (pruned positions and tokens past
    // the end); the decoders write the kept values only
    typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
    u32x4v* vt4 = reinterpret_cast<u32x4v*>(vt);
    for (int i = tid; i < vt_elems(VTR) * 2 / 16; i += 2 * kChunk) vt4[i] = u32x4v{0, 0, 0, 0};
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies
  }
  __syncthreads();
  const int ti = tid & (kChunk - 1);
  const int64_t tok = (int64_t)c * kChunk + ti;
  const bool live = tok < a.T;
  // the draft decoder of this thread's token in stream j (0: K, 1: V) over
  // the staged words; its codes from shared memory when they lie inside the
  // staged run, else from global memory
  auto init_draft = [&](KvVec<EXACT, FMT>& dec, int j) {
    const int s = 2 * h + j;
    uint32_t* base = stg + j * sw;
    uint32_t* rest = base + kChunk * (kDim / 32) + a.fcap;
    const uint64_t fbit = (uint64_t)tok * kv.k * fwid - (uint64_t)fw0 * 32;
    const uint32_t* cl = nullptr;
    uint64_t cbit = 0;
    if (FMT == CASS_FMT_C1_UNARY) {
      const uint8_t* sr = kv.spec + s * kv.sstride;
      const uint32_t* offs = reinterpret_cast<const uint32_t*>(sr + kv.so[2]);
      const uint32_t off = offs[tok];
      const unsigned long long end = tok + 1 < a.T ? (unsigned long long)offs[tok + 1]
                                                   : kv.state[2 + 2 * s];
      // (the reader looks up to three words past the code it is on)
      if (off != 0xFFFFFFFFu && end != 0xFFFFFFFFull && (int64_t)(off >> 5) >= cw0[j] &&
          (int64_t)(end >> 5) + 4 < cw0[j] + a.ccap) {
        cl = rest;
        cbit = (uint64_t)off - (uint64_t)cw0[j] * 32;
      }
    }
    dec.init_staged(kv, s, tok, base + ti * (kDim / 32), base + kChunk * (kDim / 32), fbit,
                    reinterpret_cast<const uint8_t*>(rest + ti), cl, cbit);
  };
  if (tid < kChunk) {
    float s[MAXR];
#pragma unroll
    for (int r = 0; r < MAXR; ++r) s[r] = 0.f;
    if (live) {  // scores: kept positions, then (exact) pruned positions
      KvVec<EXACT, FMT> dec;
      if (EXACT)
        dec.init(kv, 2 * h, tok);
      else
        init_draft(dec, 0);
      dec.use_tables(tabs[0], tabs[1]);
      if (!EXACT && FMT == CASS_FMT_C2_MX32 && MAXR <= 8 && kv.m <= 6 &&
          __all(dec.bm[0] != 0u && dec.bm[1] != 0u && dec.bm[2] != 0u && dec.bm[3] != 0u)) {
        dec.kept_windows_c2(kv.k, [&](uint32_t d, uint32_t bits) {
          const float kvv = bf16_bits_to_float(bits);
#pragma unroll
          for (int r = 0; r < MAXR; ++r) s[r] = __builtin_fmaf(kvv, qf[d * MAXR + r], s[r]);
        });
      } else if (!EXACT && FMT == CASS_FMT_C1_UNARY && MAXR <= 8 && kv.m <= 3 &&
          __all(dec.bm[0] != 0u && dec.bm[1] != 0u && dec.bm[2] != 0u && dec.bm[3] != 0u &&
                dec.cw_l != nullptr)) {
        dec.kept_windows(kv.k, [&](uint32_t d, uint32_t bits) {
          const float kvv = bf16_bits_to_float(bits);
#pragma unroll
          for (int r = 0; r < MAXR; ++r) s[r] = __builtin_fmaf(kvv, qf[d * MAXR + r], s[r]);
        });
      } else if (!EXACT && FMT == CASS_FMT_C1_UNARY && MAXR <= 8 &&
          __all(dec.bm[0] != 0u && dec.bm[1] != 0u && dec.bm[2] != 0u && dec.bm[3] != 0u)) {
        dec.kept_grouped(kv.k, [&](uint32_t d, uint32_t bits) {
          const float kvv = bf16_bits_to_float(bits);
#pragma unroll
          for (int r = 0; r < MAXR; ++r) s[r] = __builtin_fmaf(kvv, qf[d * MAXR + r], s[r]);
        });
      } else
      for (int w = 0; w < kDim / 32; ++w) {
        const uint32_t word = dec.bm[w];
        for (uint32_t km = word; km; km &= km - 1u) {
          const float kvv = bf16_bits_to_float(dec.kept(w));
          const int d = w * 32 + __builtin_ctz(km);
#pragma unroll
          for (int r = 0; r < MAXR; ++r) s[r] = __builtin_fmaf(kvv, qf[d * MAXR + r], s[r]);
        }
        if (EXACT) {
          for (uint32_t pm = ~word; pm; pm &= pm - 1u) {
            const float kvv = bf16_bits_to_float(dec.pruned());
            const int d = w * 32 + __builtin_ctz(pm);
#pragma unroll
            for (int r = 0; r < MAXR; ++r) s[r] = __builtin_fmaf(kvv, qf[d * MAXR + r], s[r]);
          }
        }
      }
    }
    // causal visibility: query qi sees tokens < T - nq + qi + 1
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      if (r < rows) {
        const int qi = r / a.G;
        const bool vis = live && tok < a.T - a.nq + qi + 1;
        sc[r * kChunk + ti] = vis ? s[r] * a.scale : -INFINITY;
      }
    }
  } else {
    // value tile (zero for tokens past the end): value d of the token at
    // row[d * vs] (a column of the transposed tile, or a row of the other)
    uint16_t* row = VTR ? vt + ti : vt + ti * kVStride;
    const int vs = VTR ? kVTStride : 1;
    if (live) {
      KvVec<EXACT, FMT> dec;
      if (EXACT) {
        dec.init(kv, 2 * h + 1, tok);
        dec.use_tables(tabs[2], tabs[3]);
        dec.all(kDim, row);
      } else {
        init_draft(dec, 1);
        dec.use_tables(tabs[2], tabs[3]);
        if (FMT == CASS_FMT_C2_MX32 && kv.m <= 6 &&
            __all(dec.bm[0] != 0u && dec.bm[1] != 0u && dec.bm[2] != 0u && dec.bm[3] != 0u))
          dec.kept_windows_c2(kv.k, [&](uint32_t d, uint32_t bits) { row[d * vs] = (uint16_t)bits; });
        else if (FMT == CASS_FMT_C1_UNARY && kv.m <= 3 &&
            __all(dec.bm[0] != 0u && dec.bm[1] != 0u && dec.bm[2] != 0u && dec.bm[3] != 0u &&
                  dec.cw_l != nullptr))
          dec.kept_windows(kv.k, [&](uint32_t d, uint32_t bits) { row[d * vs] = (uint16_t)bits; });
        else if (FMT == CASS_FMT_C1_UNARY &&
            __all(dec.bm[0] != 0u && dec.bm[1] != 0u && dec.bm[2] != 0u && dec.bm[3] != 0u))
          dec.kept_grouped(kv.k, [&](uint32_t d, uint32_t bits) { row[d * vs] = (uint16_t)bits; });
        else
          dec.kept_into(kDim, row, vs);
      }
    } else if (EXACT) {
      for (int d = 0; d < kDim; ++d) row[d] = 0;
    }
  }
  __syncthreads();
  // per row: max over the chunk, then p = e^{s - max}
  const int lane = tid & 63, wv = tid >> 6;
  if (tid < kChunk) {
    for (int r = 0; r < rows; ++r) {
      float mx = sc[r * kChunk + ti];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      if (lane == 0) red[r][wv] = mx;
    }
  }
  __syncthreads();
  if constexpr (VTR) {
    // p as two bf16 terms (hi, then lo = p - hi: about 2^-17 relative), rows
    // [4][kChunk] each, over the query region (no longer read); the row sums
    // by wave reductions; then o = p V on the matrix cores
    uint16_t* ph = reinterpret_cast<uint16_t*>(qf);
    if (tid < kChunk) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float p = 0.f;
        if (r < rows) {
          const float mx = fmaxf(red[r][0], red[r][1]);
          const float sv = sc[r * kChunk + ti];
          p = (mx == -INFINITY || sv == -INFINITY) ? 0.f : __expf(sv - mx);
        }
        const uint32_t hb = x1_bf16_rne(p);
        ph[r * kChunk + ti] = (uint16_t)hb;
        ph[4 * kChunk + r * kChunk + ti] = (uint16_t)x1_bf16_rne(p - __uint_as_float(hb << 16));
        float l = p;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o, 64);
        if (lane == 0) lsum[r][wv] = l;
      }
    }
    __syncthreads();
    // v_mfma_f32_16x16x32_bf16: lane (i16, kq) feeds row i16 of p (rows 4..15
    // zero) and dimension i16 of its group, tokens 8kq..8kq+7 of each 32-token
    // step; a wave takes dimension groups wv and wv + 4
    const int i16 = lane & 15, kq = lane >> 4;
    const xv8s zero = xv8s{0, 0, 0, 0, 0, 0, 0, 0};
    xv8s ahi[kChunk / 32], alo[kChunk / 32];
#pragma unroll
    for (int ks = 0; ks < kChunk / 32; ++ks) {
      const int tb = ks * 32 + 8 * kq;
      ahi[ks] = i16 < 4 ? *reinterpret_cast<const xv8s*>(ph + i16 * kChunk + tb) : zero;
      alo[ks] = i16 < 4 ? *reinterpret_cast<const xv8s*>(ph + 4 * kChunk + i16 * kChunk + tb) : zero;
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int dcol = (wv + 4 * half) * 16 + i16;
      const uint16_t* vcol = vt + dcol * kVTStride;
      xv4f acc = xv4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kChunk / 32; ++ks) {
        const xv8s bop = *reinterpret_cast<const xv8s*>(vcol + ks * 32 + 8 * kq);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(xv8bf, ahi[ks]),
                                                      __builtin_bit_cast(xv8bf, bop), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(xv8bf, alo[ks]),
                                                      __builtin_bit_cast(xv8bf, bop), acc, 0, 0, 0);
      }
      // D: lanes kq = 0 hold rows 0..3 of dimension dcol
      if (kq == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e < rows) a.part[(((int64_t)h * a.nchunks + c) * rows + e) * kDim + dcol] = acc[e];
      }
    }
    if (tid < rows) {
      float* ml = a.ml + (((int64_t)h * rows + tid) * a.nchunks + c) * 2;
      ml[0] = fmaxf(red[tid][0], red[tid][1]);
      ml[1] = lsum[tid][0] + lsum[tid][1];
    }
    return;
  }
  if (MAXR == 4) {
    // up to 4 rows: p also as [token][4] over the queries (no longer read), the
    // row sums by wave reductions; then o[r][d] = sum_t p[r][t] V[t][d] with
    // thread (d, half of the tokens) reading each value once for every row
    float* pt = qf;  // [kChunk][4]
    if (tid < kChunk) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float p = 0.f;
        if (r < rows) {
          const float mx = fmaxf(red[r][0], red[r][1]);
          const float sv = sc[r * kChunk + ti];
          p = (mx == -INFINITY || sv == -INFINITY) ? 0.f : __expf(sv - mx);
        }
        pt[ti * 4 + r] = p;
        float l = p;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o, 64);
        if (lane == 0) lsum[r][wv] = l;
      }
    }
    __syncthreads();
    const int d = tid & (kDim - 1), half = tid >> 7;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    typedef float f4v __attribute__((ext_vector_type(4)));
#pragma unroll 8
    for (int t = half * (kChunk / 2); t < (half + 1) * (kChunk / 2); ++t) {
      const float v = bf16_bits_to_float(vt[t * kVStride + d]);
      const f4v p4 = *reinterpret_cast<const f4v*>(pt + 4 * t);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(p4[r], v, acc[r]);
    }
    float* other = sc;  // [kDim][4]: the second half's sums (the scores are dead)
    if (half == 1) {
#pragma unroll
      for (int r = 0; r < 4; ++r) other[d * 4 + r] = acc[r];
    }
    __syncthreads();
    if (half == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r < rows) {
          a.part[(((int64_t)h * a.nchunks + c) * rows + r) * kDim + d] = acc[r] + other[d * 4 + r];
          if (d == 0) {
            float* ml = a.ml + (((int64_t)h * rows + r) * a.nchunks + c) * 2;
            ml[0] = fmaxf(red[r][0], red[r][1]);
            ml[1] = lsum[r][0] + lsum[r][1];
          }
        }
      }
    }
    return;
  }
  if (tid < kChunk) {
    for (int r = 0; r < rows; ++r) {
      const float mx = fmaxf(red[r][0], red[r][1]);
      const float sv = sc[r * kChunk + ti];
      sc[r * kChunk + ti] = (mx == -INFINITY || sv == -INFINITY) ? 0.f : __expf(sv - mx);
    }
  }
  __syncthreads();
  // o[r][d] = sum_t p[r][t] V[t][d]; thread = (d, half of the rows)
  const int d = tid & (kDim - 1), half = tid >> 7;
  for (int r = half; r < rows; r += 2) {
    float acc = 0.f, l = 0.f;
#pragma unroll 8
    for (int t = 0; t < kChunk; ++t) {
      const float p = sc[r * kChunk + t];
      acc = __builtin_fmaf(p, bf16_bits_to_float(vt[t * kVStride + d]), acc);
      l += p;
    }
    a.part[(((int64_t)h * a.nchunks + c) * rows + r) * kDim + d] = acc;
    if (d == 0) {
      float* ml = a.ml + (((int64_t)h * rows + r) * a.nchunks + c) * 2;
      ml[0] = fmaxf(red[r][0], red[r][1]);
      ml[1] = l;
    }
  }
}

// combine the chunk partials: o = sum_c e^{m_c - M} o_c / sum_c e^{m_c - M} l_c.
// A workgroup per (KV head, query row, range of kMergeDims dimensions); every
// workgroup of a row computes the same weights and denominator.
constexpr int kMergeDims = 32;                       // dimensions per workgroup
constexpr int kMergeSplit = kDim / kMergeDims;       // workgroups per (head, row)
constexpr int kMergeParts = 16;                      // chunk ranges summed side by side
constexpr int kMergeThreads = kMergeDims * kMergeParts;

__global__ void __launch_bounds__(kMergeThreads) k_kv_merge(AttnArgs a, int H, float* out) {
  __shared__ float wgt[kMaxChunksMerge];
  __shared__ float red[2][kMergeThreads / 64];
  __shared__ float nums[kMergeParts][kMergeDims];
  const int rows = a.nq * a.G;
  const int hr = blockIdx.x / kMergeSplit, ds = blockIdx.x % kMergeSplit;  // (h * rows + r, dims)
  const int h = hr / rows, r = hr % rows;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, nw = blockDim.x / 64;
  const float* base = a.part + ((int64_t)h * a.nchunks * rows + r) * kDim;  // chunk 0's numerator
  const int64_t cstride = (int64_t)rows * kDim;
  const float* ml = a.ml + ((int64_t)h * rows + r) * a.nchunks * 2;       // contiguous per row
  // chunk maxima and their overall maximum (the loads of every chunk in flight at once)
  float M = -INFINITY;
  for (int c = tid; c < a.nchunks; c += blockDim.x) {
    const float mc = ml[2 * c];
    wgt[c] = mc;
    M = fmaxf(M, mc);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  if (lane == 0) red[0][wv] = M;
  __syncthreads();
  M = red[0][0];
  for (int i = 1; i < nw; ++i) M = fmaxf(M, red[0][i]);
  // chunk weights e^{m_c - M} and the denominator sum_c w_c l_c (fixed order)
  float den = 0.f;
  for (int c = tid; c < a.nchunks; c += blockDim.x) {
    const float mc = wgt[c];
    const float w = mc == -INFINITY ? 0.f : __expf(mc - M);
    wgt[c] = w;
    den += w * ml[2 * c + 1];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o, 64);
  if (lane == 0) red[1][wv] = den;
  __syncthreads();
  den = 0.f;
  for (int i = 0; i < nw; ++i) den += red[1][i];
  // numerator: thread (d, part) sums chunks part, part + kMergeParts, ...
  const int dl = tid & (kMergeDims - 1), q = tid / kMergeDims, d = ds * kMergeDims + dl;
  float num = 0.f;
#pragma unroll 8
  for (int c = q; c < a.nchunks; c += kMergeParts) num += wgt[c] * base[c * cstride + d];
  nums[q][dl] = num;
  __syncthreads();
  if (q == 0) {
    float tot = 0.f;
    for (int i = 0; i < kMergeParts; ++i) tot += nums[i][dl];
    const int qi = r / a.G, g = r % a.G;
    out[((int64_t)qi * a.Hq + h * a.G + g) * kDim + d] = tot / den;
  }
}

// ---- verification attention, Cassandra-1: split decode, matrix-core products ----
// One workgroup of 8 waves per (KV head, chunk of 64 tokens): about 60 KB of
// shared memory, so two workgroups share a CU and one's copies overlap the
// other's arithmetic.
//  1. The chunk's sections of K and V are copied to shared memory with
//     coalesced loads: fields, low mantissas, pruned bytes, and the
//     speculation and pruned-exponent code runs (a run longer than its staged
//     space is read in place).
//  2. Each of the 512 threads rebuilds 32 exact values: one keep-bitmap word
//     of one token of K or V.  Its kept and pruned values start at indices the
//     popcounts of the token's earlier words give, so its fields, low mantissas
//     and pruned bytes sit at known bit positions, and its codes start after
//     that many one bits of the token's code runs (every unary code ends with
//     its one bit).  Values go to K and V tiles in shared memory.
//  3. Scores S = Q K^T for up to 32 query rows on the matrix cores
//     (v_mfma_f32_16x16x32_bf16: bf16 inputs are exact, sums in fp32), scaled
//     and masked (causal over the appended block).
//  4. Softmax per row over the chunk; o = p V on the matrix cores with p split
//     into two bf16 terms (p = hi + lo to about 2^-17 relative), fp32 sums;
//     written as a chunk partial (row maximum, sum, numerator) for k_kv_merge.
constexpr int kXChunk = 64;  // tokens per workgroup
constexpr int kXThreads = 2 * kXChunk * 4;  // (K | V, token, keep word)
constexpr int kXRows = 32;
constexpr int kXStride = 132;  // bf16 per key tile row (8-byte aligned rows, banks shifted by 2 words)
constexpr int kXVStride = kXChunk + 8;  // bf16 per row of the transposed value tile (16-byte rows)

// Staged words per stream of the split-decode attention.
struct XCaps {
  int scode, pcode;     // speculation / pruned-exponent code runs
  int field, low, pbyte;  // fields, low mantissas, pruned bytes
  __host__ __device__ int per_stream() const { return scode + pcode + field + low + pbyte; }
};

__host__ __device__ __forceinline__ int64_t x1_lds_bytes(const XCaps& cp) {
  return (int64_t)kXChunk * kXStride * 2 + (int64_t)kDim * kXVStride * 2 +
         (int64_t)kXRows * kXChunk * 4 + (int64_t)2 * cp.per_stream() * 4;
}

__global__ void __launch_bounds__(kXThreads) k_kv_attn_x1(KvDev kv, AttnArgs a, XCaps cp) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint16_t* kt = reinterpret_cast<uint16_t*>(smem);          // [token][kXStride] keys
  uint16_t* vt = kt + kXChunk * kXStride;                       // [dim][kXVStride] values, transposed
  // [32][128] scores; then per row p in bf16, hi terms then lo terms
  float* sc = reinterpret_cast<float*>(vt + kDim * kXVStride);
  uint32_t* stg = reinterpret_cast<uint32_t*>(sc + kXRows * kXChunk);  // staged sections
  __shared__ uint8_t tabs[4][256];  // rank tables: K spec, K verif, V spec, V verif
  __shared__ long long cfirst[2][2];  // first staged code word [stream][spec | pruned], -1: in place
  __shared__ float rmax[kXRows], rsum[kXRows];
  const int h = blockIdx.x, c = blockIdx.y;
  const int rows = a.nq * a.G;
  const int tid = threadIdx.x;
  const int k = kv.k, m = kv.m, np = kDim - kv.k;
  const int64_t t0 = (int64_t)c * kXChunk;
  const int64_t t1 = t0 + kXChunk < a.T ? t0 + kXChunk : a.T;  // tokens of the chunk: [t0, t1)
  const int psw = cp.per_stream();
  // staged words of stream j: codes (spec, pruned), fields, low mantissas, pruned bytes
  auto sbase = [&](int j) { return stg + j * psw; };
  // staged copies start at the 16-byte boundary at or before the chunk's first word
  const int64_t fw0 = ((t0 * k * (1 + m)) >> 5) & ~(int64_t)3,
                lw0 = ((t0 * k * (7 - m)) >> 5) & ~(int64_t)3, bw0 = ((t0 * np) >> 2) & ~(int64_t)3;
  const int l64 = tid & 63, w64 = tid >> 6;
  auto dma = [&](uint32_t* dst, const uint32_t* src, int64_t a0, int n, int64_t lim) {
    dma_words(dst, src, a0, n, lim, tid, kXThreads);
  };
  // 1. code runs of the chunk: [offset of t0, offset of t1 or the stream tail);
  // wave 0 finds them while the other waves start the fixed-width copies
  if (tid < 4) {
    const int j = tid >> 1, which = tid & 1;
    const int s = 2 * h + j;
    const uint32_t* offs = reinterpret_cast<const uint32_t*>(
        which ? kv.verif + s * kv.vstride + kv.vo[3] : kv.spec + s * kv.sstride + kv.so[2]);
    const uint32_t b0 = offs[t0];
    const unsigned long long b1 = t1 < kv.T_max && t1 < a.T ? (unsigned long long)offs[t1]
                                                            : kv.state[2 + 2 * s + which];
    const int room = (which ? cp.pcode : cp.scode) - 8;  // words a staged run may take
    long long first = -1;
    if (b0 != 0xFFFFFFFFu && b1 != 0xFFFFFFFFull && b1 >= b0 &&
        (long long)((b1 + 31) >> 5) + 4 - (long long)((b0 >> 5) & ~3u) <= room)
      first = (long long)((b0 >> 5) & ~3u);
    cfirst[j][which] = first;
  }
  if (w64 == 1) {
    // the four rank tables: 16 chunks each
    const int s = 2 * h + (l64 >> 5), which = (l64 >> 4) & 1;
    const uint8_t* src = which ? kv.verif + s * kv.vstride + kv.vo[0] : kv.spec + s * kv.sstride + kv.so[0];
    __builtin_amdgcn_global_load_lds((const void*)(src + 16 * (l64 & 15)), (lds_void*)&tabs[0][0], 16,
                                     0, 0);
  }
  for (int j = 0; j < 2; ++j) {
    const int s = 2 * h + j;
    const uint8_t* sr = kv.spec + s * kv.sstride;
    const uint8_t* vr = kv.verif + s * kv.vstride;
    uint32_t* b = sbase(j) + cp.scode + cp.pcode;
    dma(b, reinterpret_cast<const uint32_t*>(sr + kv.so[3]), fw0, cp.field - 8,
        (kv.T_max * k * (1 + m) + 31) / 32 + 4);
    b += cp.field;
    dma(b, reinterpret_cast<const uint32_t*>(vr + kv.vo[1]), lw0, cp.low - 8,
        (kv.T_max * k * (7 - m) + 31) / 32 + 4);
    b += cp.low;
    dma(b, reinterpret_cast<const uint32_t*>(vr + kv.vo[2]), bw0, cp.pbyte - 8,
        (kv.T_max * np + 3) / 4 + 4);
  }
  __syncthreads();  // the code runs' starts
  for (int j = 0; j < 2; ++j) {
    const int s = 2 * h + j;
    const uint8_t* sr = kv.spec + s * kv.sstride;
    const uint8_t* vr = kv.verif + s * kv.vstride;
    for (int which = 0; which < 2; ++which) {
      const long long first = cfirst[j][which];
      if (first < 0) continue;
      const uint32_t* src = reinterpret_cast<const uint32_t*>(which ? vr + kv.vo[4] : sr + kv.so[4]);
      const int64_t lim = ((which ? kv.vcap : kv.ccap) + 31) / 32 + 4;  // plus the zero pad
      dma(sbase(j) + (which ? cp.scode : 0), src, first, (which ? cp.pcode : cp.scode) - 8, lim);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies
  __syncthreads();

  // 2. exact values: thread = (stream j, token, keep word w)
  {
    const int j = tid / (4 * kXChunk), tl = (tid >> 2) & (kXChunk - 1), w = tid & 3;
    const int64_t tok = t0 + tl;
    // value d of the word goes to row[d * dstride]: keys by token, values by dimension
    uint16_t* row = j ? vt + w * 32 * kXVStride + tl : kt + tl * kXStride + w * 32;
    const int dstride = j ? kXVStride : 1;
    if (tok >= t1) {
      for (int i = 0; i < 32; ++i) row[i * dstride] = 0;
    } else {
      const int s = 2 * h + j;
      const uint8_t* sr = kv.spec + s * kv.sstride;
      const uint8_t* vr = kv.verif + s * kv.vstride;
      const uint32_t* bmp = reinterpret_cast<const uint32_t*>(sr + kv.so[1]) + tok * (kDim / 32);
      const uint32_t wd0 = bmp[0], wd1 = bmp[1], wd2 = bmp[2], wd3 = bmp[3];
      const uint32_t word = w == 0 ? wd0 : w == 1 ? wd1 : w == 2 ? wd2 : wd3;
      const int kb = (w > 0 ? __builtin_popcount(wd0) : 0) + (w > 1 ? __builtin_popcount(wd1) : 0) +
                     (w > 2 ? __builtin_popcount(wd2) : 0);
      const int pb = 32 * w - kb;
      const uint32_t* base = sbase(j);
      const uint32_t* fl = base + cp.scode + cp.pcode;
      const uint32_t* ll = fl + cp.field;
      const uint8_t* bl = reinterpret_cast<const uint8_t*>(ll + cp.low);
      const int64_t kin = (int64_t)tok * k + kb;
      uint32_t fpos = (uint32_t)(kin * (1 + m) - fw0 * 32);
      uint32_t lpos = (uint32_t)(kin * (7 - m) - lw0 * 32);
      uint32_t bpos = (uint32_t)((int64_t)tok * np + pb - bw0 * 4);
      // code runs: from the staged copy, or in place (a token whose codes did
      // not fit the stream reads from bit 0: meaningless values, reads inside)
      const uint32_t* cw[2];
      uint32_t cpos[2];
      for (int which = 0; which < 2; ++which) {
        const uint32_t* offs = reinterpret_cast<const uint32_t*>(
            which ? vr + kv.vo[3] : sr + kv.so[2]);
        uint32_t off = offs[tok];
        off = off == 0xFFFFFFFFu ? 0u : off;
        const long long first = cfirst[j][which];
        if (first >= 0) {
          cw[which] = base + (which ? cp.scode : 0);
          cpos[which] = off - (uint32_t)first * 32u;
        } else {
          cw[which] = reinterpret_cast<const uint32_t*>(which ? vr + kv.vo[4] : sr + kv.so[4]);
          cpos[which] = off;
        }
      }
      // (staged runs have 64 words of slack: the first 256 bits in one round trip)
      cpos[0] = cfirst[j][0] >= 0 ? skip_codes8(cw[0], cpos[0], kb) : skip_codes(cw[0], cpos[0], kb);
      cpos[1] = cfirst[j][1] >= 0 ? skip_codes8(cw[1], cpos[1], pb) : skip_codes(cw[1], cpos[1], pb);
      const uint8_t* ps = tabs[2 * j];
      const uint8_t* pv = tabs[2 * j + 1];
      const int fwd = 1 + m, lwd = 7 - m;
      const uint32_t fmask = (2u << m) - 1u, lmask = (1u << lwd) - 1u;
      // Windows held in registers: fields and low mantissas of the next
      // 32 / width values, pruned bytes four at a time, codes until the window
      // runs out of one bits (a code of 32 bits or more: the general reader).
      // Every lane refills its field, low and byte windows at the same value
      // index, so those refills do not diverge.
      {
        const int uf = 32 / fwd, ul = lwd > 0 ? 32 / lwd : 32;
        uint32_t fwin = 0, lwin = 0, cwin = window32(cw[0], cpos[0]);
        int fleft = 0, lleft = 0;
        for (uint32_t km = word; km; km &= km - 1u) {
          if (fleft == 0) {
            fwin = window32(fl, fpos);
            fleft = uf;
          }
          if (lleft == 0) {
            lwin = window32(ll, lpos);
            lleft = ul;
          }
          const uint32_t f = fwin & fmask;
          const uint32_t lo = lwin & lmask;
          fwin >>= fwd;
          lwin >>= lwd;
          --fleft;
          --lleft;
          fpos += fwd;
          lpos += lwd;
          if (cwin == 0u) cwin = window32(cw[0], cpos[0]);
          int r;
          if (cwin != 0u) {
            r = __builtin_ctz(cwin);
            cwin = (cwin >> r) >> 1;
            cpos[0] += (uint32_t)r + 1u;
          } else {
            r = unary_at(cw[0], cpos[0]);
            cwin = window32(cw[0], cpos[0]);
          }
          const uint32_t e = ps[r & 255];
          row[__builtin_ctz(km) * dstride] = (uint16_t)(((f >> m) << 15) | (e << 7) |
                                                        ((f & ((1u << m) - 1u)) << lwd) | lo);
        }
      }
      {
        const uint32_t* bw = reinterpret_cast<const uint32_t*>(bl);
        uint32_t bwin = 0, cwin = window32(cw[1], cpos[1]);
        int bleft = 0;
        for (uint32_t pm = ~word; pm; pm &= pm - 1u) {
          if (bleft == 0) {
            bwin = window32(bw, bpos * 8u);
            bleft = 4;
          }
          const uint32_t byte = bwin & 0xFFu;
          bwin >>= 8;
          --bleft;
          ++bpos;
          if (cwin == 0u) cwin = window32(cw[1], cpos[1]);
          int r;
          if (cwin != 0u) {
            r = __builtin_ctz(cwin);
            cwin = (cwin >> r) >> 1;
            cpos[1] += (uint32_t)r + 1u;
          } else {
            r = unary_at(cw[1], cpos[1]);
            cwin = window32(cw[1], cpos[1]);
          }
          const uint32_t e = pv[r & 255];
          row[__builtin_ctz(pm) * dstride] =
              (uint16_t)(((byte >> 7) << 15) | (e << 7) | (byte & 0x7F));
        }
      }
      // every window this thread read lay inside its staged section
      CASS_DCHECK((fpos >> 5) + 1 < (uint32_t)cp.field && (lpos >> 5) + 1 < (uint32_t)cp.low &&
                      ((bpos * 8u) >> 5) + 1 < (uint32_t)cp.pbyte,
                  CASS_DBG_WINDOW);
      CASS_DCHECK(cfirst[j][0] < 0 || (cpos[0] >> 5) + 1 < (uint32_t)cp.scode, CASS_DBG_WINDOW);
      CASS_DCHECK(cfirst[j][1] < 0 || (cpos[1] >> 5) + 1 < (uint32_t)cp.pcode, CASS_DBG_WINDOW);
    }
  }
  __syncthreads();

  const int lane = tid & 63, wv = tid >> 6;
  const int rg = wv >> 2, cg = wv & 3;  // 16-row group, 16-column group (tokens, then dims)
  const int i16 = lane & 15, kq = lane >> 4;
  // 3. scores: lane (i16, kq) feeds query row / token i16 of its group and
  // dimensions 8kq..8kq+7 of each 32-dimension step
  {
    const int r = rg * 16 + i16;
    const uint16_t* qrow = nullptr;
    if (r < rows) {
      const int qi = r / a.G, g = r % a.G;
      qrow = a.q + ((int64_t)qi * a.Hq + h * a.G + g) * kDim;
    }
    const uint32_t* krow = reinterpret_cast<const uint32_t*>(kt + (cg * 16 + i16) * kXStride);
    xv4f acc = xv4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kDim / 32; ++ks) {
      xv8s aop = xv8s{0, 0, 0, 0, 0, 0, 0, 0};
      if (qrow) {
        const uint16_t* qp = qrow + ks * 32 + 8 * kq;
        aop = xv8s{(short)qp[0], (short)qp[1], (short)qp[2], (short)qp[3],
                   (short)qp[4], (short)qp[5], (short)qp[6], (short)qp[7]};
      }
      const uint32_t* kp = krow + ks * 16 + 4 * kq;
      const uint32_t b0 = kp[0], b1 = kp[1], b2 = kp[2], b3 = kp[3];
      const xv8s bop = xv8s{(short)(b0 & 0xFFFF), (short)(b0 >> 16), (short)(b1 & 0xFFFF),
                            (short)(b1 >> 16), (short)(b2 & 0xFFFF), (short)(b2 >> 16),
                            (short)(b3 & 0xFFFF), (short)(b3 >> 16)};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(xv8bf, aop),
                                                    __builtin_bit_cast(xv8bf, bop), acc, 0, 0, 0);
    }
    // D: this lane holds rows rg*16 + 4kq + e, token cg*16 + i16
    const int64_t tok = t0 + cg * 16 + i16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int rr = rg * 16 + 4 * kq + e;
      if (rr < rows) {
        const int qi = rr / a.G;
        const bool vis = tok < t1 && tok < a.T - a.nq + qi + 1;
        sc[rr * kXChunk + cg * 16 + i16] = vis ? acc[e] * a.scale : -INFINITY;
      }
    }
  }
  __syncthreads();

  // 4a. softmax per row: 32 threads per row, 4 tokens each
  {
    constexpr int TPR = kXChunk / 4;  // threads per row, 4 tokens each (a row in one wave)
    const int r = tid / TPR, q = tid % TPR;
    if (r < rows) {
      float* srow = sc + r * kXChunk;
      float v0 = srow[q], v1 = srow[q + TPR], v2 = srow[q + 2 * TPR], v3 = srow[q + 3 * TPR];
      float mx = fmaxf(fmaxf(v0, v1), fmaxf(v2, v3));
#pragma unroll
      for (int o = TPR / 2; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      const bool none = mx == -INFINITY;
      v0 = none || v0 == -INFINITY ? 0.f : __expf(v0 - mx);
      v1 = none || v1 == -INFINITY ? 0.f : __expf(v1 - mx);
      v2 = none || v2 == -INFINITY ? 0.f : __expf(v2 - mx);
      v3 = none || v3 == -INFINITY ? 0.f : __expf(v3 - mx);
      // p as two bf16 terms (hi, then lo = p - hi), over the row's scores: a
      // row's 32 threads are in one wave, so every read above comes first
      uint16_t* ph = reinterpret_cast<uint16_t*>(srow);
      const float pv4[4] = {v0, v1, v2, v3};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t hb = x1_bf16_rne(pv4[i]);
        ph[q + TPR * i] = (uint16_t)hb;
        ph[kXChunk + q + TPR * i] = (uint16_t)x1_bf16_rne(pv4[i] - __uint_as_float(hb << 16));
      }
      float l = (v0 + v1) + (v2 + v3);
#pragma unroll
      for (int o = TPR / 2; o >= 1; o >>= 1) l += __shfl_xor(l, o, 64);
      if (q == 0) {
        rmax[r] = mx;
        rsum[r] = l;
      }
    }
  }
  __syncthreads();
  // 4b. o = p V: lane (i16, kq) feeds row i16 of p and column i16 of V (dims of
  // its group), tokens 8kq..8kq+7 of each 32-token step; p = hi + lo in bf16.
  // A wave takes its row group and two of the eight 16-dimension groups.
  {
    const int r = rg * 16 + i16;
    const uint16_t* ph = reinterpret_cast<const uint16_t*>(sc + r * kXChunk);
    const xv8s zero = xv8s{0, 0, 0, 0, 0, 0, 0, 0};
    xv8s ahi[kXChunk / 32], alo[kXChunk / 32];
#pragma unroll
    for (int ks = 0; ks < kXChunk / 32; ++ks) {
      const int tb = ks * 32 + 8 * kq;
      ahi[ks] = r < rows ? *reinterpret_cast<const xv8s*>(ph + tb) : zero;
      alo[ks] = r < rows ? *reinterpret_cast<const xv8s*>(ph + kXChunk + tb) : zero;
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int dcol = (cg + 4 * half) * 16 + i16;
      const uint16_t* vcol = vt + dcol * kXVStride;
      xv4f acc = xv4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kXChunk / 32; ++ks) {
        const xv8s bop = *reinterpret_cast<const xv8s*>(vcol + ks * 32 + 8 * kq);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(xv8bf, ahi[ks]),
                                                      __builtin_bit_cast(xv8bf, bop), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(xv8bf, alo[ks]),
                                                      __builtin_bit_cast(xv8bf, bop), acc, 0, 0, 0);
      }
      // D: this lane holds rows rg*16 + 4kq + e, dimension dcol
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rr = rg * 16 + 4 * kq + e;
        if (rr < rows) {
          a.part[(((int64_t)h * a.nchunks + c) * rows + rr) * kDim + dcol] = acc[e];
          if (dcol == 0) {
            float* ml = a.ml + (((int64_t)h * rows + rr) * a.nchunks + c) * 2;
            ml[0] = rmax[rr];
            ml[1] = rsum[rr];
          }
        }
      }
    }
  }
}

int64_t aln256(int64_t v) { return (v + 255) / 256 * 256; }
int64_t part_at(int64_t* pos, int64_t bytes) {
  const int64_t o = *pos;
  *pos = aln256(*pos + bytes + 16);
  return o;
}

int fmt_of(const cass_kv_params* p) {
  return p->format == 0 ? CASS_FMT_C1_UNARY : p->format;
}

int check_kv_params(const cass_kv_params* p) {
  if (!p) return report(CASS_ERR_INVALID, "kv params is NULL");
  if (p->n_kv_heads < 1 || p->n_kv_heads > 64 || p->head_dim < 32 || p->head_dim > 256 ||
      p->head_dim % 32 || p->keep < 0 || p->keep > p->head_dim || p->mant_bits < 0 ||
      p->mant_bits > 7 || p->max_tokens < 0 || p->code_cap_bits < 0 || p->vcode_cap_bits < 0 ||
      p->code_cap_bits >= ((int64_t)1 << 32) || p->vcode_cap_bits >= ((int64_t)1 << 32))
    return report(CASS_ERR_INVALID, "bad kv params");
  if (fmt_of(p) != CASS_FMT_C1_UNARY && fmt_of(p) != CASS_FMT_C2_MX32)
    return report(CASS_ERR_INVALID, "bad kv format %d", p->format);
  return CASS_OK;
}
void kv_layout(const cass_kv_params* p, int64_t* so, int64_t* vo, int64_t* sb, int64_t* vb) {
  const int64_t D = p->head_dim, k = p->keep, m = p->mant_bits, T = p->max_tokens;
  const bool c1 = fmt_of(p) == CASS_FMT_C1_UNARY;
  int64_t pos = 0;
  so[0] = part_at(&pos, 256);
  so[1] = part_at(&pos, T * D / 8);
  if (c1) {
    so[2] = part_at(&pos, 4 * T);
    so[3] = part_at(&pos, (T * k * (1 + m) + 7) / 8);
    so[4] = part_at(&pos, (p->code_cap_bits + 7) / 8);
  } else {
    so[2] = part_at(&pos, T * D / 32);
    so[3] = part_at(&pos, (T * k * (2 + m) + 7) / 8);
    so[4] = part_at(&pos, 0);
  }
  *sb = pos;
  pos = 0;
  vo[0] = part_at(&pos, 256);
  vo[1] = c1 ? part_at(&pos, (T * k * (7 - m) + 7) / 8) : part_at(&pos, (p->code_cap_bits + 7) / 8);
  vo[2] = part_at(&pos, T * (D - k));
  vo[3] = part_at(&pos, (c1 ? 4 : 8) * T);
  vo[4] = part_at(&pos, (p->vcode_cap_bits + 7) / 8);
  *vb = pos;
}

KvDev dev_of(const cass_kv* kv) {
  KvDev d;
  d.spec = (uint8_t*)kv->spec;
  d.verif = (uint8_t*)kv->verif;
  d.state = (unsigned long long*)kv->state;
  d.sstride = kv->spec_stream_bytes;
  d.vstride = kv->verif_stream_bytes;
  for (int i = 0; i < 5; ++i) {
    d.so[i] = kv->spec_part[i];
    d.vo[i] = kv->verif_part[i];
  }
  d.H = kv->p.n_kv_heads;
  d.D = kv->p.head_dim;
  d.k = kv->p.keep;
  d.m = kv->p.mant_bits;
  d.T_max = kv->p.max_tokens;
  d.ccap = kv->p.code_cap_bits;
  d.vcap = kv->p.vcode_cap_bits;
  d.fmt = fmt_of(&kv->p);
  return d;
}

int check_kv(const cass_kv* kv) {
  if (!kv) return report(CASS_ERR_INVALID, "kv is NULL");
  int st = check_kv_params(&kv->p);
  if (st) return st;
  if (!kv->spec || !kv->verif || !kv->state) return report(CASS_ERR_INVALID, "kv buffers missing");
  if (kv->tokens < 0 || kv->tokens > kv->p.max_tokens)
    return report(CASS_ERR_INVALID, "kv token count out of range");
  return CASS_OK;
}

int64_t append_ws_layout(const cass_kv* kv, int ntok, AppendWs* ws, uint8_t* base) {
  const int64_t nvec = (int64_t)ntok * 2 * kv->p.n_kv_heads;
  int64_t pos = 0;
  auto take = [&](int64_t bytes) {
    uint8_t* p = base ? base + pos : nullptr;
    pos = aln256(pos + (bytes > 0 ? bytes : 1));
    return p;
  };
  AppendWs w;
  w.bm = (uint32_t*)take(nvec * (kv->p.head_dim / 32) * 4);
  w.lens = (uint32_t*)take(nvec * 2 * 4);
  w.start = (uint32_t*)take(nvec * 2 * 4);
  w.hist = (uint32_t*)take((int64_t)2 * kv->p.n_kv_heads * 512 * 4);
  if (ws) *ws = w;
  return pos;
}

// Chunk partials of one attention call in chunks of `chunk` tokens; the
// public size is that of the smaller chunks (the verification kernel's 64).
int64_t attn_ws(const cass_kv* kv, int nq, int G, int chunk = kXChunk) {
  const int64_t nchunks = (kv->tokens + chunk - 1) / chunk;
  return (int64_t)kv->p.n_kv_heads * nchunks * nq * G * (2 + kDim) * 4;
}

unsigned grid_of(int64_t n, int per) {
  int64_t g = (n + per - 1) / per;
  return (unsigned)(g < 1 ? 1 : g);
}

template <bool EXACT, int MAXR, int FMT>
hipError_t attn_launch_f(const KvDev& d, const AttnArgs& a, int H, size_t, hipStream_t stream) {
  const size_t lds = (size_t)MAXR * kDim * 4 + (size_t)MAXR * kChunk * 4 +
                     (size_t)vt_elems(!EXACT && MAXR == 4) * 2 +
                     (EXACT ? 0 : (size_t)2 * staged_words(a.fcap, a.ccap, FMT) * 4);
  hipError_t e = hipFuncSetAttribute((const void*)&k_kv_attn<EXACT, MAXR, FMT>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  k_kv_attn<EXACT, MAXR, FMT><<<dim3(H, a.nchunks), 2 * kChunk, lds, stream>>>(d, a);
  return hipGetLastError();
}

template <bool EXACT, int MAXR>
hipError_t attn_launch(const KvDev& d, const AttnArgs& a, int H, size_t lds, hipStream_t stream) {
  return d.fmt == CASS_FMT_C1_UNARY ? attn_launch_f<EXACT, MAXR, CASS_FMT_C1_UNARY>(d, a, H, lds, stream)
                                    : attn_launch_f<EXACT, MAXR, CASS_FMT_C2_MX32>(d, a, H, lds, stream);
}

int run_attention(const cass_kv* kv, const uint16_t* q, int nq, int n_q_heads, float scale,
                  float* out, void* ws, int64_t ws_bytes, hipStream_t stream, bool exact) {
  int st = check_kv(kv);
  if (st) return st;
  const int H = kv->p.n_kv_heads;
  if (kv->p.head_dim != kDim) return report(CASS_ERR_UNSUPPORTED, "attention needs head_dim 128");
  if (n_q_heads < H || n_q_heads % H) return report(CASS_ERR_INVALID, "n_q_heads must be a multiple of n_kv_heads");
  const int G = n_q_heads / H;
  if (nq < 1 || nq * G > kMaxRows) return report(CASS_ERR_UNSUPPORTED, "nq * heads per group > 32");
  if (kv->tokens < nq) return report(CASS_ERR_INVALID, "cache holds fewer tokens than queries");
  if (!q || !out) return report(CASS_ERR_INVALID, "q or out is NULL");
  const bool x1 = exact && fmt_of(&kv->p) == CASS_FMT_C1_UNARY && option(OPT_KV_EXACT_PATH) != 1;
  const int64_t need = attn_ws(kv, nq, G, x1 ? kXChunk : kChunk);
  if (!ws || ws_bytes < need) return report(CASS_ERR_CAPACITY, "attention workspace too small");
  AttnArgs a;
  a.q = q;
  a.nq = nq;
  a.Hq = n_q_heads;
  a.G = G;
  a.scale = scale;
  a.T = kv->tokens;
  a.nchunks = (int)((kv->tokens + kChunk - 1) / kChunk);
  if ((kv->tokens + kXChunk - 1) / kXChunk > kMaxChunksMerge)
    return report(CASS_ERR_UNSUPPORTED, "attention over more than 512K tokens");
  a.part = (float*)ws;
  a.ml = a.part + (int64_t)H * a.nchunks * (nq * G) * kDim;
  {
    // draft staging: every field of the chunk, and codes averaging up to 4
    // bits per kept value (longer runs read their codes from global memory)
    const int fwid = fmt_of(&kv->p) == CASS_FMT_C1_UNARY ? 1 + kv->p.mant_bits : 2 + kv->p.mant_bits;
    // (multiples of 4 words: the staged regions stay 16-byte aligned)
    a.fcap = (int)(((int64_t)kChunk * kv->p.keep * fwid + 31) / 32 + 8 + 3) / 4 * 4;
    // (3 bits per kept value: the staged code run; a token whose codes run
    // past it reads them in place)
    a.ccap = (int)(((int64_t)kChunk * kv->p.keep * 3 / 32 + 64 + 3) / 4 * 4);
  }
  const KvDev d = dev_of(kv);
  const size_t lds = 0;  // per launch, from the row bound (attn_launch_f)
  const int rows = nq * G;
  if (x1) {
    // split decode and matrix-core scores; staged code space averaging up to
    // 4 bits per value (longer runs are read in place)
    const int64_t kk = kv->p.keep, mm = kv->p.mant_bits;
    AttnArgs ax = a;
    ax.nchunks = (int)((kv->tokens + kXChunk - 1) / kXChunk);
    ax.ml = ax.part + (int64_t)H * ax.nchunks * (nq * G) * kDim;
    XCaps cp;
    // (regions in whole 16-byte chunks; 8 words beyond what a run may take,
    // which covers a copy that starts up to 3 words early and a chunk's tail)
    auto r4 = [](int64_t w) { return (int)((w + 3) / 4 * 4); };
    cp.scode = r4((kXChunk * kk * 4 + 31) / 32 + 64 + 8);
    cp.pcode = r4((kXChunk * (kDim - kk) * 4 + 31) / 32 + 64 + 8);
    cp.field = r4((kXChunk * kk * (1 + mm) + 31) / 32 + 8 + 8);  // (a run may start mid-word)
    cp.low = r4((kXChunk * kk * (7 - mm) + 31) / 32 + 8 + 8);
    cp.pbyte = r4((kXChunk * (kDim - kk) + 3) / 4 + 8 + 8);
    const int64_t xl = x1_lds_bytes(cp);
    hipError_t e = hipFuncSetAttribute((const void*)&k_kv_attn_x1,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)xl);
    if (e == hipSuccess) {
      k_kv_attn_x1<<<dim3(H, ax.nchunks), kXThreads, (size_t)xl, stream>>>(d, ax, cp);
      e = hipGetLastError();
    }
    if (e != hipSuccess) return report(CASS_ERR_HIP, "attention: %s", hipGetErrorString(e));
    k_kv_merge<<<H * nq * G * kMergeSplit, kMergeThreads, 0, stream>>>(ax, H, out);
    if ((e = hipGetLastError()) != hipSuccess) return report(CASS_ERR_HIP, "merge: %s", hipGetErrorString(e));
    return CASS_OK;
  }
  // row bounds: one query of 4 heads (draft), 5 queries of 4 heads (verify), ...
  // (the 20-row instance of the exact Cassandra-2 kernel gave results that
  // changed from run to run in workgroups sharing a CU with another one, and
  // the cause is not known; that case takes the 32-row instance, which is
  // checked for identical results over repeated runs)
  const bool r20 = rows <= 20 && !(exact && d.fmt == CASS_FMT_C2_MX32);
  hipError_t e = exact ? (rows <= 4    ? attn_launch<true, 4>(d, a, H, lds, stream)
                          : rows <= 8  ? attn_launch<true, 8>(d, a, H, lds, stream)
                          : rows <= 16 ? attn_launch<true, 16>(d, a, H, lds, stream)
                          : r20        ? attn_launch<true, 20>(d, a, H, lds, stream)
                                       : attn_launch<true, 32>(d, a, H, lds, stream))
                       : (rows <= 4    ? attn_launch<false, 4>(d, a, H, lds, stream)
                          : rows <= 8  ? attn_launch<false, 8>(d, a, H, lds, stream)
                          : rows <= 16 ? attn_launch<false, 16>(d, a, H, lds, stream)
                          : rows <= 20 ? attn_launch<false, 20>(d, a, H, lds, stream)
                                       : attn_launch<false, 32>(d, a, H, lds, stream));
  if (e != hipSuccess) return report(CASS_ERR_HIP, "attention: %s", hipGetErrorString(e));
  k_kv_merge<<<H * nq * G * kMergeSplit, kMergeThreads, 0, stream>>>(a, H, out);
  if ((e = hipGetLastError()) != hipSuccess) return report(CASS_ERR_HIP, "merge: %s", hipGetErrorString(e));
  return CASS_OK;
}

// Fixed scratch of the allocation-free draft attention: the per-chunk
// partials live in this array instead of a caller workspace.  Each device the
// library runs on holds its own copy until the process ends; host code uses
// the address hipGetSymbolAddress returns for the current device, never the
// array's name (which on the host is only a stand-in).
constexpr int64_t kStaticScratchBytes = CASS_KV_STATIC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch (looked up once per device).
int static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return report(CASS_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return report(CASS_ERR_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return report(CASS_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return CASS_OK;
}

}  // namespace

}  // namespace cass

using namespace cass;

extern "C" {

int cass_kv_bytes(const cass_kv_params* p, int64_t* spec_bytes, int64_t* verif_bytes,
                  int64_t* state_bytes) {
  clear_error();
  int st = check_kv_params(p);
  if (st) return st;
  int64_t so[5], vo[5], sb, vb;
  kv_layout(p, so, vo, &sb, &vb);
  if (spec_bytes) *spec_bytes = sb * 2 * p->n_kv_heads;
  if (verif_bytes) *verif_bytes = vb * 2 * p->n_kv_heads;
  if (state_bytes) *state_bytes = CASS_KV_STATE_BYTES;
  return CASS_OK;
}

int cass_kv_init(cass_kv* kv, const cass_kv_params* p, void* spec, void* verif, void* state,
                 hipStream_t stream) {
  clear_error();
  int st = check_kv_params(p);
  if (st) return st;
  if (!kv || !spec || !verif || !state) return report(CASS_ERR_INVALID, "NULL argument");
  if (((uintptr_t)spec | (uintptr_t)verif | (uintptr_t)state) % 256)
    return report(CASS_ERR_INVALID, "kv buffers must be 256-byte aligned");
  memset(kv, 0, sizeof *kv);
  kv->p = *p;
  kv->spec = spec;
  kv->verif = verif;
  kv->state = state;
  kv_layout(p, kv->spec_part, kv->verif_part, &kv->spec_stream_bytes, &kv->verif_stream_bytes);
  kv->tokens = 0;
  hipError_t e;
  if ((e = launch_fill_zero(spec, kv->spec_stream_bytes * 2 * p->n_kv_heads, stream)) != hipSuccess ||
      (e = launch_fill_zero(verif, kv->verif_stream_bytes * 2 * p->n_kv_heads, stream)) != hipSuccess ||
      (e = launch_fill_zero(state, CASS_KV_STATE_BYTES, stream)) != hipSuccess)
    return report(CASS_ERR_HIP, "kv init: %s", hipGetErrorString(e));
  return CASS_OK;
}

int cass_kv_append_ws_bytes(const cass_kv* kv, int ntok, int64_t* ws_bytes) {
  clear_error();
  int st = check_kv(kv);
  if (st) return st;
  if (ntok < 0 || !ws_bytes) return report(CASS_ERR_INVALID, "bad ntok or ws_bytes");
  *ws_bytes = append_ws_layout(kv, ntok, nullptr, nullptr);
  return CASS_OK;
}

int cass_kv_append_encode(cass_kv* kv, const uint16_t* k, const uint16_t* v, int ntok, void* ws,
                          int64_t ws_bytes, hipStream_t stream) {
  clear_error();
  int st = check_kv(kv);
  if (st) return st;
  if (ntok < 0) return report(CASS_ERR_INVALID, "ntok < 0");
  if (ntok == 0) return CASS_OK;
  if (!k || !v) return report(CASS_ERR_INVALID, "k or v is NULL");
  if (kv->tokens + ntok > kv->p.max_tokens) return report(CASS_ERR_CAPACITY, "cache full");
  const int64_t need = append_ws_layout(kv, ntok, nullptr, nullptr);
  if (!ws || ws_bytes < need) return report(CASS_ERR_CAPACITY, "append workspace too small");
  AppendWs w;
  append_ws_layout(kv, ntok, &w, (uint8_t*)ws);
  const KvDev d = dev_of(kv);
  const int first = kv->tokens == 0;
  const int64_t nvec = (int64_t)ntok * 2 * kv->p.n_kv_heads;
  hipError_t e;
  if (!first && ntok <= kFusedMaxTokens && option(OPT_KV_APPEND_PATH) != 1) {
    // a decoding step's few tokens: one launch, one wave per stream
    // one wave per token: selections, lengths and packing side by side
    k_kv_append_few<<<2 * kv->p.n_kv_heads, 64 * ntok, 0, stream>>>(d, k, v, ntok, kv->tokens, w);
    if ((e = hipGetLastError()) != hipSuccess) return report(CASS_ERR_HIP, "append: %s", hipGetErrorString(e));
    kv->tokens += ntok;
    return CASS_OK;
  }
  if (first && (e = launch_fill_zero(w.hist, (int64_t)2 * kv->p.n_kv_heads * 512 * 4, stream)) != hipSuccess)
    return report(CASS_ERR_HIP, "append: %s", hipGetErrorString(e));
  k_kv_select<<<grid_of(nvec, kWaves), 64 * kWaves, 0, stream>>>(d, k, v, ntok, first, w);
  if (first) k_kv_ranks<<<2 * kv->p.n_kv_heads, 256, 0, stream>>>(d, w);
  k_kv_lengths<<<grid_of(nvec, kWaves), 64 * kWaves, 0, stream>>>(d, k, v, ntok, w);
  k_kv_scan<<<2 * kv->p.n_kv_heads, 256, 0, stream>>>(d, ntok, kv->tokens, w);
  k_kv_pack<<<grid_of(nvec, kWaves), 64 * kWaves, 0, stream>>>(d, k, v, ntok, kv->tokens, w);
  if ((e = hipGetLastError()) != hipSuccess) return report(CASS_ERR_HIP, "append: %s", hipGetErrorString(e));
  kv->tokens += ntok;
  return CASS_OK;
}

int cass_kv_truncate(cass_kv* kv, int64_t tokens, hipStream_t stream) {
  clear_error();
  int st = check_kv(kv);
  if (st) return st;
  if (tokens < 0 || tokens > kv->tokens) return report(CASS_ERR_INVALID, "truncate to %lld of %lld tokens",
                                                       (long long)tokens, (long long)kv->tokens);
  if (tokens == kv->tokens) return CASS_OK;
  k_kv_truncate<<<2 * kv->p.n_kv_heads, 256, 0, stream>>>(dev_of(kv), tokens, kv->tokens);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return report(CASS_ERR_HIP, "truncate: %s", hipGetErrorString(e));
  kv->tokens = tokens;
  return CASS_OK;
}

int cass_kv_status(const cass_kv* kv, int64_t* tokens, uint32_t* flags, hipStream_t stream) {
  clear_error();
  int st = check_kv(kv);
  if (st) return st;
  unsigned long long h[2];
  hipError_t e = hipMemcpyAsync(h, kv->state, sizeof h, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return report(CASS_ERR_HIP, "kv status: %s", hipGetErrorString(e));
  if (tokens) *tokens = (int64_t)h[0];
  if (flags) *flags = (uint32_t)h[1];
  return CASS_OK;
}

int cass_kv_decode(const cass_kv* kv, int exact, uint16_t* out, hipStream_t stream) {
  clear_error();
  int st = check_kv(kv);
  if (st) return st;
  if (kv->tokens == 0) return CASS_OK;
  if (!out) return report(CASS_ERR_INVALID, "out is NULL");
  const KvDev d = dev_of(kv);
  const int64_t n = (int64_t)2 * kv->p.n_kv_heads * kv->tokens;
  unsigned g = grid_of(n, 256);
  if (g > 65535u * 4) g = 65535u * 4;
  if (d.fmt == CASS_FMT_C1_UNARY) {
    if (exact) k_kv_decode<true, CASS_FMT_C1_UNARY><<<g, 256, 0, stream>>>(d, kv->tokens, out);
    else k_kv_decode<false, CASS_FMT_C1_UNARY><<<g, 256, 0, stream>>>(d, kv->tokens, out);
  } else {
    if (exact) k_kv_decode<true, CASS_FMT_C2_MX32><<<g, 256, 0, stream>>>(d, kv->tokens, out);
    else k_kv_decode<false, CASS_FMT_C2_MX32><<<g, 256, 0, stream>>>(d, kv->tokens, out);
  }
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? CASS_OK : report(CASS_ERR_HIP, "kv decode: %s", hipGetErrorString(e));
}

int cass_kv_attn_ws_bytes(const cass_kv* kv, int nq, int n_q_heads, int64_t* ws_bytes) {
  clear_error();
  int st = check_kv(kv);
  if (st) return st;
  if (nq < 1 || n_q_heads < kv->p.n_kv_heads || n_q_heads % kv->p.n_kv_heads || !ws_bytes)
    return report(CASS_ERR_INVALID, "bad attention shape");
  *ws_bytes = attn_ws(kv, nq, n_q_heads / kv->p.n_kv_heads);
  return CASS_OK;
}

int cass_kv_draft_attn(const cass_kv* kv, const uint16_t* q, int n_q_heads, float scale, float* out,
                       void* ws, int64_t ws_bytes, hipStream_t stream) {
  clear_error();
  return run_attention(kv, q, 1, n_q_heads, scale, out, ws, ws_bytes, stream, false);
}

int cass_kv_draft_attn_static(const cass_kv* kv, const uint16_t* q, int n_q_heads, float scale,
                              float* out, hipStream_t stream) {
  clear_error();
  int st = check_kv(kv);
  if (st) return st;
  if (n_q_heads < kv->p.n_kv_heads || n_q_heads % kv->p.n_kv_heads)
    return report(CASS_ERR_INVALID, "n_q_heads must be a multiple of n_kv_heads");
  const int64_t need = attn_ws(kv, 1, n_q_heads / kv->p.n_kv_heads, kChunk);
  if (need > kStaticScratchBytes)
    return report(CASS_ERR_CAPACITY, "draft attention needs %lld scratch bytes, the fixed scratch holds %lld",
                  (long long)need, (long long)kStaticScratchBytes);
  void* ws = nullptr;
  if ((st = static_scratch(&ws))) return st;
  return run_attention(kv, q, 1, n_q_heads, scale, out, ws, kStaticScratchBytes, stream, false);
}

int cass_kv_verify_attn(const cass_kv* kv, const uint16_t* q, int nq, int n_q_heads, float scale,
                        float* out, void* ws, int64_t ws_bytes, hipStream_t stream) {
  clear_error();
  if (nq > 8) return report(CASS_ERR_UNSUPPORTED, "nq > 8");
  return run_attention(kv, q, nq, n_q_heads, scale, out, ws, ws_bytes, stream, true);
}

}  // extern "C"
