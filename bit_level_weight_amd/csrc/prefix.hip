// Comparison exponent codecs: a length-limited canonical Huffman code and
// Cassandra-1's frequency-ranked unary code, both as prefix codes over the
// same exponent sequence, with three decoders.
//
// Method: Cassandra review (marsggbo.github.io), section 3.2 -- the unary code
// is chosen over Huffman coding although Huffman codes come out a little
// shorter, because a Huffman stream has to be parsed serially (bit by bit or
// through a table of 2^N entries, N the longest code) while unary codes can be
// decoded in parallel.  The decoders here put a number on that trade:
//   table    one thread per block of symbols, a 2^N-entry table in LDS (any
//            prefix code with N <= 12);
//   serial   one thread per block, count-trailing-zeros (unary code only);
//   parallel no block offsets at all: every 32-bit word of a unary stream is
//            decoded on its own, the symbol index of each code from a prefix
//            count of one-bits and its length from the previous one-bit.
#include <string.h>

#include <algorithm>
#include <vector>

#include "bits.hpp"
#include "internal.hpp"

namespace cass {

namespace {

constexpr int kMaxTableBits = 12;
constexpr int kPcThreads = 256;

struct CodeTable {
  uint32_t rev[256];  // code bits in stream order (first bit in bit 0)
  uint8_t len[256];
};

struct PermTable {
  uint8_t sym[256];  // unary code: symbol of rank r
};

// Bit reader that never loads past word `lim` of its section (reads there
// give zeros): a stream that ends early or holds garbage cannot make a
// decoder read outside the caller's buffer.
struct LimitedReader {
  const uint32_t* base;
  int64_t next, lim;  // next word to load; words in the buffer
  uint64_t buf;
  int n;              // valid bits in buf
  __device__ __forceinline__ uint32_t load() {
    const uint32_t v = next < lim ? base[next] : 0u;
    ++next;
    return v;
  }
  __device__ __forceinline__ void init(const uint32_t* b, int64_t words, uint64_t pos) {
    base = b;
    lim = words;
    next = (int64_t)(pos >> 5);
    const int sft = (int)(pos & 31);
    const uint32_t w0 = load(), w1 = load();
    buf = ((uint64_t)w1 << 32 | w0) >> sft;
    n = 64 - sft;
    refill();
  }
  __device__ __forceinline__ void refill() {
    if (n <= 32) {
      buf |= (uint64_t)load() << n;
      n += 32;
    }
  }
  __device__ __forceinline__ void skip(int width) {  // width in 0..32
    buf >>= width;
    n -= width;
    refill();
  }
};

CodeTable table_of(const cass_prefix_code* c) {
  CodeTable t = {};
  for (int s = 0; s < 256; ++s) {
    const int l = c->len[s];
    uint32_t r = 0;
    for (int j = 0; j < l; ++j) r |= ((c->code[s] >> (l - 1 - j)) & 1u) << j;
    t.rev[s] = r;
    t.len[s] = (uint8_t)l;
  }
  return t;
}

// ---- encoder: per-block code bits, their exclusive scan, packing ----
__global__ void __launch_bounds__(kPcThreads) k_pc_block_bits(const uint8_t* __restrict__ sym,
                                                              int64_t n, int64_t block,
                                                              CodeTable t,
                                                              uint32_t* __restrict__ bits) {
  const int64_t nblk = (n + block - 1) / block;
  for (int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; b < nblk;
       b += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i1 = (b + 1) * block < n ? (b + 1) * block : n;
    uint32_t acc = 0;
    for (int64_t i = b * block; i < i1; ++i) acc += t.len[sym[i]];
    bits[b] = acc;
  }
}

// One workgroup: exclusive scan of v[0..n) in place (u32; the host checks the
// total fits).
__global__ void __launch_bounds__(1024) k_pc_scan(uint32_t* v, int64_t n) {
  __shared__ uint32_t tmp[1024];
  __shared__ uint32_t carry_s;
  const int t = threadIdx.x;
  if (t == 0) carry_s = 0;
  __syncthreads();
  for (int64_t c0 = 0; c0 < n; c0 += 1024) {
    const int64_t i = c0 + t;
    const uint32_t x = i < n ? v[i] : 0u;
    tmp[t] = x;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
      const uint32_t add = t >= d ? tmp[t - d] : 0u;
      __syncthreads();
      tmp[t] += add;
      __syncthreads();
    }
    const uint32_t carry = carry_s;
    if (i < n) v[i] = carry + tmp[t] - x;
    __syncthreads();
    if (t == 1023) carry_s = carry + tmp[1023];
    __syncthreads();
  }
}

// Blocks whose codes would pass cap_bits (a stream sized too small) are not
// written, so the writes stay inside the caller's buffer.
__global__ void __launch_bounds__(kPcThreads) k_pc_pack(const uint8_t* __restrict__ sym, int64_t n,
                                                        int64_t block, CodeTable t,
                                                        const uint32_t* __restrict__ blkoff,
                                                        uint32_t* __restrict__ stream,
                                                        uint64_t cap_bits) {
  const int64_t nblk = (n + block - 1) / block;
  for (int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; b < nblk;
       b += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i1 = (b + 1) * block < n ? (b + 1) * block : n;
    uint64_t bits = 0;
    for (int64_t i = b * block; i < i1; ++i) bits += t.len[sym[i]];
    if ((uint64_t)blkoff[b] + bits > cap_bits) continue;
    BitWriter bw;
    bw.init(stream, blkoff[b]);
    for (int64_t i = b * block; i < i1; ++i) {
      const int s = sym[i];
      bw.put(t.rev[s], t.len[s]);
    }
    bw.finish();
  }
}

// ---- decoders writing 16 symbols at a time ----
struct Out16 {
  uint32_t w[4];
  int k;
  __device__ __forceinline__ void reset() { w[0] = w[1] = w[2] = w[3] = 0u; k = 0; }
  __device__ __forceinline__ void push(uint32_t s, uint8_t* out, int64_t base) {
    w[k >> 2] |= s << (8 * (k & 3));
    if (++k == 16) {
      *reinterpret_cast<uint4*>(out + base) = make_uint4(w[0], w[1], w[2], w[3]);
      reset();
    }
  }
};

// table: entry (len << 8) | symbol for every kMaxTableBits-bit window whose
// first len bits are that symbol's code
__global__ void __launch_bounds__(kPcThreads) k_pc_decode_table(const uint32_t* __restrict__ stream,
                                                                int64_t words,
                                                                const uint32_t* __restrict__ blkoff,
                                                                int64_t n, int64_t block, CodeTable t,
                                                                int nbits, uint8_t* __restrict__ out) {
  __shared__ uint16_t lut[1 << kMaxTableBits];
  const int size = 1 << nbits;
  for (int i = threadIdx.x; i < size; i += blockDim.x) lut[i] = 0;
  __syncthreads();
  for (int s = 0; s < 256; ++s) {
    const int l = t.len[s];
    if (l == 0) continue;
    for (int hi = threadIdx.x; hi < (size >> l); hi += blockDim.x)
      lut[(hi << l) | t.rev[s]] = (uint16_t)((l << 8) | s);
  }
  __syncthreads();
  const int64_t nblk = (n + block - 1) / block;
  const uint32_t mask = (uint32_t)size - 1u;
  for (int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; b < nblk;
       b += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i0 = b * block, i1 = i0 + block < n ? i0 + block : n;
    LimitedReader br;
    br.init(stream, words, blkoff[b]);
    Out16 o;
    o.reset();
    for (int64_t i = i0; i < i1; ++i) {
      const uint32_t e = lut[(uint32_t)br.buf & mask];
      br.skip((int)(e >> 8));
      o.push(e & 0xFFu, out, i - 15);
    }
  }
}

// unary code: rank = trailing zeros, symbol = perm[rank]
__global__ void __launch_bounds__(kPcThreads) k_pc_decode_unary(const uint32_t* __restrict__ stream,
                                                                int64_t words,
                                                                const uint32_t* __restrict__ blkoff,
                                                                int64_t n, int64_t block,
                                                                PermTable pt,
                                                                uint8_t* __restrict__ out) {
  __shared__ uint8_t perm[256];
  for (int i = threadIdx.x; i < 256; i += blockDim.x) perm[i] = pt.sym[i];
  __syncthreads();
  const int64_t nblk = (n + block - 1) / block;
  for (int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; b < nblk;
       b += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i0 = b * block, i1 = i0 + block < n ? i0 + block : n;
    LimitedReader br;
    br.init(stream, words, blkoff[b]);
    Out16 o;
    o.reset();
    for (int64_t i = i0; i < i1; ++i) {
      // codes are at most 32 bits and the buffer holds at least 33
      const uint32_t lo = (uint32_t)br.buf;
      const int r = lo ? __builtin_ctz(lo) : 31;
      br.skip(r + 1);
      o.push(perm[r], out, i - 15);
    }
  }
}

// unary, no offsets: words per workgroup of the parallel decoder
constexpr int kWordsPerThread = 8;
constexpr int64_t kWordsPerGroup = (int64_t)kPcThreads * kWordsPerThread;

// pass 1: per workgroup, the one-bits and the position of the last one
__global__ void __launch_bounds__(kPcThreads) k_pc_group_ones(const uint32_t* __restrict__ stream,
                                                              int64_t nwords,
                                                              unsigned long long* __restrict__ cnt,
                                                              long long* __restrict__ last) {
  __shared__ unsigned long long sc[kPcThreads];
  __shared__ long long sl[kPcThreads];
  const int t = threadIdx.x;
  const int64_t w0 = (int64_t)blockIdx.x * kWordsPerGroup + (int64_t)t * kWordsPerThread;
  unsigned long long c = 0;
  long long l = -1;
  for (int j = 0; j < kWordsPerThread; ++j) {
    const int64_t wi = w0 + j;
    if (wi >= nwords) break;
    const uint32_t v = stream[wi];
    c += (unsigned)__builtin_popcount(v);
    if (v) l = wi * 32 + 31 - __builtin_clz(v);
  }
  sc[t] = c;
  sl[t] = l;
  __syncthreads();
  for (int d = kPcThreads / 2; d > 0; d >>= 1) {
    if (t < d) {
      sc[t] += sc[t + d];
      sl[t] = sl[t] > sl[t + d] ? sl[t] : sl[t + d];
    }
    __syncthreads();
  }
  if (t == 0) {
    cnt[blockIdx.x] = sc[0];
    last[blockIdx.x] = sl[0];
  }
}

// pass 2 (one workgroup): exclusive prefix of the counts and of the last-one
// positions (a running maximum) over the workgroups
__global__ void __launch_bounds__(1024) k_pc_group_scan(unsigned long long* cnt, long long* last,
                                                         int64_t ng) {
  __shared__ unsigned long long tc[1024];
  __shared__ long long tl[1024];
  __shared__ unsigned long long cc;
  __shared__ long long cl;
  const int t = threadIdx.x;
  if (t == 0) {
    cc = 0;
    cl = -1;
  }
  __syncthreads();
  for (int64_t c0 = 0; c0 < ng; c0 += 1024) {
    const int64_t i = c0 + t;
    const unsigned long long x = i < ng ? cnt[i] : 0ull;
    const long long y = i < ng ? last[i] : -1ll;
    tc[t] = x;
    tl[t] = y;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
      const unsigned long long ac = t >= d ? tc[t - d] : 0ull;
      const long long al = t >= d ? tl[t - d] : -1ll;
      __syncthreads();
      tc[t] += ac;
      tl[t] = tl[t] > al ? tl[t] : al;
      __syncthreads();
    }
    const unsigned long long base_c = cc;
    const long long base_l = cl;
    if (i < ng) {
      cnt[i] = base_c + tc[t] - x;                   // ones before group i
      const long long before = t > 0 ? tl[t - 1] : -1ll;
      last[i] = before > base_l ? before : base_l;   // last one before group i
    }
    __syncthreads();
    if (t == 1023) {
      cc = base_c + tc[1023];
      cl = tl[1023] > base_l ? tl[1023] : base_l;
    }
    __syncthreads();
  }
}

// pass 3: every one-bit ends a code; its index is the ones before it, its rank
// the distance to the previous one-bit minus one
__global__ void __launch_bounds__(kPcThreads) k_pc_decode_parallel(
    const uint32_t* __restrict__ stream, int64_t nwords, int64_t n,
    const unsigned long long* __restrict__ cnt, const long long* __restrict__ last,
    PermTable pt, uint8_t* __restrict__ out) {
  __shared__ uint8_t perm[256];
  __shared__ unsigned long long sc[kPcThreads];
  __shared__ long long sl[kPcThreads];
  const int t = threadIdx.x;
  for (int i = t; i < 256; i += blockDim.x) perm[i] = pt.sym[i];
  const int64_t w0 = (int64_t)blockIdx.x * kWordsPerGroup + (int64_t)t * kWordsPerThread;
  uint32_t v[kWordsPerThread];
  unsigned long long c = 0;
  long long l = -1;
  for (int j = 0; j < kWordsPerThread; ++j) {
    const int64_t wi = w0 + j;
    v[j] = wi < nwords ? stream[wi] : 0u;
    c += (unsigned)__builtin_popcount(v[j]);
    if (v[j]) l = wi * 32 + 31 - __builtin_clz(v[j]);
  }
  sc[t] = c;
  sl[t] = l;
  __syncthreads();
  for (int d = 1; d < kPcThreads; d <<= 1) {
    const unsigned long long ac = t >= d ? sc[t - d] : 0ull;
    const long long al = t >= d ? sl[t - d] : -1ll;
    __syncthreads();
    sc[t] += ac;
    sl[t] = sl[t] > al ? sl[t] : al;
    __syncthreads();
  }
  unsigned long long idx = cnt[blockIdx.x] + sc[t] - c;
  long long prev = t > 0 ? sl[t - 1] : -1ll;
  if (last[blockIdx.x] > prev) prev = last[blockIdx.x];
  for (int j = 0; j < kWordsPerThread; ++j) {
    for (uint32_t m = v[j]; m; m &= m - 1u) {
      const long long g = (w0 + j) * 32 + __builtin_ctz(m);
      const long long r = g - prev - 1;
      if ((long long)idx < n) out[idx] = perm[r > 255 ? 255 : r];
      ++idx;
      prev = g;
    }
  }
}

int64_t nblk_of(int64_t n, int64_t block) { return (n + block - 1) / block; }

unsigned grid_of_blocks(int64_t nblk) {
  int64_t g = (nblk + kPcThreads - 1) / kPcThreads;
  return (unsigned)(g < 1 ? 1 : g);
}

bool is_unary(const cass_prefix_code* c, uint8_t perm[256]) {
  // a unary code: every length 1..256 at most once, every value 1
  int seen[257] = {0};
  for (int s = 0; s < 256; ++s) {
    const int l = c->len[s];
    if (l == 0) continue;
    if (c->code[s] != 1u || seen[l]) return false;
    seen[l] = 1;
    perm[l - 1] = (uint8_t)s;
  }
  for (int l = 1; l <= 256; ++l)  // ranks 0..r all present
    if (!seen[l]) {
      for (int m = l + 1; m <= 256; ++m)
        if (seen[m]) return false;
      break;
    }
  return true;
}

int check_code(const cass_prefix_code* c) {
  if (!c) return report(CASS_ERR_INVALID, "code is NULL");
  int maxl = 0;
  double kraft = 0.0;
  for (int s = 0; s < 256; ++s) {
    const int l = c->len[s];
    if (l > 32) return report(CASS_ERR_INVALID, "code length %d > 32", l);
    if (l > 0 && l < 32 && (c->code[s] >> l) != 0u) return report(CASS_ERR_INVALID, "code value wider than its length");
    if (l > maxl) maxl = l;
    if (l) kraft += 1.0 / (double)(1ull << l);
  }
  if (kraft > 1.0 + 1e-12) return report(CASS_ERR_INVALID, "code lengths break Kraft's inequality");
  if (maxl != c->max_len) return report(CASS_ERR_INVALID, "max_len does not match the lengths");
  return CASS_OK;
}

// Package-merge, the coin-collector form: level lists hold leaves and pairs of
// the previous level's items in weight order (leaves first among equal
// weights, leaves by (count, symbol), pairs in the order formed); a leaf's code
// length is how often it occurs in the first 2n-2 items of the last level.
struct PmItem {
  uint64_t w;
  int leaf;  // >= 0: leaf index; -1: pair of items a, b of the previous level
  int a, b;
};

void count_leaf(const std::vector<std::vector<PmItem>>& lv, int level, int i, std::vector<int>& cnt) {
  const PmItem& it = lv[level][i];
  if (it.leaf >= 0) {
    ++cnt[it.leaf];
    return;
  }
  count_leaf(lv, level - 1, it.a, cnt);
  count_leaf(lv, level - 1, it.b, cnt);
}

}  // namespace

}  // namespace cass

using namespace cass;

extern "C" {

int cass_prefix_code_huffman(const uint64_t* hist, int max_len, cass_prefix_code* out) {
  clear_error();
  if (!hist || !out) return report(CASS_ERR_INVALID, "NULL argument");
  if (max_len < 1 || max_len > 32) return report(CASS_ERR_INVALID, "max_len %d outside 1..32", max_len);
  memset(out, 0, sizeof *out);
  std::vector<int> syms;
  for (int s = 0; s < 256; ++s)
    if (hist[s]) syms.push_back(s);
  const int n = (int)syms.size();
  if (n == 1) {
    out->len[syms[0]] = 1;
    out->max_len = 1;
  }
  if (n >= 2) {
    if (max_len < 32 && (1ll << max_len) < n)
      return report(CASS_ERR_INVALID, "%d symbols need codes longer than %d bits", n, max_len);
    std::stable_sort(syms.begin(), syms.end(), [&](int a, int b) { return hist[a] < hist[b]; });
    // levels[0] is the deepest (leaves only); levels[max_len-1] the last
    std::vector<std::vector<PmItem>> levels(max_len);
    for (int i = 0; i < n; ++i) levels[0].push_back(PmItem{hist[syms[i]], i, 0, 0});
    for (int d = 1; d < max_len; ++d) {
      const std::vector<PmItem>& prev = levels[d - 1];
      const int npairs = (int)prev.size() / 2;
      std::vector<PmItem>& cur = levels[d];
      int li = 0, pi = 0;
      while (li < n || pi < npairs) {
        const uint64_t pw = pi < npairs ? prev[2 * pi].w + prev[2 * pi + 1].w : 0;
        if (li < n && (pi >= npairs || hist[syms[li]] <= pw)) {
          cur.push_back(PmItem{hist[syms[li]], li, 0, 0});
          ++li;
        } else {
          cur.push_back(PmItem{pw, -1, 2 * pi, 2 * pi + 1});
          ++pi;
        }
      }
    }
    std::vector<int> cnt(n, 0);
    const int top = max_len - 1;
    for (int i = 0; i < 2 * n - 2 && i < (int)levels[top].size(); ++i) count_leaf(levels, top, i, cnt);
    for (int i = 0; i < n; ++i) {
      out->len[syms[i]] = (uint8_t)cnt[i];
      if (cnt[i] > out->max_len) out->max_len = cnt[i];
    }
  }
  // canonical values: by (length, symbol), consecutive, shifted as lengths grow
  uint32_t c = 0;
  int prevl = 0;
  bool first = true;
  for (int l = 1; l <= 32; ++l)
    for (int s = 0; s < 256; ++s) {
      if (out->len[s] != l) continue;
      c = first ? 0u : (c + 1u) << (l - prevl);
      first = false;
      prevl = l;
      out->code[s] = c;
    }
  return CASS_OK;
}

int cass_prefix_code_unary(const uint64_t* hist, cass_prefix_code* out) {
  clear_error();
  if (!hist || !out) return report(CASS_ERR_INVALID, "NULL argument");
  memset(out, 0, sizeof *out);
  int order[256];
  for (int i = 0; i < 256; ++i) order[i] = i;
  std::stable_sort(order, order + 256, [&](int a, int b) { return hist[a] > hist[b]; });
  for (int r = 0; r < 256; ++r) {
    out->len[order[r]] = (uint8_t)(r + 1 > 32 ? 0 : r + 1);
    out->code[order[r]] = r + 1 > 32 ? 0u : 1u;
    if (r + 1 <= 32) out->max_len = r + 1;
  }
  // ranks past 32 carry no code (their symbols must not occur)
  return CASS_OK;
}

int cass_prefix_stream_bits(const cass_prefix_code* c, const uint64_t* hist, int64_t* bits) {
  clear_error();
  int st = check_code(c);
  if (st) return st;
  if (!hist || !bits) return report(CASS_ERR_INVALID, "NULL argument");
  uint64_t b = 0;
  for (int s = 0; s < 256; ++s) {
    if (hist[s] && !c->len[s]) return report(CASS_ERR_INVALID, "symbol %d has no code", s);
    b += hist[s] * c->len[s];
  }
  *bits = (int64_t)b;
  return CASS_OK;
}

int cass_prefix_encode(const cass_prefix_code* c, const uint8_t* sym, int64_t n, int64_t block,
                       void* stream, int64_t stream_bytes, uint32_t* blkoff, hipStream_t s) {
  clear_error();
  int st = check_code(c);
  if (st) return st;
  if (n < 0 || block < 16 || block % 16) return report(CASS_ERR_INVALID, "n < 0 or block not a multiple of 16");
  if (n == 0) return CASS_OK;
  if (!sym || !stream || !blkoff) return report(CASS_ERR_INVALID, "NULL buffer");
  if ((uintptr_t)stream % 16 || stream_bytes % 16 || stream_bytes < 32)
    return report(CASS_ERR_INVALID, "stream must be 16-byte aligned, a multiple of 16 bytes");
  if (stream_bytes > ((int64_t)1 << 29))
    return report(CASS_ERR_UNSUPPORTED, "streams above 2^32 bits");
  // the codes must fit before the 16 trailing zero bytes: the caller sizes the
  // stream from cass_prefix_stream_bits; every symbol's code is at most 32 bits
  if (n > (stream_bytes - 16) * 8)
    return report(CASS_ERR_CAPACITY, "stream too small for %lld symbols", (long long)n);
  if (nblk_of(n, block) > ((int64_t)1 << 31)) return report(CASS_ERR_UNSUPPORTED, "too many blocks");
  const CodeTable t = table_of(c);
  const int64_t nblk = (n + block - 1) / block;
  hipError_t e = launch_fill_zero(stream, stream_bytes, s);
  if (e != hipSuccess) return report(CASS_ERR_HIP, "fill: %s", hipGetErrorString(e));
  k_pc_block_bits<<<grid_of_blocks(nblk), kPcThreads, 0, s>>>(sym, n, block, t, blkoff);
  k_pc_scan<<<1, 1024, 0, s>>>(blkoff, nblk);
  k_pc_pack<<<grid_of_blocks(nblk), kPcThreads, 0, s>>>(sym, n, block, t, blkoff, (uint32_t*)stream,
                                                        (uint64_t)(stream_bytes - 16) * 8u);
  if ((e = hipGetLastError()) != hipSuccess) return report(CASS_ERR_HIP, "encode: %s", hipGetErrorString(e));
  return CASS_OK;
}

int cass_prefix_decode_ws_bytes(int64_t stream_bytes, int64_t* ws_bytes) {
  clear_error();
  if (stream_bytes < 0 || !ws_bytes) return report(CASS_ERR_INVALID, "bad argument");
  const int64_t ng = (stream_bytes / 4 + kWordsPerGroup - 1) / kWordsPerGroup;
  *ws_bytes = 16 * (ng > 0 ? ng : 1);  // per workgroup: ones before it, last one before it
  return CASS_OK;
}

int cass_prefix_decode(const cass_prefix_code* c, const void* stream, int64_t stream_bytes,
                       const uint32_t* blkoff, int64_t n, int64_t block, int method, uint8_t* out,
                       void* ws, int64_t ws_bytes, hipStream_t s) {
  clear_error();
  int st = check_code(c);
  if (st) return st;
  if (n < 0 || block < 16 || block % 16) return report(CASS_ERR_INVALID, "n < 0 or block not a multiple of 16");
  if (n == 0) return CASS_OK;
  if (!stream || !out) return report(CASS_ERR_INVALID, "NULL buffer");
  if ((uintptr_t)stream % 16 || stream_bytes % 16 || stream_bytes < 32 || (uintptr_t)out % 16 ||
      n % 16)
    return report(CASS_ERR_INVALID, "stream and out must be 16-byte aligned, n a multiple of 16");
  const int64_t nblk = nblk_of(n, block);
  const int64_t words = stream_bytes / 4;
  PermTable pt = {};
  hipError_t e = hipSuccess;
  if (method == CASS_PREFIX_TABLE) {
    if (!blkoff) return report(CASS_ERR_INVALID, "blkoff is NULL");
    if (c->max_len > kMaxTableBits)
      return report(CASS_ERR_UNSUPPORTED, "table decoding needs codes of at most %d bits", kMaxTableBits);
    const CodeTable t = table_of(c);
    k_pc_decode_table<<<grid_of_blocks(nblk), kPcThreads, 0, s>>>((const uint32_t*)stream, words,
                                                                 blkoff, n, block, t, c->max_len, out);
  } else if (method == CASS_PREFIX_UNARY_SERIAL) {
    if (!is_unary(c, pt.sym)) return report(CASS_ERR_INVALID, "not a unary code");
    if (!blkoff) return report(CASS_ERR_INVALID, "blkoff is NULL");
    k_pc_decode_unary<<<grid_of_blocks(nblk), kPcThreads, 0, s>>>((const uint32_t*)stream, words,
                                                                 blkoff, n, block, pt, out);
  } else if (method == CASS_PREFIX_UNARY_PARALLEL) {
    if (!is_unary(c, pt.sym)) return report(CASS_ERR_INVALID, "not a unary code");
    int64_t need = 0;
    cass_prefix_decode_ws_bytes(stream_bytes, &need);
    if (!ws || ws_bytes < need || (uintptr_t)ws % 8)
      return report(CASS_ERR_CAPACITY, "decode workspace missing or too small");
    const int64_t ng = (words + kWordsPerGroup - 1) / kWordsPerGroup;
    unsigned long long* cnt = (unsigned long long*)ws;
    long long* last = (long long*)ws + ng;
    k_pc_group_ones<<<(unsigned)ng, kPcThreads, 0, s>>>((const uint32_t*)stream, words, cnt, last);
    k_pc_group_scan<<<1, 1024, 0, s>>>(cnt, last, ng);
    k_pc_decode_parallel<<<(unsigned)ng, kPcThreads, 0, s>>>((const uint32_t*)stream, words, n, cnt,
                                                              last, pt, out);
  } else {
    return report(CASS_ERR_INVALID, "unknown method %d", method);
  }
  if ((e = hipGetLastError()) != hipSuccess) return report(CASS_ERR_HIP, "decode: %s", hipGetErrorString(e));
  return CASS_OK;
}

}  // extern "C"
