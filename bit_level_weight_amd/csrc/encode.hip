// Encoder kernels: pruning (top-k select per row), exponent statistics, code
// lengths and offsets, and packing of the two streams.
//
// Method: Cassandra review (marsggbo.github.io), section 3.1 -- value pruning
// by saliency, mantissa truncation, exponent compression, split into
// speculation and verification data; section 3.2 -- frequency-ranked unary
// exponent codes (Cassandra-1) and a shared MX exponent (Cassandra-2, OCP MX
// specification: one shared 8-bit exponent per 32 elements).
#include "bits.hpp"
#include "internal.hpp"

namespace cass {

namespace {

constexpr int kSelThreads = 256;

__device__ __forceinline__ int key_of(uint16_t b) { return b & 0x7FFF; }
__device__ __forceinline__ int exp_of(uint16_t b) { return (b >> 7) & 0xFF; }

// Exclusive scan of one value per thread over a 256-thread block.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
  const int t = threadIdx.x;
  tmp[t] = v;
  __syncthreads();
  for (int d = 1; d < kSelThreads; d <<= 1) {
    const uint32_t add = (t >= d) ? tmp[t - d] : 0u;
    __syncthreads();
    tmp[t] += add;
    __syncthreads();
  }
  const uint32_t incl = tmp[t];
  if (total) *total = tmp[kSelThreads - 1];
  __syncthreads();
  return incl - v;
}

__global__ void __launch_bounds__(256) k_fill_zero(uint4* p, int64_t n16) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

__global__ void __launch_bounds__(256) k_fill_zero_bytes(uint8_t* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

// One workgroup per row: radix select of the k largest 15-bit magnitude keys
// (high 8 bits, then low 7 bits), then the bitmap with ties at the threshold
// kept in column order.
__global__ void __launch_bounds__(kSelThreads) k_select(const uint16_t* __restrict__ w,
                                                        int64_t C, int64_t ld, int64_t k,
                                                        uint32_t* __restrict__ bitmap) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scan_tmp[kSelThreads];
  __shared__ int sh_T, sh_need;
  const int64_t row = blockIdx.x;
  const uint16_t* wr = w + row * ld;
  uint32_t* bm = bitmap + row * (C / 32);
  const int t = threadIdx.x;
  const int64_t nwords = C / 32;

  if (k == 0 || k == C) {
    const uint32_t fillv = (k == 0) ? 0u : 0xFFFFFFFFu;
    for (int64_t i = t; i < nwords; i += kSelThreads) bm[i] = fillv;
    return;
  }
  // pass 1: high byte of the key
  hist[t] = 0;
  __syncthreads();
  for (int64_t j = t; j < C; j += kSelThreads) atomicAdd(&hist[key_of(wr[j]) >> 7], 1u);
  __syncthreads();
  if (t == 0) {
    int64_t cum = 0;
    int H = 255;
    for (; H > 0; --H) {
      if (cum + hist[H] >= (uint64_t)k) break;
      cum += hist[H];
    }
    sh_T = H;
    sh_need = (int)(k - cum);
  }
  __syncthreads();
  const int H = sh_T;
  const int need1 = sh_need;
  __syncthreads();
  // pass 2: low 7 bits among keys whose high byte is H
  if (t < 128) hist[t] = 0;
  __syncthreads();
  for (int64_t j = t; j < C; j += kSelThreads) {
    const int kk = key_of(wr[j]);
    if ((kk >> 7) == H) atomicAdd(&hist[kk & 127], 1u);
  }
  __syncthreads();
  if (t == 0) {
    int cum = 0;
    int L = 127;
    for (; L > 0; --L) {
      if (cum + (int)hist[L] >= need1) break;
      cum += hist[L];
    }
    sh_T = (H << 7) | L;
    sh_need = need1 - cum;
  }
  __syncthreads();
  const int T = sh_T;
  const int need = sh_need;  // how many values equal to T are kept (lowest columns)

  // pass 3: each thread owns a contiguous run of words
  const int64_t per = (nwords + kSelThreads - 1) / kSelThreads;
  const int64_t w0 = t * per;
  const int64_t w1 = (w0 + per < nwords) ? w0 + per : nwords;
  uint32_t eq_mine = 0;
  for (int64_t wi = w0; wi < w1; ++wi)
    for (int b = 0; b < 32; ++b) eq_mine += (key_of(wr[wi * 32 + b]) == T);
  uint32_t eq_before = block_exclusive_scan(eq_mine, scan_tmp, nullptr);
  for (int64_t wi = w0; wi < w1; ++wi) {
    uint32_t word = 0;
    for (int b = 0; b < 32; ++b) {
      const int kk = key_of(wr[wi * 32 + b]);
      uint32_t keep = kk > T;
      if (kk == T) {
        keep = eq_before < (uint32_t)need;
        ++eq_before;
      }
      word |= keep << b;
    }
    bm[wi] = word;
  }
}

// Exponent histograms of kept and pruned values; for Cassandra-2 also the
// shared exponent of each 32-position group (largest max(e,1) among kept).
__global__ void __launch_bounds__(256) k_histograms(const uint16_t* __restrict__ w, int64_t nwords,
                                                    int64_t wpr, int64_t ld,
                                                    const uint32_t* __restrict__ bitmap,
                                                    unsigned long long* __restrict__ hist,
                                                    uint8_t* __restrict__ shexp) {
  __shared__ uint32_t h[512];
  for (int i = threadIdx.x; i < 512; i += blockDim.x) h[i] = 0;
  __syncthreads();
  for (int64_t wi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; wi < nwords;
       wi += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t bw = bitmap[wi];
    const uint16_t* wv = w + (wi / wpr) * ld + (wi % wpr) * 32;  // row wi / wpr
    int E = 0;
    for (int b = 0; b < 32; ++b) {
      const uint16_t v = wv[b];
      const int e = exp_of(v);
      const int kept = (bw >> b) & 1;
      atomicAdd(&h[(kept ? 0 : 256) + e], 1u);
      const int eff = e > 0 ? e : 1;
      if (kept && eff > E) E = eff;
    }
    if (shexp) shexp[wi] = (uint8_t)E;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 512; i += blockDim.x)
    if (h[i]) atomicAdd(hist + i, (unsigned long long)h[i]);
}

// Per (row, block): code bits of each variable-length section and the kept count.
__global__ void __launch_bounds__(256) k_block_bits(const uint16_t* __restrict__ w, Shape sh,
                                                    int format, RankTables rt,
                                                    const uint32_t* __restrict__ bitmap,
                                                    const uint8_t* __restrict__ shexp,
                                                    uint32_t* __restrict__ blk_a,
                                                    uint32_t* __restrict__ blk_v,
                                                    uint32_t* __restrict__ blk_kept) {
  __shared__ uint8_t rk[256], rp[256];
  for (int i = threadIdx.x; i < 256; i += blockDim.x) {
    rk[i] = rt.rank_kept[i];
    rp[i] = rt.rank_pruned[i];
  }
  __syncthreads();
  const int64_t nb = sh.cols / sh.block;
  const int64_t nblk = sh.rows * nb;
  const int m = sh.mant;
  for (int64_t bi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; bi < nblk;
       bi += (int64_t)gridDim.x * blockDim.x) {
    const int64_t pos0 = bi * sh.block;  // (row*nb + b)*B == row*C + b*B
    const uint16_t* wb = w + (bi / nb) * sh.ld + (bi % nb) * sh.block;  // the block's values
    uint32_t a = 0, v = 0, kept = 0;
    for (int64_t wi = 0; wi < sh.block / 32; ++wi) {
      const uint32_t bw = bitmap[pos0 / 32 + wi];
      for (int b = 0; b < 32; ++b) {
        const uint16_t x = wb[wi * 32 + b];
        const int e = exp_of(x);
        if ((bw >> b) & 1) {
          ++kept;
          if (format == CASS_FMT_C2_MX_TARGET) {
            // fixed-width verification sections: no code bits
          } else if (is_c1_format(format)) {
            a += rk[e] + 1u;
          } else {
            const int E = shexp[pos0 / 32 + wi];
            const int d = E - (e > 0 ? e : 1);
            const int wd = (7 - m + d < 8) ? 7 - m + d : 8;
            a += (uint32_t)(d + 1 + wd);
          }
        } else if (format != CASS_FMT_C2_MX_TARGET) {
          v += rp[e] + 1u;
        }
      }
    }
    blk_a[bi] = a;
    blk_v[bi] = v;
    blk_kept[bi] = kept;
  }
}

// One workgroup per row: exclusive scans over the row's blocks.
__global__ void __launch_bounds__(kSelThreads) k_row_scan(
    int64_t nb, const uint32_t* __restrict__ blk_a, const uint32_t* __restrict__ blk_v,
    const uint32_t* __restrict__ blk_kept, uint32_t* __restrict__ off_a,
    uint32_t* __restrict__ off_v, uint16_t* __restrict__ keptb,
    unsigned long long* __restrict__ row_a, unsigned long long* __restrict__ row_v) {
  __shared__ uint32_t tmp[kSelThreads];
  __shared__ uint32_t tot;
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t per = (nb + kSelThreads - 1) / kSelThreads;
  const int64_t b0 = t * per;
  const int64_t b1 = (b0 + per < nb) ? b0 + per : nb;
  const uint32_t* src[3] = {blk_a + row * nb, blk_v + row * nb, blk_kept + row * nb};
  for (int which = 0; which < 3; ++which) {
    uint32_t mine = 0;
    for (int64_t b = b0; b < b1; ++b) mine += src[which][b];
    uint32_t run = block_exclusive_scan(mine, tmp, &tot);
    for (int64_t b = b0; b < b1; ++b) {
      if (which == 0) off_a[row * nb + b] = run;
      else if (which == 1) off_v[row * nb + b] = run;
      else keptb[row * nb + b] = (uint16_t)run;
      run += src[which][b];
    }
    if (t == 0) {
      if (which == 0) row_a[row] = tot;
      else if (which == 1) row_v[row] = tot;
    }
    __syncthreads();
  }
}

// One workgroup: row totals -> exclusive row bases, and the grand totals.
__global__ void __launch_bounds__(1024) k_rows_scan(int64_t R, unsigned long long* row_a,
                                                    unsigned long long* row_v,
                                                    unsigned long long* totals) {
  __shared__ unsigned long long tmp[1024];
  const int t = threadIdx.x;
  const int64_t per = (R + 1023) / 1024;
  const int64_t r0 = t * per;
  const int64_t r1 = (r0 + per < R) ? r0 + per : R;
  unsigned long long* arr[2] = {row_a, row_v};
  for (int which = 0; which < 2; ++which) {
    unsigned long long mine = 0;
    for (int64_t r = r0; r < r1; ++r) mine += arr[which][r];
    tmp[t] = mine;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
      const unsigned long long add = (t >= d) ? tmp[t - d] : 0ull;
      __syncthreads();
      tmp[t] += add;
      __syncthreads();
    }
    unsigned long long run = tmp[t] - mine;
    if (t == 1023) totals[which] = tmp[t];
    __syncthreads();
    for (int64_t r = r0; r < r1; ++r) {
      const unsigned long long v = arr[which][r];
      arr[which][r] = run;
      run += v;
    }
    __syncthreads();
  }
}

// Largest offset of a block's first code bit from its superblock's first
// block, over the tensor.
__global__ void __launch_bounds__(256) k_superblock_span(const uint32_t* __restrict__ off_a,
                                                         int64_t R, int64_t nb, int sblocks,
                                                         unsigned long long* out) {
  unsigned long long mx = 0;
  for (int64_t bi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; bi < R * nb;
       bi += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = bi % nb;
    const unsigned long long d = off_a[bi] - off_a[bi - b % sblocks];
    mx = d > mx ? d : mx;
  }
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long v = __shfl_xor(mx, o, 64);
    mx = v > mx ? v : mx;
  }
  if ((threadIdx.x & 63) == 0 && mx) atomicMax(out, mx);
}

__global__ void k_write_headers(HeaderBlob hb, uint8_t* spec, int64_t spec_rank_off,
                                uint8_t* verif, int64_t verif_rank_off) {
  const int t = threadIdx.x;  // 256 threads
  spec[t] = hb.spec_hdr[t];
  verif[t] = hb.verif_hdr[t];
  if (spec_rank_off > 0) spec[spec_rank_off + t] = hb.perm_spec[t];
  if (verif_rank_off > 0) verif[verif_rank_off + t] = hb.perm_verif[t];
}

struct PackPtrs {
  uint32_t* s_bitmap;
  unsigned long long* s_rowbase;  // C-1
  uint32_t* s_blkoff;             // C-1
  uint16_t* s_keptb;
  uint32_t* s_fields;
  uint32_t* s_codes;              // C-1
  uint8_t* s_shexp;               // C-2
  unsigned long long* v_rowbase;  // C-1: pruned codes; C-2: residues
  uint32_t* v_blkoff;
  uint32_t* v_lowmant;            // C-1
  uint32_t* v_resid;              // C-2
  uint8_t* v_pruned;
  unsigned long long* v_rowbase_p;  // C-2
  uint32_t* v_blkoff_p;             // C-2
  uint32_t* v_codes;
  uint8_t* v_gexp;                  // format 3: X per 32 positions
  uint32_t* v_low;                  // format 3: kept low 7-m bits of t
  uint32_t* v_pr9;                  // format 3: pruned (s<<8)|t
  unsigned long long* s_sbbase;     // format 4: code base per superblock
  uint16_t* s_blkoff16;             // format 4: block offset from its superblock
};

// One thread per (row, block): writes every section's share of that block.
__global__ void __launch_bounds__(256) k_pack(const uint16_t* __restrict__ w, Shape sh, int format,
                                              RankTables rt, Workspace ws, PackPtrs P) {
  __shared__ uint8_t rk[256], rp[256];
  for (int i = threadIdx.x; i < 256; i += blockDim.x) {
    rk[i] = rt.rank_kept[i];
    rp[i] = rt.rank_pruned[i];
  }
  __syncthreads();
  const int64_t B = sh.block, C = sh.cols, k = sh.keep;
  const int64_t nb = C / B;
  const int64_t nblk = sh.rows * nb;
  const int m = sh.mant;
  const bool c1 = is_c1_format(format);
  const bool c3 = format == CASS_FMT_C2_MX_TARGET;
  const bool sbm = format == CASS_FMT_C1_SUPERBLOCK;
  const int64_t nsb = (nb + CASS_SUPERBLOCK_BLOCKS - 1) / CASS_SUPERBLOCK_BLOCKS;
  for (int64_t bi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; bi < nblk;
       bi += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = bi / nb, b = bi % nb;
    const int64_t pos0 = bi * B;
    const uint32_t kb = ws.keptb[bi];
    const int64_t pb = b * B - kb;  // pruned before the block in the row
    if (c3) {
      // Cassandra-2 speculation sections; the target's fixed-width verification
      // sections: X per 32 positions, low 7-m bits of each kept t, (s, t) of each
      // pruned value
      for (int64_t wi = 0; wi < B / 32; ++wi) {
        P.s_bitmap[pos0 / 32 + wi] = ws.bitmap[pos0 / 32 + wi];
        P.s_shexp[pos0 / 32 + wi] = ws.shexp[pos0 / 32 + wi];
      }
      P.s_keptb[bi] = (uint16_t)kb;
      const uint64_t kin0 = (uint64_t)row * k + kb;
      BitWriter fw, lw, pw;
      fw.init(P.s_fields, kin0 * (uint64_t)(2 + m));
      lw.init(P.v_low, kin0 * (uint64_t)(7 - m));
      pw.init(P.v_pr9, (uint64_t)(row * (C - k) + pb) * 9u);
      for (int64_t wi = 0; wi < B / 32; ++wi) {
        const uint32_t bw = ws.bitmap[pos0 / 32 + wi];
        const uint16_t* xw = w + row * sh.ld + b * B + wi * 32;
        int X = 0;
        for (int bb = 0; bb < 32; ++bb) {
          const int e = exp_of(xw[bb]);
          X = (e > 0 ? e : 1) > X ? (e > 0 ? e : 1) : X;
        }
        P.v_gexp[pos0 / 32 + wi] = (uint8_t)X;
        for (int bb = 0; bb < 32; ++bb) {
          const uint16_t x = xw[bb];
          const int s = x >> 15, e = exp_of(x), f = x & 0x7F;
          const int M = ((e > 0) << 7) | f;
          const int d = X - (e > 0 ? e : 1);
          const int t = d >= 8 ? 0 : (M >> d);
          if ((bw >> bb) & 1) {
            // a group that keeps anything has its maximum among the kept
            // values, so t's top m+1 bits are the Cassandra-2 field
            fw.put((uint32_t)((s << (m + 1)) | (t >> (7 - m))), 2 + m);
            lw.put((uint32_t)(t & ((1 << (7 - m)) - 1)), 7 - m);
          } else {
            pw.put((uint32_t)((s << 8) | t), 9);
          }
        }
      }
      fw.finish();
      lw.finish();
      pw.finish();
      continue;
    }
    const unsigned long long base_a = ws.row_a[row], base_v = ws.row_v[row];
    // fixed sections
    for (int64_t wi = 0; wi < B / 32; ++wi) P.s_bitmap[pos0 / 32 + wi] = ws.bitmap[pos0 / 32 + wi];
    P.s_keptb[bi] = (uint16_t)kb;
    if (c1) {
      if (b == 0) {
        if (!sbm) P.s_rowbase[row] = base_a;
        P.v_rowbase[row] = base_v;
      }
      if (sbm) {
        // superblock metadata: a u64 base at each superblock's first block,
        // 16-bit offsets from it (the plan checked they fit)
        const int64_t b0 = b - b % CASS_SUPERBLOCK_BLOCKS;
        const uint32_t sb_off = ws.off_a[row * nb + b0];
        if (b == b0) P.s_sbbase[row * nsb + b / CASS_SUPERBLOCK_BLOCKS] = base_a + sb_off;
        P.s_blkoff16[bi] = (uint16_t)(ws.off_a[bi] - sb_off);
      } else {
        P.s_blkoff[bi] = ws.off_a[bi];
      }
      P.v_blkoff[bi] = ws.off_v[bi];
    } else {
      for (int64_t wi = 0; wi < B / 32; ++wi) P.s_shexp[pos0 / 32 + wi] = ws.shexp[pos0 / 32 + wi];
      if (b == 0) {
        P.v_rowbase[row] = base_a;
        P.v_rowbase_p[row] = base_v;
      }
      P.v_blkoff[bi] = ws.off_a[bi];
      P.v_blkoff_p[bi] = ws.off_v[bi];
    }
    // variable sections
    const uint64_t kin0 = (uint64_t)row * k + kb;  // first kept index of the block
    BitWriter fw, cw, lw, vw;
    fw.init(P.s_fields, kin0 * (uint64_t)(c1 ? 1 + m : 2 + m));
    if (c1) {
      cw.init(P.s_codes, base_a + ws.off_a[bi]);
      lw.init(P.v_lowmant, kin0 * (uint64_t)(7 - m));
    } else {
      cw.init(P.v_resid, base_a + ws.off_a[bi]);
    }
    vw.init(P.v_codes, base_v + ws.off_v[bi]);
    int64_t pidx = row * (C - k) + pb;
    for (int64_t wi = 0; wi < B / 32; ++wi) {
      const uint32_t bw = ws.bitmap[pos0 / 32 + wi];
      const int E = c1 ? 0 : ws.shexp[pos0 / 32 + wi];
      for (int bb = 0; bb < 32; ++bb) {
        const uint16_t x = w[row * sh.ld + b * B + wi * 32 + bb];
        const int s = x >> 15, e = exp_of(x), f = x & 0x7F;
        if ((bw >> bb) & 1) {
          if (c1) {
            // sign and top m mantissa bits -> speculation; low 7-m bits -> verification
            fw.put((uint32_t)((s << m) | (f >> (7 - m))), 1 + m);
            cw.put_unary(rk[e]);
            lw.put((uint32_t)(f & ((1 << (7 - m)) - 1)), 7 - m);
          } else {
            const int eff = e > 0 ? e : 1;
            const int M = ((e > 0) << 7) | f;
            const int d = E - eff;
            const int shift = 7 - m + d;
            const int a = shift >= 8 ? 0 : (M >> shift);
            const int wd = shift < 8 ? shift : 8;
            fw.put((uint32_t)((s << (m + 1)) | a), 2 + m);
            cw.put_unary(d);
            cw.put((uint32_t)(M & ((1 << wd) - 1)), wd);
          }
        } else {
          P.v_pruned[pidx++] = (uint8_t)((s << 7) | f);
          vw.put_unary(rp[e]);
        }
      }
    }
    fw.finish();
    cw.finish();
    if (c1) lw.finish();
    vw.finish();
  }
}

int grid_for(int64_t items, int threads) {
  int64_t g = (items + threads - 1) / threads;
  const int64_t cap = (int64_t)device_cu_count() * 16;
  if (g > cap) g = cap;
  return (int)(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_fill_zero(void* p, int64_t bytes, hipStream_t s) {
  if (bytes <= 0) return hipSuccess;
  if ((bytes % 16) == 0 && ((uintptr_t)p % 16) == 0) {
    k_fill_zero<<<grid_for(bytes / 16, 256), 256, 0, s>>>((uint4*)p, bytes / 16);
  } else {
    k_fill_zero_bytes<<<grid_for(bytes, 256), 256, 0, s>>>((uint8_t*)p, bytes);
  }
  return hipGetLastError();
}

hipError_t launch_select(const uint16_t* w, const Shape& sh, uint32_t* bitmap, hipStream_t s) {
  if (sh.rows == 0) return hipSuccess;
  k_select<<<(unsigned)sh.rows, kSelThreads, 0, s>>>(w, sh.cols, sh.ld, sh.keep, bitmap);
  return hipGetLastError();
}

hipError_t launch_histograms(const uint16_t* w, const Shape& sh, int format, const Workspace& ws,
                             hipStream_t s) {
  hipError_t e = launch_fill_zero(ws.hist, 512 * sizeof(unsigned long long), s);
  if (e != hipSuccess) return e;
  const int64_t nwords = sh.rows * sh.cols / 32;
  if (nwords == 0) return hipSuccess;
  k_histograms<<<grid_for(nwords, 256), 256, 0, s>>>(
      w, nwords, sh.cols / 32, sh.ld, ws.bitmap, ws.hist,
      is_c1_format(format) ? nullptr : ws.shexp);
  return hipGetLastError();
}

hipError_t launch_block_bits(const uint16_t* w, const Shape& sh, int format, const Workspace& ws,
                             const RankTables& rt, hipStream_t s) {
  const int64_t nblk = sh.rows * (sh.cols / sh.block);
  if (nblk == 0) return hipSuccess;
  k_block_bits<<<grid_for(nblk, 256), 256, 0, s>>>(w, sh, format, rt, ws.bitmap, ws.shexp,
                                                   ws.blk_a, ws.blk_v, ws.blk_kept);
  return hipGetLastError();
}

hipError_t launch_row_scan(const Shape& sh, const Workspace& ws, hipStream_t s) {
  if (sh.rows == 0) return hipSuccess;
  k_row_scan<<<(unsigned)sh.rows, kSelThreads, 0, s>>>(sh.cols / sh.block, ws.blk_a, ws.blk_v,
                                                       ws.blk_kept, ws.off_a, ws.off_v, ws.keptb,
                                                       ws.row_a, ws.row_v);
  return hipGetLastError();
}

hipError_t launch_rows_scan(const Shape& sh, const Workspace& ws, hipStream_t s) {
  hipError_t e = launch_fill_zero(ws.totals, 3 * sizeof(unsigned long long), s);
  if (e != hipSuccess || sh.rows == 0) return e;
  k_rows_scan<<<1, 1024, 0, s>>>(sh.rows, ws.row_a, ws.row_v, ws.totals);
  return hipGetLastError();
}

hipError_t launch_superblock_span(const Shape& sh, const Workspace& ws, int sblocks, hipStream_t s) {
  const int64_t nblk = sh.rows * (sh.cols / sh.block);
  if (nblk == 0) return hipSuccess;
  k_superblock_span<<<grid_for(nblk, 256), 256, 0, s>>>(ws.off_a, sh.rows, sh.cols / sh.block,
                                                        sblocks, ws.totals + 2);
  return hipGetLastError();
}

hipError_t launch_write_headers(const HeaderBlob& hb, uint8_t* spec, int64_t spec_rank_off,
                                uint8_t* verif, int64_t verif_rank_off, hipStream_t s) {
  k_write_headers<<<1, 256, 0, s>>>(hb, spec, spec_rank_off, verif, verif_rank_off);
  return hipGetLastError();
}

hipError_t launch_pack(const uint16_t* w, const Shape& sh, int format, const Workspace& ws,
                       const RankTables& rt, uint8_t* spec, const int64_t* ss, uint8_t* verif,
                       const int64_t* vs, hipStream_t s) {
  const int64_t nblk = sh.rows * (sh.cols / sh.block);
  if (nblk == 0) return hipSuccess;
  PackPtrs P = {};
  if (is_c1_format(format)) {
    P.s_bitmap = (uint32_t*)(spec + ss[S1_BITMAP]);
    if (format == CASS_FMT_C1_SUPERBLOCK) {
      P.s_sbbase = (unsigned long long*)(spec + ss[S1_ROWBASE]);
      P.s_blkoff16 = (uint16_t*)(spec + ss[S1_BLKOFF]);
    } else {
      P.s_rowbase = (unsigned long long*)(spec + ss[S1_ROWBASE]);
      P.s_blkoff = (uint32_t*)(spec + ss[S1_BLKOFF]);
    }
    P.s_keptb = (uint16_t*)(spec + ss[S1_KEPTB]);
    P.s_fields = (uint32_t*)(spec + ss[S1_FIELDS]);
    P.s_codes = (uint32_t*)(spec + ss[S1_CODES]);
    P.v_rowbase = (unsigned long long*)(verif + vs[V1_ROWBASE]);
    P.v_blkoff = (uint32_t*)(verif + vs[V1_BLKOFF]);
    P.v_lowmant = (uint32_t*)(verif + vs[V1_LOWMANT]);
    P.v_pruned = verif + vs[V1_PRUNED];
    P.v_codes = (uint32_t*)(verif + vs[V1_CODES]);
  } else if (format == CASS_FMT_C2_MX_TARGET) {
    P.s_bitmap = (uint32_t*)(spec + ss[S2_BITMAP]);
    P.s_shexp = spec + ss[S2_SHEXP];
    P.s_keptb = (uint16_t*)(spec + ss[S2_KEPTB]);
    P.s_fields = (uint32_t*)(spec + ss[S2_FIELDS]);
    P.v_gexp = verif + vs[V3_GEXP];
    P.v_low = (uint32_t*)(verif + vs[V3_LOW]);
    P.v_pr9 = (uint32_t*)(verif + vs[V3_PRUNED]);
  } else {
    P.s_bitmap = (uint32_t*)(spec + ss[S2_BITMAP]);
    P.s_shexp = spec + ss[S2_SHEXP];
    P.s_keptb = (uint16_t*)(spec + ss[S2_KEPTB]);
    P.s_fields = (uint32_t*)(spec + ss[S2_FIELDS]);
    P.v_rowbase = (unsigned long long*)(verif + vs[V2_ROWBASE_K]);
    P.v_blkoff = (uint32_t*)(verif + vs[V2_BLKOFF_K]);
    P.v_resid = (uint32_t*)(verif + vs[V2_RESID]);
    P.v_pruned = verif + vs[V2_PRUNED];
    P.v_rowbase_p = (unsigned long long*)(verif + vs[V2_ROWBASE_P]);
    P.v_blkoff_p = (uint32_t*)(verif + vs[V2_BLKOFF_P]);
    P.v_codes = (uint32_t*)(verif + vs[V2_CODES]);
  }
  k_pack<<<grid_for(nblk, 256), 256, 0, s>>>(w, sh, format, rt, ws, P);
  return hipGetLastError();
}

}  // namespace cass
