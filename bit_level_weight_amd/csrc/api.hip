// C ABI of libcassandra: argument validation, stream layout, encoder
// orchestration and kernel launches.  See include/cassandra.h.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "internal.hpp"

namespace cass {

namespace {

thread_local std::string g_last_error;

std::atomic<int> g_options[OPT_COUNT];

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(CASS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t align256(int64_t v) { return (v + 255) / 256 * 256; }

// ---------------------------------------------------------------- layout

struct Layout {
  int nsec = 0;
  int64_t off[CASS_MAX_SECTIONS] = {};
  int64_t len[CASS_MAX_SECTIONS] = {};
  int64_t total = 0;
};

// Sections start on 256-byte boundaries, each followed by >= 16 zero bytes.
Layout lay_out(const std::vector<int64_t>& lens) {
  Layout L;
  L.nsec = (int)lens.size();
  int64_t pos = kHeaderBytes;
  for (int i = 0; i < L.nsec; ++i) {
    L.off[i] = pos;
    L.len[i] = lens[i];
    pos = align256(pos + lens[i] + 16);
  }
  L.total = pos;
  return L;
}

void stream_lengths(int format, int64_t R, int64_t C, int64_t B, int64_t k, int m,
                    uint64_t code_a, uint64_t code_v, std::vector<int64_t>& ls,
                    std::vector<int64_t>& lv) {
  const int64_t n = R * C, nb = C / B;
  if (is_c1_format(format)) {
    ls = {256, n / 8, 8 * R, 4 * R * nb, 2 * R * nb, (R * k * (1 + m) + 7) / 8,
          (int64_t)((code_a + 7) / 8)};
    lv = {256, 8 * R, 4 * R * nb, (R * k * (7 - m) + 7) / 8, R * (C - k),
          (int64_t)((code_v + 7) / 8)};
    if (format == CASS_FMT_C1_SUPERBLOCK) {  // u64 per superblock, u16 per block
      ls[S1_ROWBASE] = 8 * R * ((nb + CASS_SUPERBLOCK_BLOCKS - 1) / CASS_SUPERBLOCK_BLOCKS);
      ls[S1_BLKOFF] = 2 * R * nb;
    }
  } else if (format == CASS_FMT_C2_MX32) {
    ls = {n / 8, n / 32, 2 * R * nb, (R * k * (2 + m) + 7) / 8};
    lv = {256, 8 * R, 4 * R * nb, (int64_t)((code_a + 7) / 8), R * (C - k), 8 * R, 4 * R * nb,
          (int64_t)((code_v + 7) / 8)};
  } else {
    ls = {n / 8, n / 32, 2 * R * nb, (R * k * (2 + m) + 7) / 8};
    lv = {n / 32, (R * k * (7 - m) + 7) / 8, (R * (C - k) * 9 + 7) / 8};
  }
}

void put32(uint8_t* p, uint32_t v) { memcpy(p, &v, 4); }
void put64(uint8_t* p, int64_t v) { memcpy(p, &v, 8); }
uint32_t get32(const uint8_t* p) { uint32_t v; memcpy(&v, p, 4); return v; }
int64_t get64(const uint8_t* p) { int64_t v; memcpy(&v, p, 8); return v; }

void write_header(uint8_t* h, uint32_t magic, int format, int m, int64_t R, int64_t C, int64_t B,
                  int64_t k, const Layout& L) {
  memset(h, 0, kHeaderBytes);
  put32(h + 0, magic);
  put32(h + 4, 1);
  put32(h + 8, (uint32_t)format);
  put32(h + 12, (uint32_t)m);
  put64(h + 16, R);
  put64(h + 24, C);
  put64(h + 32, B);
  put64(h + 40, k);
  put64(h + 48, L.total);
  put32(h + 56, (uint32_t)L.nsec);
  put32(h + 60, format == CASS_FMT_C1_SUPERBLOCK ? CASS_SUPERBLOCK_BLOCKS : 0u);
  for (int s = 0; s < CASS_MAX_SECTIONS; ++s) {
    put64(h + 64 + 16 * s, L.off[s]);
    put64(h + 72 + 16 * s, L.len[s]);
  }
}

// ---------------------------------------------------------- validation

int check_shape(int64_t R, int64_t C, const cass_params* p) {
  if (!p) return fail(CASS_ERR_INVALID, "params is NULL");
  if (p->format != CASS_FMT_C1_UNARY && p->format != CASS_FMT_C2_MX32 &&
      p->format != CASS_FMT_C2_MX_TARGET && p->format != CASS_FMT_C1_SUPERBLOCK)
    return fail(CASS_ERR_INVALID, "unknown format %d", p->format);
  if (p->mant_bits < 0 || p->mant_bits > 7)
    return fail(CASS_ERR_INVALID, "mant_bits %d outside 0..7", p->mant_bits);
  if (R < 0 || C <= 0) return fail(CASS_ERR_INVALID, "bad shape %lld x %lld", (long long)R, (long long)C);
  if (C > 65536) return fail(CASS_ERR_UNSUPPORTED, "cols %lld > 65536", (long long)C);
  if (p->block < 32 || (p->block & (p->block - 1)) || C % p->block)
    return fail(CASS_ERR_INVALID, "block %lld must be a power of two >= 32 dividing cols %lld",
                (long long)p->block, (long long)C);
  if (p->keep < 0 || p->keep > C)
    return fail(CASS_ERR_INVALID, "keep %lld outside 0..cols", (long long)p->keep);
  if (R > ((int64_t)1 << 40) / C) return fail(CASS_ERR_OVERFLOW, "tensor too large");
  return CASS_OK;
}

// Closed-form lengths of a stream's sections; -1 for the variable-length code
// sections (their size depends on the data).
std::vector<int64_t> closed_lengths(bool spec, int format, int64_t R, int64_t C, int64_t B,
                                    int64_t k, int m) {
  std::vector<int64_t> ls, lv;
  stream_lengths(format, R, C, B, k, m, 0, 0, ls, lv);
  if (is_c1_format(format)) {
    ls[S1_CODES] = -1;
    lv[V1_CODES] = -1;
  } else if (format == CASS_FMT_C2_MX32) {
    lv[V2_RESID] = -1;
    lv[V2_CODES] = -1;
  }  // format 3: every section has a closed form
  return spec ? ls : lv;
}

// Every section starts on a 256-byte boundary after the header, in order, and
// a fixed-size section with its >= 16 padding bytes ends before the next
// section starts (the last one before the end of the buffer), so kernels that
// size their reads from the shape stay inside the caller's buffer.  The device
// contents (row bases, offsets, codes) are trusted: cass_tensor_validate
// checks untrusted streams on the host.
int check_sections(const char* what, const int64_t* off, int64_t bytes,
                   const std::vector<int64_t>& len) {
  const int n = (int)len.size();
  for (int s = 0; s < n; ++s) {
    const int64_t end = s + 1 < n ? off[s + 1] : bytes;
    if (off[s] < kHeaderBytes || off[s] % 256 || off[s] >= bytes || end > bytes)
      return fail(CASS_ERR_INVALID, "%s section %d offset out of range", what, s);
    if (off[s] + (len[s] < 0 ? 0 : len[s]) + 16 > end)
      return fail(CASS_ERR_INVALID, "%s section %d does not fit before %s", what, s,
                  s + 1 < n ? "the next section" : "the end of the buffer");
  }
  return CASS_OK;
}

int check_tensor(const cass_tensor* W, bool need_verif) {
  if (!W) return fail(CASS_ERR_INVALID, "tensor descriptor is NULL");
  cass_params p = {W->format, W->mant_bits, W->block, W->keep};
  int st = check_shape(W->rows, W->cols, &p);
  if (st) return st;
  if (!W->spec) return fail(CASS_ERR_INVALID, "speculation stream is NULL");
  if (need_verif && !W->verif) return fail(CASS_ERR_INVALID, "verification stream is NULL");
  if (((uintptr_t)W->spec % 16) || (W->verif && ((uintptr_t)W->verif % 16)))
    return fail(CASS_ERR_INVALID, "stream buffers must be 16-byte aligned");
  st = check_sections("speculation", W->spec_sec, W->spec_bytes,
                      closed_lengths(true, W->format, W->rows, W->cols, W->block, W->keep,
                                     W->mant_bits));
  if (st) return st;
  if (need_verif)
    st = check_sections("verification", W->verif_sec, W->verif_bytes,
                        closed_lengths(false, W->format, W->rows, W->cols, W->block, W->keep,
                                       W->mant_bits));
  return st;
}

Shape shape_of(const cass_tensor* W) {
  return Shape{W->rows, W->cols, W->block, W->keep, W->mant_bits, W->cols};
}

// Whole 16-byte units between a section start and the end of the buffer, in
// 32-bit words: the bulk copies of the staged kernels stay below this.
// The staged exact decoders serve Cassandra-1 verification and reconstruction
// unless the exact_path option selects the per-thread stream readers.
bool staged_exact_enabled() { return option(OPT_EXACT_PATH) != 1; }

int64_t word_limit(int64_t buffer_bytes, int64_t section_off) {
  return (buffer_bytes - section_off) / 16 * 4;
}

SpecViewC1 spec_c1(const cass_tensor* W) {
  const uint8_t* b = (const uint8_t*)W->spec;
  const int64_t* o = W->spec_sec;
  return SpecViewC1{b + o[S1_RANK], (const uint32_t*)(b + o[S1_BITMAP]),
                    (const unsigned long long*)(b + o[S1_ROWBASE]),
                    (const uint32_t*)(b + o[S1_BLKOFF]), (const uint16_t*)(b + o[S1_KEPTB]),
                    (const uint32_t*)(b + o[S1_FIELDS]), (const uint32_t*)(b + o[S1_CODES]),
                    word_limit(W->spec_bytes, o[S1_BITMAP]), word_limit(W->spec_bytes, o[S1_FIELDS]),
                    word_limit(W->spec_bytes, o[S1_CODES]), word_limit(W->spec_bytes, o[S1_BLKOFF]),
                    2 * word_limit(W->spec_bytes, o[S1_KEPTB]), nullptr, nullptr, -1, 0, 0};
}
// Format 4: the row-base / block-offset sections hold superblock bases and
// 16-bit block offsets.
SpecViewC1 spec_c1s(const cass_tensor* W) {
  SpecViewC1 v = spec_c1(W);
  const uint8_t* b = (const uint8_t*)W->spec;
  const int64_t nb = W->cols / W->block;
  v.sbbase = (const unsigned long long*)(b + W->spec_sec[S1_ROWBASE]);
  v.blkoff16 = (const uint16_t*)(b + W->spec_sec[S1_BLKOFF]);
  v.rowbase = nullptr;
  v.blkoff = nullptr;
  v.sb_log = 4;
  v.nsb = (nb + CASS_SUPERBLOCK_BLOCKS - 1) / CASS_SUPERBLOCK_BLOCKS;
  v.sbbase_limit = word_limit(W->spec_bytes, W->spec_sec[S1_ROWBASE]) / 2;
  return v;
}
VerifViewC1 verif_c1(const cass_tensor* W) {
  const uint8_t* b = (const uint8_t*)W->verif;
  const int64_t* o = W->verif_sec;
  return VerifViewC1{b + o[V1_RANK], (const unsigned long long*)(b + o[V1_ROWBASE]),
                     (const uint32_t*)(b + o[V1_BLKOFF]), (const uint32_t*)(b + o[V1_LOWMANT]),
                     b + o[V1_PRUNED], (const uint32_t*)(b + o[V1_CODES]),
                     word_limit(W->verif_bytes, o[V1_LOWMANT]), word_limit(W->verif_bytes, o[V1_PRUNED]),
                     word_limit(W->verif_bytes, o[V1_CODES])};
}
SpecViewC2 spec_c2(const cass_tensor* W) {
  const uint8_t* b = (const uint8_t*)W->spec;
  const int64_t* o = W->spec_sec;
  return SpecViewC2{(const uint32_t*)(b + o[S2_BITMAP]), b + o[S2_SHEXP],
                    (const uint16_t*)(b + o[S2_KEPTB]), (const uint32_t*)(b + o[S2_FIELDS]),
                    word_limit(W->spec_bytes, o[S2_BITMAP]), word_limit(W->spec_bytes, o[S2_SHEXP]),
                    word_limit(W->spec_bytes, o[S2_FIELDS]), 2 * word_limit(W->spec_bytes, o[S2_KEPTB])};
}
VerifViewC2 verif_c2(const cass_tensor* W) {
  const uint8_t* b = (const uint8_t*)W->verif;
  const int64_t* o = W->verif_sec;
  return VerifViewC2{b + o[V2_RANK], (const unsigned long long*)(b + o[V2_ROWBASE_K]),
                     (const uint32_t*)(b + o[V2_BLKOFF_K]), (const uint32_t*)(b + o[V2_RESID]),
                     b + o[V2_PRUNED], (const unsigned long long*)(b + o[V2_ROWBASE_P]),
                     (const uint32_t*)(b + o[V2_BLKOFF_P]), (const uint32_t*)(b + o[V2_CODES])};
}

VerifViewC3 verif_c3(const cass_tensor* W) {
  const uint8_t* b = (const uint8_t*)W->verif;
  const int64_t* o = W->verif_sec;
  return VerifViewC3{b + o[V3_GEXP], (const uint32_t*)(b + o[V3_LOW]),
                     (const uint32_t*)(b + o[V3_PRUNED])};
}

// frequency ranking: count descending, exponent ascending among equal counts
void rank_table(const uint64_t* hist, uint8_t* perm, uint8_t* rank) {
  int order[256];
  for (int i = 0; i < 256; ++i) order[i] = i;
  std::stable_sort(order, order + 256, [&](int a, int b) { return hist[a] > hist[b]; });
  for (int r = 0; r < 256; ++r) {
    perm[r] = (uint8_t)order[r];
    rank[order[r]] = (uint8_t)r;
  }
}

int64_t ws_layout(int64_t R, int64_t C, int64_t B, Workspace* ws, uint8_t* base) {
  const int64_t n = R * C, nb = C / B, nblk = R * nb;
  int64_t pos = 0;
  auto take = [&](int64_t bytes) {
    uint8_t* p = base ? base + pos : nullptr;
    pos = align256(pos + (bytes > 0 ? bytes : 1));
    return p;
  };
  Workspace w;
  w.bitmap = (uint32_t*)take(n / 8);
  w.shexp = take(n / 32);
  w.hist = (unsigned long long*)take(512 * 8);
  w.blk_a = (uint32_t*)take(4 * nblk);
  w.blk_v = (uint32_t*)take(4 * nblk);
  w.blk_kept = (uint32_t*)take(4 * nblk);
  w.off_a = (uint32_t*)take(4 * nblk);
  w.off_v = (uint32_t*)take(4 * nblk);
  w.keptb = (uint16_t*)take(2 * nblk);
  w.row_a = (unsigned long long*)take(8 * R);
  w.row_v = (unsigned long long*)take(8 * R);
  w.totals = (unsigned long long*)take(24);  // code bits, pruned bits, superblock span
  w.bytes = pos;
  if (ws) *ws = w;
  return pos;
}

}  // namespace

int report(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

void clear_error() { g_last_error.clear(); }

int option(Option o) { return g_options[o].load(std::memory_order_relaxed); }

Workspace carve_workspace(void* base, int64_t rows, int64_t cols, int64_t block) {
  Workspace w;
  ws_layout(rows, cols, block, &w, (uint8_t*)base);
  return w;
}

int device_cu_count() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

// Readers of the translation units' debug flag words (debug build).
std::vector<uint32_t (*)()>& debug_registry() {
  static std::vector<uint32_t (*)()> r;
  return r;
}
void debug_register(uint32_t (*read_and_clear)()) { debug_registry().push_back(read_and_clear); }

}  // namespace cass

using namespace cass;

extern "C" {

int cass_version(void) { return CASS_VERSION; }

int cass_debug_flags(uint32_t* flags) {
  g_last_error.clear();
  if (!flags) return fail(CASS_ERR_INVALID, "flags is NULL");
  *flags = 0;
#ifdef CASS_DEBUG
  for (auto f : debug_registry()) *flags |= f();
  return CASS_OK;
#else
  return fail(CASS_ERR_UNSUPPORTED, "device bounds checks are in the debug build only");
#endif
}

const char* cass_last_error(void) { return g_last_error.c_str(); }

const char* cass_status_string(int status) {
  switch (status) {
    case CASS_OK: return "ok";
    case CASS_ERR_INVALID: return "invalid argument";
    case CASS_ERR_UNSUPPORTED: return "unsupported";
    case CASS_ERR_OVERFLOW: return "overflow";
    case CASS_ERR_CORRUPT: return "corrupt stream";
    case CASS_ERR_CAPACITY: return "buffer too small";
    case CASS_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

int cass_encode_ws_bytes(int64_t rows, int64_t cols, const cass_params* p, int64_t* ws_bytes) {
  g_last_error.clear();
  int st = check_shape(rows, cols, p);
  if (st) return st;
  if (!ws_bytes) return fail(CASS_ERR_INVALID, "ws_bytes is NULL");
  *ws_bytes = ws_layout(rows, cols, p->block, nullptr, nullptr);
  return CASS_OK;
}

int cass_encode_plan(const uint16_t* w, int64_t rows, int64_t cols, int64_t ld,
                     const cass_params* p, void* ws, int64_t ws_bytes, hipStream_t stream,
                     cass_plan* plan) {
  g_last_error.clear();
  int st = check_shape(rows, cols, p);
  if (st) return st;
  if (!plan) return fail(CASS_ERR_INVALID, "plan is NULL");
  if (ld < cols) return fail(CASS_ERR_INVALID, "ld %lld < cols %lld", (long long)ld, (long long)cols);
  if (rows > 0 && !w) return fail(CASS_ERR_INVALID, "w is NULL");
  const int64_t need = ws_layout(rows, cols, p->block, nullptr, nullptr);
  if (!ws) return fail(CASS_ERR_INVALID, "workspace is NULL");
  if (ws_bytes < need)
    return fail(CASS_ERR_CAPACITY, "workspace %lld < %lld bytes", (long long)ws_bytes,
                (long long)need);
  memset(plan, 0, sizeof *plan);
  plan->rows = rows;
  plan->cols = cols;
  plan->ld = ld;
  plan->p = *p;
  plan->ws = ws;
  plan->ws_bytes = ws_bytes;
  const Shape sh{rows, cols, p->block, p->keep, p->mant_bits, ld};
  const Workspace W = carve_workspace(ws, rows, cols, p->block);
  hipError_t e;
  if ((e = launch_select(w, sh, W.bitmap, stream)) != hipSuccess) return hip_fail(e, "select");
  if ((e = launch_histograms(w, sh, p->format, W, stream)) != hipSuccess)
    return hip_fail(e, "histograms");
  unsigned long long hist[512];
  if ((e = hipMemcpyAsync(hist, W.hist, sizeof hist, hipMemcpyDeviceToHost, stream)) != hipSuccess)
    return hip_fail(e, "histogram copy");
  if ((e = hipStreamSynchronize(stream)) != hipSuccess) return hip_fail(e, "synchronize");
  RankTables rt;
  for (int i = 0; i < 256; ++i) {
    plan->hist_kept[i] = hist[i];
    plan->hist_pruned[i] = hist[256 + i];
  }
  rank_table(plan->hist_kept, plan->perm_spec, rt.rank_kept);
  rank_table(plan->hist_pruned, plan->perm_verif, rt.rank_pruned);
  if ((e = launch_block_bits(w, sh, p->format, W, rt, stream)) != hipSuccess)
    return hip_fail(e, "code lengths");
  if ((e = launch_row_scan(sh, W, stream)) != hipSuccess) return hip_fail(e, "row scan");
  if ((e = launch_rows_scan(sh, W, stream)) != hipSuccess) return hip_fail(e, "rows scan");
  if (p->format == CASS_FMT_C1_SUPERBLOCK &&
      (e = launch_superblock_span(sh, W, CASS_SUPERBLOCK_BLOCKS, stream)) != hipSuccess)
    return hip_fail(e, "superblock span");
  unsigned long long totals[3];
  if ((e = hipMemcpyAsync(totals, W.totals, sizeof totals, hipMemcpyDeviceToHost, stream)) !=
      hipSuccess)
    return hip_fail(e, "totals copy");
  if ((e = hipStreamSynchronize(stream)) != hipSuccess) return hip_fail(e, "synchronize");
  if (is_c1_format(p->format)) {
    plan->spec_code_bits = totals[0];
  } else {
    plan->resid_bits = totals[0];
  }
  if (p->format == CASS_FMT_C1_SUPERBLOCK && totals[2] > 65535)
    return fail(CASS_ERR_OVERFLOW,
                "a block starts %llu code bits after its superblock's base (16-bit offsets); use "
                "format 1", (unsigned long long)totals[2]);
  plan->verif_code_bits = totals[1];
  std::vector<int64_t> ls, lv;
  stream_lengths(p->format, rows, cols, p->block, p->keep, p->mant_bits, totals[0], totals[1], ls,
                 lv);
  const Layout Ls = lay_out(ls), Lv = lay_out(lv);
  plan->spec_bytes = Ls.total;
  plan->verif_bytes = Lv.total;
  for (int s = 0; s < CASS_MAX_SECTIONS; ++s) {
    plan->spec_sec[s] = Ls.off[s];
    plan->spec_len[s] = Ls.len[s];
    plan->verif_sec[s] = Lv.off[s];
    plan->verif_len[s] = Lv.len[s];
  }
  return CASS_OK;
}

int cass_encode_tensor(const uint16_t* w, int64_t ld, const cass_plan* plan, void* spec,
                       int64_t spec_cap, void* verif, int64_t verif_cap, hipStream_t stream,
                       cass_tensor* out) {
  g_last_error.clear();
  if (!plan) return fail(CASS_ERR_INVALID, "plan is NULL");
  int st = check_shape(plan->rows, plan->cols, &plan->p);
  if (st) return st;
  if (ld != plan->ld) return fail(CASS_ERR_INVALID, "ld %lld differs from the plan's %lld",
                                  (long long)ld, (long long)plan->ld);
  if (!spec || !verif || !out) return fail(CASS_ERR_INVALID, "NULL stream buffer or descriptor");
  if (plan->rows > 0 && !w) return fail(CASS_ERR_INVALID, "w is NULL");
  if (((uintptr_t)spec | (uintptr_t)verif) % 256)
    return fail(CASS_ERR_INVALID, "stream buffers must be 256-byte aligned");
  if (spec_cap < plan->spec_bytes || verif_cap < plan->verif_bytes)
    return fail(CASS_ERR_CAPACITY, "stream buffers smaller than the plan's sizes");
  const cass_params* p = &plan->p;
  const Shape sh{plan->rows, plan->cols, p->block, p->keep, p->mant_bits, ld};
  const Workspace W = carve_workspace((void*)plan->ws, plan->rows, plan->cols, p->block);
  RankTables rt;
  for (int r = 0; r < 256; ++r) {
    rt.rank_kept[plan->perm_spec[r]] = (uint8_t)r;
    rt.rank_pruned[plan->perm_verif[r]] = (uint8_t)r;
  }
  std::vector<int64_t> ls, lv;
  const uint64_t code_a = is_c1_format(p->format) ? plan->spec_code_bits : plan->resid_bits;
  stream_lengths(p->format, plan->rows, plan->cols, p->block, p->keep, p->mant_bits, code_a,
                 plan->verif_code_bits, ls, lv);
  const Layout Ls = lay_out(ls), Lv = lay_out(lv);
  if (Ls.total != plan->spec_bytes || Lv.total != plan->verif_bytes)
    return fail(CASS_ERR_INVALID, "plan sizes are inconsistent");
  HeaderBlob hb;
  write_header(hb.spec_hdr, kMagicSpec, p->format, p->mant_bits, plan->rows, plan->cols, p->block,
               p->keep, Ls);
  write_header(hb.verif_hdr, kMagicVerif, p->format, p->mant_bits, plan->rows, plan->cols,
               p->block, p->keep, Lv);
  memcpy(hb.perm_spec, plan->perm_spec, 256);
  memcpy(hb.perm_verif, plan->perm_verif, 256);
  hipError_t e;
  if ((e = launch_fill_zero(spec, Ls.total, stream)) != hipSuccess) return hip_fail(e, "zero fill");
  if ((e = launch_fill_zero(verif, Lv.total, stream)) != hipSuccess) return hip_fail(e, "zero fill");
  const int64_t srank = is_c1_format(p->format) ? Ls.off[S1_RANK] : 0;
  const int64_t vrank = p->format == CASS_FMT_C2_MX_TARGET ? 0 : Lv.off[V1_RANK];
  if ((e = launch_write_headers(hb, (uint8_t*)spec, srank, (uint8_t*)verif, vrank,
                                stream)) != hipSuccess)
    return hip_fail(e, "headers");
  if ((e = launch_pack(w, sh, p->format, W, rt, (uint8_t*)spec, Ls.off, (uint8_t*)verif, Lv.off,
                       stream)) != hipSuccess)
    return hip_fail(e, "pack");
  memset(out, 0, sizeof *out);
  out->format = p->format;
  out->mant_bits = p->mant_bits;
  out->rows = plan->rows;
  out->cols = plan->cols;
  out->block = p->block;
  out->keep = p->keep;
  out->spec = spec;
  out->spec_bytes = Ls.total;
  out->verif = verif;
  out->verif_bytes = Lv.total;
  for (int s = 0; s < CASS_MAX_SECTIONS; ++s) {
    out->spec_sec[s] = Ls.off[s];
    out->verif_sec[s] = Lv.off[s];
  }
  return CASS_OK;
}

int cass_tensor_describe(const void* spec_header, const void* spec, int64_t spec_bytes,
                         const void* verif_header, const void* verif, int64_t verif_bytes,
                         cass_tensor* out) {
  g_last_error.clear();
  if (!spec_header || !spec || !out) return fail(CASS_ERR_INVALID, "NULL argument");
  const uint8_t* h = (const uint8_t*)spec_header;
  if (get32(h) != kMagicSpec || get32(h + 4) != 1)
    return fail(CASS_ERR_CORRUPT, "not a version-1 speculation stream header");
  memset(out, 0, sizeof *out);
  out->format = (int32_t)get32(h + 8);
  out->mant_bits = (int32_t)get32(h + 12);
  out->rows = get64(h + 16);
  out->cols = get64(h + 24);
  out->block = get64(h + 32);
  out->keep = get64(h + 40);
  out->spec = spec;
  out->spec_bytes = spec_bytes;
  if (get64(h + 48) > spec_bytes) return fail(CASS_ERR_CORRUPT, "speculation stream truncated");
  for (int s = 0; s < CASS_MAX_SECTIONS; ++s) out->spec_sec[s] = get64(h + 64 + 16 * s);
  if (verif_header && verif) {
    const uint8_t* v = (const uint8_t*)verif_header;
    if (get32(v) != kMagicVerif || get32(v + 4) != 1 || (int32_t)get32(v + 8) != out->format ||
        (int32_t)get32(v + 12) != out->mant_bits || get64(v + 16) != out->rows ||
        get64(v + 24) != out->cols || get64(v + 32) != out->block || get64(v + 40) != out->keep)
      return fail(CASS_ERR_CORRUPT, "verification header does not match");
    if (get64(v + 48) > verif_bytes) return fail(CASS_ERR_CORRUPT, "verification stream truncated");
    out->verif = verif;
    out->verif_bytes = verif_bytes;
    for (int s = 0; s < CASS_MAX_SECTIONS; ++s) out->verif_sec[s] = get64(v + 64 + 16 * s);
  }
  if (((uintptr_t)spec % 16) || (out->verif && ((uintptr_t)out->verif % 16)))
    return fail(CASS_ERR_INVALID, "stream buffers must be 16-byte aligned");
  // the header's own section table: fixed-size sections have their closed-form
  // lengths, and every section with its padding lies inside the stream
  cass_params pp = {out->format, out->mant_bits, out->block, out->keep};
  int st = check_shape(out->rows, out->cols, &pp);
  if (st) return fail(CASS_ERR_CORRUPT, "%s", g_last_error.c_str());
  const uint32_t want_sb = out->format == CASS_FMT_C1_SUPERBLOCK ? CASS_SUPERBLOCK_BLOCKS : 0u;
  if (get32(h + 60) != want_sb || (out->verif && get32((const uint8_t*)verif_header + 60) != want_sb))
    return fail(CASS_ERR_CORRUPT, "superblock size field does not match the format");
  for (int which = 0; which < (out->verif ? 2 : 1); ++which) {
    const uint8_t* hh = which == 0 ? h : (const uint8_t*)verif_header;
    const int64_t total = get64(hh + 48);
    const std::vector<int64_t> want = closed_lengths(which == 0, out->format, out->rows,
                                                     out->cols, out->block, out->keep,
                                                     out->mant_bits);
    if ((int64_t)get32(hh + 56) != (int64_t)want.size())
      return fail(CASS_ERR_CORRUPT, "section count does not match the format");
    for (size_t s = 0; s < want.size(); ++s) {
      const int64_t off = get64(hh + 64 + 16 * s), len = get64(hh + 72 + 16 * s);
      if (len < 0 || (want[s] >= 0 && len != want[s]) || off + len + 16 > total)
        return fail(CASS_ERR_CORRUPT, "%s section %d: length %lld does not fit the shape",
                    which == 0 ? "speculation" : "verification", (int)s, (long long)len);
    }
  }
  st = check_tensor(out, out->verif != nullptr);
  if (st) return st == CASS_ERR_INVALID ? fail(CASS_ERR_CORRUPT, "%s", g_last_error.c_str()) : st;
  return CASS_OK;
}

int cass_set_option(const char* name, int64_t value) {
  g_last_error.clear();
  static const struct { const char* name; Option o; int64_t lo, hi; } table[] = {
      {"gemv_parts", OPT_GEMV_PARTS, 0, 64}, {"gemv_path", OPT_GEMV_PATH, 0, 2},
      {"gemv_sub", OPT_GEMV_SUB, 0, 64},     {"exact_path", OPT_EXACT_PATH, 0, 1},
      {"exact_blocks", OPT_EXACT_BLOCKS, 0, 2}, {"kv_exact_path", OPT_KV_EXACT_PATH, 0, 1},
      {"kv_append_path", OPT_KV_APPEND_PATH, 0, 1}};
  if (!name) return fail(CASS_ERR_INVALID, "option name is NULL");
  for (const auto& t : table)
    if (strcmp(name, t.name) == 0) {
      if (value < t.lo || value > t.hi)
        return fail(CASS_ERR_INVALID, "option %s: value %lld outside %lld..%lld", name,
                    (long long)value, (long long)t.lo, (long long)t.hi);
      g_options[t.o].store((int)value, std::memory_order_relaxed);
      return CASS_OK;
    }
  return fail(CASS_ERR_INVALID, "unknown option %s", name);
}

int cass_draft_gemv(const cass_tensor* W, const uint16_t* x, int batch, int64_t ldx, float* y,
                    int64_t ldy, hipStream_t stream) {
  g_last_error.clear();
  int st = check_tensor(W, false);
  if (st) return st;
  if (batch < 1 || batch > 8) return fail(CASS_ERR_UNSUPPORTED, "batch %d outside 1..8", batch);
  if (W->rows == 0) return CASS_OK;
  if (!x || !y) return fail(CASS_ERR_INVALID, "x or y is NULL");
  if (ldx < W->cols || ldy < W->rows) return fail(CASS_ERR_INVALID, "ldx < cols or ldy < rows");
  const Shape sh = shape_of(W);
  const int64_t code_limit = is_c1_format(W->format) ? spec_c1(W).codes_limit : 0;
  const bool staged_ok =
      W->format == CASS_FMT_C1_SUPERBLOCK
          ? draft_gemv_bal_fits(sh, batch, code_limit, spec_c1s(W).nsb)
          : draft_gemv_staged_fits(sh, batch, W->format, code_limit);
  if (!staged_ok && draft_gemv_direct_lds_bytes(sh, batch) > 150 * 1024)
    return fail(CASS_ERR_UNSUPPORTED, "batch %d x cols %lld does not fit in LDS", batch,
                (long long)W->cols);
  hipError_t e =
      W->format == CASS_FMT_C1_UNARY
          ? launch_draft_gemv_c1(spec_c1(W), sh, x, batch, ldx, y, ldy, stream)
      : W->format == CASS_FMT_C1_SUPERBLOCK
          ? launch_draft_gemv_c1(spec_c1s(W), sh, x, batch, ldx, y, ldy, stream)
          : launch_draft_gemv_c2(spec_c2(W), sh, x, batch, ldx, y, ldy, stream);
  return e == hipSuccess ? CASS_OK : hip_fail(e, "draft gemv launch");
}

int cass_verify_gemm(const cass_tensor* W, const uint16_t* X, int ntok, int64_t ldx, float* Y,
                     int64_t ldy, hipStream_t stream) {
  g_last_error.clear();
  int st = check_tensor(W, true);
  if (st) return st;
  if (ntok < 1 || ntok > 16) return fail(CASS_ERR_UNSUPPORTED, "ntok %d outside 1..16", ntok);
  if (W->rows == 0) return CASS_OK;
  if (!X || !Y) return fail(CASS_ERR_INVALID, "X or Y is NULL");
  if (ldx < W->cols || ldy < W->rows) return fail(CASS_ERR_INVALID, "ldx < cols or ldy < rows");
  const Shape sh = shape_of(W);
  hipError_t e;
  if (W->format == CASS_FMT_C1_UNARY) {
    const SpecViewC1 sv = spec_c1(W);
    const VerifViewC1 vv = verif_c1(W);
    e = staged_exact_enabled() && exact_staged_fits(sh, sv, vv)
            ? launch_verify_gemm_c1_staged(sv, vv, sh, X, ntok, ldx, Y, ldy, stream)
            : launch_verify_gemm_c1(sv, vv, sh, X, ntok, ldx, Y, ldy, stream);
  } else if (W->format == CASS_FMT_C1_SUPERBLOCK) {
    const SpecViewC1 sv = spec_c1s(W);
    const VerifViewC1 vv = verif_c1(W);
    e = staged_exact_enabled() && exact_staged_fits(sh, sv, vv)
            ? launch_verify_gemm_c1_staged(sv, vv, sh, X, ntok, ldx, Y, ldy, stream)
            : launch_verify_gemm_c1(sv, vv, sh, X, ntok, ldx, Y, ldy, stream);
  } else if (W->format == CASS_FMT_C2_MX32) {
    e = launch_verify_gemm_c2(spec_c2(W), verif_c2(W), sh, X, ntok, ldx, Y, ldy, stream);
  } else {
    e = launch_verify_gemm_c3(spec_c2(W), verif_c3(W), sh, X, ntok, ldx, Y, ldy, stream);
  }
  return e == hipSuccess ? CASS_OK : hip_fail(e, "verify gemm launch");
}

int cass_reconstruct(const cass_tensor* W, uint16_t* out, hipStream_t stream) {
  g_last_error.clear();
  int st = check_tensor(W, true);
  if (st) return st;
  if (W->rows == 0) return CASS_OK;
  if (!out || ((uintptr_t)out % 16)) return fail(CASS_ERR_INVALID, "out must be 16-byte aligned");
  const Shape sh = shape_of(W);
  hipError_t e;
  if (W->format == CASS_FMT_C1_UNARY) {
    const SpecViewC1 sv = spec_c1(W);
    const VerifViewC1 vv = verif_c1(W);
    e = staged_exact_enabled() && exact_staged_fits(sh, sv, vv)
            ? launch_reconstruct_c1_staged(sv, vv, sh, out, stream)
            : launch_decode_c1(sv, &vv, sh, out, stream);
  } else if (W->format == CASS_FMT_C1_SUPERBLOCK) {
    const SpecViewC1 sv = spec_c1s(W);
    const VerifViewC1 vv = verif_c1(W);
    e = staged_exact_enabled() && exact_staged_fits(sh, sv, vv)
            ? launch_reconstruct_c1_staged(sv, vv, sh, out, stream)
            : launch_decode_c1(sv, &vv, sh, out, stream);
  } else if (W->format == CASS_FMT_C2_MX32) {
    const VerifViewC2 vv = verif_c2(W);
    e = launch_decode_c2(spec_c2(W), &vv, sh, out, stream);
  } else {
    e = launch_decode_c3(spec_c2(W), verif_c3(W), sh, out, stream);
  }
  return e == hipSuccess ? CASS_OK : hip_fail(e, "reconstruct launch");
}

int cass_draft_decode(const cass_tensor* W, uint16_t* out, hipStream_t stream) {
  g_last_error.clear();
  int st = check_tensor(W, false);
  if (st) return st;
  if (W->rows == 0) return CASS_OK;
  if (!out || ((uintptr_t)out % 16)) return fail(CASS_ERR_INVALID, "out must be 16-byte aligned");
  const Shape sh = shape_of(W);
  hipError_t e;
  if (W->format == CASS_FMT_C1_UNARY) {
    const SpecViewC1 sv = spec_c1(W);
    const VerifViewC1 none = {};
    e = staged_exact_enabled() && exact_staged_fits(sh, sv, none)
            ? launch_draft_decode_c1_staged(sv, sh, out, stream)
            : launch_decode_c1(sv, nullptr, sh, out, stream);
  } else if (W->format == CASS_FMT_C1_SUPERBLOCK) {
    const SpecViewC1 sv = spec_c1s(W);
    const VerifViewC1 none = {};
    e = staged_exact_enabled() && exact_staged_fits(sh, sv, none)
            ? launch_draft_decode_c1_staged(sv, sh, out, stream)
            : launch_decode_c1(sv, nullptr, sh, out, stream);
  } else {
    e = launch_decode_c2(spec_c2(W), nullptr, sh, out, stream);
  }
  return e == hipSuccess ? CASS_OK : hip_fail(e, "draft decode launch");
}

}  // extern "C"
