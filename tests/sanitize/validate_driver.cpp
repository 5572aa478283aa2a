// Exercises the library's host-side stream validator (cass_tensor_validate)
// under AddressSanitizer and UndefinedBehaviorSanitizer, on streams the CPU
// oracle writes in every format and on corrupted copies of them: valid
// streams pass, corrupted ones are refused or pass, and nothing is read
// outside the buffers.  Exit status 0 on success.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "cass_oracle.h"
#include "cassandra.h"

static uint64_t st = 0x2545F4914F6CDD1Dull;
static uint64_t next_u64() {
  st ^= st << 13;
  st ^= st >> 7;
  st ^= st << 17;
  return st;
}

int main() {
  for (int fmt = 1; fmt <= 4; ++fmt) {
    const int64_t R = 6, C = 1024, k = 300, m = 3, B = 256;
    std::vector<uint16_t> w(R * C);
    for (auto& v : w) v = (uint16_t)next_u64();
    int64_t sb = 0, vb = 0;
    if (orc_encode(w.data(), R, C, k, m, B, fmt, nullptr, 0, nullptr, 0, &sb, &vb) != ORC_OK) {
      std::fprintf(stderr, "oracle sizes failed (format %d)\n", fmt);
      return 1;
    }
    std::vector<uint8_t> spec(sb), verif(vb);
    if (orc_encode(w.data(), R, C, k, m, B, fmt, spec.data(), sb, verif.data(), vb, &sb, &vb) != ORC_OK)
      continue;  // format 4 may refuse random exponents (16-bit offsets)
    if (cass_tensor_validate(spec.data(), sb, verif.data(), vb) != CASS_OK) {
      std::fprintf(stderr, "valid stream refused (format %d)\n", fmt);
      return 1;
    }
    for (int t = 0; t < 200; ++t) {
      std::vector<uint8_t> bad = (t & 1) ? verif : spec;
      bad[next_u64() % bad.size()] ^= (uint8_t)(1u << (next_u64() & 7));
      const int r = (t & 1) ? cass_tensor_validate(spec.data(), sb, bad.data(), vb)
                            : cass_tensor_validate(bad.data(), sb, verif.data(), vb);
      if (r != CASS_OK && r != CASS_ERR_CORRUPT) return 1;
    }
    if (cass_tensor_validate(spec.data(), 200, nullptr, 0) != CASS_ERR_CORRUPT) return 1;
  }
  std::printf("validate driver ok\n");
  return 0;
}
