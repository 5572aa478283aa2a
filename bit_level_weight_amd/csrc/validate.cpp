// cass_tensor_validate: host-side structural check of a stream pair held in
// host memory.  It walks every row once: bitmap counts, kept-before counts,
// and every unary code, checking that row bases and block offsets land on
// code boundaries and that no code runs past its section.
#include <string.h>

#include <string>
#include <vector>

#include "cassandra.h"

namespace {

constexpr uint32_t kMagicSpec = 0x50535343u, kMagicVerif = 0x46565343u;

struct Hdr {
  uint32_t format, mant, nsec;
  int64_t R, C, B, k, total;
  int64_t off[CASS_MAX_SECTIONS], len[CASS_MAX_SECTIONS];
};

uint32_t rd32(const uint8_t* p) { uint32_t v; memcpy(&v, p, 4); return v; }
int64_t rd64(const uint8_t* p) { int64_t v; memcpy(&v, p, 8); return v; }

bool parse(const uint8_t* b, int64_t n, uint32_t magic, Hdr* h) {
  if (!b || n < 256 || rd32(b) != magic || rd32(b + 4) != 1) return false;
  h->format = rd32(b + 8);
  h->mant = rd32(b + 12);
  h->R = rd64(b + 16);
  h->C = rd64(b + 24);
  h->B = rd64(b + 32);
  h->k = rd64(b + 40);
  h->total = rd64(b + 48);
  h->nsec = rd32(b + 56);
  if (h->format < 1 || h->format > 4) return false;
  if (rd32(b + 60) != (h->format == 4 ? (uint32_t)CASS_SUPERBLOCK_BLOCKS : 0u)) return false;
  if (h->mant > 7 || h->R < 0 || h->C <= 0 || h->C > 65536 || h->B < 32 || (h->B & (h->B - 1)) ||
      h->C % h->B || h->k < 0 || h->k > h->C || h->total > n || h->total < 256 ||
      h->nsec > CASS_MAX_SECTIONS)
    return false;
  if (h->R > ((int64_t)1 << 40) / h->C) return false;
  const bool c1f = h->format == 1 || h->format == 4;
  const uint32_t want = magic == kMagicSpec ? (c1f ? 7u : 4u)
                                            : (c1f ? 6u : h->format == 2 ? 8u : 3u);
  if (h->nsec != want) return false;
  for (int s = 0; s < CASS_MAX_SECTIONS; ++s) {
    h->off[s] = rd64(b + 64 + 16 * s);
    h->len[s] = rd64(b + 72 + 16 * s);
    if (s < (int)h->nsec &&
        (h->off[s] < 256 || h->off[s] % 256 || h->len[s] < 0 || h->off[s] + h->len[s] > h->total))
      return false;
  }
  return true;
}

struct Bits {
  const uint8_t* p;
  uint64_t nbits;
  bool get(uint64_t i) const { return (p[i >> 3] >> (i & 7)) & 1; }
  // unary code at *pos; false if it runs past the end or beyond `limit` zeros
  bool unary(uint64_t* pos, int limit, int* r) const {
    for (int z = 0; z <= limit; ++z) {
      if (*pos + z >= nbits) return false;
      if (get(*pos + z)) {
        *r = z;
        *pos += z + 1;
        return true;
      }
    }
    return false;
  }
};

Bits sec_bits(const uint8_t* b, const Hdr& h, int s) {
  return Bits{b + h.off[s], (uint64_t)h.len[s] * 8};
}

}  // namespace

extern "C" int cass_tensor_validate(const void* spec_v, int64_t spec_bytes, const void* verif_v,
                                    int64_t verif_bytes) {
  const uint8_t* spec = (const uint8_t*)spec_v;
  const uint8_t* verif = (const uint8_t*)verif_v;
  Hdr hs, hv;
  if (!parse(spec, spec_bytes, kMagicSpec, &hs)) return CASS_ERR_CORRUPT;
  const bool c1 = hs.format == 1 || hs.format == 4;
  const bool sbm = hs.format == 4;  // superblock metadata
  if (verif) {
    if (!parse(verif, verif_bytes, kMagicVerif, &hv)) return CASS_ERR_CORRUPT;
    if (hv.format != hs.format || hv.mant != hs.mant || hv.R != hs.R || hv.C != hs.C ||
        hv.B != hs.B || hv.k != hs.k)
      return CASS_ERR_CORRUPT;
  }
  const int64_t R = hs.R, C = hs.C, B = hs.B, k = hs.k, nb = C / B;
  const int m = (int)hs.mant;
  // fixed-size sections must have their closed-form lengths
  const int bm_sec = c1 ? 1 : 0, kb_sec = c1 ? 4 : 2, f_sec = c1 ? 5 : 3;
  if (hs.len[bm_sec] != R * C / 8 || hs.len[kb_sec] != 2 * R * nb ||
      hs.len[f_sec] != (R * k * (c1 ? 1 + m : 2 + m) + 7) / 8)
    return CASS_ERR_CORRUPT;
  const int64_t SB = CASS_SUPERBLOCK_BLOCKS, nsb = (nb + SB - 1) / SB;
  if (c1 && !sbm && (hs.len[0] != 256 || hs.len[2] != 8 * R || hs.len[3] != 4 * R * nb))
    return CASS_ERR_CORRUPT;
  if (sbm && (hs.len[0] != 256 || hs.len[2] != 8 * R * nsb || hs.len[3] != 2 * R * nb))
    return CASS_ERR_CORRUPT;
  if (!c1 && hs.len[1] != R * C / 32) return CASS_ERR_CORRUPT;
  if (hs.format == 3) {
    // MX-quantised target: fixed-size verification sections; each group
    // exponent is at least 1 and equals the speculation stream's shared
    // exponent wherever the group keeps a value
    const uint8_t* bmb = spec + hs.off[0];
    for (int64_t r = 0; r < R; ++r) {
      uint16_t kbv;
      int64_t kept = 0;
      for (int64_t j = 0; j < C; ++j) {
        if (j % B == 0) {
          memcpy(&kbv, spec + hs.off[2] + 2 * (r * nb + j / B), 2);
          if (kbv != (uint16_t)kept) return CASS_ERR_CORRUPT;
        }
        kept += (bmb[(r * C + j) >> 3] >> ((r * C + j) & 7)) & 1;
      }
      if (kept != k) return CASS_ERR_CORRUPT;
    }
    if (!verif) return CASS_OK;
    if (hv.len[0] != R * C / 32 || hv.len[1] != (R * k * (7 - m) + 7) / 8 ||
        hv.len[2] != (R * (C - k) * 9 + 7) / 8)
      return CASS_ERR_CORRUPT;
    const uint8_t* shexp = spec + hs.off[1];
    const uint8_t* gexp = verif + hv.off[0];
    for (int64_t g = 0; g < R * C / 32; ++g)
      if (gexp[g] < 1 || (shexp[g] != 0 && shexp[g] != gexp[g])) return CASS_ERR_CORRUPT;
    return CASS_OK;
  }
  if (verif) {
    if (hv.len[0] != 256 || hv.len[1] != 8 * R || hv.len[2] != 4 * R * nb) return CASS_ERR_CORRUPT;
    if (c1 && (hv.len[3] != (R * k * (7 - m) + 7) / 8 || hv.len[4] != R * (C - k)))
      return CASS_ERR_CORRUPT;
    if (!c1 && (hv.len[4] != R * (C - k) || hv.len[5] != 8 * R || hv.len[6] != 4 * R * nb))
      return CASS_ERR_CORRUPT;
  }
  const Bits bm = sec_bits(spec, hs, bm_sec);
  const uint8_t* keptb = spec + hs.off[kb_sec];
  Bits scodes{nullptr, 0}, vcodes{nullptr, 0}, resid{nullptr, 0};
  if (c1) scodes = sec_bits(spec, hs, 6);
  if (verif) {
    vcodes = sec_bits(verif, hv, c1 ? 5 : 7);
    if (!c1) resid = sec_bits(verif, hv, 3);
  }
  const uint8_t* shexp = c1 ? nullptr : spec + hs.off[1];
  uint64_t spos = 0, vpos = 0, kpos = 0;
  for (int64_t r = 0; r < R; ++r) {
    uint64_t sbase = spos, vbase = vpos, kbase = kpos;
    if (c1 && (uint64_t)rd64(spec + hs.off[2] + 8 * (sbm ? r * nsb : r)) != spos) return CASS_ERR_CORRUPT;
    uint64_t sb_base = spos;
    if (verif) {
      if (c1 && (uint64_t)rd64(verif + hv.off[1] + 8 * r) != vpos) return CASS_ERR_CORRUPT;
      if (!c1 && ((uint64_t)rd64(verif + hv.off[1] + 8 * r) != kpos ||
                  (uint64_t)rd64(verif + hv.off[5] + 8 * r) != vpos))
        return CASS_ERR_CORRUPT;
    }
    int64_t kept = 0;
    for (int64_t j = 0; j < C; ++j) {
      if (j % B == 0) {
        const int64_t blk = r * nb + j / B;
        uint16_t kbv;
        memcpy(&kbv, keptb + 2 * blk, 2);
        if (kbv != (uint16_t)kept) return CASS_ERR_CORRUPT;
        if (sbm) {
          if ((j / B) % SB == 0) {
            sb_base = spos;
            if ((uint64_t)rd64(spec + hs.off[2] + 8 * (r * nsb + (j / B) / SB)) != spos)
              return CASS_ERR_CORRUPT;
          }
          uint16_t o16;
          memcpy(&o16, spec + hs.off[3] + 2 * blk, 2);
          if (spos - sb_base > 65535 || o16 != (uint16_t)(spos - sb_base)) return CASS_ERR_CORRUPT;
        } else if (c1 && rd32(spec + hs.off[3] + 4 * blk) != (uint32_t)(spos - sbase)) {
          return CASS_ERR_CORRUPT;
        }
        if (verif) {
          if (c1 && rd32(verif + hv.off[2] + 4 * blk) != (uint32_t)(vpos - vbase))
            return CASS_ERR_CORRUPT;
          if (!c1 && (rd32(verif + hv.off[2] + 4 * blk) != (uint32_t)(kpos - kbase) ||
                      rd32(verif + hv.off[6] + 4 * blk) != (uint32_t)(vpos - vbase)))
            return CASS_ERR_CORRUPT;
        }
      }
      int rank;
      if (bm.get((uint64_t)(r * C + j))) {
        if (++kept > k) return CASS_ERR_CORRUPT;
        if (c1 && !scodes.unary(&spos, 255, &rank)) return CASS_ERR_CORRUPT;
        if (!c1 && verif) {
          const int E = shexp[(r * C + j) / 32];
          if (!resid.unary(&kpos, 254, &rank) || rank >= E) return CASS_ERR_CORRUPT;
          const int wd = 7 - m + rank < 8 ? 7 - m + rank : 8;
          kpos += wd;
          if (kpos > resid.nbits) return CASS_ERR_CORRUPT;
        }
      } else if (verif) {
        if (!vcodes.unary(&vpos, 255, &rank)) return CASS_ERR_CORRUPT;
      }
    }
    if (kept != k) return CASS_ERR_CORRUPT;
  }
  return CASS_OK;
}
