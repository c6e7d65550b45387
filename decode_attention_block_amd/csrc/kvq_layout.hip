// kvq_layout.hip — host-side converters of int4 block regions between the order the
// library stores (the operand order of the gfx950 matrix cores, see kvq_device.h) and
// natural order ([64 tokens][D/2 bytes], channel 2k in the low nibble of byte k). Host
// memory only, no GPU work: for callers that read a cache back or write one
// themselves.
#include <stdint.h>

#include "kvq.h"

namespace {

// Stored position of nibble q (0..7) of dword f (0..D/8-1) of lane l (0..63): byte
// ((f / 4) * 64 + l) * 16 + (f % 4) * 4 + q / 2, the low nibble for even q. That nibble
// holds, for K, channel 32 (f % (D/32)) + 8 (l / 16) + q of token 16 (f / (D/32)) + l % 16;
// for V, token 32 (f % 2) + 8 (l / 16) + q of channel 16 (f / 2) + l % 16.
template <class Visit>
void for_each_nibble(int D, bool is_v, Visit visit) {
  const int F = D / 8, KS = D / 32;
  for (int f = 0; f < F; ++f)
    for (int l = 0; l < 64; ++l)
      for (int q = 0; q < 8; ++q) {
        const int sbyte = ((f / 4) * 64 + l) * 16 + (f % 4) * 4 + q / 2;
        int t, c;
        if (!is_v) {
          t = 16 * (f / KS) + l % 16;
          c = 32 * (f % KS) + 8 * (l / 16) + q;
        } else {
          t = 32 * (f % 2) + 8 * (l / 16) + q;
          c = 16 * (f / 2) + l % 16;
        }
        visit(sbyte, q & 1, t * (D / 2) + c / 2, c & 1);
      }
}

int convert(const uint8_t* src, uint8_t* dst, int32_t head_dim, int32_t is_v, int64_t n,
            bool to_natural) {
  if (!src || !dst || n < 0) return KVQ_EINVAL;
  if (head_dim != 64 && head_dim != 128) return KVQ_ENOTSUP;
  const int64_t region = 32 * static_cast<int64_t>(head_dim);
  for (int64_t r = 0; r < n; ++r) {
    const uint8_t* s = src + r * region;
    uint8_t* d = dst + r * region;
    for (int64_t i = 0; i < region; ++i) d[i] = 0;
    for_each_nibble(head_dim, is_v != 0, [&](int sb, int sh, int nb, int nh) {
      if (to_natural)
        d[nb] = static_cast<uint8_t>(d[nb] | (((s[sb] >> (4 * sh)) & 0xF) << (4 * nh)));
      else
        d[sb] = static_cast<uint8_t>(d[sb] | (((s[nb] >> (4 * nh)) & 0xF) << (4 * sh)));
    });
  }
  return KVQ_OK;
}

}  // namespace

extern "C" int kvq_int4_to_natural(const uint8_t* stored, uint8_t* natural, int32_t head_dim,
                                   int32_t is_v, int64_t n_regions) {
  return convert(stored, natural, head_dim, is_v, n_regions, true);
}

extern "C" int kvq_int4_from_natural(const uint8_t* natural, uint8_t* stored, int32_t head_dim,
                                     int32_t is_v, int64_t n_regions) {
  return convert(natural, stored, head_dim, is_v, n_regions, false);
}
