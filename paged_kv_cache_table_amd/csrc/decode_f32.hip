// Decode kernel instances for the (q, K, V) format combination kComboF32.
#include "decode_impl.hpp"

namespace pkv {

hipError_t launch_decode_split_f32(const AttnArgs& a, int hd, int bs, int g, int64_t max_units,
                                     hipStream_t st, bool* found) {
#define PKV_CASE(HD, BS, G)                                                  \
  if (hd == HD && bs == BS && g == G) {                                      \
    *found = true;                                                           \
    return launch_split_instance<HD, BS, G, kComboF32>(a, max_units, st);      \
  }
#define PKV_CASES_G(HD, BS) PKV_CASE(HD, BS, 1) PKV_CASE(HD, BS, 2) PKV_CASE(HD, BS, 3) PKV_CASE(HD, BS, 4) PKV_CASE(HD, BS, 8)
  PKV_CASES_G(64, 16)
  PKV_CASES_G(128, 16)
  PKV_CASES_G(256, 16)
  PKV_CASES_G(128, 32)
#undef PKV_CASES_G
#undef PKV_CASE
  *found = false;
  return hipSuccess;
}

}  // namespace pkv
