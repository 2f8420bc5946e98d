// Host check of the packed-format conversions (sparse_gemm_patch_amd/csrc/layout.h),
// built with -fsanitize=address,undefined by tests/test_host_sanitizers.py.
//
// For every tile size and several tile counts: row-major pools of exactly the
// documented sizes (so that any index past a pool trips the address
// sanitizer) are converted to the device order and back; the round trip must
// be the identity, and every device-order element must be written exactly once
// (the map is a bijection).  Exit status 0 on success.
#include <stdint.h>
#include <stdio.h>

#include <vector>

#include "../../sparse_gemm_patch_amd/csrc/layout.h"

using namespace patch_layout;

static uint32_t lcg(uint32_t& s) {
  s = s * 1664525u + 1013904223u;
  return s >> 8;
}

template <typename T, typename Fwd, typename Back>
static int round_trip(const char* what, int64_t elems, Fwd to_dev, Back from_dev, uint32_t seed) {
  std::vector<T> rm(elems), dev(elems), back(elems);
  for (auto& v : rm) v = (T)lcg(seed);
  to_dev(rm.data(), dev.data());
  from_dev(dev.data(), back.data());
  int bad = 0;
  for (int64_t i = 0; i < elems; ++i) bad += rm[i] != back[i];
  if (bad) printf("%s: %d mismatches\n", what, bad);
  return bad;
}

int main() {
  int bad = 0;
  const int sizes[2] = {64, 128};
  const int64_t counts[3] = {1, 3, 17};
  for (int tn : sizes)
    for (int tk : sizes)
      for (int64_t tiles : counts) {
        const int64_t dv = tiles * tn * tk, sv = tiles * tn * tk / 2, sm = tiles * tn * tk / 8;
        bad += round_trip<uint16_t>(
            "dense", dv, [&](const uint16_t* rm, uint16_t* dev) { dense_from_row_major(rm, dev, tiles, tn, tk); },
            [&](const uint16_t* dev, uint16_t* rm) { dense_to_row_major(dev, rm, tiles, tn, tk); }, 1u + tn + tk);
        bad += round_trip<uint16_t>(
            "2:4 values", sv,
            [&](const uint16_t* rm, uint16_t* dev) { sparse_values_from_row_major(rm, dev, tiles, tn, tk); },
            [&](const uint16_t* dev, uint16_t* rm) { sparse_values_to_row_major(dev, rm, tiles, tn, tk); }, 7u + tn);
        bad += round_trip<uint8_t>(
            "2:4 codes", sm,
            [&](const uint8_t* rm, uint8_t* dev) { sparse_codes_from_row_major(rm, dev, tiles, tn, tk); },
            [&](const uint8_t* dev, uint8_t* rm) { sparse_codes_to_row_major(dev, rm, tiles, tn, tk); }, 11u + tk);
        // every device position is the image of exactly one row-major position
        std::vector<int> seen_d(dv / tiles, 0), seen_s(sv / tiles, 0), seen_m(sm / tiles, 0);
        for (int64_t r = 0; r < tn; ++r) {
          for (int64_t c = 0; c < tk; ++c) ++seen_d.at(dense_index(r, c, tn));
          for (int64_t c = 0; c < tk / 2; ++c) ++seen_s.at(sparse_value_index(r, c, tn));
          for (int64_t b = 0; b < tk / 8; ++b) ++seen_m.at(sparse_code_index(r, b, tn));
        }
        for (int v : seen_d) bad += v != 1;
        for (int v : seen_s) bad += v != 1;
        for (int v : seen_m) bad += v != 1;
      }
  printf("layout round trips: %s\n", bad ? "FAILED" : "ok");
  return bad ? 1 : 0;
}
