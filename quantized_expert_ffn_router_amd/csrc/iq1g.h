// iq1g.h -- the grid of the IQ1-style ternary codebook format (MOE_FMT_IQ1G).
//
// The pages' packs include IQ1_M GGUF tensors (basalt.jgulfo.com, "Models"),
// a codebook format of under two bits per weight whose grid the pages do not
// give.  This format defines its own: the 1024 vectors of eight values in
// {-1, 0, +1} with the fewest nonzero values, ordered by the number of nonzero
// values and then lexicographically (-1 < 0 < +1, value 0 the most
// significant): every vector with at most 3 nonzero values (577), then the
// first 447 with 4.  Entry e is the e-th such vector.
//
// Built at compile time by a counting sort on the nonzero count: every vector
// is visited in lexicographic order and placed at the next free position of
// its count's range, so equal counts keep lexicographic order.
#pragma once

#include <stdint.h>

namespace moe {

struct Iq1gGrid {
  uint16_t c[1024];  // entry e: value i nonzero at bit 2i, negative at bit 2i + 1
};

constexpr Iq1gGrid make_iq1g_grid() {
  int count[10] = {};
  for (int u = 0; u < 6561; ++u) {
    int nz = 0;
    for (int r = u, i = 0; i < 8; ++i, r /= 3) nz += (r % 3) != 1;
    ++count[nz + 1];
  }
  for (int n = 1; n < 10; ++n) count[n] += count[n - 1];  // count[n] = first slot of n nonzeros
  Iq1gGrid g{};
  for (int u = 0; u < 6561; ++u) {  // base-3 digit 7 - i is value i + 1: lexicographic order
    int nz = 0, code = 0;
    for (int i = 0, r = u; i < 8; ++i, r /= 3) {
      const int v = r % 3 - 1;  // value 7 - i
      nz += v != 0;
      if (v != 0) code |= (v < 0 ? 3 : 1) << (2 * (7 - i));
    }
    const int slot = count[nz]++;
    if (slot < 1024) g.c[slot] = (uint16_t)code;
  }
  return g;
}

#if defined(__HIPCC__)
// The grid in device memory (each translation unit that uses it keeps a copy).
static __device__ const Iq1gGrid kIq1gGridDev = make_iq1g_grid();
#endif

// Bytes per 256-weight superblock in the canonical layout: d fp16, 8 x 4-bit
// sub-block multipliers, 32 low index bytes, 8 bytes of 2-bit high index parts.
constexpr int kIq1gBlockBytes = 46;

}  // namespace moe
