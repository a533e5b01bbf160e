// iq3g.h -- the grid of the IQ3-style codebook format (MOE_FMT_IQ3G).
//
// The pages' packs include IQ3 GGUF files (basalt.jgulfo.com, "Community"),
// whose weights decode four at a time through a grid of magnitudes; the pages
// do not give that grid, so this format defines its own: the 256 smallest
// vectors of four positive odd integers (up to 15), ordered by squared norm
// and then lexicographically.  Entry e is the e-th such vector.  Its largest
// magnitude is 9 (the shells are whole up to norm 108, 247 vectors, then 9 of
// norm 116).
//
// Built at compile time by a counting sort on the squared norm: every vector
// is visited in lexicographic order and placed at the next free position of
// its norm's range, so equal norms keep lexicographic order.
#pragma once

#include <stdint.h>

namespace moe {

struct Iq3gGrid {
  uint32_t m[256];  // entry e: magnitudes m0..m3 in bytes 0..3
};

constexpr Iq3gGrid make_iq3g_grid() {
  constexpr int kMaxNorm = 4 * 15 * 15;
  int count[kMaxNorm + 2] = {};
  for (int v = 0; v < 4096; ++v) {
    int n = 0;
    for (int c = 0; c < 4; ++c) {
      const int m = 2 * ((v >> (3 * c)) & 7) + 1;
      n += m * m;
    }
    ++count[n + 1];
  }
  for (int n = 1; n <= kMaxNorm + 1; ++n) count[n] += count[n - 1];  // count[n] = first slot of norm n
  Iq3gGrid g{};
  for (int v = 0; v < 4096; ++v) {  // digit 3 (bits 9..11) is m0: lexicographic order
    const int m0 = 2 * ((v >> 9) & 7) + 1, m1 = 2 * ((v >> 6) & 7) + 1;
    const int m2 = 2 * ((v >> 3) & 7) + 1, m3 = 2 * (v & 7) + 1;
    const int slot = count[m0 * m0 + m1 * m1 + m2 * m2 + m3 * m3]++;
    if (slot < 256)
      g.m[slot] = (uint32_t)m0 | ((uint32_t)m1 << 8) | ((uint32_t)m2 << 16) | ((uint32_t)m3 << 24);
  }
  return g;
}

#if defined(__HIPCC__)
// The grid in device memory (each translation unit that uses it keeps a copy).
static __device__ const Iq3gGrid kIq3gGridDev = make_iq3g_grid();
#endif

// Bytes per 256-weight superblock in the canonical layout: d fp16, 8 x 4-bit
// sub-block multipliers, 64 grid indices, 32 sign bytes.
constexpr int kIq3gBlockBytes = 102;

}  // namespace moe
