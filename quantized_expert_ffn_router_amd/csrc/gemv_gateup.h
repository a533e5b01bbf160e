// gemv_gateup.h -- the gate/up streaming pieces of the decode-size expert
// kernels (the two-launch gate/up GEMV and the one-launch fused FFN): a
// wave streams its K-groups of 128 NVFP4 elements of one matrix through a
// register ring and accumulates per-token sums in its LDS slice.
#pragma once

#include "gemv_common.h"

namespace moe {

constexpr int kGuMT = 16;  // tokens per batch (an expert's further tokens take more batches)

// Register ring of one pass: GPS groups of 128 elements (64 code bytes and 8
// E4M3 scale bytes per lane each).
template <int GPS>
struct GURing {
  uint4 rc[GPS][4];
  uint2 rs[GPS];
};

// Issue the loads of the first D groups of a pass.
template <int GPS, int D>
__device__ __forceinline__ void gu_issue(GURing<GPS>& R, const uint8_t* pq, const uint8_t* ps,
                                         int I, size_t nc, int gb) {
#pragma unroll
  for (int gi = 0; gi < GPS && gi < D; ++gi) {
    const int g = gb + gi;
#pragma unroll
    for (int q = 0; q < 4; ++q) R.rc[gi][q] = ld16(pq + (((size_t)(4 * g + q)) * I + nc) * 16);
    R.rs[gi] = ld8(ps + ((size_t)g * I + nc) * 8);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Row offset (elements) of the token of sorted assignment p: p's token is
// sorted_asg[p] / k (k a power of two in every shipped layer; the shift is
// negative otherwise and a division is used).
__device__ __forceinline__ size_t token_row(const int32_t* __restrict__ sorted_asg, int p,
                                            int ktop, int kshift, int H) {
  const int a = sorted_asg[p];
  const int tok = kshift >= 0 ? (a >> kshift) : a / ktop;
  return (size_t)tok * H;
}

// One pass of GPS groups over the mt tokens of sorted positions p0.., the
// first D groups already in flight.  The group loop unrolls fully, so the
// ring needs no loop-carried registers; D groups of weight loads stay in
// flight ahead of use, issued in group order (scheduling barriers keep them
// apart) so that waiting for group gi never waits for a later group.  Each
// group is decoded once to bf16 pairs; the token loop is a plain loop (the
// register footprint does not grow with the batch) whose activations come
// from scalar loads and whose per-token sums accumulate in this wave's LDS
// slice acc[t * 64 + lane].
template <int GPS, int D>
__device__ __forceinline__ void gu_consume(GURing<GPS>& R, const uint16_t* __restrict__ x,
                                           const int32_t* __restrict__ sorted_asg, int p0,
                                           int ktop, int kshift, int H, int I, size_t nc,
                                           const uint8_t* pq, const uint8_t* ps, int gb, int mt,
                                           float* acc) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int gi = 0; gi < GPS; ++gi) {
    if (gi + D < GPS) {  // keep D groups in flight
      const int g2 = gb + gi + D;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        R.rc[gi + D][q] = ld16(pq + (((size_t)(4 * g2 + q)) * I + nc) * 16);
      R.rs[gi + D] = ld8(ps + ((size_t)g2 * I + nc) * 8);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int g = gb + gi;
    float sc[8];
    e4m3x8(R.rs[gi], sc);
    v2bf_t w[8][8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      e2m1x8_bf16(word_of(R.rc[gi][b >> 1], (b & 1) * 2), w[b]);
      e2m1x8_bf16(word_of(R.rc[gi][b >> 1], (b & 1) * 2 + 1), w[b] + 4);
    }
#pragma unroll 1
    for (int t = 0; t < mt; ++t) {
      const uint32_t* xp =
          reinterpret_cast<const uint32_t*>(x + token_row(sorted_asg, p0 + t, ktop, kshift, H)) +
          64 * g;
      float a = 0.0f;
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        float p = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          p = __builtin_amdgcn_fdot2_f32_bf16(as_v2bf(xp[8 * b + i]), w[b][i], p, false);
        a = fmaf(p, sc[b], a);
      }
      acc[t * 64 + lane] += a;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// K split of the gate/up streaming over S waves per matrix (the largest
// divisor of NG = H/128 up to 4; 8 when the grid of RB row blocks x
// max_slots experts leaves CUs idle, i.e. at most 256 workgroups of 16 waves)
// and passes of GP <= 8 of each wave's gps_total groups.
inline void gu_split(int H, int RB, int max_slots, int* S, int* GP, int* gps_total) {
  const int NG = H / 128;
  int s = 4;
  while (NG % s) --s;
  if (NG % 8 == 0 && (int64_t)RB * max_slots <= 256) s = 8;
  const int gt = NG / s;
  int gp = gt;
  if (gp > 8) {
    gp = 8;
    while (gt % gp) --gp;
  }
  *S = s;
  *GP = gp;
  *gps_total = gt;
}

}  // namespace moe
