// combine.hip -- gate-weighted combine of the expert outputs.
//
// The mixture's output for a token is the sum of its selected experts'
// outputs weighted by the gate weights; a token goes through only a small
// subset of the experts (basalt.jgulfo.com, section "Expert tiers").  It is
// written as a gather over
// the token's k assignments (position asg_pos[t*k+j] of the sorted expert
// outputs), summed in fp32 with j ascending, plus the optional residual, then
// rounded once to bf16 -- so the result never depends on scheduling.
#include "common.h"

namespace moe {

namespace {

// Eight columns per thread.  The k assignments are taken 8 at a time: first
// their positions and gate weights, then all their expert-output rows, so a
// token costs two dependent memory round trips per 8 assignments instead of
// two per assignment; the sum still runs over j in ascending order.  In a
// group with fewer than 8 assignments left the loads repeat the last one,
// which is never added.
template <bool YBF16>
__global__ __launch_bounds__(256) void k_combine(const void* __restrict__ y,
                                                 const int32_t* __restrict__ asg_pos,
                                                 const float* __restrict__ w, int64_t T, int k, int H,
                                                 const uint16_t* __restrict__ residual,
                                                 uint16_t* __restrict__ out) {
  const int n0 = (blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (n0 >= H) return;
  for (int64_t t = blockIdx.y; t < T; t += gridDim.y) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += 8) {
      const int nj = min(8, k - j0);
      size_t p[8];
      float wj[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const size_t a = (size_t)t * k + j0 + min(j, nj - 1);
        p[j] = (size_t)asg_pos[a];
        wj[j] = w[a];
      }
      float v[8][8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (YBF16) {
          const uint4 q = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(y) + p[j] * H + n0);
          v[j][0] = __uint_as_float(q.x << 16); v[j][1] = __uint_as_float(q.x & 0xffff0000u);
          v[j][2] = __uint_as_float(q.y << 16); v[j][3] = __uint_as_float(q.y & 0xffff0000u);
          v[j][4] = __uint_as_float(q.z << 16); v[j][5] = __uint_as_float(q.z & 0xffff0000u);
          v[j][6] = __uint_as_float(q.w << 16); v[j][7] = __uint_as_float(q.w & 0xffff0000u);
        } else {
          const float4* yp = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(y) + p[j] * H + n0);
          const float4 a = yp[0], b = yp[1];
          v[j][0] = a.x; v[j][1] = a.y; v[j][2] = a.z; v[j][3] = a.w;
          v[j][4] = b.x; v[j][5] = b.y; v[j][6] = b.z; v[j][7] = b.w;
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < nj) {
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj[j], v[j][i], acc[i]);
        }
      }
    }
    if (residual) {
      uint4 r = *reinterpret_cast<const uint4*>(residual + (size_t)t * H + n0);
      acc[0] = __uint_as_float(r.x << 16) + acc[0]; acc[1] = __uint_as_float(r.x & 0xffff0000u) + acc[1];
      acc[2] = __uint_as_float(r.y << 16) + acc[2]; acc[3] = __uint_as_float(r.y & 0xffff0000u) + acc[3];
      acc[4] = __uint_as_float(r.z << 16) + acc[4]; acc[5] = __uint_as_float(r.z & 0xffff0000u) + acc[5];
      acc[6] = __uint_as_float(r.w << 16) + acc[6]; acc[7] = __uint_as_float(r.w & 0xffff0000u) + acc[7];
    }
    uint4 o;
    o.x = (uint32_t)f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
    o.y = (uint32_t)f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
    o.z = (uint32_t)f32_to_bf16_rne(acc[4]) | ((uint32_t)f32_to_bf16_rne(acc[5]) << 16);
    o.w = (uint32_t)f32_to_bf16_rne(acc[6]) | ((uint32_t)f32_to_bf16_rne(acc[7]) << 16);
    *reinterpret_cast<uint4*>(out + (size_t)t * H + n0) = o;
  }
}

}  // namespace

hipError_t launch_combine(const void* y, int y_dtype, const int32_t* asg_pos, const float* w,
                          int64_t T, int k, int H, const uint16_t* residual, uint16_t* out,
                          hipStream_t s) {
  // Small batches: one wavefront per 512 columns, so a token is spread over
  // H / 512 workgroups (more CUs issuing its loads); large batches: 256
  // threads per workgroup.
  const unsigned threads = T <= 64 ? 64u : 256u;
  dim3 grid((unsigned)((H / 8 + threads - 1) / threads), (unsigned)(T < 65535 ? T : 65535));
  if (y_dtype == MOE_DTYPE_BF16)
    hipLaunchKernelGGL(k_combine<true>, grid, dim3(threads), 0, s, y, asg_pos, w, T, k, H, residual, out);
  else
    hipLaunchKernelGGL(k_combine<false>, grid, dim3(threads), 0, s, y, asg_pos, w, T, k, H, residual, out);
  return hipGetLastError();
}

}  // namespace moe
