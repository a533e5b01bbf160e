// combine.hip -- gate-weighted combine of the expert outputs.
//
// The mixture's output for a token is the sum of its selected experts'
// outputs weighted by the gate weights ("each token uses only a few experts":
// basalt.jgulfo.com, section "Expert tiers").  It is written as a gather over
// the token's k assignments (position asg_pos[t*k+j] of the sorted expert
// outputs), summed in fp32 with j ascending, plus the optional residual, then
// rounded once to bf16 -- so the result never depends on scheduling.
#include "common.h"

namespace moe {

namespace {

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
  for (int j = 0; j < k; ++j) {
    const size_t p = (size_t)asg_pos[(size_t)t * k + j];
    const float wj = w[(size_t)t * k + j];
    float v[8];
    if (YBF16) {
      uint4 q = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(y) + p * H + n0);
      v[0] = __uint_as_float(q.x << 16); v[1] = __uint_as_float(q.x & 0xffff0000u);
      v[2] = __uint_as_float(q.y << 16); v[3] = __uint_as_float(q.y & 0xffff0000u);
      v[4] = __uint_as_float(q.z << 16); v[5] = __uint_as_float(q.z & 0xffff0000u);
      v[6] = __uint_as_float(q.w << 16); v[7] = __uint_as_float(q.w & 0xffff0000u);
    } else {
      const float4* yp = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(y) + p * H + n0);
      float4 a = yp[0], b = yp[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, v[i], acc[i]);
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
  dim3 grid((unsigned)((H / 8 + 255) / 256), (unsigned)(T < 65535 ? T : 65535));
  if (y_dtype == MOE_DTYPE_BF16)
    hipLaunchKernelGGL(k_combine<true>, grid, dim3(256), 0, s, y, asg_pos, w, T, k, H, residual, out);
  else
    hipLaunchKernelGGL(k_combine<false>, grid, dim3(256), 0, s, y, asg_pos, w, T, k, H, residual, out);
  return hipGetLastError();
}

}  // namespace moe
