// pack.hip -- re-arrange canonical NVFP4 / Q6_K-style / Q8_0 / IQ3G / IQ1G expert bytes into the
// device blob (16-byte granules transposed from [row][granule] to
// [granule][row], see common.h).  A one-time byte permutation at load.
#include "common.h"

namespace moe {

namespace {

// dst granule (g, n) of pieces * gsz + pad bytes <- piece j < pieces from
// source granule gg = g * pieces + j of row n, at byte offset (gg / per_sb) *
// sb_stride + inner + gsz * (gg % per_sb), then pad zero bytes; one thread per
// destination byte.
__global__ void k_pack_granules(const uint8_t* __restrict__ src, size_t src_expert_stride,
                                int64_t N, int64_t G, int gsz, int pieces, int pad,
                                size_t row_stride, int per_sb, size_t sb_stride, size_t inner,
                                uint8_t* __restrict__ dst, size_t dst_expert_stride) {
  const int64_t dsz = (int64_t)gsz * pieces, dstep = dsz + pad;
  const int64_t total = N * G * dstep;
  const uint8_t* s = src + (size_t)blockIdx.y * src_expert_stride;
  uint8_t* d = dst + (size_t)blockIdx.y * dst_expert_stride;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t db = i % dstep;
    if (db >= dsz) {
      d[i] = 0;
      continue;
    }
    const int64_t gn = i / dstep;
    const int64_t n = gn % N;
    const int64_t gg = (gn / N) * pieces + db / gsz;
    const int64_t byte = db % gsz;
    d[i] = s[(size_t)n * row_stride + (size_t)(gg / per_sb) * sb_stride + inner +
             (size_t)gsz * (size_t)(gg % per_sb) + (size_t)byte];
  }
}

// Exponent s of the grouped GEMM's fp16 down weights of one expert (one
// workgroup per expert).  The fp16 path forms, per block, a scale times 2^s in
// fp16 and the weights from it:
//   Q8_0:  w * 2^s = q * (d * 2^s), |q| <= 128: with M = max |d| over the
//          expert's blocks, M * 2^s < 2^8 keeps |w| * 2^s < 2^15;
//   Q6_K:  w * 2^s = (q - 32) * 2^-10 * (d * sc * 2^(10+s)), |q - 32| <= 32:
//          with M = max |d * sc|, M * 2^s < 2^5 keeps the fp16 factor below
//          2^15 and |w| * 2^s below 2^10;
//   IQ3G:  w * 2^s = (m * (2 s_j + 1)) * (d * 2^s), m * (2 s_j + 1) <= 279:
//          with M = max |d|, M * 2^s < 2^6 keeps |w| * 2^s below 2^15;
//   IQ1G:  w * 2^s = (v * (2 s_j + 1)) * (d * 2^s), |v * (2 s_j + 1)| <= 31:
//          with M = max |d|, M * 2^s < 2^9 keeps |w| * 2^s below 2^14.
// s = P - e for M = f * 2^e (f in [0.5, 1)) is the largest such s; all-zero
// scales give s = 0.  Clamped to [-64, 64].
__global__ __launch_bounds__(256) void k_down_exponent(const uint8_t* __restrict__ src,
                                                       size_t src_expert_stride, int64_t nblocks,
                                                       int fmt, uint8_t* __restrict__ meta,
                                                       size_t dst_expert_stride) {
  __shared__ float red[256];
  const uint8_t* s = src + (size_t)blockIdx.x * src_expert_stride;
  float m = 0.0f;
  for (int64_t b = threadIdx.x; b < nblocks; b += blockDim.x) {
    if (fmt == MOE_FMT_Q8_0 || fmt == MOE_FMT_IQ3G || fmt == MOE_FMT_IQ1G) {  // d leads
      const uint8_t* blk =
          s + (size_t)b * (fmt == MOE_FMT_Q8_0 ? 34
                                               : (fmt == MOE_FMT_IQ3G ? kIq3gBlockBytes
                                                                      : kIq1gBlockBytes));
      m = fmaxf(m, fabsf(f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)))));
    } else {
      const uint8_t* blk = s + (size_t)b * 210;
      int sc = 0;
      for (int j = 0; j < 16; ++j) sc = max(sc, abs((int)(int8_t)blk[192 + j]));
      m = fmaxf(m, fabsf(f16_to_f32((uint16_t)(blk[208] | (blk[209] << 8)))) * (float)sc);
    }
  }
  red[threadIdx.x] = m;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float M = red[0];
    int e = 0;
    (void)frexpf(M, &e);
    const int P = (fmt == MOE_FMT_Q8_0)   ? 8
                  : (fmt == MOE_FMT_IQ3G) ? 6
                  : (fmt == MOE_FMT_IQ1G) ? 9
                                          : 5;
    int sx = (M > 0.0f && M <= 3.0e38f) ? P - e : 0;
    sx = sx < -64 ? -64 : (sx > 64 ? 64 : sx);
    *reinterpret_cast<int32_t*>(meta + (size_t)blockIdx.x * dst_expert_stride) = sx;
  }
}

}  // namespace

hipError_t launch_down_exponent(const uint8_t* down_q, int E, int64_t H, int64_t I, int fmt,
                                uint8_t* meta, size_t dst_expert_stride, hipStream_t s) {
  const int64_t per_row = (fmt == MOE_FMT_Q8_0) ? I / 32 : I / 256;
  const size_t bsz = (fmt == MOE_FMT_Q8_0)   ? 34
                     : (fmt == MOE_FMT_IQ3G) ? kIq3gBlockBytes
                     : (fmt == MOE_FMT_IQ1G) ? kIq1gBlockBytes
                                             : 210;
  const int64_t nblocks = H * per_row;
  hipLaunchKernelGGL(k_down_exponent, dim3((unsigned)E), dim3(256), 0, s, down_q,
                     (size_t)nblocks * bsz, nblocks, fmt, meta, dst_expert_stride);
  return hipGetLastError();
}

hipError_t launch_pack_granules(const uint8_t* src, int E, size_t src_expert_stride, int64_t N,
                                int64_t G, int gsz, size_t row_stride, int per_sb,
                                size_t sb_stride, size_t inner, uint8_t* dst,
                                size_t dst_expert_stride, hipStream_t s, int pieces, int pad) {
  const int64_t total = N * G * ((int64_t)gsz * pieces + pad);
  int64_t nblk = (total + 255) / 256;
  unsigned blocks = (unsigned)(nblk < 4096 ? nblk : 4096);
  hipLaunchKernelGGL(k_pack_granules, dim3(blocks, (unsigned)E), dim3(256), 0, s, src,
                     src_expert_stride, N, G, gsz, pieces, pad, row_stride, per_sb, sb_stride,
                     inner, dst, dst_expert_stride);
  return hipGetLastError();
}

}  // namespace moe
