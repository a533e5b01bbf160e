// pack.hip -- re-arrange canonical NVFP4 / Q6_K-style / Q8_0 expert bytes into the
// device blob (16-byte granules transposed from [row][granule] to
// [granule][row], see common.h).  A one-time byte permutation at load.
#include "common.h"

namespace moe {

namespace {

// dst granule (g, n) of pieces * gsz bytes <- piece j < pieces from source
// granule gg = g * pieces + j of row n, at byte offset (gg / per_sb) * sb_stride
// + inner + gsz * (gg % per_sb); one thread per destination byte.
__global__ void k_pack_granules(const uint8_t* __restrict__ src, size_t src_expert_stride,
                                int64_t N, int64_t G, int gsz, int pieces, size_t row_stride,
                                int per_sb, size_t sb_stride, size_t inner,
                                uint8_t* __restrict__ dst, size_t dst_expert_stride) {
  const int64_t dsz = (int64_t)gsz * pieces;
  const int64_t total = N * G * dsz;
  const uint8_t* s = src + (size_t)blockIdx.y * src_expert_stride;
  uint8_t* d = dst + (size_t)blockIdx.y * dst_expert_stride;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t db = i % dsz;
    const int64_t gn = i / dsz;
    const int64_t n = gn % N;
    const int64_t gg = (gn / N) * pieces + db / gsz;
    const int64_t byte = db % gsz;
    d[i] = s[(size_t)n * row_stride + (size_t)(gg / per_sb) * sb_stride + inner +
             (size_t)gsz * (size_t)(gg % per_sb) + (size_t)byte];
  }
}

}  // namespace

hipError_t launch_pack_granules(const uint8_t* src, int E, size_t src_expert_stride, int64_t N,
                                int64_t G, int gsz, size_t row_stride, int per_sb,
                                size_t sb_stride, size_t inner, uint8_t* dst,
                                size_t dst_expert_stride, hipStream_t s, int pieces) {
  const int64_t total = N * G * gsz * pieces;
  int64_t nblk = (total + 255) / 256;
  unsigned blocks = (unsigned)(nblk < 4096 ? nblk : 4096);
  hipLaunchKernelGGL(k_pack_granules, dim3(blocks, (unsigned)E), dim3(256), 0, s, src,
                     src_expert_stride, N, G, gsz, pieces, row_stride, per_sb, sb_stride, inner, dst,
                     dst_expert_stride);
  return hipGetLastError();
}

}  // namespace moe
