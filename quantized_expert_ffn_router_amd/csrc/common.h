// common.h -- internal declarations of libmoe (not part of the C ABI).
//
// Packed expert blob: the canonical NVFP4 / Q6_K-style bytes re-arranged so
// that a wavefront load of 64 lanes x 16 bytes covers the same K-slice of 64
// consecutive output rows ("lane per row").  Every section is a transpose of
// fixed-size byte granules from [row][granule] to [granule][row]:
//
//   NVFP4 matrix [N][K]:  codes  granule (c, n), c < K/32,  16 bytes = the
//                         32 elements 32c..32c+31 of row n (canonical bytes
//                         16c..16c+15 of the row);
//                         scales granule (g, n), g < K/128, 8 bytes = the E4M3
//                         scales of elements 128g..128g+127 of row n.
//   Q6_K matrix [N][K]:   ql granule (c, n), c < K/32: ql bytes of elements
//                         32c..32c+31 (superblock c/8, ql bytes 16*(c%8)..);
//                         qh granule (c, n), c < K/64: qh bytes of elements
//                         64c..64c+63 (superblock c/4, qh bytes 16*(c%4)..);
//                         sc granule (s, n), s < K/256: the 16 int8 sub-scales;
//                         d  granule (s, n), s < K/256: the fp16 scale (2 bytes).
//   Q8_0 matrix [N][K]:   codes  granule (c, n), c < K/16, 16 bytes = the int8
//                         codes of elements 16c..16c+15 (block c/2, code
//                         bytes 16*(c%2)..);
//                         scales granule (g, n), g < K/128, 8 bytes = the fp16
//                         scales of blocks 4g..4g+3.
//   IQ3G matrix [N][K]:   idx  granule (c, n), c < K/64, 16 bytes = the grid
//                         indices of elements 64c..64c+63 (superblock c/4);
//                         sign granule (c, n), c < K/128, 16 bytes = the sign
//                         bits of elements 128c..128c+127 (superblock c/2);
//                         sc granule (s, n), s < K/256, 8 bytes = d (fp16) and
//                         the 8 nibble multipliers of superblock s, 2 zero bytes.
//
// Blob = gate, up (NVFP4, [I][H]) then down ([H][I], NVFP4, Q6_K, Q8_0 or
// IQ3G); each section starts on a 256-byte boundary.  Q6_K, Q8_0 and IQ3G
// blobs end with a
// 256-byte meta section whose first int32 is the expert's down-weight exponent
// s (written by moe_pack_experts): the grouped GEMM forms its fp16 down
// weights as w * 2^s, s chosen from the expert's largest block scale so that
// no weight of the expert can overflow fp16, and takes 2^-s out in fp32.

#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"
#include "iq1g.h"
#include "iq3g.h"

namespace moe {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v, size_t a = kAlign) { return (v + a - 1) / a * a; }

struct BlobLayout {
  size_t gate_q, gate_s, up_q, up_s;
  size_t down_q, down_s;  // NVFP4 or Q8_0 down; IQ3G: grid indices, signs; IQ1G: index
                          // low bytes, 2-bit high parts
  size_t down_ql, down_qh, down_sc, down_d;  // Q6_K down; IQ3G / IQ1G: down_sc (d and multipliers)
  size_t down_meta;  // Q6_K / Q8_0 / IQ3G / IQ1G: int32 fp16-path exponent (0 for NVFP4)
  size_t total;
};

inline BlobLayout blob_layout(int64_t H, int64_t I, int fmt_down) {
  BlobLayout b{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  b.gate_q = take((size_t)I * H / 2);
  b.gate_s = take((size_t)I * H / 16);
  b.up_q = take((size_t)I * H / 2);
  b.up_s = take((size_t)I * H / 16);
  if (fmt_down == MOE_FMT_NVFP4) {
    b.down_q = take((size_t)H * I / 2);
    b.down_s = take((size_t)H * I / 16);
  } else if (fmt_down == MOE_FMT_Q8_0) {
    b.down_q = take((size_t)H * I);
    b.down_s = take((size_t)H * I / 16);
    b.down_meta = take(4);
  } else if (fmt_down == MOE_FMT_IQ3G) {
    b.down_q = take((size_t)H * I / 4);
    b.down_s = take((size_t)H * I / 8);
    b.down_sc = take((size_t)H * I / 32);
    b.down_meta = take(4);
  } else if (fmt_down == MOE_FMT_IQ1G) {
    b.down_q = take((size_t)H * I / 8);   // [I/128][H][16]: index low bytes of 16 groups of 8
    b.down_s = take((size_t)H * I / 32);  // [I/128][H][4]: their 2-bit high parts
    b.down_sc = take((size_t)H * I / 32); // [I/256][H][8]: d, 8 nibble multipliers, 2 zero bytes
    b.down_meta = take(4);
  } else {
    b.down_ql = take((size_t)H * I / 2);
    b.down_qh = take((size_t)H * I / 4);
    b.down_sc = take((size_t)H * I / 16);
    b.down_d = take((size_t)H * I / 128);
    b.down_meta = take(4);
  }
  b.total = off;
  return b;
}

// ---------------------------------------------------------------- device

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

// fp32 -> bf16, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// E4M3 (fn) byte -> fp32: normal (1 + m/8) * 2^(e-7), subnormal m * 2^-9.
// 0x7f/0xff (NaN) never occur in valid scales.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1.0p-9f;
  return (b & 0x80u) ? -mag : mag;
}

// IEEE binary16 bits -> fp32 (exact).
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, h);
  return (float)v;
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// 64-bit ballot over the wavefront.
__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

}  // namespace moe

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; arguments are pre-validated.

namespace moe {

// Per-expert exponent of the grouped GEMM's fp16 down weights (Q6_K, Q8_0, IQ3G)
// from the canonical down bytes, into the blob's meta section.
hipError_t launch_down_exponent(const uint8_t* down_q, int E, int64_t H, int64_t I, int fmt,
                                uint8_t* meta, size_t dst_expert_stride, hipStream_t s);

// pad: zero bytes after each destination granule (granule size gsz * pieces + pad).
hipError_t launch_pack_granules(const uint8_t* src, int E, size_t src_expert_stride,
                                int64_t N, int64_t G, int gsz, size_t row_stride,
                                int per_sb, size_t sb_stride, size_t inner, uint8_t* dst,
                                size_t dst_expert_stride, hipStream_t s, int pieces = 1,
                                int pad = 0);

hipError_t launch_router(const uint16_t* x, int64_t T, int H, const float* Wr,
                         const float* bias, int E, float* logits, hipStream_t s);

// Top-k + bucketing (+ histogram when hist is not null) in one launch, for
// E <= 256 and T * k <= 256 (gate_fused_fits).
bool gate_fused_fits(int64_t T, int E, int k);
hipError_t launch_gate_fused(const float* logits, int64_t T, int E, int k, int renorm,
                             int32_t* idx, float* w, const moe_buckets* b, uint32_t* hist, int ds,
                             int us, hipStream_t s);
hipError_t launch_topk(const float* logits, int64_t T, int E, int k, int renorm, int32_t* idx,
                       float* w, hipStream_t s);

size_t bucket_ws_bytes(int E, int64_t A);
hipError_t launch_bucket(const int32_t* idx, int64_t A, int E, const moe_buckets* b, void* ws,
                         hipStream_t s);

hipError_t launch_hist(const uint32_t* counts, int E, uint32_t* hist, int ds, int us,
                       hipStream_t s);

hipError_t launch_combine(const void* y, int y_dtype, const int32_t* asg_pos, const float* w,
                          int64_t T, int k, int H, const uint16_t* residual, uint16_t* out,
                          hipStream_t s);

}  // namespace moe
