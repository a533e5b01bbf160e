// ffn_gemv.hip -- expert FFNs for decode-sized batches: dequant-fused GEMV.
//
// Routed experts are block-quantized (NVFP4; GGUF Q6_K in the DQ6_K packs:
// basalt.jgulfo.com, sections "Models" and "Quick start"), and only the
// experts a token selected are touched ("each token uses only a few experts":
// "Expert tiers").  At 1..8 tokens per step (one per request slot) the work is
// bound by reading each active expert's weight bytes once from HBM, so the
// kernels stream the packed codes with 16-byte loads and dequantize in
// registers:
//   - one workgroup per (active expert, 64 output rows); lane l of every wave
//     owns output row 64*blockIdx.x + l, so a wave-wide 16-byte load reads the
//     same 32-element K-slice of 64 consecutive rows (the packed blob stores
//     exactly that contiguously) and no cross-lane reduction is needed;
//   - the K dimension is split over the NW waves (groups of 128 elements,
//     strided over waves) and the NW partial sums are added through LDS in
//     wave order;
//   - the expert's tokens (gathered through the bucket permutation) are staged
//     in LDS as fp32 and read as wave-uniform broadcasts;
//   - NVFP4: E2M1 pairs are converted with the gfx950 packed FP4->F32
//     conversion (scale 1.0, exact); each 16-element block sum is scaled by
//     its E4M3 scale, and the fp32 per-tensor scale is applied to the total.
//   - Q6_K: 6-bit codes are assembled from the low-nibble and high-bit planes;
//     each 16-element sub-block sum of x * (q - 32) is scaled by d * sc.
// Workgroups of experts with no tokens exit at once.
#include "common.h"

namespace moe {

namespace {

typedef float v2f __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// 8 E2M1 codes of one 32-bit word (element 2b in the low nibble of byte b)
// -> 8 floats, exact.
__device__ __forceinline__ void e2m1x8(uint32_t c, float* o) {
  v2f p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
  v2f p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
  v2f p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2);
  v2f p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
  o[0] = p0.x; o[1] = p0.y; o[2] = p1.x; o[3] = p1.y;
  o[4] = p2.x; o[5] = p2.y; o[6] = p3.x; o[7] = p3.y;
}

__device__ __forceinline__ float dot16(const float* w, const float* x) {
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s = fmaf(w[i], x[i], s);
  return s;
}

__device__ __forceinline__ void bf16x8_to_f32(const uint4& v, float* d) {
  d[0] = __uint_as_float(v.x << 16); d[1] = __uint_as_float(v.x & 0xffff0000u);
  d[2] = __uint_as_float(v.y << 16); d[3] = __uint_as_float(v.y & 0xffff0000u);
  d[4] = __uint_as_float(v.z << 16); d[5] = __uint_as_float(v.z & 0xffff0000u);
  d[6] = __uint_as_float(v.w << 16); d[7] = __uint_as_float(v.w & 0xffff0000u);
}

// ------------------------------------------------------------ gate / up

template <int NW, int MT>
__global__ __launch_bounds__(NW * 64) void k_gemv_gateup_nvfp4(
    const uint16_t* __restrict__ x, int H, int I, int ktop,
    const moe_expert_ref* __restrict__ experts, size_t off_gq, size_t off_gs, size_t off_uq,
    size_t off_us, const uint32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_asg, float* __restrict__ hout) {
  extern __shared__ float sm[];
  const int e = blockIdx.y;
  const int cnt = (int)counts[e];
  if (cnt == 0) return;
  const int base = offsets[e];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = blockIdx.x * 64 + lane;
  const bool row_ok = n < I;
  const size_t nc = row_ok ? (size_t)n : 0;
  const moe_expert_ref ref = experts[e];
  const uint8_t* blob = (const uint8_t*)ref.blob;
  const uint8_t* gq = blob + off_gq;
  const uint8_t* gs = blob + off_gs;
  const uint8_t* uq = blob + off_uq;
  const uint8_t* us = blob + off_us;
  const int NG = H >> 7;
  const int vpr = H >> 3;

  for (int c0 = 0; c0 < cnt; c0 += MT) {
    const int mt = min(MT, cnt - c0);
    if (c0 > 0) __syncthreads();
    for (int i = tid; i < mt * vpr; i += NW * 64) {
      int r = i / vpr, c = i - r * vpr;
      int tok = sorted_asg[base + c0 + r] / ktop;
      uint4 v = *reinterpret_cast<const uint4*>(x + (size_t)tok * H + 8 * c);
      float d[8];
      bf16x8_to_f32(v, d);
      float4* dst = reinterpret_cast<float4*>(sm + (size_t)r * H + 8 * c);
      dst[0] = make_float4(d[0], d[1], d[2], d[3]);
      dst[1] = make_float4(d[4], d[5], d[6], d[7]);
    }
    __syncthreads();

    float ag[MT], au[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) { ag[t] = 0.0f; au[t] = 0.0f; }

    for (int g = wave; g < NG; g += NW) {
      uint4 cg[4], cu[4];
      uint2 sg = make_uint2(0, 0), su = make_uint2(0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        cg[q] = make_uint4(0, 0, 0, 0);
        cu[q] = make_uint4(0, 0, 0, 0);
      }
      if (row_ok) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          cg[q] = *reinterpret_cast<const uint4*>(gq + (((size_t)(4 * g + q)) * I + nc) * 16);
          cu[q] = *reinterpret_cast<const uint4*>(uq + (((size_t)(4 * g + q)) * I + nc) * 16);
        }
        sg = *reinterpret_cast<const uint2*>(gs + ((size_t)g * I + nc) * 8);
        su = *reinterpret_cast<const uint2*>(us + ((size_t)g * I + nc) * 8);
      }
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const uint32_t sgw = (b < 4) ? sg.x : sg.y, suw = (b < 4) ? su.x : su.y;
        const float scg = e4m3_to_f32((sgw >> (8 * (b & 3))) & 0xffu);
        const float scu = e4m3_to_f32((suw >> (8 * (b & 3))) & 0xffu);
        float wg[16], wu[16];
        e2m1x8(word_of(cg[b >> 1], (b & 1) * 2), wg);
        e2m1x8(word_of(cg[b >> 1], (b & 1) * 2 + 1), wg + 8);
        e2m1x8(word_of(cu[b >> 1], (b & 1) * 2), wu);
        e2m1x8(word_of(cu[b >> 1], (b & 1) * 2 + 1), wu + 8);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          if (t < mt) {
            const float4* xp = reinterpret_cast<const float4*>(sm + (size_t)t * H + 128 * g + 16 * b);
            float xv[16];
            float4 a0 = xp[0], a1 = xp[1], a2 = xp[2], a3 = xp[3];
            xv[0] = a0.x; xv[1] = a0.y; xv[2] = a0.z; xv[3] = a0.w;
            xv[4] = a1.x; xv[5] = a1.y; xv[6] = a1.z; xv[7] = a1.w;
            xv[8] = a2.x; xv[9] = a2.y; xv[10] = a2.z; xv[11] = a2.w;
            xv[12] = a3.x; xv[13] = a3.y; xv[14] = a3.z; xv[15] = a3.w;
            ag[t] = fmaf(dot16(wg, xv), scg, ag[t]);
            au[t] = fmaf(dot16(wu, xv), scu, au[t]);
          }
        }
      }
    }

    __syncthreads();
    float* red = sm;  // [NW][MT][2][64]
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (t < mt) {
        red[((wave * MT + t) * 2 + 0) * 64 + lane] = ag[t];
        red[((wave * MT + t) * 2 + 1) * 64 + lane] = au[t];
      }
    }
    __syncthreads();
    for (int o = tid; o < mt * 64; o += NW * 64) {
      const int t = o >> 6, r = o & 63;
      const int n2 = blockIdx.x * 64 + r;
      if (n2 < I) {
        float gsum = 0.0f, usum = 0.0f;
        for (int w = 0; w < NW; ++w) {
          gsum += red[((w * MT + t) * 2 + 0) * 64 + r];
          usum += red[((w * MT + t) * 2 + 1) * 64 + r];
        }
        gsum *= ref.ts_gate;
        usum *= ref.ts_up;
        hout[(size_t)(base + c0 + t) * I + n2] = gsum / (1.0f + expf(-gsum)) * usum;
      }
    }
  }
}

// ------------------------------------------------------------ down

template <bool BF16>
__device__ __forceinline__ void store_y(void* y, size_t i, float v) {
  if (BF16) reinterpret_cast<uint16_t*>(y)[i] = f32_to_bf16_rne(v);
  else reinterpret_cast<float*>(y)[i] = v;
}

// Stage rows base+c0 .. +mt of h (fp32 [A][I], sorted order) into LDS.
__device__ __forceinline__ void stage_h(const float* __restrict__ hin, int I, int row0, int mt,
                                        float* sm, int nthreads) {
  const int vpr = I >> 2;
  for (int i = threadIdx.x; i < mt * vpr; i += nthreads) {
    int r = i / vpr, c = i - r * vpr;
    reinterpret_cast<float4*>(sm + (size_t)r * I)[c] =
        reinterpret_cast<const float4*>(hin + (size_t)(row0 + r) * I)[c];
  }
}

template <int NW, int MT, bool BF16>
__global__ __launch_bounds__(NW * 64) void k_gemv_down_nvfp4(
    const float* __restrict__ hin, int H, int I, const moe_expert_ref* __restrict__ experts,
    size_t off_dq, size_t off_ds, const uint32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, void* __restrict__ y) {
  extern __shared__ float sm[];
  const int e = blockIdx.y;
  const int cnt = (int)counts[e];
  if (cnt == 0) return;
  const int base = offsets[e];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = blockIdx.x * 64 + lane;
  const bool row_ok = n < H;
  const size_t nc = row_ok ? (size_t)n : 0;
  const moe_expert_ref ref = experts[e];
  const uint8_t* blob = (const uint8_t*)ref.blob;
  const uint8_t* dq = blob + off_dq;
  const uint8_t* ds = blob + off_ds;
  const int NG = I >> 7;

  for (int c0 = 0; c0 < cnt; c0 += MT) {
    const int mt = min(MT, cnt - c0);
    if (c0 > 0) __syncthreads();
    stage_h(hin, I, base + c0, mt, sm, NW * 64);
    __syncthreads();
    float acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = 0.0f;
    for (int g = wave; g < NG; g += NW) {
      uint4 cq[4];
      uint2 sc = make_uint2(0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) cq[q] = make_uint4(0, 0, 0, 0);
      if (row_ok) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          cq[q] = *reinterpret_cast<const uint4*>(dq + (((size_t)(4 * g + q)) * H + nc) * 16);
        sc = *reinterpret_cast<const uint2*>(ds + ((size_t)g * H + nc) * 8);
      }
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const uint32_t sw = (b < 4) ? sc.x : sc.y;
        const float s = e4m3_to_f32((sw >> (8 * (b & 3))) & 0xffu);
        float w[16];
        e2m1x8(word_of(cq[b >> 1], (b & 1) * 2), w);
        e2m1x8(word_of(cq[b >> 1], (b & 1) * 2 + 1), w + 8);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          if (t < mt) {
            const float4* xp = reinterpret_cast<const float4*>(sm + (size_t)t * I + 128 * g + 16 * b);
            float xv[16];
            float4 a0 = xp[0], a1 = xp[1], a2 = xp[2], a3 = xp[3];
            xv[0] = a0.x; xv[1] = a0.y; xv[2] = a0.z; xv[3] = a0.w;
            xv[4] = a1.x; xv[5] = a1.y; xv[6] = a1.z; xv[7] = a1.w;
            xv[8] = a2.x; xv[9] = a2.y; xv[10] = a2.z; xv[11] = a2.w;
            xv[12] = a3.x; xv[13] = a3.y; xv[14] = a3.z; xv[15] = a3.w;
            acc[t] = fmaf(dot16(w, xv), s, acc[t]);
          }
        }
      }
    }
    __syncthreads();
    float* red = sm;  // [NW][MT][64]
#pragma unroll
    for (int t = 0; t < MT; ++t)
      if (t < mt) red[(wave * MT + t) * 64 + lane] = acc[t];
    __syncthreads();
    for (int o = tid; o < mt * 64; o += NW * 64) {
      const int t = o >> 6, r = o & 63;
      const int n2 = blockIdx.x * 64 + r;
      if (n2 < H) {
        float s = 0.0f;
        for (int w = 0; w < NW; ++w) s += red[(w * MT + t) * 64 + r];
        store_y<BF16>(y, (size_t)(base + c0 + t) * H + n2, s * ref.ts_down);
      }
    }
  }
}

template <int NW, int MT, bool BF16>
__global__ __launch_bounds__(NW * 64) void k_gemv_down_q6k(
    const float* __restrict__ hin, int H, int I, const moe_expert_ref* __restrict__ experts,
    size_t off_ql, size_t off_qh, size_t off_sc, size_t off_d,
    const uint32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    void* __restrict__ y) {
  extern __shared__ float sm[];
  const int e = blockIdx.y;
  const int cnt = (int)counts[e];
  if (cnt == 0) return;
  const int base = offsets[e];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = blockIdx.x * 64 + lane;
  const bool row_ok = n < H;
  const size_t nc = row_ok ? (size_t)n : 0;
  const moe_expert_ref ref = experts[e];
  const uint8_t* blob = (const uint8_t*)ref.blob;
  const uint8_t* pql = blob + off_ql;
  const uint8_t* pqh = blob + off_qh;
  const uint8_t* psc = blob + off_sc;
  const uint8_t* pd = blob + off_d;
  const int NS = I >> 8;  // superblocks per row

  for (int c0 = 0; c0 < cnt; c0 += MT) {
    const int mt = min(MT, cnt - c0);
    if (c0 > 0) __syncthreads();
    stage_h(hin, I, base + c0, mt, sm, NW * 64);
    __syncthreads();
    float acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = 0.0f;
    for (int sb = wave; sb < NS; sb += NW) {
      uint4 ql[8], qh[4], scv = make_uint4(0, 0, 0, 0);
      uint16_t dbits = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) ql[q] = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) qh[q] = make_uint4(0, 0, 0, 0);
      if (row_ok) {
#pragma unroll
        for (int q = 0; q < 8; ++q)
          ql[q] = *reinterpret_cast<const uint4*>(pql + (((size_t)(8 * sb + q)) * H + nc) * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          qh[q] = *reinterpret_cast<const uint4*>(pqh + (((size_t)(4 * sb + q)) * H + nc) * 16);
        scv = *reinterpret_cast<const uint4*>(psc + ((size_t)sb * H + nc) * 16);
        dbits = *reinterpret_cast<const uint16_t*>(pd + ((size_t)sb * H + nc) * 2);
      }
      const float d = f16_to_f32(dbits);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t lo0 = word_of(ql[j >> 1], (j & 1) * 2);
        const uint32_t lo1 = word_of(ql[j >> 1], (j & 1) * 2 + 1);
        const uint32_t hi = word_of(qh[j >> 2], j & 3);
        const int8_t scj = (int8_t)((word_of(scv, j >> 2) >> (8 * (j & 3))) & 0xffu);
        const float s = d * (float)scj;
        float w[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          uint32_t lo = ((i < 8 ? lo0 : lo1) >> (4 * (i & 7))) & 15u;
          uint32_t h2 = (hi >> (2 * i)) & 3u;
          w[i] = (float)((int)(lo | (h2 << 4)) - 32);
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          if (t < mt) {
            const float4* xp = reinterpret_cast<const float4*>(sm + (size_t)t * I + 256 * sb + 16 * j);
            float xv[16];
            float4 a0 = xp[0], a1 = xp[1], a2 = xp[2], a3 = xp[3];
            xv[0] = a0.x; xv[1] = a0.y; xv[2] = a0.z; xv[3] = a0.w;
            xv[4] = a1.x; xv[5] = a1.y; xv[6] = a1.z; xv[7] = a1.w;
            xv[8] = a2.x; xv[9] = a2.y; xv[10] = a2.z; xv[11] = a2.w;
            xv[12] = a3.x; xv[13] = a3.y; xv[14] = a3.z; xv[15] = a3.w;
            acc[t] = fmaf(dot16(w, xv), s, acc[t]);
          }
        }
      }
    }
    __syncthreads();
    float* red = sm;
#pragma unroll
    for (int t = 0; t < MT; ++t)
      if (t < mt) red[(wave * MT + t) * 64 + lane] = acc[t];
    __syncthreads();
    for (int o = tid; o < mt * 64; o += NW * 64) {
      const int t = o >> 6, r = o & 63;
      const int n2 = blockIdx.x * 64 + r;
      if (n2 < H) {
        float s = 0.0f;
        for (int w = 0; w < NW; ++w) s += red[(w * MT + t) * 64 + r];
        store_y<BF16>(y, (size_t)(base + c0 + t) * H + n2, s);
      }
    }
  }
}

// ------------------------------------------------------------ launchers

template <int NW, int MT>
hipError_t gateup_t(const moe_layer_desc* L, const uint16_t* x, const moe_buckets* b,
                    const BlobLayout& lay, float* h, hipStream_t s) {
  dim3 grid((unsigned)((L->I + 63) / 64), (unsigned)L->E);
  size_t lds = sizeof(float) * (size_t)max(MT * L->H, NW * MT * 2 * 64);
  hipLaunchKernelGGL((k_gemv_gateup_nvfp4<NW, MT>), grid, dim3(NW * 64), lds, s, x, L->H, L->I,
                     L->k, L->experts, lay.gate_q, lay.gate_s, lay.up_q, lay.up_s, b->counts,
                     b->offsets, b->sorted_asg, h);
  return hipGetLastError();
}

template <int NW, int MT, bool BF16>
hipError_t down_t(const moe_layer_desc* L, const float* h, const moe_buckets* b,
                  const BlobLayout& lay, void* y, hipStream_t s) {
  dim3 grid((unsigned)((L->H + 63) / 64), (unsigned)L->E);
  size_t lds = sizeof(float) * (size_t)max(MT * L->I, NW * MT * 64);
  if (L->fmt_down == MOE_FMT_NVFP4) {
    hipLaunchKernelGGL((k_gemv_down_nvfp4<NW, MT, BF16>), grid, dim3(NW * 64), lds, s, h, L->H,
                       L->I, L->experts, lay.down_q, lay.down_s, b->counts, b->offsets, y);
  } else {
    hipLaunchKernelGGL((k_gemv_down_q6k<NW, MT, BF16>), grid, dim3(NW * 64), lds, s, h, L->H,
                       L->I, L->experts, lay.down_ql, lay.down_qh, lay.down_sc, lay.down_d,
                       b->counts, b->offsets, y);
  }
  return hipGetLastError();
}

// Waves per workgroup: one per K-group (128 elements NVFP4, 256 Q6_K), <= 16.
template <int MT>
hipError_t gateup_nw(const moe_layer_desc* L, const uint16_t* x, const moe_buckets* b,
                     const BlobLayout& lay, float* h, hipStream_t s) {
  int ng = L->H / 128;
  if (ng >= 16) return gateup_t<16, MT>(L, x, b, lay, h, s);
  if (ng >= 8) return gateup_t<8, MT>(L, x, b, lay, h, s);
  if (ng >= 4) return gateup_t<4, MT>(L, x, b, lay, h, s);
  if (ng >= 2) return gateup_t<2, MT>(L, x, b, lay, h, s);
  return gateup_t<1, MT>(L, x, b, lay, h, s);
}

template <int MT, bool BF16>
hipError_t down_nw(const moe_layer_desc* L, const float* h, const moe_buckets* b,
                   const BlobLayout& lay, void* y, hipStream_t s) {
  int ng = (L->fmt_down == MOE_FMT_NVFP4) ? L->I / 128 : L->I / 256;
  if (ng >= 16) return down_t<16, MT, BF16>(L, h, b, lay, y, s);
  if (ng >= 8) return down_t<8, MT, BF16>(L, h, b, lay, y, s);
  if (ng >= 6 && ng % 6 == 0) return down_t<6, MT, BF16>(L, h, b, lay, y, s);
  if (ng >= 4) return down_t<4, MT, BF16>(L, h, b, lay, y, s);
  if (ng >= 2) return down_t<2, MT, BF16>(L, h, b, lay, y, s);
  return down_t<1, MT, BF16>(L, h, b, lay, y, s);
}

}  // namespace

// Tokens staged per pass: the fp32 tile MT x K stays within 64 KiB of LDS.
hipError_t launch_gemv_ffn(const moe_layer_desc* L, const uint16_t* x, const moe_buckets* b,
                           float* h, void* y, int y_dtype, hipStream_t s) {
  const BlobLayout lay = blob_layout(L->H, L->I, L->fmt_down);
  hipError_t err;
  if (L->H <= 2048) err = gateup_nw<8>(L, x, b, lay, h, s);
  else if (L->H <= 4096) err = gateup_nw<4>(L, x, b, lay, h, s);
  else err = gateup_nw<2>(L, x, b, lay, h, s);
  if (err != hipSuccess) return err;
  const bool bf = (y_dtype == MOE_DTYPE_BF16);
  if (L->I <= 2048) return bf ? down_nw<8, true>(L, h, b, lay, y, s) : down_nw<8, false>(L, h, b, lay, y, s);
  if (L->I <= 4096) return bf ? down_nw<4, true>(L, h, b, lay, y, s) : down_nw<4, false>(L, h, b, lay, y, s);
  return bf ? down_nw<2, true>(L, h, b, lay, y, s) : down_nw<2, false>(L, h, b, lay, y, s);
}

}  // namespace moe
