// gemv_down_q6k.hip -- decode-size down projection with Q6_K-style weights
// (256-element superblocks: 6-bit codes in a low-nibble plane and a 2-bit
// plane, 16 int8 sub-scales, one fp16 scale; the DQ6_K packs of
// basalt.jgulfo.com, "Quick start").  For each 16-element sub-block the sum
// of h * (q - 32) is taken in fp32 (q - 32 is a small exact integer) and
// scaled by d * sc, exact in fp32.  Work split: gemv_common.h, with groups of
// one superblock.
#include "gemv_common.h"

namespace moe {

namespace {

template <int NW, int GPW, bool BF16>
__global__ __launch_bounds__(NW * 64) void k_gemv_down_q6k(
    const float* __restrict__ hin, int H, int I, int mt_max,
    const moe_expert_ref* __restrict__ experts, size_t off_ql, size_t off_qh, size_t off_sc,
    size_t off_d, const uint32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ active, const int32_t* __restrict__ n_active,
    void* __restrict__ y) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* hs = reinterpret_cast<float*>(smem);
  float* red = hs + (size_t)mt_max * I;

  SlotInfo si;
  if (!slot_info(active, n_active, counts, offsets, experts, &si)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = blockIdx.x * 64 + lane;
  const bool row_ok = n < H;
  const size_t nc = row_ok ? (size_t)n : 0;
  const uint8_t* blob = (const uint8_t*)si.ref.blob;
  const uint8_t* pql = blob + off_ql;
  const uint8_t* pqh = blob + off_qh;
  const uint8_t* psc = blob + off_sc;
  const uint8_t* pd = blob + off_d;
  const int NS = I >> 8;
  const int n_sets = (NS + NW * GPW - 1) / (NW * GPW);

  for (int c0 = 0; c0 < si.cnt; c0 += mt_max) {
    const int mt = min(mt_max, si.cnt - c0);
    float acc[kMaxMT];
#pragma unroll
    for (int t = 0; t < kMaxMT; ++t) acc[t] = 0.0f;
    for (int s = 0; s < n_sets; ++s) {
      const int g0 = (s * NW + wave) * GPW;
      uint4 ql[GPW][8], qh[GPW][4], scv[GPW];
      uint32_t dbits[GPW];
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi) {
        const int sb = g0 + gi;
        if (row_ok && sb < NS) {
#pragma unroll
          for (int q = 0; q < 8; ++q)
            ql[gi][q] = *reinterpret_cast<const uint4*>(pql + (((size_t)(8 * sb + q)) * H + nc) * 16);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            qh[gi][q] = *reinterpret_cast<const uint4*>(pqh + (((size_t)(4 * sb + q)) * H + nc) * 16);
          scv[gi] = *reinterpret_cast<const uint4*>(psc + ((size_t)sb * H + nc) * 16);
          dbits[gi] = *reinterpret_cast<const uint16_t*>(pd + ((size_t)sb * H + nc) * 2);
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) ql[gi][q] = make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int q = 0; q < 4; ++q) qh[gi][q] = make_uint4(0, 0, 0, 0);
          scv[gi] = make_uint4(0, 0, 0, 0);
          dbits[gi] = 0;
        }
      }
      if (s == 0) {
        stage_rows_f32(hin, I, si.base + c0, mt, hs, NW * 64);
        __syncthreads();
      }
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi) {
        const int sb = g0 + gi;
        if (sb >= NS) break;
        const float d = f16_to_f32((uint16_t)dbits[gi]);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const uint32_t lo0 = word_of(ql[gi][j >> 1], (j & 1) * 2);
          const uint32_t lo1 = word_of(ql[gi][j >> 1], (j & 1) * 2 + 1);
          const uint32_t hi = word_of(qh[gi][j >> 2], j & 3);
          const int8_t scj = (int8_t)((word_of(scv[gi], j >> 2) >> (8 * (j & 3))) & 0xffu);
          const float scale = d * (float)scj;
          float w[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const uint32_t lo = ((i < 8 ? lo0 : lo1) >> (4 * (i & 7))) & 15u;
            const uint32_t h2 = (hi >> (2 * i)) & 3u;
            w[i] = (float)((int)(lo | (h2 << 4)) - 32);
          }
#pragma unroll
          for (int t = 0; t < kMaxMT; ++t) {
            if (t < mt) {
              float xv[16];
              load_f32x16(hs + (size_t)t * I + 256 * sb + 16 * j, xv);
              acc[t] = fmaf(dot16_f32(w, xv), scale, acc[t]);
            }
          }
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kMaxMT; ++t)
      if (t < mt) red[(wave * kMaxMT + t) * 64 + lane] = acc[t];
    __syncthreads();
    for (int o = tid; o < mt * 64; o += NW * 64) {
      const int t = o >> 6, r = o & 63;
      const int n2 = blockIdx.x * 64 + r;
      if (n2 < H) {
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) sum += red[(w * kMaxMT + t) * 64 + r];
        store_y<BF16>(y, (size_t)(si.base + c0 + t) * H + n2, sum);
      }
    }
  }
}

template <int NW, int GPW>
hipError_t down_q6k_t(const moe_layer_desc* L, const float* h, const moe_buckets* b,
                      int max_slots, void* y, int y_dtype, hipStream_t s) {
  const BlobLayout lay = blob_layout(L->H, L->I, L->fmt_down);
  const int mt_max = min(kMaxMT, 8192 / L->I);
  dim3 grid((unsigned)((L->H + 63) / 64), (unsigned)max_slots);
  size_t lds = sizeof(float) * ((size_t)mt_max * L->I + NW * kMaxMT * 64);
  if (y_dtype == MOE_DTYPE_BF16)
    hipLaunchKernelGGL((k_gemv_down_q6k<NW, GPW, true>), grid, dim3(NW * 64), lds, s, h, L->H,
                       L->I, mt_max, L->experts, lay.down_ql, lay.down_qh, lay.down_sc,
                       lay.down_d, b->counts, b->offsets, b->active, b->n_active, y);
  else
    hipLaunchKernelGGL((k_gemv_down_q6k<NW, GPW, false>), grid, dim3(NW * 64), lds, s, h, L->H,
                       L->I, mt_max, L->experts, lay.down_ql, lay.down_qh, lay.down_sc,
                       lay.down_d, b->counts, b->offsets, b->active, b->n_active, y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_down_q6k(const moe_layer_desc* L, const float* h, const moe_buckets* b,
                                int max_slots, void* y, int y_dtype, hipStream_t s) {
  switch (L->I / 256) {  // superblocks along K = I
    case 1: return down_q6k_t<1, 1>(L, h, b, max_slots, y, y_dtype, s);
    case 2: return down_q6k_t<2, 1>(L, h, b, max_slots, y, y_dtype, s);
    case 3: return down_q6k_t<3, 1>(L, h, b, max_slots, y, y_dtype, s);
    default: return down_q6k_t<4, 1>(L, h, b, max_slots, y, y_dtype, s);
  }
}

}  // namespace moe
