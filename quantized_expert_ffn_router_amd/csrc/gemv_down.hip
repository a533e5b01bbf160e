// gemv_down.hip -- decode-size down projection of the routed experts with
// NVFP4 weights: y[p] = (h[p] . dq(Wd)^T) for each sorted assignment p of the
// expert.  h stays fp32 (staged in LDS); E2M1 pairs are converted to fp32 with
// the gfx950 packed FP4 conversion and each 16-element block sum is scaled by
// its E4M3 scale, the per-tensor scale by the total.  Work split:
// gemv_common.h.
#include "gemv_common.h"

namespace moe {

namespace {

template <int NW, int GPW, bool BF16>
__global__ __launch_bounds__(NW * 64) void k_gemv_down_nvfp4(
    const float* __restrict__ hin, int H, int I, int mt_max,
    const moe_expert_ref* __restrict__ experts, size_t off_dq, size_t off_ds,
    const uint32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ active, const int32_t* __restrict__ n_active,
    void* __restrict__ y) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* hs = reinterpret_cast<float*>(smem);                  // [mt_max][I]
  float* red = hs + (size_t)mt_max * I;                        // [NW][MT][64]

  SlotInfo si;
  if (!slot_info(active, n_active, counts, offsets, experts, &si)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = blockIdx.x * 64 + lane;
  const bool row_ok = n < H;
  const size_t nc = row_ok ? (size_t)n : 0;
  const uint8_t* blob = (const uint8_t*)si.ref.blob;
  const uint8_t* dq = blob + off_dq;
  const uint8_t* ds = blob + off_ds;
  const int NG = I >> 7;
  const int n_sets = (NG + NW * GPW - 1) / (NW * GPW);

  for (int c0 = 0; c0 < si.cnt; c0 += mt_max) {
    const int mt = min(mt_max, si.cnt - c0);
    float acc[kMaxMT];
#pragma unroll
    for (int t = 0; t < kMaxMT; ++t) acc[t] = 0.0f;
    for (int s = 0; s < n_sets; ++s) {
      const int g0 = (s * NW + wave) * GPW;
      uint4 cq[GPW][4];
      uint2 sc[GPW];
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi) {
        const int g = g0 + gi;
        if (row_ok && g < NG) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            cq[gi][q] = *reinterpret_cast<const uint4*>(dq + (((size_t)(4 * g + q)) * H + nc) * 16);
          sc[gi] = *reinterpret_cast<const uint2*>(ds + ((size_t)g * H + nc) * 8);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) cq[gi][q] = make_uint4(0, 0, 0, 0);
          sc[gi] = make_uint2(0, 0);
        }
      }
      if (s == 0) {
        stage_rows_f32(hin, I, si.base + c0, mt, hs, NW * 64);
        __syncthreads();
      }
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi) {
        const int g = g0 + gi;
        if (g >= NG) break;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const uint32_t sw = (b < 4) ? sc[gi].x : sc[gi].y;
          const float scale = e4m3_to_f32((sw >> (8 * (b & 3))) & 0xffu);
          float w[16];
          e2m1x8_f32(word_of(cq[gi][b >> 1], (b & 1) * 2), w);
          e2m1x8_f32(word_of(cq[gi][b >> 1], (b & 1) * 2 + 1), w + 8);
#pragma unroll
          for (int t = 0; t < kMaxMT; ++t) {
            if (t < mt) {
              float xv[16];
              load_f32x16(hs + (size_t)t * I + 128 * g + 16 * b, xv);
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
        store_y<BF16>(y, (size_t)(si.base + c0 + t) * H + n2, sum * si.ref.ts_down);
      }
    }
  }
}

template <int NW, int GPW>
hipError_t down_t(const moe_layer_desc* L, const float* h, const moe_buckets* b, int max_slots,
                  void* y, int y_dtype, hipStream_t s) {
  const BlobLayout lay = blob_layout(L->H, L->I, L->fmt_down);
  const int mt_max = min(kMaxMT, 8192 / L->I);  // fp32 h tile <= 32 KiB
  dim3 grid((unsigned)((L->H + 63) / 64), (unsigned)max_slots);
  size_t lds = sizeof(float) * ((size_t)mt_max * L->I + NW * kMaxMT * 64);
  if (y_dtype == MOE_DTYPE_BF16)
    hipLaunchKernelGGL((k_gemv_down_nvfp4<NW, GPW, true>), grid, dim3(NW * 64), lds, s, h, L->H,
                       L->I, mt_max, L->experts, lay.down_q, lay.down_s, b->counts, b->offsets,
                       b->active, b->n_active, y);
  else
    hipLaunchKernelGGL((k_gemv_down_nvfp4<NW, GPW, false>), grid, dim3(NW * 64), lds, s, h, L->H,
                       L->I, mt_max, L->experts, lay.down_q, lay.down_s, b->counts, b->offsets,
                       b->active, b->n_active, y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_down(const moe_layer_desc* L, const float* h, const moe_buckets* b,
                            int max_slots, void* y, int y_dtype, hipStream_t s) {
  switch (L->I / 128) {  // groups of 128 along K = I
    case 1: return down_t<1, 1>(L, h, b, max_slots, y, y_dtype, s);
    case 2: return down_t<2, 1>(L, h, b, max_slots, y, y_dtype, s);
    case 3: return down_t<3, 1>(L, h, b, max_slots, y, y_dtype, s);
    case 4: return down_t<4, 1>(L, h, b, max_slots, y, y_dtype, s);
    case 6: return down_t<3, 2>(L, h, b, max_slots, y, y_dtype, s);
    case 8: return down_t<4, 2>(L, h, b, max_slots, y, y_dtype, s);
    default: return down_t<4, 4>(L, h, b, max_slots, y, y_dtype, s);
  }
}

}  // namespace moe
