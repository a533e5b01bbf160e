// gemv_gateup.hip -- decode-size gate/up projections of the routed experts,
// NVFP4 weights dequantized in registers, SwiGLU in the epilogue:
//   g = x . dq(Wg)^T, u = x . dq(Wu)^T, h = silu(g * ts_g) * (u * ts_u).
// E2M1 codes become exact bf16 pairs and meet the bf16 activations in
// v_dot2_f32_bf16 (two products per instruction, fp32 accumulation); each
// 16-element block sum is scaled by its E4M3 scale.  Layout and work split:
// gemv_common.h.
#include "gemv_common.h"

namespace moe {

namespace {

template <int NW, int GPW>
__global__ __launch_bounds__(NW * 64) void k_gemv_gateup_nvfp4(
    const uint16_t* __restrict__ x, int H, int I, int ktop, int mt_max,
    const moe_expert_ref* __restrict__ experts, size_t off_gq, size_t off_gs, size_t off_uq,
    size_t off_us, const uint32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_asg, const int32_t* __restrict__ active,
    const int32_t* __restrict__ n_active, float* __restrict__ hout) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                         // [mt_max][H] bf16
  float* red = reinterpret_cast<float*>(smem + (size_t)mt_max * H * 2);     // [NW][MT][2][64]

  SlotInfo si;
  if (!slot_info(active, n_active, counts, offsets, experts, &si)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = blockIdx.x * 64 + lane;
  const bool row_ok = n < I;
  const size_t nc = row_ok ? (size_t)n : 0;
  const uint8_t* blob = (const uint8_t*)si.ref.blob;
  const uint8_t* gq = blob + off_gq;
  const uint8_t* gs = blob + off_gs;
  const uint8_t* uq = blob + off_uq;
  const uint8_t* us = blob + off_us;
  const int NG = H >> 7;
  const int n_sets = (NG + NW * GPW - 1) / (NW * GPW);
  const int vpr = H >> 3;

  for (int c0 = 0; c0 < si.cnt; c0 += mt_max) {
    const int mt = min(mt_max, si.cnt - c0);
    float ag[kMaxMT], au[kMaxMT];
#pragma unroll
    for (int t = 0; t < kMaxMT; ++t) { ag[t] = 0.0f; au[t] = 0.0f; }

    for (int s = 0; s < n_sets; ++s) {
      const int g0 = (s * NW + wave) * GPW;
      uint4 cg[GPW][4], cu[GPW][4];
      uint2 sg[GPW], su[GPW];
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi) {
        const int g = g0 + gi;
        if (row_ok && g < NG) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            cg[gi][q] = *reinterpret_cast<const uint4*>(gq + (((size_t)(4 * g + q)) * I + nc) * 16);
            cu[gi][q] = *reinterpret_cast<const uint4*>(uq + (((size_t)(4 * g + q)) * I + nc) * 16);
          }
          sg[gi] = *reinterpret_cast<const uint2*>(gs + ((size_t)g * I + nc) * 8);
          su[gi] = *reinterpret_cast<const uint2*>(us + ((size_t)g * I + nc) * 8);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            cg[gi][q] = make_uint4(0, 0, 0, 0);
            cu[gi][q] = make_uint4(0, 0, 0, 0);
          }
          sg[gi] = make_uint2(0, 0);
          su[gi] = make_uint2(0, 0);
        }
      }
      if (s == 0) {
        // Gather this pass's token rows (bf16) into LDS while the weights fly.
        for (int i = tid; i < mt * vpr; i += NW * 64) {
          int r = i / vpr, c = i - r * vpr;
          int tok = sorted_asg[si.base + c0 + r] / ktop;
          reinterpret_cast<uint4*>(xs + (size_t)r * H)[c] =
              reinterpret_cast<const uint4*>(x + (size_t)tok * H)[c];
        }
        __syncthreads();
      }
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi) {
        const int g = g0 + gi;
        if (g >= NG) break;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const uint32_t sgw = (b < 4) ? sg[gi].x : sg[gi].y;
          const uint32_t suw = (b < 4) ? su[gi].x : su[gi].y;
          const float scg = e4m3_to_f32((sgw >> (8 * (b & 3))) & 0xffu);
          const float scu = e4m3_to_f32((suw >> (8 * (b & 3))) & 0xffu);
          v2bf_t wg[8], wu[8];
          e2m1x8_bf16(word_of(cg[gi][b >> 1], (b & 1) * 2), wg);
          e2m1x8_bf16(word_of(cg[gi][b >> 1], (b & 1) * 2 + 1), wg + 4);
          e2m1x8_bf16(word_of(cu[gi][b >> 1], (b & 1) * 2), wu);
          e2m1x8_bf16(word_of(cu[gi][b >> 1], (b & 1) * 2 + 1), wu + 4);
#pragma unroll
          for (int t = 0; t < kMaxMT; ++t) {
            if (t < mt) {
              const uint4* xp = reinterpret_cast<const uint4*>(xs + (size_t)t * H + 128 * g + 16 * b);
              const uint4 xa = xp[0], xb = xp[1];
              const uint32_t xw[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
              float pg = 0.0f, pu = 0.0f;
#pragma unroll
              for (int i = 0; i < 8; ++i) {
                pg = __builtin_amdgcn_fdot2_f32_bf16(wg[i], as_v2bf(xw[i]), pg, false);
                pu = __builtin_amdgcn_fdot2_f32_bf16(wu[i], as_v2bf(xw[i]), pu, false);
              }
              ag[t] = fmaf(pg, scg, ag[t]);
              au[t] = fmaf(pu, scu, au[t]);
            }
          }
        }
      }
    }

    __syncthreads();
#pragma unroll
    for (int t = 0; t < kMaxMT; ++t) {
      if (t < mt) {
        red[((wave * kMaxMT + t) * 2 + 0) * 64 + lane] = ag[t];
        red[((wave * kMaxMT + t) * 2 + 1) * 64 + lane] = au[t];
      }
    }
    __syncthreads();
    for (int o = tid; o < mt * 64; o += NW * 64) {
      const int t = o >> 6, r = o & 63;
      const int n2 = blockIdx.x * 64 + r;
      if (n2 < I) {
        float gsum = 0.0f, usum = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          gsum += red[((w * kMaxMT + t) * 2 + 0) * 64 + r];
          usum += red[((w * kMaxMT + t) * 2 + 1) * 64 + r];
        }
        gsum *= si.ref.ts_gate;
        usum *= si.ref.ts_up;
        hout[(size_t)(si.base + c0 + t) * I + n2] = gsum / (1.0f + expf(-gsum)) * usum;
      }
    }
  }
}

template <int NW, int GPW>
hipError_t gateup_t(const moe_layer_desc* L, const uint16_t* x, const moe_buckets* b,
                    int max_slots, float* h, hipStream_t s) {
  const BlobLayout lay = blob_layout(L->H, L->I, L->fmt_down);
  const int mt_max = min(kMaxMT, 16384 / L->H);  // bf16 token tile <= 32 KiB
  dim3 grid((unsigned)((L->I + 63) / 64), (unsigned)max_slots);
  size_t lds = (size_t)mt_max * L->H * 2 + sizeof(float) * NW * kMaxMT * 2 * 64;
  hipLaunchKernelGGL((k_gemv_gateup_nvfp4<NW, GPW>), grid, dim3(NW * 64), lds, s, x, L->H, L->I,
                     L->k, mt_max, L->experts, lay.gate_q, lay.gate_s, lay.up_q, lay.up_s,
                     b->counts, b->offsets, b->sorted_asg, b->active, b->n_active, h);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_gateup(const moe_layer_desc* L, const uint16_t* x, const moe_buckets* b,
                              int max_slots, float* h, hipStream_t s) {
  switch (L->H / 128) {  // groups of 128 along K = H
    case 1: return gateup_t<1, 1>(L, x, b, max_slots, h, s);
    case 2: return gateup_t<2, 1>(L, x, b, max_slots, h, s);
    case 3: return gateup_t<3, 1>(L, x, b, max_slots, h, s);
    case 4: return gateup_t<4, 1>(L, x, b, max_slots, h, s);
    case 8: return gateup_t<4, 2>(L, x, b, max_slots, h, s);
    case 12: return gateup_t<4, 3>(L, x, b, max_slots, h, s);
    default: return gateup_t<4, 4>(L, x, b, max_slots, h, s);  // 16 and above (strided sets)
  }
}

}  // namespace moe
