// gemv_gateup.hip -- decode-size gate/up projections of the routed experts,
// NVFP4 weights dequantized in registers, SwiGLU in the epilogue:
//   g = x . dq(Wg)^T, u = x . dq(Wu)^T, h = silu(g * ts_g) * (u * ts_u).
// A workgroup owns 64 rows of one active expert: waves [0, S) stream the gate
// matrix and waves [S, 2S) the up matrix, each over 1/S of K (gemv_common.h).
// E2M1 codes become exact bf16 pairs that meet the bf16 activations in
// v_dot2_f32_bf16 (fp32 accumulation); each 16-element block sum is scaled by
// its E4M3 scale (hardware conversion), the per-tensor scale by the total.
#include "gemv_common.h"

namespace moe {

namespace {

// One pass over the mt staged tokens.  GPS groups per wave (the group loop
// unrolls fully, so the prefetch needs no loop-carried registers), D groups of
// weight loads in flight ahead of use.  Each group's codes and scales are
// decoded right after they arrive, before any per-token branch, so the load
// registers die at once and nothing waits on memory inside the token loop.
template <int GPS, int D>
__device__ __forceinline__ void gateup_pass(const uint16_t* xs, int H, int I, size_t nc,
                                            const uint8_t* pq, const uint8_t* ps, int gb,
                                            int mt, float* acc) {
  uint4 rc[GPS][4];
  uint2 rs[GPS];
  // Group loads are issued in group order (scheduling barriers keep them
  // apart) so that waiting for group gi never waits for a later group.
#pragma unroll
  for (int gi = 0; gi < GPS && gi < D; ++gi) {
    const int g = gb + gi;
#pragma unroll
    for (int q = 0; q < 4; ++q) rc[gi][q] = ld16(pq + (((size_t)(4 * g + q)) * I + nc) * 16);
    rs[gi] = ld8(ps + ((size_t)g * I + nc) * 8);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int gi = 0; gi < GPS; ++gi) {
    if (gi + D < GPS) {  // keep D groups in flight
      const int g2 = gb + gi + D;
#pragma unroll
      for (int q = 0; q < 4; ++q) rc[gi + D][q] = ld16(pq + (((size_t)(4 * g2 + q)) * I + nc) * 16);
      rs[gi + D] = ld8(ps + ((size_t)g2 * I + nc) * 8);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int g = gb + gi;
    float sc[8];
    e4m3x8(rs[gi], sc);
    v2bf_t w[8][8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      e2m1x8_bf16(word_of(rc[gi][b >> 1], (b & 1) * 2), w[b]);
      e2m1x8_bf16(word_of(rc[gi][b >> 1], (b & 1) * 2 + 1), w[b] + 4);
    }
#pragma unroll
    for (int t = 0; t < kMaxMT; ++t) {
      if (t < mt) {
        const uint4* xp = reinterpret_cast<const uint4*>(xs + (size_t)t * H + 128 * g);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const uint4 xa = xp[2 * b], xb = xp[2 * b + 1];
          float p = 0.0f;
          p = __builtin_amdgcn_fdot2_f32_bf16(w[b][0], as_v2bf(xa.x), p, false);
          p = __builtin_amdgcn_fdot2_f32_bf16(w[b][1], as_v2bf(xa.y), p, false);
          p = __builtin_amdgcn_fdot2_f32_bf16(w[b][2], as_v2bf(xa.z), p, false);
          p = __builtin_amdgcn_fdot2_f32_bf16(w[b][3], as_v2bf(xa.w), p, false);
          p = __builtin_amdgcn_fdot2_f32_bf16(w[b][4], as_v2bf(xb.x), p, false);
          p = __builtin_amdgcn_fdot2_f32_bf16(w[b][5], as_v2bf(xb.y), p, false);
          p = __builtin_amdgcn_fdot2_f32_bf16(w[b][6], as_v2bf(xb.z), p, false);
          p = __builtin_amdgcn_fdot2_f32_bf16(w[b][7], as_v2bf(xb.w), p, false);
          acc[t] = fmaf(p, sc[b], acc[t]);
        }
      }
    }
  }
}

template <int GPS, int D>
__global__ __launch_bounds__(512, 3) void k_gemv_gateup_nvfp4(
    const uint16_t* __restrict__ x, int H, int I, int ktop, int mt_max, int S, int gps_total,
    const moe_expert_ref* __restrict__ experts, size_t off_gq, size_t off_gs, size_t off_uq,
    size_t off_us, const uint32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_asg, const int32_t* __restrict__ active,
    const int32_t* __restrict__ n_active, float* __restrict__ hout) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                       // [mt_max][H]
  float* red = reinterpret_cast<float*>(smem + (size_t)mt_max * H * 2);   // [2S][mt_max][64]

  SlotInfo si;
  if (!slot_info(active, n_active, counts, offsets, experts, &si)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nthreads = 2 * S * 64;
  const int mat = wave / S, ks = wave - mat * S;
  const int n = blockIdx.x * 64 + lane;
  const size_t nc = (n < I) ? (size_t)n : 0;  // rows past the end read row 0, never stored
  const uint8_t* blob = (const uint8_t*)si.ref.blob;
  const uint8_t* pq = blob + (mat ? off_uq : off_gq);
  const uint8_t* ps = blob + (mat ? off_us : off_gs);
  const int gb = ks * gps_total;
  const int vpr = H >> 3;

  for (int c0 = 0; c0 < si.cnt; c0 += mt_max) {
    const int mt = min(mt_max, si.cnt - c0);
    // Gather this pass's token rows (bf16) into LDS before the weight loads
    // (memory counters retire in order).
    for (int i = tid; i < mt * vpr; i += nthreads) {
      const int r = i / vpr, c = i - r * vpr;
      const int tok = sorted_asg[si.base + c0 + r] / ktop;
      reinterpret_cast<uint4*>(xs + (size_t)r * H)[c] =
          reinterpret_cast<const uint4*>(x + (size_t)tok * H)[c];
    }
    __syncthreads();

    float acc[kMaxMT];
#pragma unroll
    for (int t = 0; t < kMaxMT; ++t) acc[t] = 0.0f;
    for (int sg = 0; sg < gps_total; sg += GPS)  // passes of GPS groups
      gateup_pass<GPS, D>(xs, H, I, nc, pq, ps, gb + sg, mt, acc);

    __syncthreads();
#pragma unroll
    for (int t = 0; t < kMaxMT; ++t)
      if (t < mt) red[(wave * mt_max + t) * 64 + lane] = acc[t];
    __syncthreads();
    for (int o = tid; o < mt * 64; o += nthreads) {
      const int t = o >> 6, r = o & 63;
      const int n2 = blockIdx.x * 64 + r;
      if (n2 < I) {
        float gsum = 0.0f, usum = 0.0f;
        for (int w = 0; w < S; ++w) {
          gsum += red[(w * mt_max + t) * 64 + r];
          usum += red[((S + w) * mt_max + t) * 64 + r];
        }
        gsum *= si.ref.ts_gate;
        usum *= si.ref.ts_up;
        hout[(size_t)(si.base + c0 + t) * I + n2] = gsum / (1.0f + expf(-gsum)) * usum;
      }
    }
  }
}

}  // namespace

hipError_t launch_gemv_gateup(const moe_layer_desc* L, const uint16_t* x, const moe_buckets* b,
                              int max_slots, int mt_max, float* h, hipStream_t s) {
  const BlobLayout lay = blob_layout(L->H, L->I, L->fmt_down);
  const int NG = L->H / 128;
  const int RB = (L->I + 63) / 64;
  // K split over S <= 4 waves per matrix (divisor of NG, within the wave
  // budget); each wave takes NG/S groups in passes of GP <= 8 groups.
  const int S = choose_split(max_slots * RB, 2, NG, 4);
  const int gps_total = NG / S;
  int GP = gps_total;
  if (GP > 8) {
    GP = 8;
    while (gps_total % GP) --GP;
  }
  dim3 grid((unsigned)RB, (unsigned)max_slots);
  dim3 block((unsigned)(2 * S * 64));
  size_t lds = (size_t)mt_max * L->H * 2 + sizeof(float) * 2 * S * mt_max * 64;
#define GU_LAUNCH(G)                                                                          \
  hipLaunchKernelGGL((k_gemv_gateup_nvfp4<G, (G < 2 ? G : 2)>), grid, block, lds, s, x, L->H, \
                     L->I, L->k, mt_max, S, gps_total, L->experts, lay.gate_q, lay.gate_s, lay.up_q,      \
                     lay.up_s, b->counts, b->offsets, b->sorted_asg, b->active, b->n_active, h)
  switch (GP) {
    case 1: GU_LAUNCH(1); break;
    case 2: GU_LAUNCH(2); break;
    case 3: GU_LAUNCH(3); break;
    case 4: GU_LAUNCH(4); break;
    case 5: GU_LAUNCH(5); break;
    case 6: GU_LAUNCH(6); break;
    case 7: GU_LAUNCH(7); break;
    default: GU_LAUNCH(8); break;
  }
#undef GU_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
