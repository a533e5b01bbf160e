// gemv_gateup.hip -- decode-size gate/up projections of the routed experts,
// NVFP4 weights dequantized in registers, SwiGLU in the epilogue:
//   g = x . dq(Wg)^T, u = x . dq(Wu)^T, h = silu(g * ts_g) * (u * ts_u).
// A workgroup owns 64 rows of one active expert: waves [0, S) stream the gate
// matrix and waves [S, 2S) the up matrix, each over 1/S of K (gemv_common.h).
// E2M1 codes become exact bf16 pairs that meet the bf16 activations in
// v_dot2_f32_bf16 (fp32 accumulation); each 16-element block sum is scaled by
// its E4M3 scale (hardware conversion), the per-tensor scale by the total.
//
// Every lane of a wave needs the same activations (lanes are rows), so they
// are read with wave-uniform addresses: the compiler turns those into scalar
// loads through the scalar cache and feeds them to v_dot2 as SGPR operands.
// A broadcast from LDS instead costs a full 64-lane LDS read per 8 values,
// which measured as the limit of the kernel at batch 8.
// h leaves rounded to bf16 (the operand type of v_dot2 in the down
// projection), as in the prefill path.
#include "gemv_gateup.h"

namespace moe {

namespace {

template <int GPS, int D, int W>
__global__ __launch_bounds__(64 * W) void k_gemv_gateup_nvfp4(
    const uint16_t* __restrict__ x, int H, int I, int ktop, int kshift, int S, int gps_total,
    const moe_expert_ref* __restrict__ experts, size_t off_gq, size_t off_gs, size_t off_uq,
    size_t off_us, const uint32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_asg, const int32_t* __restrict__ active,
    const int32_t* __restrict__ n_active, uint16_t* __restrict__ hout) {
  __shared__ float red[W][kGuMT][64];  // [wave][token][row] partial sums over K

  int e;
  moe_expert_ref ref;
  if (!slot_expert(active, n_active, experts, &e, &ref)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int nthreads = 2 * S * 64;
  const int mat = wave / S, ks = wave - mat * S;
  const int n = blockIdx.x * 64 + lane;
  const size_t nc = (n < I) ? (size_t)n : 0;  // rows past the end read row 0, never stored
  const uint8_t* blob = (const uint8_t*)ref.blob;
  const uint8_t* pq = blob + (mat ? off_uq : off_gq);
  const uint8_t* ps = blob + (mat ? off_us : off_gs);
  const int gb = ks * gps_total;
  float* acc = &red[wave][0][0];

  // Batches of kGuMT tokens.  An active expert has at least one token, so the
  // first batch always runs; its first pass's weights are requested before
  // the token count and offset are read (see slot_expert).
  int cnt = 1, base = 0, mt = 0;
  for (int c0 = 0; c0 < cnt; c0 += kGuMT) {
    if (c0 > 0) __syncthreads();  // the previous batch's reads of red are done
    for (int sg = 0; sg < gps_total; sg += GPS) {  // passes of GPS groups
      GURing<GPS> R;
      gu_issue<GPS, D>(R, pq, ps, I, nc, gb + sg);
      __builtin_amdgcn_sched_barrier(0);
      if (sg == 0) {
        if (c0 == 0) {
          cnt = (int)counts[e];
          base = offsets[e];
        }
        mt = min(kGuMT, cnt - c0);
        for (int t = 0; t < mt; ++t) acc[t * 64 + lane] = 0.0f;  // this wave's slice only
      }
      {  // the pass's activations of the first 4 tokens (4 lines per group)
        uint32_t tch = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (t < mt)
            tch ^= touch_lines<4 * GPS>(
                reinterpret_cast<const uint32_t*>(
                    x + token_row(sorted_asg, base + c0 + t, ktop, kshift, H)) +
                64 * (gb + sg));
        keep_scalar(tch);
      }
      gu_consume<GPS, D>(R, x, sorted_asg, base + c0, ktop, kshift, H, I, nc, pq, ps, gb + sg,
                         mt, acc);
    }
    __syncthreads();
    for (int o = tid; o < mt * 64; o += nthreads) {
      const int t = o >> 6, r = o & 63;
      const int n2 = blockIdx.x * 64 + r;
      if (n2 < I) {
        float gsum = 0.0f, usum = 0.0f;
        for (int w = 0; w < S; ++w) {
          gsum += red[w][t][r];
          usum += red[S + w][t][r];
        }
        gsum *= ref.ts_gate;
        usum *= ref.ts_up;
        const float h = swiglu(gsum, usum);
        hout[(size_t)(base + c0 + t) * I + n2] = f32_to_bf16_rne(h);
      }
    }
  }
}

}  // namespace

hipError_t launch_gemv_gateup(const moe_layer_desc* L, const uint16_t* x, const moe_buckets* b,
                              int max_slots, uint16_t* h, hipStream_t s) {
  const BlobLayout lay = blob_layout(L->H, L->I, L->fmt_down);
  const int RB = (L->I + 63) / 64;
  int S, GP, gps_total;
  gu_split(L->H, RB, max_slots, &S, &GP, &gps_total);
  int kshift = -1;
  for (int i = 0; i < 31; ++i)
    if ((1 << i) == L->k) kshift = i;
  dim3 grid((unsigned)RB, (unsigned)max_slots);
  dim3 block((unsigned)(2 * S * 64));
#define GU_LAUNCH_W(G, W)                                                                       \
  hipLaunchKernelGGL((k_gemv_gateup_nvfp4<G, (G < 2 ? G : 2), W>), grid, block, 0, s, x, L->H, \
                     L->I, L->k, kshift, S, gps_total, L->experts, lay.gate_q, lay.gate_s,      \
                     lay.up_q, lay.up_s, b->counts, b->offsets, b->sorted_asg, b->active,       \
                     b->n_active, h)
#define GU_LAUNCH(G)          \
  if (S == 8) {               \
    GU_LAUNCH_W(G, 16);       \
  } else {                    \
    GU_LAUNCH_W(G, 8);        \
  }
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
#undef GU_LAUNCH_W
  return hipGetLastError();
}

}  // namespace moe
