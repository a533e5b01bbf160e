// gemv_gateup32.hip -- decode-size gate/up projections of the routed experts
// in 32-row (or, for the smallest batches, 24-row) slices, all of a
// workgroup's weight loads issued when it starts.
//
// A workgroup (8 waves) owns one active expert and one slice of R = 32 (or
// 24, see g32_rows) consecutive rows of its intermediate dimension (slice j:
// rows Rj..Rj+R-1), and computes h = silu(g * ts_g) * (u * ts_u) for those
// rows and the expert's tokens:
//   - in every wave lanes 0..31 are the gate rows and lanes 32..63 the same
//     up rows (with R = 24, lanes 24..31 and 56..63 repeat the last row and
//     are not stored), and wave w takes K granules (32 elements) w, w + 8, w + 16,
//     ...: all lanes of a wave use the same activations, which are read with
//     wave-uniform addresses (scalar loads, SGPR operands of v_dot2);
//   - each lane's granules (8 of 16 bytes for H = 2048, with their E4M3 scale
//     pairs) are all requested when the workgroup starts, before the expert's
//     token count is even read; per token they are decoded to exact bf16
//     pairs (the decode is redone per token, so the decoded pairs of only one
//     granule are live at a time);
//   - the 8 waves' partial sums are added in wave order through LDS, SwiGLU
//     pairs lane n (gate) with lane n + 32 (up), and h is stored rounded to
//     bf16, the operand type of the down GEMV.
// Against the 64-row GEMV (gemv_gateup.hip) this doubles the workgroups
// (192 at batch 1, about 1,200 at batch 8) and keeps a workgroup's whole
// working set in flight from its start: a probe streaming the same bytes with
// that shape (512 threads, 50-150 KB per workgroup, all loads up front) runs
// at 4.9 TB/s for the batch-1 bytes and 6.1-6.5 TB/s for the batch-8 bytes.
//
// Workgroup order: 4 consecutive slices of an expert run on one XCD one
// after another (block ids 8 apart), sharing that XCD's L2 for the expert's
// token rows.
//
// k_gemv_gate_gateup32 starts with the decode gating (gate_common.h) from the
// router logits: each workgroup runs the top-k and bucketing of the whole
// batch into its LDS, finds its slot's expert there and goes on as above;
// workgroup 0 also writes the gating outputs (top-k, buckets, histogram).
// One launch fewer per layer step than gating and gate/up apart, the same
// results bit for bit.
#include <mutex>

#include "gate_common.h"
#include "gemv_gateup.h"

namespace moe {

namespace {

constexpr int kG32Waves = 8;
constexpr int kG32Threads = 64 * kG32Waves;

// Slice of workgroup b: groups of 4 consecutive slices on XCD b % 8, the 4
// consecutive on it (block ids 8 apart).
__device__ __forceinline__ bool g32_item(int NS, int max_slots, int* slot, int* j) {
  const int b = blockIdx.x, x = b & 7, r = b >> 3;
  const int group = (r >> 2) * 8 + x, q = r & 3;
  const int gps = NS >> 2;  // groups per expert
  *slot = group / gps;
  *j = (group - *slot * gps) * 4 + q;
  return *slot < max_slots;
}

template <int NP>
struct G32A {  // a lane's weights: NP granules (32 elements) and their scale pairs
  uint4 c[NP];
  uint32_t s[NP];  // the two E4M3 scales of each granule (low 16 bits)
};

// Loads at a wave-uniform address plus a 32-bit per-lane byte offset.  The
// empty asm makes the lane offset opaque at each load, so the address is
// formed right there from the uniform part (scalar registers) and one VGPR
// instead of the compiler precomputing and holding (or spilling) the
// addresses of every load.
__device__ __forceinline__ uint4 bl16(const uint8_t* blob, uint32_t uoff, uint32_t lane_off) {
  __asm__ volatile("" : "+v"(lane_off));
  return ld16(blob + (lane_off + uoff));
}
__device__ __forceinline__ uint32_t bl2(const uint8_t* blob, uint32_t uoff, uint32_t lane_off) {
  __asm__ volatile("" : "+v"(lane_off));
  return ld2(blob + (lane_off + uoff));
}

// Granule i of wave w: K granule cg = w + 8 i of the lane's matrix (gate for
// lanes < 32, up otherwise).  oq / os: the lane's byte offsets of its
// matrix's code and scale planes plus its row (n * 16, n * 8).
template <int NP>
__device__ __forceinline__ void g32_load(G32A<NP>& r, const uint8_t* blob, uint32_t oq,
                                         uint32_t os, int I, int w) {
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int cg = w + kG32Waves * i;
    r.c[i] = bl16(blob, (uint32_t)cg * (uint32_t)I * 16u, oq);
    r.s[i] = bl2(blob, (uint32_t)(cg >> 2) * (uint32_t)I * 8u + 2u * (uint32_t)(cg & 3), os);
  }
}

// Token row offset (elements) of sorted assignment p.
__device__ __forceinline__ uint32_t g32_row(const int32_t* __restrict__ sorted_asg, int p, int ktop,
                                            int kshift, int H) {
  const int a = sorted_asg[p];
  return (uint32_t)(kshift >= 0 ? (a >> kshift) : a / ktop) * (uint32_t)H;
}

// One token: the lane's dot products over its granules (each decoded to exact
// bf16 pairs, 16 v_dot2 with the token's activations as scalar operands, the
// two block scales applied in fp32).
template <int NP>
__device__ __forceinline__ float g32_token(const G32A<NP>& r, const uint16_t* __restrict__ x,
                                           uint32_t xrow, int w) {
  float acc = 0.0f;
  const uint16_t* xr = x + xrow;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int cg = w + kG32Waves * i;
    // The decode is the same for every token; the opaque copy keeps it
    // inside the caller's token loop (hoisted, the decoded pairs of all
    // granules would take 16 registers each).
    uint4 c = r.c[i];
    uint32_t sw = r.s[i];
    __asm__ volatile("" : "+v"(c.x), "+v"(c.y), "+v"(c.z), "+v"(c.w), "+v"(sw));
    v2bf_t wv[16];
    e2m1x8_bf16(c.x, wv);
    e2m1x8_bf16(c.y, wv + 4);
    e2m1x8_bf16(c.z, wv + 8);
    e2m1x8_bf16(c.w, wv + 12);
    const v2f_t sc = e4m3x2<false>(sw);
    const uint32_t* xp = reinterpret_cast<const uint32_t*>(xr) + 16 * cg;
    float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      p0 = __builtin_amdgcn_fdot2_f32_bf16(as_v2bf(xp[k]), wv[k], p0, false);
      p1 = __builtin_amdgcn_fdot2_f32_bf16(as_v2bf(xp[8 + k]), wv[8 + k], p1, false);
    }
    acc = fmaf(p1, sc.y, fmaf(p0, sc.x, acc));
    __builtin_amdgcn_sched_barrier(0);  // one granule's decoded pairs live at a time
  }
  return acc;
}

template <int NP, int R>
__global__ __launch_bounds__(kG32Threads) __attribute__((amdgpu_waves_per_eu(4))) void
k_gemv_gateup32_nvfp4(const uint16_t* __restrict__ x, int H, int I, int ktop, int kshift, int NS,
                      int max_slots, int nparts, const moe_expert_ref* __restrict__ experts,
                      size_t off_gq, size_t off_gs, size_t off_uq, size_t off_us,
                      const uint32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
                      const int32_t* __restrict__ sorted_asg, const int32_t* __restrict__ active,
                      const int32_t* __restrict__ n_active, uint16_t* __restrict__ hout) {
  __shared__ float red[kG32Waves][kGuMT][64];  // [wave][token][lane] partial sums

  int slot, j;
  if (!g32_item(NS, max_slots, &slot, &j)) return;
  const int na = __builtin_nontemporal_load(n_active);
  const int e = __builtin_nontemporal_load(active + slot);
  asm volatile("" ::"s"(na), "s"(e), "s"(experts));
  if (slot >= na) return;
  const moe_expert_ref ref = experts[e];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool up = lane >= 32;
  // row of the slice (R rows: lanes past R in each half repeat row R - 1's
  // loads, in bounds, and their sums are never stored)
  const uint32_t n = (uint32_t)j * (uint32_t)R + (uint32_t)min(lane & 31, R - 1);
  const uint8_t* blob = (const uint8_t*)ref.blob;  // wave-uniform
  const uint32_t aq = (uint32_t)(up ? off_uq : off_gq) + n * 16u;
  const uint32_t as = (uint32_t)(up ? off_us : off_gs) + n * 8u;
  const bool part = wave < nparts;  // waves past the K parts of a small H stay idle

  // Batches of kGuMT tokens (an active expert has at least one).  Each batch
  // starts by issuing all of the lane's weight loads (unconditionally here,
  // so the compiler does not keep them live across the loop); for the first
  // batch that is before the expert's token count and offset are read.
  int c0 = 0, cnt = 1, base = 0;
  do {
    if (c0 > 0) __syncthreads();  // the previous batch's reads of red are done
    G32A<NP> ra;
    if (part) g32_load<NP>(ra, blob, aq, as, I, wave);
    __builtin_amdgcn_sched_barrier(0);
    if (c0 == 0) {
      cnt = (int)counts[e];
      base = offsets[e];
    }
    const int mt = min(kGuMT, cnt - c0);
    if (part) {
      // One word of each 64-byte activation line this wave will read, for
      // the first 4 tokens, while the weights are still in flight: the lines
      // are then in the scalar cache when the dot products need them (else
      // each token's first reads would wait a memory round trip after the
      // weights have arrived).
      uint32_t tch = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t < mt) {
          const uint32_t* xp = reinterpret_cast<const uint32_t*>(
              x + g32_row(sorted_asg, base + c0 + t, ktop, kshift, H));
#pragma unroll
          for (int i = 0; i < NP; ++i) tch ^= xp[16 * (wave + kG32Waves * i)];
        }
      }
      keep_scalar(tch);
#pragma unroll 1
      for (int t = 0; t < mt; ++t)
        red[wave][t][lane] =
            g32_token<NP>(ra, x, g32_row(sorted_asg, base + c0 + t, ktop, kshift, H), wave);
    }
    __syncthreads();
    for (int o = tid; o < mt * 32; o += kG32Threads) {
      const int t = o >> 5, r = o & 31;
      if (r >= R) continue;
      float g = 0.0f, u = 0.0f;
      for (int w = 0; w < nparts; ++w) {
        g += red[w][t][r];
        u += red[w][t][32 + r];
      }
      hout[(size_t)(base + c0 + t) * I + j * R + r] =
          f32_to_bf16_rne(swiglu(g * ref.ts_gate, u * ref.ts_up));
    }
    c0 += kGuMT;
  } while (c0 < cnt);
}

// The gating of the batch (all T tokens) by every workgroup, then its slice
// of gate/up as in k_gemv_gateup32_nvfp4 (T <= kGateGemvMaxT: one pass of
// tokens).
template <int NP, int NV, int R>
__global__ __launch_bounds__(kG32Threads) __attribute__((amdgpu_waves_per_eu(4))) void
k_gemv_gate_gateup32(const uint16_t* __restrict__ x, int H, int I, int ktop, int NS,
                     int max_slots, int nparts, const moe_expert_ref* __restrict__ experts,
                     size_t off_gq, size_t off_gs, size_t off_uq, size_t off_us,
                     const float* __restrict__ logits, int T, int E, int renorm, GateOut out,
                     uint16_t* __restrict__ hout) {
  __shared__ float red[kG32Waves][kGuMT][64];  // [wave][token][lane] partial sums
  __shared__ GateLds gl;
  __shared__ int s_tok[kGuMT];  // the expert's tokens, ascending

  int slot, j;
  if (!g32_item(NS, max_slots, &slot, &j)) return;  // block 0 has slot 0
  const int tid = threadIdx.x, lane = tid & 63;
  gate_block<NV>(gl, logits, T, E, ktop, renorm, out, blockIdx.x == 0, tid, kG32Threads);
  if (slot >= gl.n_active) return;
  const int e = gl.active[slot];
  const moe_expert_ref ref = experts[e];
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool up = lane >= 32;
  // row of the slice (as in k_gemv_gateup32_nvfp4)
  const uint32_t n = (uint32_t)j * (uint32_t)R + (uint32_t)min(lane & 31, R - 1);
  const uint8_t* blob = (const uint8_t*)ref.blob;  // wave-uniform
  const uint32_t aq = (uint32_t)(up ? off_uq : off_gq) + n * 16u;
  const uint32_t as = (uint32_t)(up ? off_us : off_gs) + n * 8u;
  const bool part = wave < nparts;

  G32A<NP> ra;
  if (part) g32_load<NP>(ra, blob, aq, as, I, wave);
  __builtin_amdgcn_sched_barrier(0);
  const unsigned long long m = gl.tmask[e];
  const int cnt = __popcll(m), base = gl.off[e];
  if (tid < T && ((m >> tid) & 1ull)) s_tok[__popcll(m & ((1ull << tid) - 1ull))] = tid;
  __syncthreads();
  if (part) {
    // the first 4 tokens' activation lines, while the weights are in flight
    uint32_t tch = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < cnt) {
        const uint32_t* xp = reinterpret_cast<const uint32_t*>(x + (size_t)s_tok[t] * H);
#pragma unroll
        for (int i = 0; i < NP; ++i) tch ^= xp[16 * (wave + kG32Waves * i)];
      }
    }
    keep_scalar(tch);
#pragma unroll 1
    for (int t = 0; t < cnt; ++t)
      red[wave][t][lane] = g32_token<NP>(ra, x, (uint32_t)s_tok[t] * (uint32_t)H, wave);
  }
  __syncthreads();
  for (int o = tid; o < cnt * 32; o += kG32Threads) {
    const int t = o >> 5, r = o & 31;
    if (r >= R) continue;
    float g = 0.0f, u = 0.0f;
    for (int w = 0; w < nparts; ++w) {
      g += red[w][t][r];
      u += red[w][t][32 + r];
    }
    hout[(size_t)(base + t) * I + j * R + r] =
        f32_to_bf16_rne(swiglu(g * ref.ts_gate, u * ref.ts_up));
  }
}

}  // namespace

namespace {

// CUs of the current device, looked up once per device (0 if unknown).
constexpr int kG32MaxDevices = 64;
std::once_flag g_g32_cu_once[kG32MaxDevices];
int g_g32_cus[kG32MaxDevices];

int g32_device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kG32MaxDevices) return 0;
  std::call_once(g_g32_cu_once[dev], [dev] {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) c = 0;
    g_g32_cus[dev] = c;
  });
  return g_g32_cus[dev];
}

// Rows per slice: 32, or 24 when the 32-row grid would give the CUs at most
// 1.5 workgroups each (decode batches of 1 and 2 tokens at I = 768: 192 and
// 384 workgroups on 256 CUs) and I splits into groups of 4 such slices.  A
// workgroup then carries 3/4 of the bytes, the busiest CU pulls fewer of
// them (batch 1: 256 workgroups of 55 KB instead of 192 of 74 KB), and the
// idle lanes (8 of each 32) cost nothing that is not already waiting on
// memory at these batch sizes.
int g32_rows(const moe_layer_desc* L, int max_slots) {
  if (L->I % 96 != 0) return 32;
  const int cus = g32_device_cus();
  return (cus > 0 && 2 * (int64_t)max_slots * (L->I / 32) <= 3 * (int64_t)cus) ? 24 : 32;
}

}  // namespace

bool gemv_gateup32_fits(const moe_layer_desc* L) {
  // whole granules per wave (H/32 <= 8, or a multiple of 8 granules) and at
  // most 8 of them per lane (H <= 2048); 128-row groups of slices
  const int ngran = L->H / 32;
  return L->fmt_gate_up == MOE_FMT_NVFP4 && L->H % 32 == 0 && L->H <= 8 * kG32Threads / 2 &&
         (ngran <= kG32Waves || ngran % kG32Waves == 0) && L->I % 128 == 0;
}

hipError_t launch_gemv_gateup32(const moe_layer_desc* L, const uint16_t* x, const moe_buckets* b,
                                int max_slots, uint16_t* h, hipStream_t s) {
  const BlobLayout lay = blob_layout(L->H, L->I, L->fmt_down);
  const int R = g32_rows(L, max_slots);
  const int NS = L->I / R;
  // K parts: one per wave (H/32 granules over at most 8 waves), NP <= 8 each
  const int ngran = L->H / 32;
  const int nparts = ngran < kG32Waves ? ngran : kG32Waves;
  const int NP = ngran / nparts;
  int kshift = -1;
  for (int i = 0; i < 31; ++i)
    if ((1 << i) == L->k) kshift = i;
  // 4-slice groups: max_slots * NS / 4 of them, 8 XCD lanes x 4 slices each
  const int groups = max_slots * (NS / 4);
  const unsigned nblocks = (unsigned)(((groups + 7) / 8) * 32);
#define G32R(P, RR)                                                                            \
  hipLaunchKernelGGL((k_gemv_gateup32_nvfp4<P, RR>), dim3(nblocks), dim3(kG32Threads), 0, s, x, \
                     L->H, L->I, L->k, kshift, NS, max_slots, nparts, L->experts, lay.gate_q,   \
                     lay.gate_s, lay.up_q, lay.up_s, b->counts, b->offsets, b->sorted_asg,      \
                     b->active, b->n_active, h)
#define G32(P)        \
  if (R == 24)        \
    G32R(P, 24);      \
  else                \
    G32R(P, 32)
  switch (NP) {
    case 1: G32(1); break;
    case 2: G32(2); break;
    case 3: G32(3); break;
    case 4: G32(4); break;
    case 5: G32(5); break;
    case 6: G32(6); break;
    case 7: G32(7); break;
    default: G32(8); break;
  }
#undef G32
#undef G32R
  return hipGetLastError();
}

// Every workgroup repeats the batch's gating before it knows its expert: at
// batch 8 that put about 3 us more in front of each workgroup's weight loads
// than the separate gating launch costs (step 44.4 against 41.6 us), while up
// to 4 tokens it saves 0.8-1.0 us per step.
constexpr int kGateGemvMaxT = 4;

bool gemv_gate_gateup32_fits(const moe_layer_desc* L, int64_t T) {
  return gemv_gateup32_fits(L) && gate_fused_fits(T, L->E, L->k) && T <= kGateGemvMaxT;
}

hipError_t launch_gemv_gate_gateup32(const moe_layer_desc* L, const uint16_t* x, int64_t T,
                                     const float* logits, int32_t* idx, float* w,
                                     const moe_buckets* b, uint32_t* hist, int ds, int us,
                                     int max_slots, uint16_t* h, hipStream_t s) {
  const BlobLayout lay = blob_layout(L->H, L->I, L->fmt_down);
  const int R = g32_rows(L, max_slots);
  const int NS = L->I / R;
  const int ngran = L->H / 32;
  const int nparts = ngran < kG32Waves ? ngran : kG32Waves;
  const int NP = ngran / nparts;
  const int groups = max_slots * (NS / 4);
  const unsigned nblocks = (unsigned)(((groups + 7) / 8) * 32);
  const GateOut out = {idx, w, b->counts, b->offsets, b->active, b->n_active, b->sorted_asg,
                       b->asg_pos, hist, ds, us};
#define GGR(P, V, RR)                                                                           \
  hipLaunchKernelGGL((k_gemv_gate_gateup32<P, V, RR>), dim3(nblocks), dim3(kG32Threads), 0, s,  \
                     x, L->H, L->I, L->k, NS, max_slots, nparts, L->experts, lay.gate_q,        \
                     lay.gate_s, lay.up_q, lay.up_s, logits, (int)T, L->E, L->renormalize, out, h)
#define GG(P, V)         \
  if (R == 24)           \
    GGR(P, V, 24);       \
  else                   \
    GGR(P, V, 32)
#define GG_NP(V)                 \
  switch (NP) {                  \
    case 1: GG(1, V); break;     \
    case 2: GG(2, V); break;     \
    case 3: GG(3, V); break;     \
    case 4: GG(4, V); break;     \
    case 5: GG(5, V); break;     \
    case 6: GG(6, V); break;     \
    case 7: GG(7, V); break;     \
    default: GG(8, V); break;    \
  }
  if (L->E <= 64) {
    GG_NP(1);
  } else if (L->E <= 128) {
    GG_NP(2);
  } else {
    GG_NP(4);
  }
#undef GG_NP
#undef GG
#undef GGR
  return hipGetLastError();
}

}  // namespace moe
