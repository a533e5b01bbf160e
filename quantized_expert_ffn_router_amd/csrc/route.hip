// route.hip -- router logits and top-k gating.
//
// Each token picks a few experts out of many (basalt.jgulfo.com, section
// "Expert tiers").  The router is an fp32 linear map; its logits are summed in
// double precision in one fixed order so that the selected experts are
// reproducible bit for bit:
//   partial j (lane j of a wavefront) adds x[h] * W[e][h] for h = j, j+64, ...
//   in ascending h (every bf16 x fp32 product is exact in double), the 64
//   partials are combined pairwise p[j] += p[j+w] for w = 32, 16, ..., 1, the
//   bias is added and the total is rounded once to fp32.
// A wavefront computes TB tokens x EB experts at once; the 64 partials of all
// TB*EB values are reduced with a transposed butterfly: at the level with
// partner lane^w each lane hands half of its values to the partner and keeps
// the other half, so the reduction costs about one shuffle per value and ends
// with value v on lane v * (64 / (TB*EB)).  The pairing at every level is the
// same as in the tree above, so the result is that tree's sum exactly.
#include "gate_common.h"

namespace moe {

namespace {

constexpr int kRouterWaves = 4;

// One level of the transposed butterfly with partner lane ^ W while NV values
// per lane remain: the lane with bit W clear keeps values [0, NV/2), the other
// keeps [NV/2, NV); each adds the partner's copy.  Once one value is left the
// remaining levels are plain pairwise sums.  All indices are compile time.
template <int NV, int W>
__device__ __forceinline__ void tb_level(double* acc, int lane) {
  if constexpr ((W == 32 || W == 16) && NV > 1) {
    // Across 32- or 16-lane groups the exchange is a register-half swap:
    // permlane{32,16}_swap(a, b) gives the lower group (a, partner's a) and
    // the upper group (partner's b, b), so a + b is keep + partner's copy on
    // both sides, as in the generic step below.
    constexpr int HALF = NV / 2;
#pragma unroll
    for (int i = 0; i < HALF; ++i) {
      const uint2 a = __builtin_bit_cast(uint2, acc[i]), b = __builtin_bit_cast(uint2, acc[i + HALF]);
      uint2 na, nb;
      if constexpr (W == 32) {
        const auto lo = __builtin_amdgcn_permlane32_swap(a.x, b.x, false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap(a.y, b.y, false, false);
        na = make_uint2(lo[0], hi[0]);
        nb = make_uint2(lo[1], hi[1]);
      } else {
        const auto lo = __builtin_amdgcn_permlane16_swap(a.x, b.x, false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap(a.y, b.y, false, false);
        na = make_uint2(lo[0], hi[0]);
        nb = make_uint2(lo[1], hi[1]);
      }
      acc[i] = __builtin_bit_cast(double, na) + __builtin_bit_cast(double, nb);
    }
    tb_level<HALF, W / 2>(acc, lane);
  } else if constexpr (W >= 1) {
    if constexpr (NV > 1) {
      constexpr int HALF = NV / 2;
      const bool upper = (lane & W) != 0;
#pragma unroll
      for (int i = 0; i < HALF; ++i) {
        const double send = upper ? acc[i] : acc[i + HALF];
        const double keep = upper ? acc[i + HALF] : acc[i];
        acc[i] = keep + __shfl_xor(send, W);
      }
      tb_level<HALF, W / 2>(acc, lane);
    } else {
      acc[0] = acc[0] + __shfl_xor(acc[0], W);
      tb_level<1, W / 2>(acc, lane);
    }
  }
}

// The 64-lane tree sum of one double per lane (lane j adds lane j + w for
// w = 32, 16, ..., 1), result in lane 0, without LDS-routed shuffles: the
// two cross-row levels swap register halves between lane groups
// (v_permlane32_swap, v_permlane16_swap; each lane then adds its partner's
// value, and lanes below w get exactly p[j] + p[j + w]), the levels within a
// row of 16 use DPP row shifts left (lane j reads lane j + w).
template <int W>
__device__ __forceinline__ double row_shl_f64(double v) {
  const uint2 u = __builtin_bit_cast(uint2, v);
  uint2 r;
  r.x = __builtin_amdgcn_update_dpp(0u, u.x, 0x100 | W, 0xf, 0xf, true);  // row_shl:W
  r.y = __builtin_amdgcn_update_dpp(0u, u.y, 0x100 | W, 0xf, 0xf, true);
  return __builtin_bit_cast(double, r);
}
__device__ __forceinline__ double tree_sum_lane0(double v) {
  uint2 u = __builtin_bit_cast(uint2, v);
  {  // w = 32
    const auto lo = __builtin_amdgcn_permlane32_swap(u.x, u.x, false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap(u.y, u.y, false, false);
    v = __builtin_bit_cast(double, make_uint2(lo[0], hi[0])) +
        __builtin_bit_cast(double, make_uint2(lo[1], hi[1]));
  }
  u = __builtin_bit_cast(uint2, v);
  {  // w = 16
    const auto lo = __builtin_amdgcn_permlane16_swap(u.x, u.x, false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap(u.y, u.y, false, false);
    v = __builtin_bit_cast(double, make_uint2(lo[0], hi[0])) +
        __builtin_bit_cast(double, make_uint2(lo[1], hi[1]));
  }
  v = v + row_shl_f64<8>(v);
  v = v + row_shl_f64<4>(v);
  v = v + row_shl_f64<2>(v);
  v = v + row_shl_f64<1>(v);
  return v;
}

template <int TB, int EB>
__global__ __launch_bounds__(kRouterWaves * 64) void k_router_logits(
    const uint16_t* __restrict__ x, int T, int H, const float* __restrict__ Wr,
    const float* __restrict__ bias, int E, float* __restrict__ logits) {
  constexpr int V = TB * EB;
  static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "TB*EB must be a power of two <= 64");
  extern __shared__ uint16_t xs[];  // [TB][H] bf16 bits
  // blockIdx.x = expert group, blockIdx.y = token block: the token blocks of
  // one expert group are 8-aligned strides of the linear workgroup id apart,
  // so they run on the same XCD (workgroup w on XCD w % 8) and share its L2
  // for the group's router rows.
  const int t0 = blockIdx.y * TB;
  if ((int)blockIdx.x * kRouterWaves * EB >= E) return;  // padding group: whole workgroup
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int e0 = (blockIdx.x * kRouterWaves + wave) * EB;

  const float* wrow[EB];
#pragma unroll
  for (int q = 0; q < EB; ++q) wrow[q] = Wr + (size_t)min(e0 + q, E - 1) * H;

  // Router weights are fetched CH strides at a time (all loads in flight
  // before the first use); terms are still added in ascending h.  The first
  // batch is issued before the token rows are staged, so the two memory
  // round trips overlap.
  constexpr int CH = (EB == 1) ? 32 : 8;
  float wv[CH][EB];
  auto load_w = [&](int h0) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      // Unconditional loads from a clamped (in-bounds) index keep every load
      // of the batch in flight; out-of-range strides are never added below.
      const int hc = min(h0 + 64 * c, H - 1);
#pragma unroll
      for (int q = 0; q < EB; ++q) wv[c][q] = wrow[q][hc];
    }
  };
  load_w(lane);

  // Stage the token block (rows past T are zero) with 16-byte loads.
  const int vec_per_row = H / 8;
  for (int i = tid; i < TB * vec_per_row; i += kRouterWaves * 64) {
    int r = i / vec_per_row, c = i % vec_per_row;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (t0 + r < T) v = *reinterpret_cast<const uint4*>(x + (size_t)(t0 + r) * H + 8 * c);
    *reinterpret_cast<uint4*>(xs + (size_t)r * H + 8 * c) = v;
  }
  __syncthreads();
  if (e0 >= E) return;

  double acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.0;

  for (int h0 = lane; h0 < H; h0 += 64 * CH) {
    if (h0 != lane) load_w(h0);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int h = h0 + 64 * c;
      if (h < H) {
#pragma unroll
        for (int i = 0; i < TB; ++i) {
          const double xv = (double)bf16_to_f32(xs[i * H + h]);
#pragma unroll
          for (int q = 0; q < EB; ++q)
            acc[i * EB + q] = __fma_rn(xv, (double)wv[c][q], acc[i * EB + q]);
        }
      }
    }
  }

  if constexpr (V == 1) {
    const double s0 = tree_sum_lane0(acc[0]);
    if (lane == 0 && t0 < T) {
      double s = s0;
      if (bias) s += (double)bias[e0];
      logits[(size_t)t0 * E + e0] = (float)s;
    }
    return;
  }
  // Transposed butterfly (see file comment).
  tb_level<V, 32>(acc, lane);
  constexpr int kShift = (V == 1) ? 6 : (V == 2) ? 5 : (V == 4) ? 4 : (V == 8) ? 3 : (V == 16) ? 2 : (V == 32) ? 1 : 0;
  if ((lane & ((1 << kShift) - 1)) == 0) {
    const int v = lane >> kShift;
    const int t = t0 + v / EB, e = e0 + v % EB;
    if (t < T && e < E) {
      double s = acc[0];
      if (bias) s += (double)bias[e];
      logits[(size_t)t * E + e] = (float)s;
    }
  }
}

// Router logits for batches past decode size.  A wavefront computes 8 tokens x
// 8 experts: per h, a lane converts the 8 activations and the 8 router weights
// of its h to double once and does 64 fmas, so conversions cost a quarter of
// the fma count.  The workgroup's 8 tokens are staged in LDS as fp32,
// transposed to [h][8], so a lane reads them with two 16-byte LDS reads; the
// four waves of a workgroup take 32 consecutive experts.  H is walked in
// chunks of at most kRtChunk so the tile fits in 64 KiB; every lane still adds
// its terms in ascending h, as in the file comment, and the result is
// bit-identical to k_router_logits.
//
// Workgroup w runs on XCD w % 8.  The expert groups of one token block are
// given to workgroups w, w + 8, w + 16, ..., all on one XCD, so the block's
// activations are read from HBM once and then hit that XCD's L2.
constexpr int kRtTok = 8, kRtExp = 8, kRtWaves = 4, kRtChunk = 2048;

struct RtOperands {
  float4 x0, x1;      // 8 activations (fp32) of one h
  float w[kRtExp];    // 8 router weights of the same h
};

// Operands of one lane h-step.  The router rows are wave-uniform base
// pointers plus a 32-bit byte offset kept opaque to the compiler, so each load
// is one instruction on a scalar base instead of a 64-bit vector address.
__device__ __forceinline__ void rt_load(RtOperands& o, const float4* xs, const float* const* wq,
                                        uint32_t boff, int i) {
  uint32_t off = boff + 256u * (uint32_t)i;
  asm volatile("" : "+v"(off));
  o.x0 = xs[128 * i];
  o.x1 = xs[128 * i + 1];
#pragma unroll
  for (int q = 0; q < kRtExp; ++q)
    o.w[q] = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(wq[q]) + off);
}

__device__ __forceinline__ void rt_fma(double* acc, const RtOperands& o) {
  double wd[kRtExp];
#pragma unroll
  for (int q = 0; q < kRtExp; ++q) wd[q] = (double)o.w[q];
  const float xv[kRtTok] = {o.x0.x, o.x0.y, o.x0.z, o.x0.w, o.x1.x, o.x1.y, o.x1.z, o.x1.w};
#pragma unroll
  for (int t = 0; t < kRtTok; ++t) {
    const double xd = (double)xv[t];
#pragma unroll
    for (int q = 0; q < kRtExp; ++q) acc[t * kRtExp + q] = __fma_rn(xd, wd[q], acc[t * kRtExp + q]);
  }
}

__global__ __launch_bounds__(kRtWaves * 64) void k_router_logits_blk(
    const uint16_t* __restrict__ x, int T, int H, const float* __restrict__ Wr,
    const float* __restrict__ bias, int E, float* __restrict__ logits, int n_tb, int n_eg) {
  extern __shared__ float4 xs4[];  // [h][8] fp32: two float4 per h
  const int wg = blockIdx.x;
  const int j = wg >> 3;
  const int tb = (j / n_eg) * 8 + (wg & 7);
  if (tb >= n_tb) return;  // whole workgroup: no barrier has been reached
  const int eg = j % n_eg;
  const int t0 = tb * kRtTok;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int e0 = (eg * kRtWaves + wave) * kRtExp;
  const bool live = e0 < E;  // wave-uniform; dead waves still take the barriers

  const float* wq[kRtExp];  // wave-uniform row pointers
#pragma unroll
  for (int q = 0; q < kRtExp; ++q) wq[q] = Wr + (size_t)min(e0 + q, E - 1) * H;
  // Token rows past T are read from row T - 1 and masked to zero.
  const uint16_t* xr[kRtTok];
  uint32_t xmask[kRtTok];
#pragma unroll
  for (int t = 0; t < kRtTok; ++t) {
    xr[t] = x + (size_t)min(t0 + t, T - 1) * H;
    xmask[t] = (t0 + t < T) ? 0xffffffffu : 0u;
  }

  double acc[kRtTok * kRtExp];
#pragma unroll
  for (int v = 0; v < kRtTok * kRtExp; ++v) acc[v] = 0.0;

  for (int hc0 = 0; hc0 < H; hc0 += kRtChunk) {
    const int hc = min(kRtChunk, H - hc0);  // multiple of 128
    if (hc0 > 0) __syncthreads();           // previous chunk fully read
    // Stage: thread p takes the h pair (2p, 2p+1) of all 8 tokens; rows past T
    // are zero.  bf16 -> fp32 is exact (bits << 16).
    for (int p = tid; p < hc / 2; p += kRtWaves * 64) {
      uint32_t v[kRtTok];
#pragma unroll
      for (int t = 0; t < kRtTok; ++t)
        v[t] = *reinterpret_cast<const uint32_t*>(xr[t] + hc0 + 2 * p) & xmask[t];
      float lo[kRtTok], hi[kRtTok];
#pragma unroll
      for (int t = 0; t < kRtTok; ++t) {
        lo[t] = __uint_as_float(v[t] << 16);
        hi[t] = __uint_as_float(v[t] & 0xffff0000u);
      }
      xs4[4 * p + 0] = make_float4(lo[0], lo[1], lo[2], lo[3]);
      xs4[4 * p + 1] = make_float4(lo[4], lo[5], lo[6], lo[7]);
      xs4[4 * p + 2] = make_float4(hi[0], hi[1], hi[2], hi[3]);
      xs4[4 * p + 3] = make_float4(hi[4], hi[5], hi[6], hi[7]);
    }
    __syncthreads();
    if (live) {
      // Lane h-steps i = 0 .. hc/64 - 1 (h = hc0 + lane + 64 i), operands
      // loaded two steps ahead.
      const float4* xl = xs4 + 2 * lane;
      const uint32_t boff = 4u * (uint32_t)(hc0 + lane);
      const int n = hc / 64;  // even
      // Each step's operands are loaded one step ahead, into the register set
      // the previous step has finished with; past the last step the loads
      // repeat step n - 1 (in bounds, unused).
      // Scheduling fences keep each group of loads ahead of the fmas that do
      // not need it (the scheduler would otherwise pull every load to the top
      // of the loop and wait on it at once).
      RtOperands a, b;
      rt_load(a, xl, wq, boff, 0);
      for (int i = 0; i < n; i += 2) {
        rt_load(b, xl, wq, boff, i + 1);
        __builtin_amdgcn_sched_barrier(0);
        rt_fma(acc, a);
        __builtin_amdgcn_sched_barrier(0);
        rt_load(a, xl, wq, boff, min(i + 2, n - 1));
        __builtin_amdgcn_sched_barrier(0);
        rt_fma(acc, b);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if (!live) return;

  // 64 values, 64 lanes: after the transposed butterfly value v is on lane v.
  tb_level<kRtTok * kRtExp, 32>(acc, lane);
  const int t = t0 + lane / kRtExp, e = e0 + lane % kRtExp;
  if (t < T && e < E) {
    double s = acc[0];
    if (bias) s += (double)bias[e];
    logits[(size_t)t * E + e] = (float)s;
  }
}

// One wavefront per token: k rounds of a wave-wide arg-max with key
// (logit desc, expert asc), then the gate weights.
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int T, int E,
                                              int k, int renorm, int32_t* __restrict__ idx,
                                              float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* l = logits + (size_t)t * E;
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    int e = lane + 64 * i;
    v[i] = (e < E) ? l[e] : 0.0f;
  }
  uint32_t taken = 0;
  for (int i = 0; i < 16; ++i)
    if (lane + 64 * i >= E) taken |= 1u << i;

  float my_v = 0.0f, top = 0.0f;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (!(taken & (1u << i))) {
        int e = lane + 64 * i;
        if (v[i] > bv || (v[i] == bv && e < be)) { bv = v[i]; be = e; }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      float ov = __shfl_xor(bv, off);
      int oe = __shfl_xor(be, off);
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (j == 0) top = bv;
    if (lane == j) { my_v = bv; my_e = be; }
  }

  float ex = (lane < k) ? expf(my_v - top) : 0.0f;
  float den;
  if (renorm) {
    den = ex;
  } else {
    den = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (lane + 64 * i < E) den += expf(v[i] - top);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);
  if (lane < k) {
    idx[(size_t)t * k + lane] = my_e;
    wout[(size_t)t * k + lane] = ex / den;
  }
}

template <int NV>
__device__ __forceinline__ void topk_wave(const float* __restrict__ l, int E, int k, int renorm,
                                          int lane, int* e_out, float* w_out) {
  float v[NV];
  topk_load<NV>(l, E, lane, v);
  topk_select<NV>(v, E, k, renorm, lane, e_out, w_out);
}

// One wavefront per token.
template <int NV>
__global__ __launch_bounds__(256) void k_topk_dpp(const float* __restrict__ logits, int T, int E,
                                                  int k, int renorm, int32_t* __restrict__ idx,
                                                  float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int e;
  float w;
  topk_wave<NV>(logits + (size_t)t * E, E, k, renorm, lane, &e, &w);
  if (lane < k) {
    idx[(size_t)t * k + lane] = e;
    wout[(size_t)t * k + lane] = w;
  }
}

// Decode-sized gating step in one workgroup (gate_common.h).
template <int NV>
__global__ __launch_bounds__(1024) void k_gate_fused(
    const float* __restrict__ logits, int T, int E, int k, int renorm,
    int32_t* __restrict__ idx, float* __restrict__ wout, uint32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ active, int32_t* __restrict__ n_active,
    int32_t* __restrict__ sorted, int32_t* __restrict__ pos, uint32_t* __restrict__ hist, int ds,
    int us, int nthr) {
  __shared__ GateLds g;
  // nthr = blockDim.x, passed as an argument so that no dispatch-packet field is read.
  const GateOut o = {idx, wout, counts, offsets, active, n_active, sorted, pos, hist, ds, us};
  gate_block<NV>(g, logits, T, E, k, renorm, o, true, threadIdx.x, nthr);
}

template <int TB, int EB>
hipError_t launch_router_t(const uint16_t* x, int64_t T, int H, const float* Wr,
                           const float* bias, int E, float* logits, hipStream_t s) {
  // x: expert groups rounded up to a multiple of 8 (see the kernel), y: token blocks
  const unsigned n_eg = (unsigned)((E + EB * kRouterWaves - 1) / (EB * kRouterWaves));
  dim3 grid((n_eg + 7u) & ~7u, (unsigned)((T + TB - 1) / TB));
  size_t lds = (size_t)TB * H * sizeof(uint16_t);
  hipLaunchKernelGGL((k_router_logits<TB, EB>), grid, dim3(kRouterWaves * 64), lds, s, x, (int)T,
                     H, Wr, bias, E, logits);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router(const uint16_t* x, int64_t T, int H, const float* Wr,
                         const float* bias, int E, float* logits, hipStream_t s) {
  // Decode-sized batches: one (token, expert) pair per wavefront -- many short
  // waves finish sooner than a few long ones.
  if (T <= 64) return launch_router_t<1, 1>(x, T, H, Wr, bias, E, logits, s);
  // Larger batches: 8 tokens x 8 experts per wavefront (H % 128 == 0).
  const int n_tb = (int)((T + kRtTok - 1) / kRtTok);
  const int n_eg = (E + kRtWaves * kRtExp - 1) / (kRtWaves * kRtExp);
  const int64_t n_wg = (int64_t)((n_tb + 7) / 8) * 8 * n_eg;
  const size_t lds = (size_t)min(H, kRtChunk) * kRtTok * sizeof(float);
  hipLaunchKernelGGL(k_router_logits_blk, dim3((unsigned)n_wg), dim3(kRtWaves * 64), lds, s, x,
                     (int)T, H, Wr, bias, E, logits, n_tb, n_eg);
  return hipGetLastError();
}

bool gate_fused_fits(int64_t T, int E, int k) {
  return E <= 256 && T <= 64 && T * k <= 256;
}

hipError_t launch_gate_fused(const float* logits, int64_t T, int E, int k, int renorm,
                             int32_t* idx, float* w, const moe_buckets* b, uint32_t* hist, int ds,
                             int us, hipStream_t s) {
  const unsigned threads = (unsigned)(64 * (T < 16 ? T : 16));
#define GF(NV)                                                                                   \
  hipLaunchKernelGGL(k_gate_fused<NV>, dim3(1), dim3(threads), 0, s, logits, (int)T, E, k,      \
                     renorm, idx, w, b->counts, b->offsets, b->active, b->n_active,      \
                     b->sorted_asg, b->asg_pos, hist, ds, us, (int)threads)
  if (E <= 64) GF(1);
  else if (E <= 128) GF(2);
  else GF(4);
#undef GF
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int64_t T, int E, int k, int renorm, int32_t* idx,
                       float* w, hipStream_t s) {
  dim3 grid((unsigned)((T + 3) / 4));
  if (E <= 64)
    hipLaunchKernelGGL(k_topk_dpp<1>, grid, dim3(256), 0, s, logits, (int)T, E, k, renorm, idx, w);
  else if (E <= 128)
    hipLaunchKernelGGL(k_topk_dpp<2>, grid, dim3(256), 0, s, logits, (int)T, E, k, renorm, idx, w);
  else if (E <= 256)
    hipLaunchKernelGGL(k_topk_dpp<4>, grid, dim3(256), 0, s, logits, (int)T, E, k, renorm, idx, w);
  else
    hipLaunchKernelGGL(k_topk, grid, dim3(256), 0, s, logits, (int)T, E, k, renorm, idx, w);
  return hipGetLastError();
}

}  // namespace moe
