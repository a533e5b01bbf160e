// gate_common.h -- top-k gating and decode-sized bucketing as device
// functions: the gating kernels (route.hip) and the gate/up kernel that does
// its own gating (gemv_gateup32.hip) share them, so both produce the same
// experts, weights and buckets bit for bit.
//
// Each token picks a few experts out of many (basalt.jgulfo.com, section
// "Expert tiers"): the k largest logits under the order (logit desc, index
// asc), weighted by a softmax restricted to them (renormalize = 1) or over
// all E (renormalize = 0).
#pragma once

#include <limits.h>

#include "common.h"

namespace moe {

// Orderable key of a logit: signed-integer order equals float order, -0
// and +0 get the same key (they compare equal as floats), NaN gets the
// lowest key.  key_to_float inverts it (a -0 comes back as +0, which gives
// the same gate weights).
__device__ __forceinline__ int logit_key(float f) {
  int b = __float_as_int(f);
  b = (b == (int)0x80000000) ? 0 : b;
  const int k = b ^ ((b >> 31) & 0x7fffffff);
  return (f != f) ? INT_MIN : k;
}
__device__ __forceinline__ float key_to_float(int k) {
  return __int_as_float(k ^ ((k >> 31) & 0x7fffffff));
}

// Wave-wide maximum with DPP moves (a few cycles each, unlike LDS-routed
// shuffles): lane pairs, quads, rows of 16 (rotate by 4 and 8), then row
// broadcasts; lane 63 ends with the maximum, broadcast with readlane.
// Lanes a row mask leaves out read INT_MIN (the identity of max), which lets
// the compiler fold the move into one v_max_i32 with a DPP source.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_max(int v) {
  return max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, CTRL, ROW_MASK, 0xf, false));
}

__device__ __forceinline__ int wave_max(int v) {
  v = dpp_max<0xb1, 0xf>(v);   // quad_perm [1,0,3,2]
  v = dpp_max<0x4e, 0xf>(v);   // quad_perm [2,3,0,1]
  v = dpp_max<0x124, 0xf>(v);  // row_ror:4
  v = dpp_max<0x128, 0xf>(v);  // row_ror:8 -> every lane holds its row's maximum
  v = dpp_max<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_max<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3 -> lane 63 holds the maximum
  return __builtin_amdgcn_readlane(v, 63);
}

// Top-k of one token's logits l[0..E) by one wavefront (E <= 64*NV): k
// rounds.  Expert e sits in slot e / 64 of lane e % 64.  A round takes the
// wave-wide maximum key m among the logits not yet taken, then the lowest
// expert index holding m among them (ballot per slot, lowest slot first,
// lowest set bit): the arg-max under the order (logit desc, index asc).
// Lane j < k gets the j-th expert and its weight.
template <int NV>
__device__ __forceinline__ void topk_load(const float* __restrict__ l, int E, int lane, float* v) {
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = l[min(lane + 64 * i, E - 1)];  // clamped, unconditional
}

template <int NV>
__device__ __forceinline__ void topk_select(const float* v, int E, int k, int renorm, int lane,
                                            int* e_out, float* w_out) {
  int key[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) key[i] = logit_key(v[i]);
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (lane + 64 * i >= E) taken |= 1u << i;

  float my_v = 0.0f, top = 0.0f;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    int bk = INT_MIN;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (!(taken & (1u << i))) bk = max(bk, key[i]);
    const int m = wave_max(bk);
    int be = -1;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const unsigned long long b = __ballot(!(taken & (1u << i)) && key[i] == m);
      if (be < 0 && b != 0ull) be = 64 * i + __ffsll((long long)b) - 1;
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    const float mv = key_to_float(m);
    if (j == 0) top = mv;
    if (lane == j) { my_v = mv; my_e = be; }
  }

  float ex = (lane < k) ? expf(my_v - top) : 0.0f;
  float den;
  if (renorm) {
    den = ex;
  } else {
    den = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (lane + 64 * i < E) den += expf(v[i] - top);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);
  *e_out = my_e;
  *w_out = ex / den;
}

// Wave-wide inclusive prefix sum with DPP (rows of 16 by shifts 1, 2, 4, 8,
// then row broadcasts 15 and 31 carry the row totals up).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return v;
}

// Results of gate_block kept in LDS for the calling workgroup.
struct GateLds {
  int keys[256];                  // expert of assignment a = t*k + j
  unsigned long long tmask[256];  // bit t set: token t is routed to expert e
  int off[256];                   // first sorted position of expert e
  int active[256];                // the active experts, ascending (first n_active)
  int n_active;
};

// Global outputs of gate_block (the moe_route_bucket outputs); hist may be
// NULL.
struct GateOut {
  int32_t* idx;
  float* w;
  uint32_t* counts;
  int32_t* offsets;
  int32_t* active;
  int32_t* n_active;
  int32_t* sorted;
  int32_t* pos;
  uint32_t* hist;
  int ds, us;
};

// Decode-sized gating step by one workgroup of nthr threads (a multiple of
// 64; E <= 256, T*k <= 256, T <= 64): top-k of every token (a wavefront per
// token), then the same bucketing as moe_bucket, computed in parallel: each
// token's wavefront sets bit t of tmask[e] for its k experts (LDS atomics; a
// token's experts are distinct), so counts[e] = popcount(tmask[e]) and
// assignment (t, j) of expert e sits at offsets[e] + popcount(tmask[e] below
// bit t) -- ascending t within an expert, which is ascending a = t*k + j, the
// stable order.  The usage histogram is updated from the counts.  The LDS
// results are visible to the whole workgroup on return; the global outputs
// (out, passed by value so that it stays in registers) are written only when
// write is true.
template <int NV>
__device__ __forceinline__ void gate_block(GateLds& g, const float* __restrict__ logits, int T,
                                           int E, int k, int renorm, GateOut out, bool write,
                                           int tid, int nthr) {
  const int lane = tid & 63, wave = tid >> 6, nw = nthr >> 6;
  // The histogram words are loaded now, so their latency hides behind top-k
  // (E <= 256 <= 4 * nthr).
  uint32_t hv[4];
  const bool hist = write && out.hist != nullptr;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = tid + j * nthr;
    hv[j] = (hist && e < E) ? out.hist[e] : 0u;
  }
  // The first token's logits of each wave are requested before the LDS
  // clear and its barrier.
  float v0[NV];
  topk_load<NV>(logits + (size_t)min(wave, T - 1) * E, E, lane, v0);
  for (int e = tid; e < E; e += nthr) g.tmask[e] = 0ull;
  __syncthreads();
  for (int t = wave; t < T; t += nw) {
    int e;
    float w;
    float v[NV];
    if (t == wave) {
#pragma unroll
      for (int i = 0; i < NV; ++i) v[i] = v0[i];
    } else {
      topk_load<NV>(logits + (size_t)t * E, E, lane, v);
    }
    topk_select<NV>(v, E, k, renorm, lane, &e, &w);
    if (lane < k) {
      if (write) {
        out.idx[(size_t)t * k + lane] = e;
        out.w[(size_t)t * k + lane] = w;
      }
      g.keys[t * k + lane] = e;
      atomicOr(&g.tmask[e], 1ull << t);
    }
  }
  __syncthreads();
  if (wave == 0) {  // counts, offsets and the active list: lane owns experts 4*lane .. +4
    int c[4], sc = 0, sa = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      c[i] = (e < E) ? __popcll(g.tmask[e]) : 0;
      sc += c[i];
      sa += c[i] > 0;
    }
    const int ic = wave_incl_scan(sc), ia = wave_incl_scan(sa);
    int run = ic - sc, arun = ia - sa;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      if (e < E) {
        if (write) {
          out.counts[e] = (uint32_t)c[i];
          out.offsets[e] = run;
          if (c[i] > 0) out.active[arun] = e;
        }
        g.off[e] = run;
        if (c[i] > 0) g.active[arun++] = e;
        run += c[i];
      }
    }
    if (lane == 63) {
      if (write) {
        out.offsets[E] = ic;
        *out.n_active = ia;
      }
      g.n_active = ia;
    }
  }
  __syncthreads();
  if (!write) return;
  for (int a = tid; a < T * k; a += nthr) {
    const int t = a / k, e = g.keys[a];
    const int p = g.off[e] + __popcll(g.tmask[e] & ((1ull << t) - 1ull));
    out.sorted[p] = a;
    out.pos[a] = p;
  }
  if (!hist) return;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = tid + j * nthr;
    if (e < E) out.hist[e] = hv[j] - (hv[j] >> out.ds) + ((uint32_t)__popcll(g.tmask[e]) << out.us);
  }
}

}  // namespace moe
