// gemv_down.hip -- decode-size down projection of the routed experts:
// y[p] = h[p] . dq(Wd)^T for each sorted assignment p of an active expert.
//   NVFP4: E2M1 codes, E4M3 scale per 16 elements, fp32 per-tensor scale.
//   Q6_K-style (the DQ6_K packs of basalt.jgulfo.com, "Quick start"):
//     256-element superblocks, 6-bit codes q in a low-nibble plane and a
//     2-bit plane, int8 sub-scale per 16 elements, fp16 scale d:
//     w = d * sc * (q - 32).
//   Q8_0 (the 8-bit GGUF blocks of basalt.jgulfo.com, "All the numbers"):
//     32-element blocks, fp16 scale d, int8 codes q: w = d * q.
//   IQ3G (IQ3-style codebook, own grid, iq3g.h): per 4 elements an 8-bit index
//     into a grid of odd magnitudes m <= 9, a sign bit per element, an odd
//     multiplier 2 s + 1 per 32 and fp16 d per 256: w = d * (2 s + 1) * +-m.
//   IQ1G (IQ1-style codebook, own grid, iq1g.h): per 8 elements a 10-bit index
//     into a grid of ternary vectors v in {-1, 0, +1}^8, an odd multiplier
//     2 s + 1 per 32 and fp16 d per 256: w = d * (2 s + 1) * v.
// Weights are decoded exactly to bf16 (E2M1 has 2 significant bits, q - 32 is
// a 6-bit integer, an int8 code has at most 8) and meet h (bf16, from the gate/up kernel) in
// v_dot2_f32_bf16 with fp32 accumulation.  Each 16-element block sum is scaled
// by its block scale (E4M3, or d * sc).  A workgroup owns 64 rows of one
// active expert; its S waves split K into 128-element groups (gemv_common.h),
// loads kept D groups ahead in group order.  Every lane needs every h value of
// its K-slice (lanes are rows), so h is read with wave-uniform addresses:
// scalar loads, SGPR operands of v_dot2, no per-value VALU broadcast (the
// kernel is otherwise close to its VALU budget).  Each wave accumulates its
// per-token sums in its own LDS slice.
#include "gemv_common.h"

namespace moe {

namespace {

constexpr int kDnMT = 16;  // tokens per batch (an expert's further tokens take more batches)

// Raw bytes of one 128-element group of a row.
template <int FMT>
struct Group;

template <>
struct Group<MOE_FMT_NVFP4> {
  uint4 c[4];  // 64 code bytes
  uint2 s;     // 8 E4M3 scales
};

template <>
struct Group<MOE_FMT_Q6K> {
  uint4 ql[4];  // low nibbles of the half superblock
  uint4 qh[2];  // 2-bit high parts
  uint2 sc;     // 8 int8 sub-scales
  uint32_t d;   // fp16 superblock scale
};

template <>
struct Group<MOE_FMT_Q8_0> {
  uint4 c[8];  // 128 int8 codes, 16 per granule
  uint2 s;     // fp16 scales of the group's 4 blocks of 32
};

template <>
struct Group<MOE_FMT_IQ3G> {
  uint4 q[2];  // 32 grid indices
  uint4 sg;    // 128 sign bits
  uint2 sc;    // d fp16 and the superblock's 8 nibble multipliers
};

template <>
struct Group<MOE_FMT_IQ1G> {
  uint4 q;      // low bytes of the 16 grid indices (8 elements each)
  uint32_t qh;  // their 2-bit high parts
  uint2 sc;     // d fp16 and the superblock's 8 nibble multipliers
};

struct Planes {
  const uint8_t* a;  // NVFP4 codes | Q6_K ql | Q8_0 codes | IQ3G indices | IQ1G index low bytes
  const uint8_t* b;  // NVFP4 scales | Q6_K qh | Q8_0 scales | IQ3G signs | IQ1G index high bits
  const uint8_t* c;  // Q6_K sc | IQ3G, IQ1G d and multipliers
  const uint8_t* d;  // Q6_K d
};

__device__ __forceinline__ void load_group(Group<MOE_FMT_NVFP4>& r, const Planes& P, int H,
                                           size_t nc, int g) {
#pragma unroll
  for (int q = 0; q < 4; ++q) r.c[q] = ld16(P.a + (((size_t)(4 * g + q)) * H + nc) * 16);
  r.s = ld8(P.b + ((size_t)g * H + nc) * 8);
}

__device__ __forceinline__ void load_group(Group<MOE_FMT_Q6K>& r, const Planes& P, int H,
                                           size_t nc, int g) {
  const int sb = g >> 1, half = g & 1;  // half superblock
#pragma unroll
  for (int q = 0; q < 4; ++q) r.ql[q] = ld16(P.a + (((size_t)(4 * g + q)) * H + nc) * 16);
#pragma unroll
  for (int q = 0; q < 2; ++q) r.qh[q] = ld16(P.b + (((size_t)(2 * g + q)) * H + nc) * 16);
  r.sc = ld8(P.c + ((size_t)sb * H + nc) * 16 + 8 * half);
  r.d = ld2(P.d + ((size_t)sb * H + nc) * 2);
}

__device__ __forceinline__ void load_group(Group<MOE_FMT_Q8_0>& r, const Planes& P, int H,
                                           size_t nc, int g) {
#pragma unroll
  for (int q = 0; q < 8; ++q) r.c[q] = ld16(P.a + (((size_t)(8 * g + q)) * H + nc) * 16);
  r.s = ld8(P.b + ((size_t)g * H + nc) * 8);
}

__device__ __forceinline__ void load_group(Group<MOE_FMT_IQ3G>& r, const Planes& P, int H,
                                           size_t nc, int g) {
#pragma unroll
  for (int q = 0; q < 2; ++q) r.q[q] = ld16(P.a + (((size_t)(2 * g + q)) * H + nc) * 16);
  r.sg = ld16(P.b + ((size_t)g * H + nc) * 16);
  r.sc = ld8(P.c + ((size_t)(g >> 1) * H + nc) * 8);
}

__device__ __forceinline__ void load_group(Group<MOE_FMT_IQ1G>& r, const Planes& P, int H,
                                           size_t nc, int g) {
  r.q = ld16(P.a + ((size_t)g * H + nc) * 16);
  r.qh = ld4(P.b + ((size_t)g * H + nc) * 4);
  r.sc = ld8(P.c + ((size_t)(g >> 1) * H + nc) * 8);
}

// Exact bf16 pairs w[b][0..8) of the 8 blocks of 16 and their fp32 scales.
__device__ __forceinline__ void decode_group(const Group<MOE_FMT_NVFP4>& r, float ts,
                                             v2bf_t (*w)[8], float* sc) {
  e4m3x8(r.s, sc);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    sc[b] *= ts;
    e2m1x8_bf16(word_of(r.c[b >> 1], (b & 1) * 2), w[b]);
    e2m1x8_bf16(word_of(r.c[b >> 1], (b & 1) * 2 + 1), w[b] + 4);
  }
}

// The codes of 8 values (one 32-bit word of low nibbles, 16 high bits) in
// byte lanes: byte p of qe = value 2p, of qo = value 2p + 1.
__device__ __forceinline__ void q6_bytes(uint32_t lo, uint32_t h16, uint32_t& qe, uint32_t& qo) {
  uint32_t t = (h16 | (h16 << 8)) & 0x00ff00ffu;  // nibble p of h16 into byte p
  t = (t | (t << 4)) & 0x0f0f0f0fu;
  qe = (lo & 0x0f0f0f0fu) | ((t & 0x03030303u) << 4);
  qo = ((lo >> 4) & 0x0f0f0f0fu) | (((t >> 2) & 0x03030303u) << 4);
}

// Code byte p of a word -> q - 32 as an exact float: one byte permute puts
// the code in bits 16..21 under the exponent byte 0x43, which is the float
// 128 + q; subtracting 160 leaves q - 32.
template <int P>
__device__ __forceinline__ float q6_value(uint32_t q) {
  // result bytes: [0, 0, byte P of q, 0x43] (selector 0..3: q, 4..7: 0x43.., 0x0c: zero)
  const uint32_t bits = __builtin_amdgcn_perm(0x43434343u, q, 0x04000c0cu | ((uint32_t)P << 16));
  return __uint_as_float(bits) - 160.0f;
}

__device__ __forceinline__ void decode_group(const Group<MOE_FMT_Q6K>& r, float /*ts*/,
                                             v2bf_t (*w)[8], float* sc) {
  const float d = f16_to_f32((uint16_t)r.d);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    sc[j] = d * (float)(int8_t)((((j < 4) ? r.sc.x : r.sc.y) >> (8 * (j & 3))) & 0xffu);
    const uint32_t hi = word_of(r.qh[j >> 2], j & 3);  // 2 bits per element
#pragma unroll
    for (int hw = 0; hw < 2; ++hw) {  // elements 8hw .. 8hw + 8
      uint32_t qe, qo;
      q6_bytes(word_of(r.ql[j >> 1], (j & 1) * 2 + hw), (hi >> (16 * hw)) & 0xffffu, qe, qo);
      w[j][4 * hw + 0] = to_v2bf(q6_value<0>(qe), q6_value<0>(qo));
      w[j][4 * hw + 1] = to_v2bf(q6_value<1>(qe), q6_value<1>(qo));
      w[j][4 * hw + 2] = to_v2bf(q6_value<2>(qe), q6_value<2>(qo));
      w[j][4 * hw + 3] = to_v2bf(q6_value<3>(qe), q6_value<3>(qo));
    }
  }
}

// Half hf of a Q8_0 group: the 4 blocks of 16 codes 4hf..4hf+3 as exact bf16
// pairs (an int8 is exact in bf16) and their fp32 scales (block 2b covers
// blocks of 16 2b, 2b + 1).  A signed byte converts to float in one
// sub-dword conversion.
template <int HF>
__device__ __forceinline__ void decode_half_q8(const Group<MOE_FMT_Q8_0>& r, v2bf_t (*w)[8],
                                               float* sc) {
  const uint32_t dw = HF ? r.s.y : r.s.x;
  sc[0] = sc[1] = f16_to_f32((uint16_t)(dw & 0xffffu));
  sc[2] = sc[3] = f16_to_f32((uint16_t)(dw >> 16));
#pragma unroll
  for (int b = 0; b < 4; ++b) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t v = word_of(r.c[4 * HF + b], i >> 1);
      const int sh = 16 * (i & 1);
      w[b][i] = to_v2bf((float)(int8_t)(v >> sh), (float)(int8_t)(v >> (sh + 8)));
    }
  }
}

// The grid as bf16 pairs in LDS: entry e = {(m0, m1), (m2, m3)}, exact (odd
// integers up to 15 need 4 significant bits).
__device__ __forceinline__ void iq3g_table_bf16(uint2* tab, int tid, int nthreads) {
  for (int e = tid; e < 256; e += nthreads) {
    const uint32_t m = kIq3gGridDev.m[e];
    auto bf = [](uint32_t v) { return __float_as_uint((float)v) >> 16; };
    tab[e] = make_uint2(bf(m & 255u) | (bf((m >> 8) & 255u) << 16),
                        bf((m >> 16) & 255u) | (bf(m >> 24) << 16));
  }
}


// Exact bf16 pairs of a 128-element group (half h = g & 1 of its superblock)
// and the fp32 scales d * (2 s + 1) of its 8 blocks of 16.
__device__ __forceinline__ void decode_group_iq3g(const Group<MOE_FMT_IQ3G>& r, int h,
                                                  const uint2* tab, v2bf_t (*w)[8], float* sc) {
  const float d = f16_to_f32((uint16_t)(r.sc.x & 0xffffu));
  const uint32_t mul = (r.sc.x >> 16) | (r.sc.y << 16);  // nibble j: multiplier of sub-block j
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int j = 4 * h + (b >> 1);
    sc[b] = d * (float)(2u * ((mul >> (4 * j)) & 15u) + 1u);
    const uint32_t idx = word_of(r.q[b >> 2], b & 3);  // entries 4b .. 4b + 3
    const uint32_t sw = word_of(r.sg, b >> 1);         // sign bits of blocks 2(b/2), +1
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint2 v = tab[(idx >> (8 * i)) & 255u];
      const int p = 16 * (b & 1) + 4 * i;  // bit of the entry's first value
      w[b][2 * i] = as_v2bf(v.x ^ pair_sign_at(sw, p));
      w[b][2 * i + 1] = as_v2bf(v.y ^ pair_sign_at(sw, p + 2));
    }
  }
}

// The IQ1G grid as bf16 pairs in LDS: entry e = the pairs (v0, v1) .. (v6, v7)
// of values -1, 0, +1 (exact).
__device__ __forceinline__ void iq1g_table_bf16(uint4* tab, int tid, int nthreads) {
  for (int e = tid; e < 1024; e += nthreads) {
    const uint32_t c = kIq1gGridDev.c[e];
    auto pair = [c](int p) {  // values 2p, 2p + 1
      const uint32_t lo = ((c >> (4 * p)) & 1u) * 0x3f80u | ((c >> (4 * p + 1)) & 1u) << 15;
      const uint32_t hi = ((c >> (4 * p + 2)) & 1u) * 0x3f80u | ((c >> (4 * p + 3)) & 1u) << 15;
      return lo | (hi << 16);
    };
    tab[e] = make_uint4(pair(0), pair(1), pair(2), pair(3));
  }
}

// Exact bf16 pairs of a 128-element IQ1G group (half h = g & 1 of its
// superblock) and the fp32 scales d * (2 s + 1) of its 8 blocks of 16.
__device__ __forceinline__ void decode_group_iq1g(const Group<MOE_FMT_IQ1G>& r, int h,
                                                  const uint4* tab, v2bf_t (*w)[8], float* sc) {
  const float d = f16_to_f32((uint16_t)(r.sc.x & 0xffffu));
  const uint32_t mul = (r.sc.x >> 16) | (r.sc.y << 16);  // nibble j: multiplier of sub-block j
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int j = 4 * h + (b >> 1);
    sc[b] = d * (float)(2u * ((mul >> (4 * j)) & 15u) + 1u);
    const uint32_t lo = word_of(r.q, b >> 1);  // index low bytes of groups 4(b/2) .. +3
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // the block's groups of 8: 2b, 2b + 1
      const int gi = 2 * b + i;
      const uint32_t idx = ((lo >> (8 * (gi & 3))) & 255u) | (((r.qh >> (2 * gi)) & 3u) << 8);
      const uint4 v = tab[idx];
      w[b][4 * i] = as_v2bf(v.x);
      w[b][4 * i + 1] = as_v2bf(v.y);
      w[b][4 * i + 2] = as_v2bf(v.z);
      w[b][4 * i + 3] = as_v2bf(v.w);
    }
  }
}

// Issue the loads of the first D groups of a pass.
template <int FMT, int GP, int D>
__device__ __forceinline__ void dn_issue(Group<FMT> (&r)[GP], const Planes& P, int H, size_t nc,
                                         int gb) {
#pragma unroll
  for (int gi = 0; gi < GP && gi < D; ++gi) {
    load_group(r[gi], P, H, nc, gb + gi);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One pass of GP groups over the mt rows of h at sorted positions p0..
// (wave-uniform addresses, so scalar loads), the first D groups already in
// flight; the rest are issued D groups ahead of use.  The token loop is a
// plain loop (the register footprint does not grow with the batch); per-token
// sums accumulate in acc[t * 64 + lane].
template <int FMT, int GP, int D>
__device__ __forceinline__ void dn_consume(Group<FMT> (&r)[GP], const uint16_t* __restrict__ h,
                                           int p0, int H, int I, size_t nc, const Planes& P,
                                           float ts, int gb, int mt, float* acc,
                                           const uint2* tab, const uint4* tab1) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int gi = 0; gi < GP; ++gi) {
    if (gi + D < GP) {
      load_group(r[gi + D], P, H, nc, gb + gi + D);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int g = gb + gi;
    if constexpr (FMT == MOE_FMT_Q8_0) {
      // Half a group at a time (the decoded group would not fit beside the
      // next group's 136 bytes in flight).
      auto half = [&](auto HF_) {
        constexpr int HF = decltype(HF_)::value;
        v2bf_t w[4][8];
        float sc[4];
        decode_half_q8<HF>(r[gi], w, sc);
#pragma unroll 1
        for (int t = 0; t < mt; ++t) {
          const uint32_t* hp =
              reinterpret_cast<const uint32_t*>(h + (size_t)(p0 + t) * I) + 64 * g + 32 * HF;
          float a = 0.0f;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            float p = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
              p = __builtin_amdgcn_fdot2_f32_bf16(as_v2bf(hp[8 * b + i]), w[b][i], p, false);
            a = fmaf(p, sc[b], a);
          }
          acc[t * 64 + lane] += a;
        }
      };
      half(std::integral_constant<int, 0>{});
      half(std::integral_constant<int, 1>{});
      __builtin_amdgcn_sched_barrier(0);
    } else {
      v2bf_t w[8][8];
      float sc[8];
      if constexpr (FMT == MOE_FMT_IQ3G) decode_group_iq3g(r[gi], g & 1, tab, w, sc);
      else if constexpr (FMT == MOE_FMT_IQ1G) decode_group_iq1g(r[gi], g & 1, tab1, w, sc);
      else decode_group(r[gi], ts, w, sc);
#pragma unroll 1
      for (int t = 0; t < mt; ++t) {
        const uint32_t* hp = reinterpret_cast<const uint32_t*>(h + (size_t)(p0 + t) * I) + 64 * g;
        float a = 0.0f;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          float p = 0.0f;
#pragma unroll
          for (int i = 0; i < 8; ++i)
            p = __builtin_amdgcn_fdot2_f32_bf16(as_v2bf(hp[8 * b + i]), w[b][i], p, false);
          a = fmaf(p, sc[b], a);
        }
        acc[t * 64 + lane] += a;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <int FMT, int GP, int D, bool BF16>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void k_gemv_down(
    const uint16_t* __restrict__ h, int H, int I, int S, int gps_total, Planes P0,
    const moe_expert_ref* __restrict__ experts, const uint32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ active,
    const int32_t* __restrict__ n_active, void* __restrict__ y) {
  extern __shared__ __align__(16) float red[];  // [S][kDnMT][64]
  __shared__ uint2 tab[FMT == MOE_FMT_IQ3G ? 256 : 1];    // IQ3G grid as bf16 pairs
  __shared__ uint4 tab1[FMT == MOE_FMT_IQ1G ? 1024 : 1];  // IQ1G grid as bf16 pairs

  int e;
  moe_expert_ref ref;
  if (!slot_expert(active, n_active, experts, &e, &ref)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int nthreads = S * 64;
  const int n = blockIdx.x * 64 + lane;
  const size_t nc = (n < H) ? (size_t)n : 0;  // rows past the end read row 0, never stored
  const uintptr_t blob = (uintptr_t)ref.blob;
  const Planes P = {(const uint8_t*)(blob + (uintptr_t)P0.a), (const uint8_t*)(blob + (uintptr_t)P0.b),
                    (const uint8_t*)(blob + (uintptr_t)P0.c), (const uint8_t*)(blob + (uintptr_t)P0.d)};
  const float ts = (FMT == MOE_FMT_NVFP4) ? ref.ts_down : 1.0f;
  const int gb = wave * gps_total;
  float* acc = red + (size_t)wave * kDnMT * 64;

  // Batches of kDnMT tokens.  An active expert has at least one token, so the
  // first batch always runs; its first pass's weights are requested before
  // the token count and offset are read (see slot_expert).
  int cnt = 1, base = 0, mt = 0;
  for (int c0 = 0; c0 < cnt; c0 += kDnMT) {
    if (c0 > 0) __syncthreads();  // the previous batch's reads of red are done
    for (int sg = 0; sg < gps_total; sg += GP) {
      Group<FMT> r[GP];
      dn_issue<FMT, GP, D>(r, P, H, nc, gb + sg);
      __builtin_amdgcn_sched_barrier(0);
      if (sg == 0) {
        if (c0 == 0) {
          cnt = (int)counts[e];
          base = offsets[e];
        }
        mt = min(kDnMT, cnt - c0);
        for (int t = 0; t < mt; ++t) acc[t * 64 + lane] = 0.0f;  // this wave's slice only
        if constexpr (FMT == MOE_FMT_IQ3G) {
          if (c0 == 0) {  // the grid, while the first weights are in flight
            iq3g_table_bf16(tab, tid, nthreads);
            __syncthreads();
          }
        }
        if constexpr (FMT == MOE_FMT_IQ1G) {
          if (c0 == 0) {
            iq1g_table_bf16(tab1, tid, nthreads);
            __syncthreads();
          }
        }
      }
      {  // the pass's h values of the first 4 tokens (4 lines per group)
        uint32_t tch = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (t < mt)
            tch ^= touch_lines<4 * GP>(reinterpret_cast<const uint32_t*>(
                                           h + (size_t)(base + c0 + t) * I) +
                                       64 * (gb + sg));
        keep_scalar(tch);
      }
      dn_consume<FMT, GP, D>(r, h, base + c0, H, I, nc, P, ts, gb + sg, mt, acc, tab, tab1);
    }
    __syncthreads();
    for (int o = tid; o < mt * 64; o += nthreads) {
      const int t = o >> 6, rr = o & 63;
      const int n2 = blockIdx.x * 64 + rr;
      if (n2 < H) {
        float sum = 0.0f;
        for (int w = 0; w < S; ++w) sum += red[((size_t)w * kDnMT + t) * 64 + rr];
        store_y<BF16>(y, (size_t)(base + c0 + t) * H + n2, sum);
      }
    }
  }
}

template <int FMT, int GP>
hipError_t down_t(const moe_layer_desc* L, const uint16_t* h, const moe_buckets* b,
                  int max_slots, int S, int gps_total, void* y, int y_dtype, hipStream_t s) {
  constexpr int D = GP < 2 ? GP : 2;
  const BlobLayout lay = blob_layout(L->H, L->I, L->fmt_down);
  Planes P;
  if (FMT == MOE_FMT_NVFP4 || FMT == MOE_FMT_Q8_0) {
    P = {(const uint8_t*)lay.down_q, (const uint8_t*)lay.down_s, nullptr, nullptr};
  } else if (FMT == MOE_FMT_IQ3G || FMT == MOE_FMT_IQ1G) {
    P = {(const uint8_t*)lay.down_q, (const uint8_t*)lay.down_s, (const uint8_t*)lay.down_sc,
         nullptr};
  } else {
    P = {(const uint8_t*)lay.down_ql, (const uint8_t*)lay.down_qh, (const uint8_t*)lay.down_sc,
         (const uint8_t*)lay.down_d};
  }
  dim3 grid((unsigned)((L->H + 63) / 64), (unsigned)max_slots);
  const size_t lds = sizeof(float) * (size_t)S * kDnMT * 64;
  if (y_dtype == MOE_DTYPE_BF16)
    hipLaunchKernelGGL((k_gemv_down<FMT, GP, D, true>), grid, dim3(S * 64), lds, s, h, L->H, L->I,
                       S, gps_total, P, L->experts, b->counts, b->offsets, b->active,
                       b->n_active, y);
  else
    hipLaunchKernelGGL((k_gemv_down<FMT, GP, D, false>), grid, dim3(S * 64), lds, s, h, L->H,
                       L->I, S, gps_total, P, L->experts, b->counts, b->offsets, b->active,
                       b->n_active, y);
  return hipGetLastError();
}

template <int FMT>
hipError_t down_fmt(const moe_layer_desc* L, const uint16_t* h, const moe_buckets* b,
                    int max_slots, void* y, int y_dtype, hipStream_t s) {
  const int NG = L->I / 128;
  // One row block of 64 rows per workgroup; S waves split K (the largest
  // divisor of NG up to 8 that leaves each wave at least two groups; Q6_K,
  // whose decode is VALU-heavy, takes one group per wave up to NG = 4).
  int S = 1;
  for (int c = 2; c <= 8; ++c)
    if (NG % c == 0 && (NG / c >= 2 || (FMT == MOE_FMT_Q6K && NG <= 4))) S = c;
  const int gps_total = NG / S;
  const int gp_max = (FMT == MOE_FMT_NVFP4) ? 4 : 2;  // register budget (no spills)
  int GP = gps_total > gp_max ? gp_max : gps_total;
  while (gps_total % GP) --GP;
  if (GP == 1) return down_t<FMT, 1>(L, h, b, max_slots, S, gps_total, y, y_dtype, s);
  if constexpr (FMT != MOE_FMT_NVFP4) {
    return down_t<FMT, 2>(L, h, b, max_slots, S, gps_total, y, y_dtype, s);
  } else {
    switch (GP) {
      case 2: return down_t<FMT, 2>(L, h, b, max_slots, S, gps_total, y, y_dtype, s);
      case 3: return down_t<FMT, 3>(L, h, b, max_slots, S, gps_total, y, y_dtype, s);
      default: return down_t<FMT, 4>(L, h, b, max_slots, S, gps_total, y, y_dtype, s);
    }
  }
}

// Down projection and gate-weighted combine in one kernel, for decode
// batches: a workgroup owns 64 rows of one token's output and has one wave
// per expert slot j < NJ = min(k, 8) (slots j, j + 8, ... when k > 8).  A
// wave takes its experts' 64 rows of Wd over the whole of K (the same group
// decode and pass schedule as k_gemv_down, one token), multiplies each
// expert's sum by its gate weight in slot order, and the waves' sums are
// added in wave order, then the residual:
//   out[t][n] = bf16_rne( residual[t][n] + sum_w sum_{j = w mod NJ, j < k} w_tj y_tj[n] ).
// A fixed order, so the result does not depend on scheduling; y never goes
// to memory.  Workgroups of one row block sit 32 or more ids apart per
// token, on one XCD, so an expert that several tokens picked is read once
// into that XCD's L2.
template <int FMT, int GP, int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void k_gemv_down_combine(
    const uint16_t* __restrict__ h, int H, int I, int NG, Planes P0,
    const moe_expert_ref* __restrict__ experts, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ asg_pos, const float* __restrict__ topk_w, int k, int NJ,
    const uint16_t* __restrict__ residual, uint16_t* __restrict__ out) {
  __shared__ float acc_s[8][64];   // a wave's running dot products of the current expert
  __shared__ float part_s[8][64];  // the waves' gate-weighted sums
  __shared__ uint2 tab[FMT == MOE_FMT_IQ3G ? 256 : 1];
  __shared__ uint4 tab1[FMT == MOE_FMT_IQ1G ? 1024 : 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = blockIdx.y;
  const int n = blockIdx.x * 64 + lane;
  const size_t nc = (n < H) ? (size_t)n : 0;  // rows past the end read row 0, never stored
  if constexpr (FMT == MOE_FMT_IQ3G) iq3g_table_bf16(tab, tid, 64 * NJ);
  if constexpr (FMT == MOE_FMT_IQ1G) iq1g_table_bf16(tab1, tid, 64 * NJ);
  if constexpr (FMT == MOE_FMT_IQ3G || FMT == MOE_FMT_IQ1G) __syncthreads();
  float* acc = &acc_s[wave][0];
  float part = 0.0f;
  for (int j = wave; j < k; j += NJ) {
    const size_t a = (size_t)t * k + j;
    const int e = idx[a], p = asg_pos[a];
    const float wj = topk_w[a];
    const moe_expert_ref ref = experts[e];
    const uintptr_t blob = (uintptr_t)ref.blob;
    const Planes P = {(const uint8_t*)(blob + (uintptr_t)P0.a), (const uint8_t*)(blob + (uintptr_t)P0.b),
                      (const uint8_t*)(blob + (uintptr_t)P0.c), (const uint8_t*)(blob + (uintptr_t)P0.d)};
    const float ts = (FMT == MOE_FMT_NVFP4) ? ref.ts_down : 1.0f;
    acc[lane] = 0.0f;
    for (int sg = 0; sg < NG; sg += GP) {
      Group<FMT> r[GP];
      dn_issue<FMT, GP, D>(r, P, H, nc, sg);
      __builtin_amdgcn_sched_barrier(0);
      keep_scalar(touch_lines<4 * GP>(reinterpret_cast<const uint32_t*>(h + (size_t)p * I) +
                                      64 * sg));
      dn_consume<FMT, GP, D>(r, h, p, H, I, nc, P, ts, sg, 1, acc, tab, tab1);
    }
    part = fmaf(wj, acc[lane], part);
  }
  part_s[wave][lane] = part;
  __syncthreads();
  if (wave != 0 || n >= H) return;
  float sum = part_s[0][lane];
  for (int w = 1; w < NJ; ++w) sum += part_s[w][lane];
  if (residual) sum = bf16_to_f32(residual[(size_t)t * H + n]) + sum;
  out[(size_t)t * H + n] = f32_to_bf16_rne(sum);
}

template <int FMT, int GP>
hipError_t down_combine_t(const moe_layer_desc* L, const uint16_t* h, int64_t T,
                          const int32_t* idx, const int32_t* asg_pos, const float* topk_w,
                          const uint16_t* residual, uint16_t* out, hipStream_t s) {
  constexpr int D = GP < 2 ? GP : 2;
  const BlobLayout lay = blob_layout(L->H, L->I, L->fmt_down);
  Planes P;
  if (FMT == MOE_FMT_NVFP4 || FMT == MOE_FMT_Q8_0) {
    P = {(const uint8_t*)lay.down_q, (const uint8_t*)lay.down_s, nullptr, nullptr};
  } else if (FMT == MOE_FMT_IQ3G || FMT == MOE_FMT_IQ1G) {
    P = {(const uint8_t*)lay.down_q, (const uint8_t*)lay.down_s, (const uint8_t*)lay.down_sc,
         nullptr};
  } else {
    P = {(const uint8_t*)lay.down_ql, (const uint8_t*)lay.down_qh, (const uint8_t*)lay.down_sc,
         (const uint8_t*)lay.down_d};
  }
  const int NJ = L->k < 8 ? L->k : 8;
  dim3 grid((unsigned)((L->H + 63) / 64), (unsigned)T);
  hipLaunchKernelGGL((k_gemv_down_combine<FMT, GP, D>), grid, dim3(64 * NJ), 0, s, h, L->H, L->I,
                     L->I / 128, P, L->experts, idx, asg_pos, topk_w, L->k, NJ, residual, out);
  return hipGetLastError();
}

template <int FMT>
hipError_t down_combine_fmt(const moe_layer_desc* L, const uint16_t* h, int64_t T,
                            const int32_t* idx, const int32_t* asg_pos, const float* topk_w,
                            const uint16_t* residual, uint16_t* out, hipStream_t s) {
  // One wave runs all of K: passes of GP groups (the register budgets of
  // k_gemv_down), the largest that divides the group count.  (Splitting K
  // over two waves per expert, 16 waves per workgroup, measured no faster.)
  const int NG = L->I / 128;
  const int gp_max = (FMT == MOE_FMT_NVFP4) ? 4 : 2;
  int GP = NG > gp_max ? gp_max : NG;
  while (NG % GP) --GP;
#define DC(G) down_combine_t<FMT, G>(L, h, T, idx, asg_pos, topk_w, residual, out, s)
  if (GP == 1) return DC(1);
  if constexpr (FMT != MOE_FMT_NVFP4) {
    return DC(2);
  } else {
    switch (GP) {
      case 2: return DC(2);
      case 3: return DC(3);
      default: return DC(4);
    }
  }
#undef DC
}

}  // namespace

hipError_t launch_gemv_down(const moe_layer_desc* L, const uint16_t* h, const moe_buckets* b,
                            int max_slots, void* y, int y_dtype, hipStream_t s) {
  if (L->fmt_down == MOE_FMT_Q6K) return down_fmt<MOE_FMT_Q6K>(L, h, b, max_slots, y, y_dtype, s);
  if (L->fmt_down == MOE_FMT_Q8_0) return down_fmt<MOE_FMT_Q8_0>(L, h, b, max_slots, y, y_dtype, s);
  if (L->fmt_down == MOE_FMT_IQ3G) return down_fmt<MOE_FMT_IQ3G>(L, h, b, max_slots, y, y_dtype, s);
  if (L->fmt_down == MOE_FMT_IQ1G) return down_fmt<MOE_FMT_IQ1G>(L, h, b, max_slots, y, y_dtype, s);
  return down_fmt<MOE_FMT_NVFP4>(L, h, b, max_slots, y, y_dtype, s);
}

hipError_t launch_gemv_down_combine(const moe_layer_desc* L, const uint16_t* h, int64_t T,
                                   const int32_t* idx, const int32_t* asg_pos,
                                   const float* topk_w, const uint16_t* residual, uint16_t* out,
                                   hipStream_t s) {
  switch (L->fmt_down) {
    case MOE_FMT_Q6K: return down_combine_fmt<MOE_FMT_Q6K>(L, h, T, idx, asg_pos, topk_w, residual, out, s);
    case MOE_FMT_Q8_0: return down_combine_fmt<MOE_FMT_Q8_0>(L, h, T, idx, asg_pos, topk_w, residual, out, s);
    case MOE_FMT_IQ3G: return down_combine_fmt<MOE_FMT_IQ3G>(L, h, T, idx, asg_pos, topk_w, residual, out, s);
    case MOE_FMT_IQ1G: return down_combine_fmt<MOE_FMT_IQ1G>(L, h, T, idx, asg_pos, topk_w, residual, out, s);
    default: return down_combine_fmt<MOE_FMT_NVFP4>(L, h, T, idx, asg_pos, topk_w, residual, out, s);
  }
}

}  // namespace moe
