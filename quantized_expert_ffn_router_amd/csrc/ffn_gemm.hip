// ffn_gemm.hip -- expert FFNs for prefill-sized batches: grouped GEMM on
// MFMA with the block-quantized weights dequantized in registers.
//
// With thousands of tokens the routed experts (NVFP4; Q6_K in the DQ6_K
// packs: basalt.jgulfo.com, "Models" and "Quick start") are a real dense
// contraction per expert: the m_e tokens routed to expert e (rows of x in
// bucket order) times the expert's weights.  One launch per projection covers
// all experts:
//   - row blocks (expert, 128 rows) are listed on the device from the bucket
//     counts (no host round trip); each gets a record and tables of token row
//     offsets and row scales;
//   - persistent workgroups (two per CU) walk tiles (row block x column
//     tile); each XCD takes a contiguous range, so the column tiles of a row
//     block share that XCD's L2 for the re-read token rows;
//   - per K step of 128: the A tile (token rows, or h rows for the down
//     projection) is copied global -> LDS by the load unit; each wave loads
//     its B fragments from the packed weight blob (one 16-byte granule per
//     lane and column tile for NVFP4, see "B fragments"; more for Q6_K and
//     Q8_0 and IQ3G) and dequantizes them in registers;
//   - operands are fp16 (NVFP4 weights are exact in fp16; token rows carry
//     an exact per-row power-of-two scale, see k_rows_to_f16; Q6_K and Q8_0
//     weights are rounded once to fp16 after an exact per-expert power-of-two
//     scale, see k_down_exponent) except for the bf16 recompute path;
//   - 8 waves, each 128 rows x 32 columns = 8 x 2 v_mfma_f32_16x16x32 tiles
//     with fp32 accumulation;
//   - gate/up: each wave's two column tiles are the same 16 rows of gate and
//     of up, so SwiGLU runs in registers; h is stored in 16 bits.  Down:
//     y = acc * ts_d in bf16 or fp32.
#include <mutex>
#include <type_traits>

#include "gemv_common.h"

namespace moe {

namespace {

typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));
typedef _Float16 v8h_t __attribute__((ext_vector_type(8)));
typedef _Float16 v2h_t __attribute__((ext_vector_type(2)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

constexpr int BM = 128;       // token rows per tile
constexpr int kThreads = 512; // 8 waves

// Tile list: entry i = (expert, first row of the block); built from counts.
__global__ __launch_bounds__(1024) void k_build_tiles(const uint32_t* __restrict__ counts,
                                                      int E, int bm, int2* __restrict__ tiles,
                                                      int* __restrict__ n_tiles) {
  __shared__ int pre[1025];
  const int e = threadIdx.x;
  const int nt = (e < E) ? (int)((counts[e] + bm - 1) / bm) : 0;
  // inclusive scan over experts (E <= 1024) in LDS, simple Hillis-Steele
  pre[e] = nt;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int v = (e >= off) ? pre[e - off] : 0;
    __syncthreads();
    pre[e] += v;
    __syncthreads();
  }
  const int start = pre[e] - nt;
  for (int i = 0; i < nt; ++i) tiles[start + i] = make_int2(e, i * bm);
  if (e == 1023) {
    n_tiles[0] = pre[1023];
    n_tiles[1] = 0;  // fp16 h overflow flag of this call
  }
}

// fp16 copy of the token rows for the gate/up GEMM, one wave per row.  Each
// row is scaled by 2^-e, e chosen so that its largest magnitude lands in
// [2^14, 2^15): every value above 2^-29 of the row maximum converts exactly
// (bf16 carries 8 significant bits, fp16 11) and nothing can overflow.
// xscale[t] = 2^e scales the row's products back in the epilogue.  Rows that
// hold an inf or NaN keep e = 0 and carry it through as the bf16 path would.
__global__ __launch_bounds__(256) void k_rows_to_f16(const uint16_t* __restrict__ x, int64_t T,
                                                     int H, uint16_t* __restrict__ xh,
                                                     float* __restrict__ xscale) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + t * H);
  uint4* dst = reinterpret_cast<uint4*>(xh + t * H);
  const int nch = H / 8;
  uint32_t mx = 0;  // largest |x| as bf16 magnitude bits (ordered like the values)
  for (int c = lane; c < nch; c += 64) {
    const uint4 v = src[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = max(mx, max(w[i] & 0x7fffu, (w[i] >> 16) & 0x7fffu));
  }
#pragma unroll
  for (int o = 32; o; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
  const int eb = (int)(mx >> 7);  // biased exponent (bf16 and fp32 share it)
  int e = (mx == 0 || eb == 0xff) ? 0 : eb - 141;  // 2^(eb-127) * 2^-e in [2^14, 2^15)
  e = e < -126 ? -126 : (e > 126 ? 126 : e);
  const float down = __uint_as_float((uint32_t)(127 - e) << 23);
  if (lane == 0) xscale[t] = __uint_as_float((uint32_t)(127 + e) << 23);
  for (int c = lane; c < nch; c += 64) {
    const uint4 v = src[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const _Float16 lo = (_Float16)(__uint_as_float(w[i] << 16) * down);
      const _Float16 hi = (_Float16)(__uint_as_float(w[i] & 0xffff0000u) * down);
      o[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
             ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    dst[c] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// Row block (tile row) record: the expert and the block's rows in bucket order.
struct TileRec {
  moe_expert_ref ref;  // blob and per-tensor scales of the expert
  int srow;            // first row of the block in bucket (sorted) order
  int nrows;           // valid rows, 1..128
};
static_assert(sizeof(TileRec) == 32, "TileRec layout");

// Row tables of the row blocks, one workgroup of 128 threads per block:
// record, token row offset of each row (row r -> token * H; rows past the
// block's end repeat row 0, read but never stored) and that token's fp16 row
// scale.  For Q6_K and Q8_0 down weights the record's ref.reserved carries
// the expert's fp16-path exponent, read from the blob's meta section at
// off_meta (0: none).
__global__ __launch_bounds__(128) void k_tile_rows(
    const int2* __restrict__ tiles, const int* __restrict__ n_tiles,
    const uint32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const moe_expert_ref* __restrict__ experts, const int32_t* __restrict__ sorted_asg, int ktop,
    int H, const float* __restrict__ xscale, size_t off_meta, TileRec* __restrict__ recs,
    uint32_t* __restrict__ toff, float* __restrict__ rsc) {
  const int mt = blockIdx.x;
  if (mt >= *n_tiles) return;
  const int2 te = tiles[mt];
  const int e = te.x, m0 = te.y;
  const int nrows = min((int)counts[e] - m0, 128);
  const int srow = offsets[e] + m0;
  const int r = threadIdx.x;
  const int tok = sorted_asg[srow + (r < nrows ? r : 0)] / ktop;
  toff[(size_t)mt * 128 + r] = (uint32_t)tok * (uint32_t)H;
  rsc[(size_t)mt * 128 + r] = xscale[tok];
  if (r == 0) {
    TileRec t;
    t.ref = experts[e];
    t.ref.reserved =
        off_meta ? *reinterpret_cast<const uint32_t*>((const uint8_t*)t.ref.blob + off_meta) : 0u;
    t.srow = srow;
    t.nrows = nrows;
    recs[mt] = t;
  }
}

// ---------------------------------------------------------------- B fragments
// The K loop runs in steps of 128 = 4 MFMA sub-steps of 32.  Within a step
// the k index is permuted so that a lane's weights come from one 16-byte
// granule: lane l (column n0 + l%16, group q = l/16) supplies, in sub-step s,
// the 8 K-elements 32q + 8s .. +8 of the step -- word s of granule
// (step*4 + q, n).  The A operand uses the same permutation (it is read from
// LDS at k = 32q + 8s), so the product is unchanged and one 16-byte load per
// lane covers a column tile for the whole step.

#if defined(__HIP_DEVICE_COMPILE__)
typedef __attribute__((address_space(1))) uint4 g128_t;
typedef __attribute__((address_space(1))) uint2 g64_t;
typedef __attribute__((address_space(1))) uint16_t g16_t;
__device__ __forceinline__ uint4 gl16(const uint8_t* p) { return *(const g128_t*)(uintptr_t)p; }
__device__ __forceinline__ uint2 gl8(const uint8_t* p) { return *(const g64_t*)(uintptr_t)p; }
__device__ __forceinline__ uint32_t gl2(const uint8_t* p) { return *(const g16_t*)(uintptr_t)p; }
typedef __attribute__((address_space(1))) uint32_t g32_t;
__device__ __forceinline__ uint32_t gl4(const uint8_t* p) { return *(const g32_t*)(uintptr_t)p; }
#else
__device__ uint4 gl16(const uint8_t* p);
__device__ uint2 gl8(const uint8_t* p);
__device__ uint32_t gl2(const uint8_t* p);
__device__ uint32_t gl4(const uint8_t* p);
#endif

struct FragNvfp4 {
  uint4 code;      // 32 E2M1 codes: word s = sub-step s
  uint32_t scale;  // the two E4M3 block scales of the granule (low 16 bits)
};

__device__ __forceinline__ void load_frag(FragNvfp4& f, const uint8_t* q, const uint8_t* sc, int N,
                                          int n, int step) {
  const int grp = (threadIdx.x & 63) >> 4;
  f.code = gl16(q + ((size_t)(4 * step + grp) * N + n) * 16);
  f.scale = gl2(sc + ((size_t)step * N + n) * 8 + 2 * grp);
}

// Lane parts of the NVFP4 fragment addresses (column lane%16, group lane/16),
// computed once: per step only a wave-uniform part is added.
struct BLane {
  uint32_t q, s;
};
__device__ __forceinline__ BLane blane(int N) {
  const int lane = threadIdx.x & 63, grp = lane >> 4, n = lane & 15;
  return BLane{(uint32_t)(grp * N + n) * 16u, (uint32_t)(n * 8 + 2 * grp)};
}
// Fragments of column tile cb.. of two matrices (gate and up: the same rows).
__device__ __forceinline__ void load_frag_gu(FragNvfp4 (&f)[2], const uint8_t* q0,
                                             const uint8_t* s0, const uint8_t* q1,
                                             const uint8_t* s1, int N, int cb, int step,
                                             BLane bl) {
  const size_t uq = ((size_t)(4 * step) * N + cb) * 16, us = ((size_t)step * N + cb) * 8;
  f[0].code = gl16(q0 + uq + bl.q);
  f[1].code = gl16(q1 + uq + bl.q);
  f[0].scale = gl2(s0 + us + bl.s) | (gl2(s1 + us + bl.s) << 16);  // both tiles' scales
  f[1].scale = 0;
}
// Column tiles cb.. and cb + 16.. of one matrix: the second pair of addresses
// is the first plus a constant, folded into the load offsets.
__device__ __forceinline__ void load_frag_pair(FragNvfp4 (&f)[2], const uint8_t* q,
                                               const uint8_t* sc, int N, int cb, int step,
                                               BLane bl) {
  // The empty asm makes the lane offsets opaque, so the compiler rebuilds the
  // addresses here (2 adds) rather than keeping them live across the loop.
  uint32_t oq = bl.q, os = bl.s;
  __asm__ volatile("" : "+v"(oq), "+v"(os));
  const uint8_t* pq = q + ((size_t)(4 * step) * N + cb) * 16 + oq;
  const uint8_t* ps = sc + ((size_t)step * N + cb) * 8 + os;
  f[0].code = gl16(pq);
  f[1].code = gl16(pq + 16 * 16);
  f[0].scale = gl2(ps) | (gl2(ps + 16 * 8) << 16);  // both tiles' scales
  f[1].scale = 0;
}

// Sub-step s: 8 exact bf16 values (an E2M1 value has at most 2 significant
// bits and an E4M3 scale at most 4, so their product has at most 6).
template <int S>
__device__ __forceinline__ v8bf_t dequant_frag(const FragNvfp4& f) {
  const float s = e4m3x2<false>(f.scale)[S >> 1];  // block 0 for words 0, 1; block 1 for 2, 3
  const uint32_t w = S == 0 ? f.code.x : S == 1 ? f.code.y : S == 2 ? f.code.z : f.code.w;
  float v[8];
  e2m1x8_f32(w, v);
  v8bf_t r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const v2bf_t b = to_v2bf(v[2 * p] * s, v[2 * p + 1] * s);
    r[2 * p] = b[0];
    r[2 * p + 1] = b[1];
  }
  return r;
}

// The same 8 values as fp16 -- also exact (E2M1 x E4M3 lies in [2^-10, 2688]
// with at most 6 significant bits, e.g. 1.5 x 1.875): the codes convert to fp16
// pairs and one packed fp16 multiply applies the block scale, 2 VALU per pair
// instead of 4.
// The fp16 path keeps the scale bytes of both column tiles of a wave in one
// register (tile j in 16-bit half j), so J selects the half.
template <int S, int J>
__device__ __forceinline__ v8h_t dequant_frag_h(const FragNvfp4& f, uint32_t scale2) {
  const v2h_t s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scale2, 1.0f, J != 0);
  const _Float16 sc = s2[S >> 1];
  const v2h_t ss = {sc, sc};
  const uint32_t w = S == 0 ? f.code.x : S == 1 ? f.code.y : S == 2 ? f.code.z : f.code.w;
  const v2h_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
  const v2h_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
  const v2h_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
  const v2h_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
  return v8h_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

struct FragQ6k {
  uint4 lo;     // 32 low nibbles: word s = sub-step s
  uint2 hi;     // 32 x 2 high bits: 16 bits per sub-step
  uint32_t sc;  // the two int8 sub-scales of the granule (low 16 bits), fp16 d (high 16)
};

__device__ __forceinline__ void load_frag_q6k(FragQ6k& f, const uint8_t* ql, const uint8_t* qh,
                                              const uint8_t* sc, const uint8_t* dd, int N, int n,
                                              int step) {
  const int grp = (threadIdx.x & 63) >> 4;
  const int c = 4 * step + grp, sb = c >> 3;
  f.lo = gl16(ql + ((size_t)c * N + n) * 16);
  f.hi = gl8(qh + ((size_t)(c >> 1) * N + n) * 16 + 8 * (c & 1));
  f.sc = gl2(sc + ((size_t)sb * N + n) * 16 + 2 * (c & 7)) | (gl2(dd + ((size_t)sb * N + n) * 2) << 16);
}

template <int S>
__device__ __forceinline__ v8bf_t dequant_frag_q6k(const FragQ6k& f) {
  const float s = f16_to_f32((uint16_t)(f.sc >> 16)) * (float)(int8_t)((f.sc >> (8 * (S >> 1))) & 0xffu);
  const uint32_t lo = S == 0 ? f.lo.x : S == 1 ? f.lo.y : S == 2 ? f.lo.z : f.lo.w;
  const uint32_t h16 = ((S < 2 ? f.hi.x : f.hi.y) >> (16 * (S & 1))) & 0xffffu;
  v8bf_t r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t byte = (lo >> (8 * p)) & 0xffu;
    const int q0 = (int)((byte & 15u) | (((h16 >> (4 * p)) & 3u) << 4));
    const int q1 = (int)((byte >> 4) | (((h16 >> (4 * p + 2)) & 3u) << 4));
    const v2bf_t b = to_v2bf((float)(q0 - 32) * s, (float)(q1 - 32) * s);
    r[2 * p] = b[0];
    r[2 * p + 1] = b[1];
  }
  return r;
}

// The same 8 weights times 2^sx as fp16 for the fp16 path (sx: the expert's
// exponent, k_down_exponent).  The six-bit codes are built in byte lanes (even
// values of the sub-step in qe, odd in qo), then each pair is placed by one
// byte permute as two fp16 subnormals q * 2^-24; one packed fma gives
// (q - 32) * 2^-10 exactly and one packed multiply applies d * sc * 2^(10+sx)
// (below 2^15 for every block of the expert; rounded once to fp16, then the
// product once: about 2^-11 relative, finer than the bf16 path's 2^-9).
// Needs fp16 denormals, the default mode.
template <int S>
__device__ __forceinline__ v8h_t dequant_frag_q6k_h(const FragQ6k& f, int sx) {
  const float s32 = __builtin_amdgcn_ldexpf(
      f16_to_f32((uint16_t)(f.sc >> 16)) * (float)(int8_t)((f.sc >> (8 * (S >> 1))) & 0xffu),
      10 + sx);
  const _Float16 sh = (_Float16)s32;
  const v2h_t ss = {sh, sh};
  const uint32_t lo = S == 0 ? f.lo.x : S == 1 ? f.lo.y : S == 2 ? f.lo.z : f.lo.w;
  const uint32_t h16 = ((S < 2 ? f.hi.x : f.hi.y) >> (16 * (S & 1))) & 0xffffu;
  // nibble p of h16 (high bits of values 2p, 2p+1) into byte p
  uint32_t t = (h16 | (h16 << 8)) & 0x00ff00ffu;
  t = (t | (t << 4)) & 0x0f0f0f0fu;
  const uint32_t qe = (lo & 0x0f0f0f0fu) | ((t & 0x03030303u) << 4);
  const uint32_t qo = ((lo >> 4) & 0x0f0f0f0fu) | (((t >> 2) & 0x03030303u) << 4);
  const v2h_t k14 = {(_Float16)16384.0f, (_Float16)16384.0f};
  const v2h_t m32 = {(_Float16)-0.03125f, (_Float16)-0.03125f};
  v8h_t r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    // bytes [qe.p, 0, qo.p, 0]: selector 0..3 picks qe (second operand), 4..7 qo
    const uint32_t sel = 0x0c000c00u | (uint32_t)p | ((uint32_t)(4 + p) << 16);
    const uint32_t raw = __builtin_amdgcn_perm(qo, qe, sel);
    const v2h_t q = __builtin_bit_cast(v2h_t, raw);
    const v2h_t v = __builtin_elementwise_fma(q, k14, m32) * ss;
    r[2 * p] = v[0];
    r[2 * p + 1] = v[1];
  }
  return r;
}

// Q8_0: a lane group's 32 values of a K step are exactly one block of 32
// (block 4 * step + lane/16), so one fp16 scale per fragment.
struct FragQ8 {
  uint4 lo, hi;  // the block's 32 int8 codes: sub-steps 0, 1 in lo, 2, 3 in hi
  uint32_t sc;   // fp16 scale d (low 16 bits)
};

__device__ __forceinline__ void load_frag_q8(FragQ8& f, const uint8_t* q, const uint8_t* sc, int N,
                                             int n, int step) {
  const int grp = (threadIdx.x & 63) >> 4;
  const int c = 4 * step + grp;  // block of 32
  f.lo = gl16(q + ((size_t)(2 * c) * N + n) * 16);
  f.hi = gl16(q + ((size_t)(2 * c + 1) * N + n) * 16);
  f.sc = gl2(sc + ((size_t)step * N + n) * 8 + 2 * grp);
}

// Both column tiles n and n + 16 of the fp16 path; their scales share
// f[0].sc (tile j in the 16-bit half j), one register fewer per step.
__device__ __forceinline__ void load_frag_q8_pair(FragQ8 (&f)[2], const uint8_t* q,
                                                  const uint8_t* sc, int N, int n, int step) {
  const int grp = (threadIdx.x & 63) >> 4;
  const int c = 4 * step + grp;
  const uint8_t* p0 = q + ((size_t)(2 * c) * N + n) * 16;
  const uint8_t* p1 = q + ((size_t)(2 * c + 1) * N + n) * 16;
  f[0].lo = gl16(p0);
  f[0].hi = gl16(p1);
  f[1].lo = gl16(p0 + 16 * 16);
  f[1].hi = gl16(p1 + 16 * 16);
  const uint8_t* ps = sc + ((size_t)step * N + n) * 8 + 2 * grp;
  f[0].sc = gl2(ps) | (gl2(ps + 16 * 8) << 16);
  f[1].sc = 0;
}

template <int S>
__device__ __forceinline__ void q8_words(const FragQ8& f, uint32_t& w0, uint32_t& w1) {
  const uint4& v = S < 2 ? f.lo : f.hi;
  w0 = (S & 1) ? v.z : v.x;
  w1 = (S & 1) ? v.w : v.y;
}

template <int S>
__device__ __forceinline__ v8bf_t dequant_frag_q8(const FragQ8& f) {
  const float d = f16_to_f32((uint16_t)(f.sc & 0xffffu));
  uint32_t w[2];
  q8_words<S>(f, w[0], w[1]);
  v8bf_t r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t v = w[p >> 1] >> (16 * (p & 1));
    const v2bf_t b = to_v2bf((float)(int8_t)v * d, (float)(int8_t)(v >> 8) * d);
    r[2 * p] = b[0];
    r[2 * p + 1] = b[1];
  }
  return r;
}

// fp16 path: the codes, offset to unsigned bytes u = q + 128, are placed by
// one byte permute under the fp16 exponent of 1024 (0x64: 1024 + u exactly),
// one packed add leaves q and one packed multiply applies d * 2^sx (sx: the
// expert's exponent, k_down_exponent; an exact ldexp of the fp16 d, below
// 2^8 for every block of the expert), rounding the product once.  So the
// weights times 2^sx stay below 2^15 whatever the scales; the epilogue takes
// the 2^sx out in fp32.
template <int S, int J>
__device__ __forceinline__ v8h_t dequant_frag_q8_h(const FragQ8& f, uint32_t sc2, int sx) {
  const _Float16 dh =
      __builtin_amdgcn_ldexph(__builtin_bit_cast(_Float16, (uint16_t)(sc2 >> (16 * J))), sx);
  const v2h_t ds = {dh, dh};
  const v2h_t off = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  uint32_t w[2];
  q8_words<S>(f, w[0], w[1]);
  v8h_t r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t u = w[p >> 1] ^ 0x80808080u;
    const uint32_t b0 = 2 * (p & 1);
    // bytes [u.b0, 0x64, u.b0+1, 0x64] (selector 0..3: u, 4: 0x64)
    const uint32_t raw = __builtin_amdgcn_perm(0x64646464u, u, 0x04000400u | b0 | ((b0 + 1) << 16));
    const v2h_t v = (__builtin_bit_cast(v2h_t, raw) + off) * ds;
    r[2 * p] = v[0];
    r[2 * p + 1] = v[1];
  }
  return r;
}

// IQ3G (iq3g.h): a lane group's 32 values of a K step are exactly one
// sub-block (one odd multiplier 2 s + 1): 8 grid indices, 32 sign bits, and
// the superblock's d with its multipliers.
struct FragIq3g {
  uint2 idx;  // grid indices of elements 32q .. 32q + 31 of the step (q = lane / 16)
  uint32_t sg;  // their sign bits
  uint2 sc;   // d fp16 (low 16 bits of x), then the superblock's 8 nibble multipliers
};

__device__ __forceinline__ void load_frag_iq3g(FragIq3g& f, const uint8_t* qi, const uint8_t* qs,
                                               const uint8_t* qc, int N, int n, int step) {
  const int grp = (threadIdx.x & 63) >> 4;
  f.idx = gl8(qi + ((size_t)(2 * step + (grp >> 1)) * N + n) * 16 + 8 * (grp & 1));
  f.sg = gl4(qs + ((size_t)step * N + n) * 16 + 4 * grp);
  f.sc = gl8(qc + ((size_t)(step >> 1) * N + n) * 8);
}

// Both column tiles cb.. and cb + 16.. (cb wave-uniform): the lane parts of
// the three addresses are 32-bit offsets made opaque at each use (the
// compiler then rebuilds them with one add instead of keeping 64-bit
// addresses live across the K loop); tile 1 is tile 0 plus a constant.
__device__ __forceinline__ void load_frag_iq3g_pair(FragIq3g (&f)[2], const uint8_t* qi,
                                                    const uint8_t* qs, const uint8_t* qc, int N,
                                                    int cb, int step) {
  const int lane = threadIdx.x & 63, grp = lane >> 4, n = lane & 15;
  uint32_t oi = (uint32_t)(((grp >> 1) * N + n) * 16 + 8 * (grp & 1));
  uint32_t os = (uint32_t)(n * 16 + 4 * grp), oc = (uint32_t)(n * 8);
  __asm__ volatile("" : "+v"(oi), "+v"(os), "+v"(oc));
  const uint8_t* pi = qi + ((size_t)(2 * step) * N + cb) * 16 + oi;
  const uint8_t* ps = qs + ((size_t)step * N + cb) * 16 + os;
  const uint8_t* pc = qc + ((size_t)(step >> 1) * N + cb) * 8 + oc;
  f[0].idx = gl8(pi);
  f[1].idx = gl8(pi + 16 * 16);
  f[0].sg = gl4(ps);
  f[1].sg = gl4(ps + 16 * 16);
  f[0].sc = gl8(pc);
  f[1].sc = gl8(pc + 16 * 8);
}

// Odd multiplier 2 s + 1 of the lane group's sub-block (4 * (step % 2) + q).
__device__ __forceinline__ uint32_t iq3g_mult(const FragIq3g& f, int step) {
  const int j = 4 * (step & 1) + ((threadIdx.x & 63) >> 4);
  const uint32_t mul = (f.sc.x >> 16) | (f.sc.y << 16);
  return 2u * ((mul >> (4 * j)) & 15u) + 1u;
}

// Sub-step S of the fp16 path: entries 2S, 2S + 1 of the lane's 8 as fp16
// pairs from the LDS grid (tab: {(m0, m1), (m2, m3)} per entry), signs
// applied, times 2 s + 1 (exact: at most 9 * 31 = 279) and then d * 2^sx (an
// exact ldexp of the fp16 d; below 2^6 for every superblock of the expert,
// see k_down_exponent), rounding each weight once.
// The step's two fp16 factors of a column tile in one register: 2 s + 1 (low
// half) and d * 2^sx (high half), formed once per step so that the
// fragment's scale bytes are dead before the sub-steps.
__device__ __forceinline__ uint32_t iq3g_factors(const FragIq3g& f, int step, int sx) {
  const _Float16 m = (_Float16)(float)iq3g_mult(f, step);
  const _Float16 dh = __builtin_amdgcn_ldexph(__builtin_bit_cast(_Float16, (uint16_t)(f.sc.x & 0xffffu)), sx);
  return (uint32_t)__builtin_bit_cast(uint16_t, m) | ((uint32_t)__builtin_bit_cast(uint16_t, dh) << 16);
}

template <int S>
__device__ __forceinline__ v8h_t dequant_frag_iq3g_h(const FragIq3g& f, const uint2* tab,
                                                     uint32_t fac) {
  const v2h_t f2 = __builtin_bit_cast(v2h_t, fac);
  const v2h_t ms = {f2[0], f2[0]}, ds = {f2[1], f2[1]};
  const uint32_t iw = (S < 2) ? f.idx.x : f.idx.y;
  v8h_t r;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const uint2 v = tab[(iw >> (16 * (S & 1) + 8 * e)) & 255u];
    const int p = 8 * S + 4 * e;  // sign bit of the entry's first value
    const v2h_t lo = __builtin_bit_cast(v2h_t, v.x ^ pair_sign_at(f.sg, p)) * ms * ds;
    const v2h_t hi = __builtin_bit_cast(v2h_t, v.y ^ pair_sign_at(f.sg, p + 2)) * ms * ds;
    r[4 * e] = lo[0];
    r[4 * e + 1] = lo[1];
    r[4 * e + 2] = hi[0];
    r[4 * e + 3] = hi[1];
  }
  return r;
}

// bf16 path (the fp16-h overflow fallback): w = +-m * (2 s + 1) * d in fp32,
// rounded once to bf16.
template <int S>
__device__ __forceinline__ v8bf_t dequant_frag_iq3g(const FragIq3g& f, const uint2* tab,
                                                    float mult) {
  const float sc = f16_to_f32((uint16_t)(f.sc.x & 0xffffu)) * mult;
  const uint32_t iw = (S < 2) ? f.idx.x : f.idx.y;
  const uint32_t sb = f.sg >> (8 * S);
  float v[8];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const uint2 t = tab[(iw >> (16 * (S & 1) + 8 * e)) & 255u];
    const uint32_t w4[2] = {t.x, t.y};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const _Float16 m = __builtin_bit_cast(_Float16, (uint16_t)(w4[c >> 1] >> (16 * (c & 1))));
      const float x = (float)m * sc;
      v[4 * e + c] = ((sb >> (4 * e + c)) & 1u) ? -x : x;
    }
  }
  v8bf_t r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const v2bf_t b = to_v2bf(v[2 * p], v[2 * p + 1]);
    r[2 * p] = b[0];
    r[2 * p + 1] = b[1];
  }
  return r;
}

// The grid as fp16 pairs in LDS (exact: odd integers up to 15).
__device__ __forceinline__ void iq3g_table_f16(uint2* tab, int tid) {
  if (tid < 256) {
    const uint32_t m = kIq3gGridDev.m[tid];
    auto h = [](uint32_t v) {
      return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(float)v);
    };
    tab[tid] = make_uint2(h(m & 255u) | (h((m >> 8) & 255u) << 16),
                          h((m >> 16) & 255u) | (h(m >> 24) << 16));
  }
}

// IQ1G (iq1g.h): a lane group's 32 values of a K step are one sub-block (one
// odd multiplier 2 s + 1) made of 4 groups of 8, one grid entry each: 4 index
// low bytes, their 2-bit high parts (one byte of the step's 4-byte record) and
// the superblock's d with its multipliers.
struct FragIq1g {
  uint32_t lo;  // index low bytes of groups 4q .. 4q + 3 of the step (q = lane / 16)
  uint32_t hi;  // the step's 16 two-bit high parts (group g at bits 2g, 2g + 1)
  uint2 sc;     // d fp16 (low 16 bits of x), then the superblock's 8 nibble multipliers
};

__device__ __forceinline__ void load_frag_iq1g(FragIq1g& f, const uint8_t* qi, const uint8_t* qh,
                                               const uint8_t* qc, int N, int n, int step) {
  const int grp = (threadIdx.x & 63) >> 4;
  f.lo = gl4(qi + ((size_t)step * N + n) * 16 + 4 * grp);
  f.hi = gl4(qh + ((size_t)step * N + n) * 4);
  f.sc = gl8(qc + ((size_t)(step >> 1) * N + n) * 8);
}

// Both column tiles cb.. and cb + 16.. (cb wave-uniform), lane offsets made
// opaque as in load_frag_iq3g_pair.
__device__ __forceinline__ void load_frag_iq1g_pair(FragIq1g (&f)[2], const uint8_t* qi,
                                                    const uint8_t* qh, const uint8_t* qc, int N,
                                                    int cb, int step) {
  const int lane = threadIdx.x & 63, grp = lane >> 4, n = lane & 15;
  uint32_t oi = (uint32_t)(n * 16 + 4 * grp), oh = (uint32_t)(n * 4), oc = (uint32_t)(n * 8);
  __asm__ volatile("" : "+v"(oi), "+v"(oh), "+v"(oc));
  const uint8_t* pi = qi + ((size_t)step * N + cb) * 16 + oi;
  const uint8_t* ph = qh + ((size_t)step * N + cb) * 4 + oh;
  const uint8_t* pc = qc + ((size_t)(step >> 1) * N + cb) * 8 + oc;
  f[0].lo = gl4(pi);
  f[1].lo = gl4(pi + 16 * 16);
  f[0].hi = gl4(ph);
  f[1].hi = gl4(ph + 16 * 4);
  f[0].sc = gl8(pc);
  f[1].sc = gl8(pc + 16 * 8);
}

// Odd multiplier 2 s + 1 of the lane group's sub-block (4 * (step % 2) + q).
__device__ __forceinline__ uint32_t iq1g_mult(const FragIq1g& f, int step) {
  const int j = 4 * (step & 1) + ((threadIdx.x & 63) >> 4);
  const uint32_t mul = (f.sc.x >> 16) | (f.sc.y << 16);
  return 2u * ((mul >> (4 * j)) & 15u) + 1u;
}

// The step's two fp16 factors of a column tile (2 s + 1, d * 2^sx), as for
// IQ3G.
__device__ __forceinline__ uint32_t iq1g_factors(const FragIq1g& f, int step, int sx) {
  const _Float16 m = (_Float16)(float)iq1g_mult(f, step);
  const _Float16 dh = __builtin_amdgcn_ldexph(__builtin_bit_cast(_Float16, (uint16_t)(f.sc.x & 0xffffu)), sx);
  return (uint32_t)__builtin_bit_cast(uint16_t, m) | ((uint32_t)__builtin_bit_cast(uint16_t, dh) << 16);
}

// Grid entry of sub-step S's group (4q + S of the step).
template <int S>
__device__ __forceinline__ uint32_t iq1g_entry(const FragIq1g& f) {
  const int q = (threadIdx.x & 63) >> 4;
  return ((f.lo >> (8 * S)) & 255u) | (((f.hi >> (8 * q + 2 * S)) & 3u) << 8);
}

// Sub-step S of the fp16 path: the group's 8 values -1, 0, +1 as fp16 pairs
// (LDS entry: byte i = the high byte of value i's fp16; one byte permute per
// pair), times 2 s + 1 and then d * 2^sx (exact up to the last product,
// rounded once; |2 s + 1| <= 31 and d * 2^sx < 2^9, see k_down_exponent).
template <int S>
__device__ __forceinline__ v8h_t dequant_frag_iq1g_h(const FragIq1g& f, const uint2* tab,
                                                     uint32_t fac) {
  const v2h_t f2 = __builtin_bit_cast(v2h_t, fac);
  const v2h_t ms = {f2[0], f2[0]}, ds = {f2[1], f2[1]};
  const uint2 t = tab[iq1g_entry<S>(f)];
  v8h_t r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t src = p < 2 ? t.x : t.y, b0 = 2 * (p & 1);
    // result bytes [0, src.b0, 0, src.b0+1] (selector 0x0c: zero)
    const uint32_t raw = __builtin_amdgcn_perm(0u, src, 0x000c000cu | (b0 << 8) | ((b0 + 1) << 24));
    const v2h_t v = __builtin_bit_cast(v2h_t, raw) * ms * ds;
    r[2 * p] = v[0];
    r[2 * p + 1] = v[1];
  }
  return r;
}

// bf16 path (the fp16-h overflow fallback): w = v * (2 s + 1) * d in fp32,
// rounded once to bf16.
template <int S>
__device__ __forceinline__ v8bf_t dequant_frag_iq1g(const FragIq1g& f, const uint2* tab,
                                                    float mult) {
  const float sc = f16_to_f32((uint16_t)(f.sc.x & 0xffffu)) * mult;
  const uint2 t = tab[iq1g_entry<S>(f)];
  v8bf_t r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t w = p < 2 ? t.x : t.y;
    float v[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint32_t hb = (w >> (8 * (2 * (p & 1) + c))) & 255u;  // 0x00, 0x3c or 0xbc
      v[c] = hb == 0u ? 0.0f : ((hb & 0x80u) ? -sc : sc);
    }
    const v2bf_t b = to_v2bf(v[0], v[1]);
    r[2 * p] = b[0];
    r[2 * p + 1] = b[1];
  }
  return r;
}

// The IQ1G grid in LDS, 8 bytes per entry: byte i = the high byte of value
// i's fp16 (0x00, 0x3c = +1, 0xbc = -1; the low bytes are zero).
__device__ __forceinline__ void iq1g_table_f16(uint2* tab, int tid, int nthreads) {
  for (int e = tid; e < 1024; e += nthreads) {
    const uint32_t c = kIq1gGridDev.c[e];
    auto byte = [c](int i) {
      return ((c >> (2 * i)) & 1u) ? (((c >> (2 * i + 1)) & 1u) ? 0xbcu : 0x3cu) : 0u;
    };
    tab[e] = make_uint2(byte(0) | (byte(1) << 8) | (byte(2) << 16) | (byte(3) << 24),
                        byte(4) | (byte(5) << 8) | (byte(6) << 16) | (byte(7) << 24));
  }
}

// ---------------------------------------------------------------- main loop
// Persistent workgroups of 8 waves.  A tile is 128 token rows x 8*NC*16
// columns; wave w owns all 128 rows and column tiles j < NC (NC = 2: 64
// accumulators per lane, 4 waves per SIMD).  K runs in steps of 128.
//   - A (token rows, 16-bit) lives in LDS as 256-byte rows whose 16-byte
//     chunks are XOR-swizzled (chunk c of row r at c ^ (r & 15)), so the
//     fragment reads (16 rows, one chunk) hit distinct banks.  The load unit
//     copies it global -> LDS itself (global_load_lds_dwordx4: lane i of a
//     wave writes LDS slot i); two buffers, loads one step ahead.
//   - B fragments go global -> registers one step ahead and are dequantized
//     right before their MFMAs.
//   - The operands enter the MFMA as (B, A), so the accumulator holds the
//     transposed tile: lane l has row l%16 and the 4 consecutive columns
//     4*(l/16) .. +4 of each 16 x 16 block, stored with one 8- or 16-byte
//     store.
//   - Each workgroup walks a list of tiles.  The step stream does not stop
//     at tile boundaries: the last step of a tile already loads step 0 of the
//     next one, whose row table (token row offsets, row scales) was copied
//     into LDS during the tile's first step, so no tile waits on a chain of
//     dependent metadata loads, and the epilogue overlaps the next loads.
constexpr int GBM = 128, GBK = 128;
constexpr int ARB = GBK;  // 16-bit values per LDS row (no padding: swizzled)

__device__ __forceinline__ int aswz(int r, int c) { return r * ARB + 8 * (c ^ (r & 15)); }

// s_waitcnt vmcnt(n) (gfx9 encoding; expcnt and lgkmcnt not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Weight planes of one column tile: NVFP4 (codes, scales) or Q6_K (ql, qh,
// sc, d) of one matrix.
struct Planes {
  const uint8_t* p[4];
};

template <int FMT>
using FragOf = typename std::conditional<
    FMT == MOE_FMT_NVFP4, FragNvfp4,
    typename std::conditional<
        FMT == MOE_FMT_Q8_0, FragQ8,
        typename std::conditional<
            FMT == MOE_FMT_IQ3G, FragIq3g,
            typename std::conditional<FMT == MOE_FMT_IQ1G, FragIq1g, FragQ6k>::type>::type>::type>::type;

template <int FMT>
__device__ __forceinline__ void load_b_tile(FragOf<FMT>& f, const Planes& P, int N, int n,
                                            int step) {
  if constexpr (FMT == MOE_FMT_NVFP4) load_frag(f, P.p[0], P.p[1], N, n, step);
  else if constexpr (FMT == MOE_FMT_Q8_0) load_frag_q8(f, P.p[0], P.p[1], N, n, step);
  else if constexpr (FMT == MOE_FMT_IQ3G) load_frag_iq3g(f, P.p[0], P.p[1], P.p[2], N, n, step);
  else if constexpr (FMT == MOE_FMT_IQ1G) load_frag_iq1g(f, P.p[0], P.p[1], P.p[2], N, n, step);
  else load_frag_q6k(f, P.p[0], P.p[1], P.p[2], P.p[3], N, n, step);
}

// Rows 16w + 4k + lane/16 (k < 4) of the A tile: slot lane%16 of row r holds
// chunk (lane%16) ^ (r & 15).  off[k]: element offset of that row's values.
__device__ __forceinline__ void load_a_tile(const uint16_t* base, const uint32_t (&off)[4], int k0,
                                            uint16_t* Abuf, int wave, int lane) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = 16 * wave + 4 * k + (lane >> 4);
    const int c = (lane & 15) ^ (r & 15);
    __builtin_amdgcn_global_load_lds(
        (const void*)(base + off[k] + k0 + 8 * c),
        (void __attribute__((address_space(3)))*)(Abuf + (16 * wave + 4 * k) * ARB), 16, 0, 0);
  }
}

// Half h (0, 1) of load_a_tile: rows k = 2h, 2h + 1.
__device__ __forceinline__ void load_a_half(const uint16_t* base, const uint32_t (&off)[4], int k0,
                                            uint16_t* Abuf, int wave, int lane, int h) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int k = 2 * h + kk;
    const int r = 16 * wave + 4 * k + (lane >> 4);
    const int c = (lane & 15) ^ (r & 15);
    __builtin_amdgcn_global_load_lds(
        (const void*)(base + off[k] + k0 + 8 * c),
        (void __attribute__((address_space(3)))*)(Abuf + (16 * wave + 4 * k) * ARB), 16, 0, 0);
  }
}

// The 4 sub-steps of one K step on A buffer Ab: acc[i][j] += tile i of A x
// column tile j of B, computed transposed (see above).  issue(S) runs before
// the MFMAs of sub-step S: the next step's loads are spread over the step, so
// no wave stalls on a full memory queue right after the barrier.
template <int FMT, int NC, bool F16, typename Issue>
__device__ __forceinline__ void step_mfma(const FragOf<FMT> (&bcur)[NC], const uint16_t* Ab,
                                          int lane, v4f_t (*acc)[NC], int sx, Issue issue,
                                          const uint2* tab = nullptr, int st = 0) {
  const int r = lane & 15, cq = 4 * (lane >> 4);
  // IQ3G: each column tile's factors for this step (fp16 path: 2 s + 1 and
  // d * 2^sx in one register; bf16 path: the multiplier)
  uint32_t imul[NC] = {};
  if constexpr (FMT == MOE_FMT_IQ3G) {
#pragma unroll
    for (int j = 0; j < NC; ++j)
      imul[j] = F16 ? iq3g_factors(bcur[j], st, sx) : iq3g_mult(bcur[j], st);
  } else if constexpr (FMT == MOE_FMT_IQ1G) {
#pragma unroll
    for (int j = 0; j < NC; ++j)
      imul[j] = F16 ? iq1g_factors(bcur[j], st, sx) : iq1g_mult(bcur[j], st);
  }
  auto sub = [&](auto S_) {
    constexpr int S = decltype(S_)::value;
    if constexpr (F16) {
      v8h_t bf[NC];
      static_assert(NC == 2, "fp16 path: two column tiles");
      if constexpr (FMT == MOE_FMT_NVFP4) {  // scales of both tiles paired in bcur[0]
        bf[0] = dequant_frag_h<S, 0>(bcur[0], bcur[0].scale);
        bf[1] = dequant_frag_h<S, 1>(bcur[1], bcur[0].scale);
      } else if constexpr (FMT == MOE_FMT_Q8_0) {
        bf[0] = dequant_frag_q8_h<S, 0>(bcur[0], bcur[0].sc, sx);
        bf[1] = dequant_frag_q8_h<S, 1>(bcur[1], bcur[0].sc, sx);
      } else if constexpr (FMT == MOE_FMT_IQ3G) {
        bf[0] = dequant_frag_iq3g_h<S>(bcur[0], tab, imul[0]);
        bf[1] = dequant_frag_iq3g_h<S>(bcur[1], tab, imul[1]);
      } else if constexpr (FMT == MOE_FMT_IQ1G) {
        bf[0] = dequant_frag_iq1g_h<S>(bcur[0], tab, imul[0]);
        bf[1] = dequant_frag_iq1g_h<S>(bcur[1], tab, imul[1]);
      } else {
        bf[0] = dequant_frag_q6k_h<S>(bcur[0], sx);
        bf[1] = dequant_frag_q6k_h<S>(bcur[1], sx);
      }
      __builtin_amdgcn_sched_barrier(0);
      issue(S_);
      __builtin_amdgcn_sched_barrier(0);
      // A fragments are read one row tile ahead of their MFMAs; the fences
      // keep the compiler from serializing read -> wait -> MFMA under the
      // 128-register budget of 4 waves per SIMD.
      // (Q8_0 and Q6_K fragments take 9 and 7 registers per column tile: no
      // A read-ahead, which would push more of the K loop into spills.)
      constexpr bool kPre = FMT == MOE_FMT_NVFP4;  // (also none for IQ3G)
      v8h_t an = *reinterpret_cast<const v8h_t*>(Ab + aswz(r, cq + S));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const v8h_t af = kPre ? an : *reinterpret_cast<const v8h_t*>(Ab + aswz(16 * i + r, cq + S));
        if (kPre && i + 1 < 8) an = *reinterpret_cast<const v8h_t*>(Ab + aswz(16 * (i + 1) + r, cq + S));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NC; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf[j], af, acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      issue(S_);
      __builtin_amdgcn_sched_barrier(0);
      v8bf_t bf[NC];
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        if constexpr (FMT == MOE_FMT_NVFP4) bf[j] = dequant_frag<S>(bcur[j]);
        else if constexpr (FMT == MOE_FMT_Q8_0) bf[j] = dequant_frag_q8<S>(bcur[j]);
        else if constexpr (FMT == MOE_FMT_IQ3G) bf[j] = dequant_frag_iq3g<S>(bcur[j], tab, (float)imul[j]);
        else if constexpr (FMT == MOE_FMT_IQ1G) bf[j] = dequant_frag_iq1g<S>(bcur[j], tab, (float)imul[j]);
        else bf[j] = dequant_frag_q6k<S>(bcur[j]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const v8bf_t af = *reinterpret_cast<const v8bf_t*>(Ab + aswz(16 * i + r, cq + S));
#pragma unroll
        for (int j = 0; j < NC; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[j], af, acc[i][j], 0, 0, 0);
      }
    }
  };
  sub(std::integral_constant<int, 0>{});
  sub(std::integral_constant<int, 1>{});
  sub(std::integral_constant<int, 2>{});
  sub(std::integral_constant<int, 3>{});
}

// fp16 h of a token is stored as h * 2^hexp, hexp = -21 - 2e where 2^e is the
// token's x row scale (2^-e * max|x| in [2^14, 2^15)): h grows like |x|^2, so
// the stored values sit near 2^8 * h / max|x|^2 whatever the activations'
// magnitude, far from both ends of the fp16 range.  Exact powers of two.
__device__ __forceinline__ int h_exp(float xscale) {
  const int e = (int)((__float_as_uint(xscale) >> 23) & 0xffu) - 127;
  const int k = -21 - 2 * e;
  return k < -126 ? -126 : (k > 126 ? 126 : k);
}
__device__ __forceinline__ float pow2f(int k) { return __uint_as_float((uint32_t)(k + 127) << 23); }

// Two values rounded to bf16 (hardware round-to-nearest-even) in one word.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, to_v2bf(a, b));
}
// Two values rounded to fp16 (round-to-nearest-even), clamped to +-65504.
__device__ __forceinline__ uint32_t pack_f16x2_sat(float a, float b) {
  const v2f_t f = {__builtin_amdgcn_fmed3f(a, -65504.0f, 65504.0f),
                   __builtin_amdgcn_fmed3f(b, -65504.0f, 65504.0f)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, v2h_t));
}

// Lane groups g = lane / 16 hold 4 consecutive outputs of a row each (the
// transposed accumulator).  With rows of two 16-lane groups swapped between
// two registers (a of the odd group <-> b of the even group below it), lane
// group g ends up with 8 consecutive outputs in (a, b): the even group keeps
// its a and gets the odd group's a, the odd group gets the even group's b and
// keeps its b.  One 16-byte store then replaces two 8-byte ones, so a store
// instruction covers 64-byte instead of 32-byte pieces of each row.
__device__ __forceinline__ void swap_row_pairs(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

// Tiles of this workgroup.  Workgroup w runs on XCD w % 8 (all workgroups of
// the grid are resident, dispatched round robin); each XCD takes a contiguous
// 1/8 of the logical tiles, in which consecutive tiles are the column tiles of
// one row block, so those share the XCD's L2 for the row block's A rows.
struct TileRange {
  int first, end, stride;
};
__device__ __forceinline__ TileRange tile_range(int n_logical) {
  const int x = blockIdx.x & 7, j = blockIdx.x >> 3, per8 = (n_logical + 7) >> 3;
  TileRange t;
  t.first = x * per8 + j;
  t.end = min((x + 1) * per8, n_logical);
  t.stride = (int)(gridDim.x >> 3);
  return t;
}

// ------------------------------------------------------------------ gate/up
// Tile columns: 128 consecutive rows n0.. of gate and the same rows of up;
// wave w takes gate rows n0 + 16w .. +16 (tile j = 0) and the same up rows
// (tile j = 1), so each lane holds matching g and u values.
//
// h goes out as fp16 (every down format's GEMM runs on fp16 operands), scaled
// per token (h_exp).  fp16 keeps 3 more mantissa bits than bf16 but tops out
// at 65504: a value beyond that is saturated and raises the call's overflow
// flag, and then the FALLBACK instance (launched right after, idle unless the
// flag is set) recomputes all of h as bf16 for a bf16 down GEMM, so the range
// is bf16's.

template <bool HF16, bool FALLBACK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_gemm_gateup_nvfp4(
    const uint16_t* __restrict__ xh, int H, int I, size_t off_gq, size_t off_gs, size_t off_uq,
    size_t off_us, const TileRec* __restrict__ recs, const uint32_t* __restrict__ toff,
    const float* __restrict__ rsc, const int* __restrict__ n_tiles, int* ovf,
    uint16_t* __restrict__ hout) {
  if (FALLBACK && *ovf == 0) return;
  __shared__ __align__(16) uint16_t As[2 * GBM * ARB];
  __shared__ uint32_t st_off[3][GBM];  // row tables of up to 3 tiles in flight
  __shared__ float st_rs[3][GBM];
  const int NT = I / 128;
  const TileRange tr = tile_range(*n_tiles * NT);
  if (tr.first >= tr.end) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nsteps = H / GBK;

  // Copy the row table of row block mt into LDS slot s (waves 0-3, async).
  auto stage_rows = [&](int mt, int s) {
    if (wave < 4) {
      const int half = wave & 1;
      const void* src = (wave < 2) ? (const void*)(toff + (size_t)mt * GBM + 64 * half + lane)
                                   : (const void*)(rsc + (size_t)mt * GBM + 64 * half + lane);
      void* dst = (wave < 2) ? (void*)&st_off[s][64 * half] : (void*)&st_rs[s][64 * half];
      __builtin_amdgcn_global_load_lds(src, (void __attribute__((address_space(3)))*)dst, 4, 0, 0);
    }
  };
  auto read_rows = [&](int s, uint32_t (&off)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) off[k] = st_off[s][16 * wave + 4 * k + (lane >> 4)];
  };
  auto planes_of = [&](const uint8_t* blob, Planes (&P)[2]) {
    P[0].p[0] = blob + off_gq; P[0].p[1] = blob + off_gs;
    P[1].p[0] = blob + off_uq; P[1].p[1] = blob + off_us;
  };

  // First tile: row table and step 0 loaded up front.
  int L = tr.first, slot = 0, buf = 0;
  const int mt = L / NT;
  int cb = (L - mt * NT) * 128 + 16 * wave;
  TileRec cur = recs[mt];
  Planes P[2];
  planes_of((const uint8_t*)cur.ref.blob, P);
  stage_rows(mt, 0);
  wait_vmcnt<0>();
  __syncthreads();
  uint32_t off[4];
  read_rows(0, off);
  FragNvfp4 bnext[2];
  const BLane bl = blane(I);
  load_a_tile(xh, off, 0, As, wave, lane);
  __builtin_amdgcn_sched_barrier(0);
  load_frag_gu(bnext, P[0].p[0], P[0].p[1], P[1].p[0], P[1].p[1], I, cb, 0, bl);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<4>();  // step 0's rows are in LDS (its weight loads may still fly)
  __syncthreads();

  int cbl = cb;  // column base of the weight loads (switches to the next tile early)
  for (;;) {
    const int Ln = L + tr.stride;
    const bool has_next = Ln < tr.end;
    const int mtn = Ln / NT, cbn = (Ln - mtn * NT) * 128 + 16 * wave;
    const int slotn = slot == 2 ? 0 : slot + 1;
    TileRec nxt = cur;
    if (has_next) {  // the next tile's record and row table, read in its last step
      nxt = recs[mtn];
      stage_rows(mtn, slotn);
      if (nsteps == 1) {
        wait_vmcnt<0>();
        __syncthreads();
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    v4f_t acc[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i][0] = acc[i][1] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int st = 0; st < nsteps; ++st) {
      FragNvfp4 bcur[2] = {bnext[0], bnext[1]};
      const bool more = st + 1 < nsteps;
      if (!more && has_next) {
        read_rows(slotn, off);
        planes_of((const uint8_t*)nxt.ref.blob, P);
        cbl = cbn;
      }
      const bool ld = more || has_next;
      const int stn = more ? st + 1 : 0;
      uint16_t* Anext = As + (buf ^ 1) * GBM * ARB;
      // Next step: weights first (they come from farther away), rows after.
      step_mfma<MOE_FMT_NVFP4, 2, true>(bcur, As + buf * GBM * ARB, lane, acc, 0, [&](auto S_) {
        constexpr int S = decltype(S_)::value;
        if (!ld) return;
        if constexpr (S == 0) {
          load_frag_gu(bnext, P[0].p[0], P[0].p[1], P[1].p[0], P[1].p[1], I, cbl, stn, bl);
        } else if constexpr (S == 1) {
          load_a_half(xh, off, stn * GBK, Anext, wave, lane, 0);
        } else if constexpr (S == 2) {
          load_a_half(xh, off, stn * GBK, Anext, wave, lane, 1);
        }
      });
      __builtin_amdgcn_sched_barrier(0);
      if (ld) wait_vmcnt<0>();  // the next step's rows are in LDS
      __syncthreads();
      buf ^= 1;
    }

    // SwiGLU epilogue: lane holds row 16i + lane%16, columns cb + 4*(lane/16) .. +4.
    // Row sets 2p and 2p+1 are computed for every lane (rows past nrows are
    // never stored), then swapped so that lane group g stores columns
    // cb + 8*(g/2) .. +8 of row set 2p + g%2.
    const float tg = cur.ref.ts_gate, tu = cur.ref.ts_up;
    const int grp = lane >> 4;
    bool big = false;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t hv[2][2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int i = 2 * p + s2;
        const int r = 16 * i + (lane & 15);
        const float rs = st_rs[slot][r];
        const float hs = HF16 ? pow2f(h_exp(rs)) : 1.0f;
#pragma unroll
        for (int q = 0; q < 4; q += 2) {
          float h2[2];
#pragma unroll
          for (int d = 0; d < 2; ++d) {
            const float g = acc[i][0][q + d] * (tg * rs), u = acc[i][1][q + d] * (tu * rs);
            h2[d] = swiglu(g, u) * hs;
          }
          if constexpr (HF16) {
            big |= (r < cur.nrows) && fmaxf(fabsf(h2[0]), fabsf(h2[1])) > 65504.0f;
            hv[s2][q >> 1] = pack_f16x2_sat(h2[0], h2[1]);
          } else {
            hv[s2][q >> 1] = pack_bf16x2(h2[0], h2[1]);
          }
        }
      }
      swap_row_pairs(hv[0][0], hv[1][0]);
      swap_row_pairs(hv[0][1], hv[1][1]);
      const int r = 16 * (2 * p + (grp & 1)) + (lane & 15);
      if (r < cur.nrows)
        *reinterpret_cast<uint4*>(hout + (size_t)(cur.srow + r) * I + cb + 8 * (grp >> 1)) =
            make_uint4(hv[0][0], hv[0][1], hv[1][0], hv[1][1]);
    }
    if (HF16 && big) *ovf = 1;
    if (!has_next) break;
    L = Ln; cb = cbn; slot = slotn; cur = nxt;
  }
}

// ------------------------------------------------------------------ down
// Tile columns: 256 consecutive rows of the down weights (output features);
// wave w takes columns n0 + 32w .. +32 (tiles j = 0, 1).  The A rows are the
// tile's rows of h, contiguous in bucket order.

// AF16: h is fp16 (NVFP4 weights only).  RUN: 0 always; 1 only when the
// call's fp16 h overflow flag is clear; 2 only when it is set.
template <int FMT, bool OUT_BF16, bool AF16, int RUN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_gemm_down(
    const uint16_t* __restrict__ h, int H, int I, size_t off_a, size_t off_b, size_t off_c,
    size_t off_d, const TileRec* __restrict__ recs, const float* __restrict__ rsc,
    const int* __restrict__ n_tiles, const int* ovf, void* __restrict__ y) {
  if (RUN == 1 && *ovf != 0) return;
  if (RUN == 2 && *ovf == 0) return;
  __shared__ __align__(16) uint16_t As[2 * GBM * ARB];
  __shared__ float st_rs[AF16 ? 3 : 1][GBM];  // x row scales of up to 3 tiles (fp16 h)
  // IQ3G grid (16-bit pairs) or IQ1G grid (fp16 high bytes)
  __shared__ uint2 gtab[FMT == MOE_FMT_IQ3G ? 256 : (FMT == MOE_FMT_IQ1G ? 1024 : 1)];
  const int NT = H / 256;
  const TileRange tr = tile_range(*n_tiles * NT);
  if (tr.first >= tr.end) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nsteps = I / GBK;
  constexpr int kB = (FMT == MOE_FMT_NVFP4) ? 2 : (FMT == MOE_FMT_Q6K ? 4 : 3);  // weight loads per column tile

  auto rows_of = [&](const TileRec& t, uint32_t (&off)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {  // rows past nrows read a valid row, never stored
      const int r = 16 * wave + 4 * k + (lane >> 4);
      off[k] = (uint32_t)(t.srow + (r < t.nrows ? r : 0)) * (uint32_t)I;
    }
  };
  auto planes_of = [&](const uint8_t* blob, Planes& P) {
    P.p[0] = blob + off_a; P.p[1] = blob + off_b; P.p[2] = blob + off_c; P.p[3] = blob + off_d;
  };
  // Row scales of row block mt into LDS slot s (waves 0-1, async), fp16 h only.
  auto stage_rs = [&](int mt, int s) {
    if (AF16 && wave < 2)
      __builtin_amdgcn_global_load_lds(
          (const void*)(rsc + (size_t)mt * GBM + 64 * wave + lane),
          (void __attribute__((address_space(3)))*)&st_rs[s][64 * wave], 4, 0, 0);
  };

  int L = tr.first, buf = 0, slot = 0;
  const int mt = L / NT;
  int cb = (L - mt * NT) * 256 + 32 * wave;
  TileRec cur = recs[mt];
  Planes P;
  planes_of((const uint8_t*)cur.ref.blob, P);
  uint32_t off[4];
  rows_of(cur, off);
  stage_rs(mt, 0);
  FragOf<FMT> bnext[2];
  const BLane bl = blane(H);
  load_a_tile(h, off, 0, As, wave, lane);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (AF16 && FMT == MOE_FMT_NVFP4) {
    load_frag_pair(bnext, P.p[0], P.p[1], H, cb, 0, bl);
  } else if constexpr (FMT == MOE_FMT_IQ3G) {
    load_frag_iq3g_pair(bnext, P.p[0], P.p[1], P.p[2], H, cb, 0);
  } else if constexpr (FMT == MOE_FMT_IQ1G) {
    load_frag_iq1g_pair(bnext, P.p[0], P.p[1], P.p[2], H, cb, 0);
  } else if constexpr (AF16 && FMT == MOE_FMT_Q8_0) {
    load_frag_q8_pair(bnext, P.p[0], P.p[1], H, cb + (lane & 15), 0);
  } else {
    load_b_tile<FMT>(bnext[0], P, H, cb + (lane & 15), 0);
    load_b_tile<FMT>(bnext[1], P, H, cb + 16 + (lane & 15), 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (FMT == MOE_FMT_IQ3G) iq3g_table_f16(gtab, tid);  // visible after the barrier below
  if constexpr (FMT == MOE_FMT_IQ1G) iq1g_table_f16(gtab, tid, kThreads);
  wait_vmcnt<2 * kB>();
  __syncthreads();

  int cbl = cb;  // column base of the weight loads (switches to the next tile early)
  for (;;) {
    const int Ln = L + tr.stride;
    const bool has_next = Ln < tr.end;
    const int mtn = Ln / NT, cbn = (Ln - mtn * NT) * 256 + 32 * wave;
    const int slotn = slot == 2 ? 0 : slot + 1;
    TileRec nxt = cur;
    if (has_next) {
      nxt = recs[mtn];
      stage_rs(mtn, slotn);  // read in the tile's epilogue, after its steps' barriers
    }
    const int sx = (int)cur.ref.reserved;  // fp16-path exponent of Q6_K / Q8_0 weights
    v4f_t acc[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i][0] = acc[i][1] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int st = 0; st < nsteps; ++st) {
      FragOf<FMT> bcur[2] = {bnext[0], bnext[1]};
      const bool more = st + 1 < nsteps;
      if (!more && has_next) {
        rows_of(nxt, off);
        planes_of((const uint8_t*)nxt.ref.blob, P);
        cbl = cbn;
      }
      const bool ld = more || has_next;
      const int stn = more ? st + 1 : 0;
      uint16_t* Anext = As + (buf ^ 1) * GBM * ARB;
      step_mfma<FMT, 2, AF16>(bcur, As + buf * GBM * ARB, lane, acc, sx, [&](auto S_) {
        constexpr int S = decltype(S_)::value;
        if (!ld) return;
        if constexpr (AF16 && FMT == MOE_FMT_Q8_0) {
          // weights after sub-step 1's dequant, when this step's first 16
          // codes are dead: 8 registers fewer live (the compiler's spills in
          // the K loop drop from 15 scratch operations to 3)
          if constexpr (S == 0) load_a_half(h, off, stn * GBK, Anext, wave, lane, 0);
          else if constexpr (S == 1)
            load_frag_q8_pair(bnext, P.p[0], P.p[1], H, cbl + (lane & 15), stn);
          else if constexpr (S == 2) load_a_half(h, off, stn * GBK, Anext, wave, lane, 1);
        } else if constexpr (AF16 && FMT == MOE_FMT_IQ1G) {
          // token rows first, the weights (4 registers per tile) after
          // sub-step 1 (issued at sub-step 3 as for IQ3G, the compiler
          // spilled 75 registers; here 8, as in the NVFP4 kernel)
          if constexpr (S == 0) {
            load_a_half(h, off, stn * GBK, Anext, wave, lane, 0);
            load_a_half(h, off, stn * GBK, Anext, wave, lane, 1);
          } else if constexpr (S == 1) {
            load_frag_iq1g_pair(bnext, P.p[0], P.p[1], P.p[2], H, cbl, stn);
          }
        } else if constexpr (AF16 && FMT == MOE_FMT_IQ3G) {
          // token rows first; the weights after sub-step 3's dequant, when
          // this step's fragments are dead and the next step's can take their
          // registers (issued at sub-step 1 or 2 they made the compiler spill
          // 60 registers, with scratch traffic in every step)
          if constexpr (S == 0) {
            load_a_half(h, off, stn * GBK, Anext, wave, lane, 0);
            load_a_half(h, off, stn * GBK, Anext, wave, lane, 1);
          } else if constexpr (S == 3) {
            load_frag_iq3g_pair(bnext, P.p[0], P.p[1], P.p[2], H, cbl, stn);
          }
        } else if constexpr (AF16 && FMT == MOE_FMT_Q6K) {  // the same schedule
          if constexpr (S == 0) load_a_half(h, off, stn * GBK, Anext, wave, lane, 0);
          else if constexpr (S == 1) {
            load_b_tile<FMT>(bnext[0], P, H, cbl + (lane & 15), stn);
            load_b_tile<FMT>(bnext[1], P, H, cbl + 16 + (lane & 15), stn);
          } else if constexpr (S == 2) load_a_half(h, off, stn * GBK, Anext, wave, lane, 1);
        } else if constexpr (AF16) {  // spread over the step (see gate/up)
          if constexpr (S == 0) {
            if constexpr (FMT == MOE_FMT_NVFP4) {
              load_frag_pair(bnext, P.p[0], P.p[1], H, cbl, stn, bl);
            } else {
              load_b_tile<FMT>(bnext[0], P, H, cbl + (lane & 15), stn);
              load_b_tile<FMT>(bnext[1], P, H, cbl + 16 + (lane & 15), stn);
            }
          } else if constexpr (S == 1) {
            load_a_half(h, off, stn * GBK, Anext, wave, lane, 0);
          } else if constexpr (S == 2) {
            load_a_half(h, off, stn * GBK, Anext, wave, lane, 1);
          }
        } else if constexpr (S == 0) {  // all at once: fewer live registers
          load_b_tile<FMT>(bnext[0], P, H, cbl + (lane & 15), stn);
          load_b_tile<FMT>(bnext[1], P, H, cbl + 16 + (lane & 15), stn);
          load_a_tile(h, off, stn * GBK, Anext, wave, lane);
        }
      }, gtab, st);
      __builtin_amdgcn_sched_barrier(0);
      if (ld) wait_vmcnt<0>();
      __syncthreads();
      buf ^= 1;
    }

    // Epilogue: lane holds row 16i + lane%16, columns cb + 16j + 4*(lane/16) .. +4.
    // bf16: the two column tiles are swapped between lane groups so that
    // group g stores columns cb + 8*(g/2) + 16*(g%2) .. +8 of its row.
    const float ts = (FMT == MOE_FMT_NVFP4) ? cur.ref.ts_down : (AF16 ? pow2f(-sx) : 1.0f);
    const int grp = lane >> 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 16 * i + (lane & 15);
      const float tr_s = AF16 ? ts * pow2f(-h_exp(st_rs[slot][r])) : ts;
      const v4f_t v0 = acc[i][0] * tr_s, v1 = acc[i][1] * tr_s;
      if constexpr (OUT_BF16) {
        uint32_t a0 = pack_bf16x2(v0[0], v0[1]), a1 = pack_bf16x2(v0[2], v0[3]);
        uint32_t b0 = pack_bf16x2(v1[0], v1[1]), b1 = pack_bf16x2(v1[2], v1[3]);
        swap_row_pairs(a0, b0);
        swap_row_pairs(a1, b1);
        if (r < cur.nrows)
          *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(y) + (size_t)(cur.srow + r) * H + cb +
                                    8 * (grp >> 1) + 16 * (grp & 1)) = make_uint4(a0, a1, b0, b1);
      } else if (r < cur.nrows) {
        float* yo = reinterpret_cast<float*>(y) + (size_t)(cur.srow + r) * H + cb + 4 * grp;
        *reinterpret_cast<float4*>(yo) = make_float4(v0[0], v0[1], v0[2], v0[3]);
        *reinterpret_cast<float4*>(yo + 16) = make_float4(v1[0], v1[1], v1[2], v1[3]);
      }
    }
    if (!has_next) break;
    L = Ln; cb = cbn; cur = nxt; slot = slotn;
  }
}

// Workgroups of a persistent launch: 2 per CU of the device (rounded up to
// a multiple of 8 XCDs), looked up once per device.
constexpr int kMaxDevices = 64;
std::once_flag g_slots_once[kMaxDevices];
int g_gemm_slots[kMaxDevices];
hipError_t g_slots_err[kMaxDevices];

}  // namespace

size_t gemm_tiles_bytes(int E, int64_t A) {
  const size_t mt = (size_t)(A / BM + E + 1);
  return align_up(mt * sizeof(int2)) + align_up(2 * sizeof(int)) + align_up(mt * sizeof(TileRec)) +
         2 * align_up(mt * GBM * sizeof(uint32_t));
}

// Grouped-GEMM expert FFN.  hbuf: h [A][I] (fp16 or bf16, see gate/up); xh: fp16 [T][H]; xscale: [T];
// tiles_ws: gemm_tiles_bytes().
hipError_t launch_gemm_ffn(const moe_layer_desc* L, const uint16_t* x, int64_t T,
                           const moe_buckets* b, uint16_t* hbuf, uint16_t* xh, float* xscale,
                           void* tiles_ws, void* y, int y_dtype, hipStream_t s) {
  const BlobLayout lay = blob_layout(L->H, L->I, L->fmt_down);
  const int64_t A = T * L->k;
  const size_t mtmax = (size_t)(A / BM + L->E + 1);
  char* w = (char*)tiles_ws;
  int2* tiles = (int2*)w;
  w += align_up(mtmax * sizeof(int2));
  int* n_tiles = (int*)w;  // [0]: row blocks, [1]: fp16 h overflow flag
  int* ovf = n_tiles + 1;
  w += align_up(2 * sizeof(int));
  TileRec* recs = (TileRec*)w;
  w += align_up(mtmax * sizeof(TileRec));
  uint32_t* toff = (uint32_t*)w;
  w += align_up(mtmax * GBM * sizeof(uint32_t));
  float* rsc = (float*)w;
  int dev = 0;
  hipError_t derr = hipGetDevice(&dev);
  if (derr != hipSuccess) return derr;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_slots_once[dev], [dev] {
    int cus = 0;
    g_slots_err[dev] = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    g_gemm_slots[dev] = (2 * cus + 7) / 8 * 8;
  });
  if (g_slots_err[dev] != hipSuccess) return g_slots_err[dev];
  const int slots = g_gemm_slots[dev];
  const int max_mtiles = (int)(A / BM) + L->E;
  hipLaunchKernelGGL(k_build_tiles, dim3(1), dim3(1024), 0, s, b->counts, L->E, BM, tiles, n_tiles);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_rows_to_f16, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, x, T, L->H, xh,
                     xscale);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(k_tile_rows, dim3((unsigned)max_mtiles), dim3(GBM), 0, s, tiles, n_tiles,
                     b->counts, b->offsets, L->experts, b->sorted_asg, L->k, L->H, xscale,
                     lay.down_meta, recs, toff, rsc);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const dim3 grid((unsigned)slots), block(kThreads);
  const bool bf = (y_dtype == MOE_DTYPE_BF16);
#define GU_ARGS                                                                                   \
  xh, L->H, L->I, lay.gate_q, lay.gate_s, lay.up_q, lay.up_s, recs, toff, rsc, n_tiles, ovf, hbuf
#define DOWN(F, B, A16, R, P0, P1, P2, P3)                                                        \
  hipLaunchKernelGGL((k_gemm_down<F, B, A16, R>), grid, block, 0, s, hbuf, L->H, L->I, P0, P1, P2, \
                     P3, recs, rsc, n_tiles, ovf, y)
  if (L->fmt_down == MOE_FMT_NVFP4) {
    // fp16 h; on overflow the bf16 instances redo the layer's FFN (see above)
    hipLaunchKernelGGL((k_gemm_gateup_nvfp4<true, false>), grid, block, 0, s, GU_ARGS);
    hipLaunchKernelGGL((k_gemm_gateup_nvfp4<false, true>), grid, block, 0, s, GU_ARGS);
    const size_t q = lay.down_q, sc = lay.down_s, z = 0;
    if (bf) {
      DOWN(MOE_FMT_NVFP4, true, true, 1, q, sc, z, z);
      DOWN(MOE_FMT_NVFP4, true, false, 2, q, sc, z, z);
    } else {
      DOWN(MOE_FMT_NVFP4, false, true, 1, q, sc, z, z);
      DOWN(MOE_FMT_NVFP4, false, false, 2, q, sc, z, z);
    }
  } else if (L->fmt_down == MOE_FMT_Q8_0) {
    hipLaunchKernelGGL((k_gemm_gateup_nvfp4<true, false>), grid, block, 0, s, GU_ARGS);
    hipLaunchKernelGGL((k_gemm_gateup_nvfp4<false, true>), grid, block, 0, s, GU_ARGS);
    const size_t q = lay.down_q, sc = lay.down_s, z = 0;
    if (bf) {
      DOWN(MOE_FMT_Q8_0, true, true, 1, q, sc, z, z);
      DOWN(MOE_FMT_Q8_0, true, false, 2, q, sc, z, z);
    } else {
      DOWN(MOE_FMT_Q8_0, false, true, 1, q, sc, z, z);
      DOWN(MOE_FMT_Q8_0, false, false, 2, q, sc, z, z);
    }
  } else if (L->fmt_down == MOE_FMT_IQ3G) {
    hipLaunchKernelGGL((k_gemm_gateup_nvfp4<true, false>), grid, block, 0, s, GU_ARGS);
    hipLaunchKernelGGL((k_gemm_gateup_nvfp4<false, true>), grid, block, 0, s, GU_ARGS);
    const size_t qi = lay.down_q, qs = lay.down_s, qc = lay.down_sc, z = 0;
    if (bf) {
      DOWN(MOE_FMT_IQ3G, true, true, 1, qi, qs, qc, z);
      DOWN(MOE_FMT_IQ3G, true, false, 2, qi, qs, qc, z);
    } else {
      DOWN(MOE_FMT_IQ3G, false, true, 1, qi, qs, qc, z);
      DOWN(MOE_FMT_IQ3G, false, false, 2, qi, qs, qc, z);
    }
  } else if (L->fmt_down == MOE_FMT_IQ1G) {
    hipLaunchKernelGGL((k_gemm_gateup_nvfp4<true, false>), grid, block, 0, s, GU_ARGS);
    hipLaunchKernelGGL((k_gemm_gateup_nvfp4<false, true>), grid, block, 0, s, GU_ARGS);
    const size_t qi = lay.down_q, qh = lay.down_s, qc = lay.down_sc, z = 0;
    if (bf) {
      DOWN(MOE_FMT_IQ1G, true, true, 1, qi, qh, qc, z);
      DOWN(MOE_FMT_IQ1G, true, false, 2, qi, qh, qc, z);
    } else {
      DOWN(MOE_FMT_IQ1G, false, true, 1, qi, qh, qc, z);
      DOWN(MOE_FMT_IQ1G, false, false, 2, qi, qh, qc, z);
    }
  } else {
    hipLaunchKernelGGL((k_gemm_gateup_nvfp4<true, false>), grid, block, 0, s, GU_ARGS);
    hipLaunchKernelGGL((k_gemm_gateup_nvfp4<false, true>), grid, block, 0, s, GU_ARGS);
    const size_t a = lay.down_ql, b2 = lay.down_qh, c = lay.down_sc, d = lay.down_d;
    if (bf) {
      DOWN(MOE_FMT_Q6K, true, true, 1, a, b2, c, d);
      DOWN(MOE_FMT_Q6K, true, false, 2, a, b2, c, d);
    } else {
      DOWN(MOE_FMT_Q6K, false, true, 1, a, b2, c, d);
      DOWN(MOE_FMT_Q6K, false, false, 2, a, b2, c, d);
    }
  }
#undef GU_ARGS
#undef DOWN
  return hipGetLastError();
}

}  // namespace moe
