// gemv_common.h -- shared pieces of the decode-size expert kernels.
//
// Routed experts are block-quantized (NVFP4; GGUF Q6_K in the DQ6_K packs:
// basalt.jgulfo.com, sections "Models" and "Quick start"), and a token touches
// only the experts it selected (same page, "Expert tiers").  With 1..8 tokens
// per step
// (one per request slot) the expert FFN is bound by reading each active
// expert's weight bytes once from HBM, so these kernels stream the packed
// codes with 16-byte loads and dequantize in registers:
//   - grid = (row blocks of 64, slots of the active-expert list[, matrix]); a
//     workgroup whose slot is past n_active exits at once, so no workgroup is
//     spent on an expert without tokens;
//   - lane l of every wave owns output row 64*blockIdx.x + l: a wave-wide
//     16-byte load reads the same 32-element K-slice of 64 consecutive rows,
//     which the packed blob stores contiguously -- no cross-lane reduction;
//   - K is cut into groups (128 elements NVFP4, 256 Q6_K) and split over the
//     S waves of a workgroup; each wave streams its GPS = groups/S groups
//     through a ring of D register slots (the loads of D groups are always in
//     flight), so a workgroup never holds more than D groups per lane and
//     every workgroup of the launch can be resident at once.  S is chosen on
//     the host from the number of workgroups (small batches split K more);
//   - the S partial sums of a row are added through LDS in wave order.
#pragma once

#include "common.h"

namespace moe {

typedef float v2f_t __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));

constexpr int kMaxMT = 8;  // tokens per pass (register arrays are sized for this)

// Weight loads: global address space (the expert blob pointer comes from a
// table, so the compiler would otherwise emit flat loads, which also count
// against the LDS wait counter) and nontemporal (each weight byte is read once
// per step, so the lines are not kept in the caches; streaming reads run
// markedly faster this way on MI355X).
// (These helpers only exist in device code; the host pass never sees them.)
#if defined(__HIP_DEVICE_COMPILE__)
typedef unsigned v4u_t __attribute__((ext_vector_type(4)));
typedef unsigned v2u_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) v4u_t g_v4u;
typedef __attribute__((address_space(1))) v2u_t g_v2u;
typedef __attribute__((address_space(1))) uint16_t g_u16;
typedef __attribute__((address_space(1))) uint32_t g_u32;
__device__ __forceinline__ uint4 ld16(const uint8_t* p) {
  const v4u_t t = __builtin_nontemporal_load((const g_v4u*)(uintptr_t)p);
  return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ uint2 ld8(const uint8_t* p) {
  const v2u_t t = __builtin_nontemporal_load((const g_v2u*)(uintptr_t)p);
  return make_uint2(t.x, t.y);
}
__device__ __forceinline__ uint32_t ld4(const uint8_t* p) {
  return __builtin_nontemporal_load((const g_u32*)(uintptr_t)p);
}
__device__ __forceinline__ uint16_t ld2(const uint8_t* p) {
  return __builtin_nontemporal_load((const g_u16*)(uintptr_t)p);
}
#else
__device__ uint4 ld16(const uint8_t* p);
__device__ uint2 ld8(const uint8_t* p);
__device__ uint32_t ld4(const uint8_t* p);
__device__ uint16_t ld2(const uint8_t* p);
#endif

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// 8 E2M1 codes of a 32-bit word (element 2b in the low nibble of byte b) ->
// 8 exact floats (gfx950 packed FP4 -> F32 conversion, scale 1.0).
__device__ __forceinline__ void e2m1x8_f32(uint32_t c, float* o) {
  v2f_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
  v2f_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
  v2f_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2);
  v2f_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
  o[0] = p0.x; o[1] = p0.y; o[2] = p1.x; o[3] = p1.y;
  o[4] = p2.x; o[5] = p2.y; o[6] = p3.x; o[7] = p3.y;
}

// Same codes -> 4 bf16 pairs (exact: E2M1 values have 2 significant bits).
__device__ __forceinline__ void e2m1x8_bf16(uint32_t c, v2bf_t* o) {
  o[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, 0);
  o[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, 1);
  o[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, 2);
  o[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, 3);
}

__device__ __forceinline__ v2bf_t as_v2bf(uint32_t u) { return __builtin_bit_cast(v2bf_t, u); }

// Sign masks of a pair of 16-bit values from bits p and p + 1 of w: bit p to
// bit 15 (low value), bit p + 1 to bit 31 (high value).  p is a constant once
// the callers' loops are unrolled, so this is two shifts and a bit select.
__device__ __forceinline__ uint32_t pair_sign_at(uint32_t w, int p) {
  const uint32_t lo = p <= 15 ? (w << (15 - p)) : (w >> (p - 15));
  const uint32_t hi = p <= 30 ? (w << (30 - p)) : (w >> (p - 30));
  return (lo & 0x8000u) | (hi & 0x80000000u);
}

// Two floats -> bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
// silu(g) * u = g * u / (1 + e^-g) with the hardware exp2 and reciprocal
// (about 1 ulp each; h is rounded to bf16 right after, 2^-9 relative).  Large
// |g| give the right limits: e^-g -> 0 or inf, so the factor -> 1 or 0.
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f)) * u;
}

__device__ __forceinline__ v2bf_t to_v2bf(float a, float b) {
  v2f_t f = {a, b};
  return __builtin_convertvector(f, v2bf_t);
}

__device__ __forceinline__ float dot16_f32(const float* w, const float* x) {
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s = fmaf(w[i], x[i], s);
  return s;
}

__device__ __forceinline__ void load_f32x16(const float* p, float* xv) {
  const float4* q = reinterpret_cast<const float4*>(p);
  float4 a0 = q[0], a1 = q[1], a2 = q[2], a3 = q[3];
  xv[0] = a0.x; xv[1] = a0.y; xv[2] = a0.z; xv[3] = a0.w;
  xv[4] = a1.x; xv[5] = a1.y; xv[6] = a1.z; xv[7] = a1.w;
  xv[8] = a2.x; xv[9] = a2.y; xv[10] = a2.z; xv[11] = a2.w;
  xv[12] = a3.x; xv[13] = a3.y; xv[14] = a3.z; xv[15] = a3.w;
}

template <bool BF16>
__device__ __forceinline__ void store_y(void* y, size_t i, float v) {
  if (BF16) reinterpret_cast<uint16_t*>(y)[i] = f32_to_bf16_rne(v);
  else reinterpret_cast<float*>(y)[i] = v;
}

// Stage rows row0 .. row0+mt of h (fp32 [A][K], sorted order) into LDS.
__device__ __forceinline__ void stage_rows_f32(const float* __restrict__ hin, int K, int row0,
                                               int mt, float* sm, int nthreads) {
  const int vpr = K >> 2;
  for (int i = threadIdx.x; i < mt * vpr; i += nthreads) {
    int r = i / vpr, c = i - r * vpr;
    reinterpret_cast<float4*>(sm + (size_t)r * K)[c] =
        reinterpret_cast<const float4*>(hin + (size_t)(row0 + r) * K)[c];
  }
}

// Per-slot header shared by the kernels: expert id, token count and offset.
// The expert of this workgroup's slot (blockIdx.y) and its table entry: false
// for a slot past n_active.  The expert's token count and first sorted
// position are loaded separately by the caller, after it has issued its
// first weight loads: they were just written by the gating step, while the
// table entry is usually in L2, so the weights need not wait for them.
__device__ __forceinline__ bool slot_expert(const int32_t* __restrict__ active,
                                            const int32_t* __restrict__ n_active,
                                            const moe_expert_ref* __restrict__ experts, int* e,
                                            moe_expert_ref* ref) {
  const int slot = blockIdx.y;
  // Both loads in one round trip: active[] has E >= gridDim.y entries, so
  // active[slot] is in bounds even for a slot past n_active (then unused).
  const int na = __builtin_nontemporal_load(n_active);
  const int ee = __builtin_nontemporal_load(active + slot);
  // Both values (and the table's address, a kernel argument) are consumed
  // here, so both loads are issued before the first wait (left alone, the
  // compiler tests na first and then loads active[slot]: two round trips).
  asm volatile("" ::"s"(na), "s"(ee), "s"(experts));
  if (slot >= na) return false;
  *e = ee;
  *ref = experts[ee];
  return true;
}

// Activations are read with wave-uniform addresses through the scalar cache,
// one 128-element group at a time, each group's reads waiting on the
// previous ones; a first read that misses the cache costs a round trip per
// group.  touch_lines reads one word of each of NL consecutive 64-byte lines
// at p (wave-uniform) right after a pass's weight loads are issued, so the
// lines are in the scalar cache by the time the groups are consumed: one
// round trip, under the weights' own latency.  The xor of the words goes to
// keep_scalar, which only makes the compiler keep (and wait for) the loads.
template <int NL>
__device__ __forceinline__ uint32_t touch_lines(const uint32_t* __restrict__ p) {
  uint32_t t = 0;
#pragma unroll
  for (int l = 0; l < NL; ++l) t ^= p[16 * l];
  return t;
}
__device__ __forceinline__ void keep_scalar(uint32_t v) { asm volatile("" ::"s"(v)); }

// E4M3 scale bytes 2i, 2i+1 (lo) or 2i+2, 2i+3 (hi) of a word -> fp32 pair, exact
// (gfx950 converts OCP E4M3).
template <bool HI>
__device__ __forceinline__ v2f_t e4m3x2(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
}

// The 8 E4M3 scales of a group (one per 16-element block) -> fp32.
__device__ __forceinline__ void e4m3x8(const uint2& s, float* sc) {
  v2f_t a = e4m3x2<false>(s.x), b = e4m3x2<true>(s.x);
  v2f_t c = e4m3x2<false>(s.y), e = e4m3x2<true>(s.y);
  sc[0] = a.x; sc[1] = a.y; sc[2] = b.x; sc[3] = b.y;
  sc[4] = c.x; sc[5] = c.y; sc[6] = e.x; sc[7] = e.y;
}

// Split of NG K-groups over S waves: the largest divisor of NG that is at most
// max_s and keeps items * waves_per_item * S within the wave budget.
inline int choose_split(int items, int waves_per_item, int NG, int max_s) {
  const int budget = 4096;
  int best = 1;
  for (int s = 1; s <= max_s && s <= NG; ++s)
    if (NG % s == 0 && (long)items * waves_per_item * s <= budget) best = s;
  return best;
}

// Launch helpers (one per kernel family), defined in their .hip files.
size_t gemm_tiles_bytes(int E, int64_t A);
hipError_t launch_gemm_ffn(const moe_layer_desc* L, const uint16_t* x, int64_t T,
                           const moe_buckets* b, uint16_t* hbuf, uint16_t* xh, float* xscale,
                           void* tiles_ws, void* y, int y_dtype, hipStream_t s);

// h passes from the gate/up kernel to the down kernel as bf16 [A][I] (sorted
// order).
hipError_t launch_gemv_gateup(const moe_layer_desc* L, const uint16_t* x, const moe_buckets* b,
                              int max_slots, uint16_t* h, hipStream_t s);
hipError_t launch_gemv_down(const moe_layer_desc* L, const uint16_t* h, const moe_buckets* b,
                            int max_slots, void* y, int y_dtype, hipStream_t s);
// Down projection fused with the gate-weighted combine for decode batches
// (gemv_down.hip): out bf16 [T][H] straight from h, no y.
hipError_t launch_gemv_down_combine(const moe_layer_desc* L, const uint16_t* h, int64_t T,
                                   const int32_t* idx, const int32_t* asg_pos,
                                   const float* topk_w, const uint16_t* residual, uint16_t* out,
                                   hipStream_t s);
// Gate/up in 32-row slices (gemv_gateup32.hip), for the layers it fits; the
// same h as launch_gemv_gateup.
bool gemv_gateup32_fits(const moe_layer_desc* L);
hipError_t launch_gemv_gateup32(const moe_layer_desc* L, const uint16_t* x, const moe_buckets* b,
                                int max_slots, uint16_t* h, hipStream_t s);
// The decode gating (as launch_gate_fused: top-k, buckets, histogram, from
// the router logits) and then the 32-row gate/up, in one launch; for the
// layers and batches gemv_gate_gateup32_fits accepts.
bool gemv_gate_gateup32_fits(const moe_layer_desc* L, int64_t T);
hipError_t launch_gemv_gate_gateup32(const moe_layer_desc* L, const uint16_t* x, int64_t T,
                                     const float* logits, int32_t* idx, float* w,
                                     const moe_buckets* b, uint32_t* hist, int ds, int us,
                                     int max_slots, uint16_t* h, hipStream_t s);


}  // namespace moe
