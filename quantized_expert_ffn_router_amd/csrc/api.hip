// api.hip -- the extern "C" entry points of libmoe: argument validation
// (before any launch), error reporting and kernel dispatch.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "gemv_common.h"

// Workspace of moe_expert_ffn_noalloc: one copy per GPU, held until the
// process ends.  Host code never passes this name to a kernel or a copy (on
// the host it is only a stand-in for the symbol); it uses the device address
// that hipGetSymbolAddress returns for the current device (scratch_ptr).
constexpr size_t kScratchBytes = MOE_NOALLOC_WORKSPACE_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

moe_status hip_status(const char* where, hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

#define CHECK_PTR(p, where) \
  if (!(p)) return fail(MOE_ERR_INVALID_ARG, "%s: %s is NULL", where, #p)

moe_status check_shape(int E, int k, int H, int I, int fmt_gu, int fmt_down, const char* where) {
  if (E < 1 || k < 1 || H < 1 || I < 1)
    return fail(MOE_ERR_INVALID_ARG, "%s: E=%d k=%d H=%d I=%d must be positive", where, E, k, H, I);
  if (k > E) return fail(MOE_ERR_INVALID_ARG, "%s: k=%d > E=%d", where, k, E);
  if (E > 1024) return fail(MOE_ERR_UNSUPPORTED, "%s: E=%d > 1024", where, E);
  if (k > 64) return fail(MOE_ERR_UNSUPPORTED, "%s: k=%d > 64", where, k);
  if (H % 128 != 0 || H > 8192)
    return fail(MOE_ERR_UNSUPPORTED, "%s: H=%d must be a multiple of 128 and <= 8192", where, H);
  if (fmt_gu != MOE_FMT_NVFP4)
    return fail(MOE_ERR_UNSUPPORTED, "%s: gate/up format %d (only NVFP4)", where, fmt_gu);
  if (fmt_down == MOE_FMT_NVFP4 || fmt_down == MOE_FMT_Q8_0) {
    if (I % 128 != 0 || I > 8192)
      return fail(MOE_ERR_UNSUPPORTED, "%s: I=%d must be a multiple of 128 and <= 8192", where, I);
  } else if (fmt_down == MOE_FMT_Q6K || fmt_down == MOE_FMT_IQ3G || fmt_down == MOE_FMT_IQ1G) {
    if (I % 256 != 0 || I > 8192)
      return fail(MOE_ERR_UNSUPPORTED,
                  "%s: I=%d must be a multiple of 256 and <= 8192 for %s", where, I,
                  fmt_down == MOE_FMT_Q6K ? "Q6_K" : (fmt_down == MOE_FMT_IQ3G ? "IQ3G" : "IQ1G"));
  } else {
    return fail(MOE_ERR_UNSUPPORTED, "%s: down format %d", where, fmt_down);
  }
  return MOE_OK;
}

moe_status check_layer(const moe_layer_desc* L, const char* where) {
  CHECK_PTR(L, where);
  moe_status st = check_shape(L->E, L->k, L->H, L->I, L->fmt_gate_up, L->fmt_down, where);
  if (st != MOE_OK) return st;
  if (L->renormalize != 0 && L->renormalize != 1)
    return fail(MOE_ERR_INVALID_ARG, "%s: renormalize=%d must be 0 or 1", where, L->renormalize);
  if (L->ffn_mode != MOE_FFN_AUTO && L->ffn_mode != MOE_FFN_GEMV && L->ffn_mode != MOE_FFN_GEMM)
    return fail(MOE_ERR_INVALID_ARG, "%s: ffn_mode=%d", where, L->ffn_mode);
  return MOE_OK;
}

moe_status check_buckets(const moe_layer_desc* L, const moe_buckets* b, int64_t T,
                         const char* where) {
  CHECK_PTR(b, where);
  if (b->E != L->E || b->k != L->k)
    return fail(MOE_ERR_INVALID_ARG, "%s: buckets carved for E=%d k=%d, layer has E=%d k=%d", where,
                b->E, b->k, L->E, L->k);
  if (T > b->T_max)
    return fail(MOE_ERR_WORKSPACE, "%s: T=%lld exceeds bucket capacity %lld", where, (long long)T,
                (long long)b->T_max);
  if (!b->counts || !b->offsets || !b->sorted_asg || !b->asg_pos || !b->active || !b->n_active)
    return fail(MOE_ERR_INVALID_ARG, "%s: bucket field is NULL (use moe_buckets_carve)", where);
  return MOE_OK;
}

constexpr int64_t kMaxT = (int64_t)1 << 24;

moe_status check_T(int64_t T, int k, const char* where) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "%s: T=%lld < 0", where, (long long)T);
  if (T > kMaxT || T * k > INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "%s: T=%lld too large", where, (long long)T);
  return MOE_OK;
}

// Workspace of moe_expert_ffn: h (bf16 [T*k][I], both paths), then for the
// grouped GEMM an fp16 copy of x ([T][H]), its row scales ([T]) and the tile list.
struct FfnWs {
  size_t h, xh, xscale, tiles, total;
};
FfnWs ffn_ws_layout(const moe_layer_desc* L, int64_t T) {
  const size_t A = (size_t)T * L->k;
  FfnWs w;
  w.h = 0;
  w.xh = moe::align_up(A * (size_t)L->I * sizeof(uint16_t));
  w.xscale = w.xh + moe::align_up((size_t)T * L->H * sizeof(uint16_t));
  w.tiles = w.xscale + moe::align_up((size_t)T * sizeof(float));
  w.total = w.tiles + moe::gemm_tiles_bytes(L->E, (int64_t)A);
  return w;
}
size_t ffn_ws(const moe_layer_desc* L, int64_t T) { return ffn_ws_layout(L, T).total; }

// The grouped GEMM needs 256-column down tiles and 32-bit element offsets
// of the token rows (x: T*H values) and of h (T*k*I values).
bool gemm_fits(const moe_layer_desc* L, int64_t T) {
  return L->H % 256 == 0 && (uint64_t)T * (uint64_t)L->H <= UINT32_MAX &&
         (uint64_t)T * (uint64_t)L->k * (uint64_t)L->I <= UINT32_MAX;
}

// Grouped GEMM once experts average >= 16 tokens (and the batch is not a
// decode step); dequant-fused GEMV otherwise.
// Batches of 2 to 8 tokens run the down projection and the combine as one
// kernel in moe_layer_forward (graph-replayed steps: batch 8 39.0 against
// 41.8 us, batch 4 27.7 against 29.5; at batch 1 its 32 workgroups pull
// each CU's 221 KB of expert rows too slowly, 20.0 against 19.2 us, and at
// batch 16 the experts that several tokens share are read once per token).
constexpr int64_t kDownCombineMinT = 2, kDownCombineMaxT = 8;

bool use_gemm(const moe_layer_desc* L, int64_t T) {
  if (L->ffn_mode == MOE_FFN_GEMV) return false;
  if (L->ffn_mode == MOE_FFN_GEMM) return true;
  return T > 64 && T * L->k >= 16 * (int64_t)L->E && gemm_fits(L, T);
}

}  // namespace

namespace moe {
moe_status tier_fail(moe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}
}  // namespace moe

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_last_error(void) { return g_err; }

size_t moe_expert_blob_bytes(int32_t H, int32_t I, int32_t fmt_gate_up, int32_t fmt_down) {
  if (check_shape(1, 1, H, I, fmt_gate_up, fmt_down, "moe_expert_blob_bytes") != MOE_OK) return 0;
  return moe::blob_layout(H, I, fmt_down).total;
}

moe_status moe_pack_experts(int32_t E, int32_t H, int32_t I, int32_t fmt_gate_up,
                            int32_t fmt_down, const uint8_t* gate_q, const uint8_t* gate_s,
                            const uint8_t* up_q, const uint8_t* up_s, const uint8_t* down_q,
                            const uint8_t* down_s, void* blobs, size_t blob_stride,
                            hipStream_t stream) {
  const char* W = "moe_pack_experts";
  moe_status st = check_shape(E, 1, H, I, fmt_gate_up, fmt_down, W);
  if (st != MOE_OK) return st;
  CHECK_PTR(gate_q, W); CHECK_PTR(gate_s, W); CHECK_PTR(up_q, W); CHECK_PTR(up_s, W);
  CHECK_PTR(down_q, W); CHECK_PTR(blobs, W);
  if (fmt_down == MOE_FMT_NVFP4) CHECK_PTR(down_s, W);
  const moe::BlobLayout lay = moe::blob_layout(H, I, fmt_down);
  if (blob_stride < lay.total || blob_stride % moe::kAlign != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: blob_stride %zu must be >= %zu and a multiple of 256", W,
                blob_stride, lay.total);
  uint8_t* d = (uint8_t*)blobs;
  const size_t gu_q = (size_t)I * H / 2, gu_s = (size_t)I * H / 16;
  hipError_t e;
  // gate / up: N = I rows, K = H
  e = moe::launch_pack_granules(gate_q, E, gu_q, I, H / 32, 16, H / 2, 1, 16, 0, d + lay.gate_q, blob_stride, stream);
  if (e == hipSuccess) e = moe::launch_pack_granules(gate_s, E, gu_s, I, H / 128, 8, H / 16, 1, 8, 0, d + lay.gate_s, blob_stride, stream);
  if (e == hipSuccess) e = moe::launch_pack_granules(up_q, E, gu_q, I, H / 32, 16, H / 2, 1, 16, 0, d + lay.up_q, blob_stride, stream);
  if (e == hipSuccess) e = moe::launch_pack_granules(up_s, E, gu_s, I, H / 128, 8, H / 16, 1, 8, 0, d + lay.up_s, blob_stride, stream);
  if (e != hipSuccess) return hip_status(W, e);
  if (fmt_down == MOE_FMT_NVFP4) {
    // down: N = H rows, K = I
    e = moe::launch_pack_granules(down_q, E, (size_t)H * I / 2, H, I / 32, 16, I / 2, 1, 16, 0, d + lay.down_q, blob_stride, stream);
    if (e == hipSuccess) e = moe::launch_pack_granules(down_s, E, (size_t)H * I / 16, H, I / 128, 8, I / 16, 1, 8, 0, d + lay.down_s, blob_stride, stream);
  } else if (fmt_down == MOE_FMT_Q8_0) {
    // 34-byte blocks: codes in two 16-byte granules per block, the 4 scales of
    // a 128-element group gathered into one 8-byte granule
    const size_t row = (size_t)(I / 32) * 34, ex = (size_t)H * row;
    e = moe::launch_pack_granules(down_q, E, ex, H, I / 16, 16, row, 2, 34, 2, d + lay.down_q, blob_stride, stream);
    if (e == hipSuccess) e = moe::launch_pack_granules(down_q, E, ex, H, I / 128, 2, row, 1, 34, 0, d + lay.down_s, blob_stride, stream, 4);
    if (e == hipSuccess) e = moe::launch_down_exponent(down_q, E, H, I, fmt_down, d + lay.down_meta, blob_stride, stream);
  } else if (fmt_down == MOE_FMT_IQ3G) {
    // 102-byte superblocks: grid indices in 16-byte granules of 64 elements,
    // sign bits in 16-byte granules of 128 elements, and d with the 4-bit
    // multipliers (6 bytes) in an 8-byte granule per superblock
    const size_t row = (size_t)(I / 256) * moe::kIq3gBlockBytes, ex = (size_t)H * row;
    e = moe::launch_pack_granules(down_q, E, ex, H, I / 64, 16, row, 4, moe::kIq3gBlockBytes, 6, d + lay.down_q, blob_stride, stream);
    if (e == hipSuccess) e = moe::launch_pack_granules(down_q, E, ex, H, I / 128, 16, row, 2, moe::kIq3gBlockBytes, 70, d + lay.down_s, blob_stride, stream);
    if (e == hipSuccess) e = moe::launch_pack_granules(down_q, E, ex, H, I / 256, 6, row, 1, moe::kIq3gBlockBytes, 0, d + lay.down_sc, blob_stride, stream, 1, 2);
    if (e == hipSuccess) e = moe::launch_down_exponent(down_q, E, H, I, fmt_down, d + lay.down_meta, blob_stride, stream);
  } else if (fmt_down == MOE_FMT_IQ1G) {
    // 46-byte superblocks: index low bytes in 16-byte granules of 128
    // elements, their 2-bit high parts in 4-byte granules of 128 elements,
    // and d with the 4-bit multipliers (6 bytes) in an 8-byte granule per
    // superblock
    const size_t row = (size_t)(I / 256) * moe::kIq1gBlockBytes, ex = (size_t)H * row;
    e = moe::launch_pack_granules(down_q, E, ex, H, I / 128, 16, row, 2, moe::kIq1gBlockBytes, 6, d + lay.down_q, blob_stride, stream);
    if (e == hipSuccess) e = moe::launch_pack_granules(down_q, E, ex, H, I / 128, 4, row, 2, moe::kIq1gBlockBytes, 38, d + lay.down_s, blob_stride, stream);
    if (e == hipSuccess) e = moe::launch_pack_granules(down_q, E, ex, H, I / 256, 6, row, 1, moe::kIq1gBlockBytes, 0, d + lay.down_sc, blob_stride, stream, 1, 2);
    if (e == hipSuccess) e = moe::launch_down_exponent(down_q, E, H, I, fmt_down, d + lay.down_meta, blob_stride, stream);
  } else {
    const size_t row = (size_t)(I / 256) * 210, ex = (size_t)H * row;
    e = moe::launch_pack_granules(down_q, E, ex, H, I / 32, 16, row, 8, 210, 0, d + lay.down_ql, blob_stride, stream);
    if (e == hipSuccess) e = moe::launch_pack_granules(down_q, E, ex, H, I / 64, 16, row, 4, 210, 128, d + lay.down_qh, blob_stride, stream);
    if (e == hipSuccess) e = moe::launch_pack_granules(down_q, E, ex, H, I / 256, 16, row, 1, 210, 192, d + lay.down_sc, blob_stride, stream);
    if (e == hipSuccess) e = moe::launch_pack_granules(down_q, E, ex, H, I / 256, 2, row, 1, 210, 208, d + lay.down_d, blob_stride, stream);
    if (e == hipSuccess) e = moe::launch_down_exponent(down_q, E, H, I, fmt_down, d + lay.down_meta, blob_stride, stream);
  }
  return hip_status(W, e);
}

size_t moe_buckets_bytes(int32_t E, int64_t T_max, int32_t k) {
  if (E < 1 || k < 1 || T_max < 0) return 0;
  size_t A = (size_t)T_max * k;
  return moe::align_up((size_t)E * 4) + moe::align_up((size_t)(E + 1) * 4) +
         moe::align_up(A * 4) * 2 + moe::align_up((size_t)E * 4) + moe::align_up(4);
}

moe_status moe_buckets_carve(void* buf, size_t bytes, int32_t E, int64_t T_max, int32_t k,
                             moe_buckets* out) {
  const char* W = "moe_buckets_carve";
  CHECK_PTR(buf, W);
  CHECK_PTR(out, W);
  if (E < 1 || k < 1 || T_max < 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: E=%d k=%d T_max=%lld", W, E, k, (long long)T_max);
  if ((uintptr_t)buf % moe::kAlign != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: buffer not 256-byte aligned", W);
  size_t need = moe_buckets_bytes(E, T_max, k);
  if (bytes < need) return fail(MOE_ERR_WORKSPACE, "%s: %zu bytes < %zu needed", W, bytes, need);
  size_t A = (size_t)T_max * k;
  char* p = (char*)buf;
  out->counts = (uint32_t*)p; p += moe::align_up((size_t)E * 4);
  out->offsets = (int32_t*)p; p += moe::align_up((size_t)(E + 1) * 4);
  out->sorted_asg = (int32_t*)p; p += moe::align_up(A * 4);
  out->asg_pos = (int32_t*)p; p += moe::align_up(A * 4);
  out->active = (int32_t*)p; p += moe::align_up((size_t)E * 4);
  out->n_active = (int32_t*)p;
  out->T_max = T_max;
  out->E = E;
  out->k = k;
  return MOE_OK;
}

size_t moe_workspace_bytes(const moe_layer_desc* L, int64_t T_max) {
  if (check_layer(L, "moe_workspace_bytes") != MOE_OK || T_max < 0) return 0;
  size_t a = moe::bucket_ws_bytes(L->E, T_max * L->k);
  size_t b = ffn_ws(L, T_max);
  size_t w = a > b ? a : b;
  return w ? w : moe::kAlign;
}

moe_status moe_route(const moe_layer_desc* L, const uint16_t* x, int64_t T, float* logits,
                     int32_t* topk_idx, float* topk_w, hipStream_t stream) {
  const char* W = "moe_route";
  moe_status st = check_layer(L, W);
  if (st != MOE_OK) return st;
  if ((st = check_T(T, L->k, W)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  CHECK_PTR(x, W); CHECK_PTR(logits, W); CHECK_PTR(topk_idx, W); CHECK_PTR(topk_w, W);
  CHECK_PTR(L->w_router, W);
  hipError_t e = moe::launch_router(x, T, L->H, L->w_router, L->router_bias, L->E, logits, stream);
  if (e == hipSuccess) e = moe::launch_topk(logits, T, L->E, L->k, L->renormalize, topk_idx, topk_w, stream);
  return hip_status(W, e);
}

moe_status moe_bucket(const moe_layer_desc* L, const int32_t* topk_idx, int64_t T,
                      const moe_buckets* b, void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* W = "moe_bucket";
  moe_status st = check_layer(L, W);
  if (st != MOE_OK) return st;
  if ((st = check_T(T, L->k, W)) != MOE_OK) return st;
  if ((st = check_buckets(L, b, T, W)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  CHECK_PTR(topk_idx, W);
  size_t need = moe::bucket_ws_bytes(L->E, T * L->k);
  if (need > 0) {
    CHECK_PTR(ws, W);
    if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu < %zu", W, ws_bytes, need);
  }
  return hip_status(W, moe::launch_bucket(topk_idx, T * L->k, L->E, b, ws, stream));
}

}  // extern "C"

namespace {

// Argument checks shared by moe_expert_ffn and moe_expert_ffn_noalloc.
moe_status ffn_check(const char* W, const moe_layer_desc* L, const uint16_t* x, int64_t T,
                     const moe_buckets* b, const void* y, int32_t y_dtype) {
  moe_status st = check_layer(L, W);
  if (st != MOE_OK) return st;
  if ((st = check_T(T, L->k, W)) != MOE_OK) return st;
  if ((st = check_buckets(L, b, T, W)) != MOE_OK) return st;
  if (y_dtype != MOE_DTYPE_F32 && y_dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "%s: y_dtype=%d", W, y_dtype);
  if (T == 0) return MOE_OK;
  CHECK_PTR(x, W); CHECK_PTR(y, W); CHECK_PTR(L->experts, W);
  if (use_gemm(L, T) && !gemm_fits(L, T))
    return fail(MOE_ERR_UNSUPPORTED, "%s: grouped GEMM needs H %% 256 == 0, T*H and T*k*I < 2^32",
                W);
  return MOE_OK;
}

// The GEMV family's gate/up into h (bf16 [T*k][I], sorted order): 32-row
// slices for up to 16 tokens (it redoes the weight decode per token, which
// costs more than it saves once experts hold many tokens), else 64-row blocks.
hipError_t gemv_gateup_launch(const moe_layer_desc* L, const uint16_t* x, int64_t T,
                              const moe_buckets* b, int max_slots, uint16_t* h,
                              hipStream_t stream) {
  return (T <= 16 && moe::gemv_gateup32_fits(L))
             ? moe::launch_gemv_gateup32(L, x, b, max_slots, h, stream)
             : moe::launch_gemv_gateup(L, x, b, max_slots, h, stream);
}

// The FFN's launches (checks done, T > 0, ws holds ffn_ws(L, T) bytes).
moe_status ffn_launch(const char* W, const moe_layer_desc* L, const uint16_t* x, int64_t T,
                      const moe_buckets* b, void* y, int32_t y_dtype, void* ws,
                      hipStream_t stream) {
  if (use_gemm(L, T)) {
    const FfnWs w = ffn_ws_layout(L, T);
    char* c = (char*)ws;
    return hip_status(W, moe::launch_gemm_ffn(L, x, T, b, (uint16_t*)(c + w.h),
                                               (uint16_t*)(c + w.xh), (float*)(c + w.xscale),
                                               c + w.tiles, y, y_dtype, stream));
  }
  // Worst-case number of active experts; workgroups past n_active exit.
  const int max_slots = (int)((T * L->k < L->E) ? T * L->k : L->E);
  uint16_t* h = (uint16_t*)ws;  // bf16 [T*k][I], sorted order
  hipError_t e = gemv_gateup_launch(L, x, T, b, max_slots, h, stream);
  if (e == hipSuccess) e = moe::launch_gemv_down(L, h, b, max_slots, y, y_dtype, stream);
  return hip_status(W, e);
}

// Device address of `scratch` on each device, looked up on the first
// moe_expert_ffn_noalloc call made with that device current.
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

moe_status scratch_ptr(const char* W, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(W, e);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "%s: device %d beyond %d", W, dev, kMaxDevices);
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess) return hip_status(W, g_scratch_err[dev]);
  if (!g_scratch_ptr[dev]) return fail(MOE_ERR_HIP, "%s: no device address for the scratch", W);
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_expert_ffn(const moe_layer_desc* L, const uint16_t* x, int64_t T,
                          const moe_buckets* b, void* y, int32_t y_dtype, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  const char* W = "moe_expert_ffn";
  moe_status st = ffn_check(W, L, x, T, b, y, y_dtype);
  if (st != MOE_OK || T == 0) return st;
  CHECK_PTR(ws, W);
  const size_t need = ffn_ws(L, T);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu < %zu", W, ws_bytes, need);
  return ffn_launch(W, L, x, T, b, y, y_dtype, ws, stream);
}

moe_status moe_expert_ffn_noalloc(const moe_layer_desc* L, const uint16_t* x, int64_t T,
                                  const moe_buckets* b, void* y, int32_t y_dtype,
                                  hipStream_t stream) {
  const char* W = "moe_expert_ffn_noalloc";
  moe_status st = ffn_check(W, L, x, T, b, y, y_dtype);
  if (st != MOE_OK || T == 0) return st;
  const size_t need = ffn_ws(L, T);
  if (need > kScratchBytes)
    return fail(MOE_ERR_WORKSPACE,
                "%s: this call needs %zu bytes of workspace, above the library's static %zu "
                "(use moe_expert_ffn with a caller workspace)",
                W, need, kScratchBytes);
  void* ws = nullptr;
  if ((st = scratch_ptr(W, &ws)) != MOE_OK) return st;
  return ffn_launch(W, L, x, T, b, y, y_dtype, ws, stream);
}

moe_status moe_combine(const moe_layer_desc* L, const void* y, int32_t y_dtype,
                       const moe_buckets* b, const float* topk_w, int64_t T,
                       const uint16_t* residual, uint16_t* out, hipStream_t stream) {
  const char* W = "moe_combine";
  moe_status st = check_layer(L, W);
  if (st != MOE_OK) return st;
  if ((st = check_T(T, L->k, W)) != MOE_OK) return st;
  if ((st = check_buckets(L, b, T, W)) != MOE_OK) return st;
  if (y_dtype != MOE_DTYPE_F32 && y_dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "%s: y_dtype=%d", W, y_dtype);
  if (T == 0) return MOE_OK;
  CHECK_PTR(y, W); CHECK_PTR(topk_w, W); CHECK_PTR(out, W);
  return hip_status(W, moe::launch_combine(y, y_dtype, b->asg_pos, topk_w, T, L->k, L->H, residual,
                                           out, stream));
}

moe_status moe_route_bucket(const moe_layer_desc* L, const uint16_t* x, int64_t T,
                            float* logits, int32_t* topk_idx, float* topk_w, const moe_buckets* b,
                            void* ws, size_t ws_bytes, uint32_t* hist, int32_t decay_shift,
                            int32_t unit_shift, hipStream_t stream) {
  const char* W = "moe_route_bucket";
  moe_status st = check_layer(L, W);
  if (st != MOE_OK) return st;
  if ((st = check_T(T, L->k, W)) != MOE_OK) return st;
  if ((st = check_buckets(L, b, T, W)) != MOE_OK) return st;
  if (hist && (decay_shift < 0 || decay_shift > 31 || unit_shift < 0 || unit_shift > 31))
    return fail(MOE_ERR_INVALID_ARG, "%s: shifts (%d, %d) must be in [0, 31]", W, decay_shift,
                unit_shift);
  if (T == 0) return MOE_OK;
  CHECK_PTR(x, W); CHECK_PTR(logits, W); CHECK_PTR(topk_idx, W); CHECK_PTR(topk_w, W);
  CHECK_PTR(L->w_router, W);
  const size_t need = moe::bucket_ws_bytes(L->E, T * L->k);
  if (need > 0) {
    CHECK_PTR(ws, W);
    if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu < %zu", W, ws_bytes, need);
  }
  hipError_t e = moe::launch_router(x, T, L->H, L->w_router, L->router_bias, L->E, logits, stream);
  if (e != hipSuccess) return hip_status(W, e);
  if (moe::gate_fused_fits(T, L->E, L->k))
    return hip_status(W, moe::launch_gate_fused(logits, T, L->E, L->k, L->renormalize, topk_idx,
                                                 topk_w, b, hist, decay_shift, unit_shift, stream));
  e = moe::launch_topk(logits, T, L->E, L->k, L->renormalize, topk_idx, topk_w, stream);
  if (e == hipSuccess) e = moe::launch_bucket(topk_idx, T * L->k, L->E, b, ws, stream);
  if (e == hipSuccess && hist)
    e = moe::launch_hist(b->counts, L->E, hist, decay_shift, unit_shift, stream);
  return hip_status(W, e);
}

moe_status moe_route_ffn(const moe_layer_desc* L, const uint16_t* x, int64_t T, float* logits,
                         int32_t* topk_idx, float* topk_w, const moe_buckets* b, uint32_t* hist,
                         int32_t decay_shift, int32_t unit_shift, void* y, int32_t y_dtype,
                         void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* W = "moe_route_ffn";
  moe_status st = ffn_check(W, L, x, T, b, y, y_dtype);
  if (st != MOE_OK) return st;
  if (hist && (decay_shift < 0 || decay_shift > 31 || unit_shift < 0 || unit_shift > 31))
    return fail(MOE_ERR_INVALID_ARG, "%s: shifts (%d, %d) must be in [0, 31]", W, decay_shift,
                unit_shift);
  if (T == 0) return MOE_OK;
  CHECK_PTR(logits, W); CHECK_PTR(topk_idx, W); CHECK_PTR(topk_w, W); CHECK_PTR(ws, W);
  CHECK_PTR(L->w_router, W);
  const size_t need = ffn_ws(L, T);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu < %zu", W, ws_bytes, need);
  if (use_gemm(L, T) || !moe::gemv_gate_gateup32_fits(L, T)) {  // the two calls
    st = moe_route_bucket(L, x, T, logits, topk_idx, topk_w, b, ws, ws_bytes, hist, decay_shift,
                          unit_shift, stream);
    if (st != MOE_OK) return st;
    return ffn_launch(W, L, x, T, b, y, y_dtype, ws, stream);
  }
  const int max_slots = (int)((T * L->k < L->E) ? T * L->k : L->E);
  uint16_t* h = (uint16_t*)ws;  // bf16 [T*k][I], sorted order
  hipError_t e = moe::launch_router(x, T, L->H, L->w_router, L->router_bias, L->E, logits, stream);
  if (e == hipSuccess)
    e = moe::launch_gemv_gate_gateup32(L, x, T, logits, topk_idx, topk_w, b, hist, decay_shift,
                                       unit_shift, max_slots, h, stream);
  if (e == hipSuccess) e = moe::launch_gemv_down(L, h, b, max_slots, y, y_dtype, stream);
  return hip_status(W, e);
}

moe_status moe_layer_forward(const moe_layer_desc* L, const uint16_t* x, int64_t T,
                             const uint16_t* residual, uint16_t* out, float* logits,
                             int32_t* topk_idx, float* topk_w, const moe_buckets* b,
                             uint32_t* hist, int32_t decay_shift, int32_t unit_shift, void* y,
                             int32_t y_dtype, void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* W = "moe_layer_forward";
  moe_status st = ffn_check(W, L, x, T, b, y, y_dtype);
  if (st != MOE_OK) return st;
  if (hist && (decay_shift < 0 || decay_shift > 31 || unit_shift < 0 || unit_shift > 31))
    return fail(MOE_ERR_INVALID_ARG, "%s: shifts (%d, %d) must be in [0, 31]", W, decay_shift,
                unit_shift);
  if (T == 0) return MOE_OK;
  CHECK_PTR(out, W); CHECK_PTR(logits, W); CHECK_PTR(topk_idx, W); CHECK_PTR(topk_w, W);
  CHECK_PTR(ws, W); CHECK_PTR(L->w_router, W);
  const size_t need = ffn_ws(L, T);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu < %zu", W, ws_bytes, need);
  if (use_gemm(L, T) || T < kDownCombineMinT || T > kDownCombineMaxT) {  // the two calls
    st = moe_route_ffn(L, x, T, logits, topk_idx, topk_w, b, hist, decay_shift, unit_shift, y,
                       y_dtype, ws, ws_bytes, stream);
    if (st != MOE_OK) return st;
    return moe_combine(L, y, y_dtype, b, topk_w, T, residual, out, stream);
  }
  const int max_slots = (int)((T * L->k < L->E) ? T * L->k : L->E);
  uint16_t* h = (uint16_t*)ws;  // bf16 [T*k][I], sorted order
  hipError_t e;
  if (moe::gemv_gate_gateup32_fits(L, T)) {
    e = moe::launch_router(x, T, L->H, L->w_router, L->router_bias, L->E, logits, stream);
    if (e == hipSuccess)
      e = moe::launch_gemv_gate_gateup32(L, x, T, logits, topk_idx, topk_w, b, hist, decay_shift,
                                         unit_shift, max_slots, h, stream);
  } else {
    st = moe_route_bucket(L, x, T, logits, topk_idx, topk_w, b, ws, ws_bytes, hist, decay_shift,
                          unit_shift, stream);
    if (st != MOE_OK) return st;
    e = gemv_gateup_launch(L, x, T, b, max_slots, h, stream);
  }
  if (e == hipSuccess)
    e = moe::launch_gemv_down_combine(L, h, T, topk_idx, b->asg_pos, topk_w, residual, out,
                                      stream);
  return hip_status(W, e);
}

moe_status moe_expert_hist(const moe_layer_desc* L, const moe_buckets* b, uint32_t* hist,
                           int32_t decay_shift, int32_t unit_shift, hipStream_t stream) {
  const char* W = "moe_expert_hist";
  moe_status st = check_layer(L, W);
  if (st != MOE_OK) return st;
  CHECK_PTR(b, W);
  if (b->E != L->E) return fail(MOE_ERR_INVALID_ARG, "%s: buckets carved for E=%d", W, b->E);
  CHECK_PTR(b->counts, W);
  CHECK_PTR(hist, W);
  if (decay_shift < 0 || decay_shift > 31 || unit_shift < 0 || unit_shift > 31)
    return fail(MOE_ERR_INVALID_ARG, "%s: shifts (%d, %d) must be in [0, 31]", W, decay_shift,
                unit_shift);
  return hip_status(W, moe::launch_hist(b->counts, L->E, hist, decay_shift, unit_shift, stream));
}

}  // extern "C"
