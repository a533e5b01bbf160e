// tier.hip -- optional cold-expert tier: experts that do not fit the HBM
// budget stay in pinned host RAM and are copied in on demand; the most-used
// experts of each layer keep resident slots (see the moe_tier_* declarations
// for the contract and the pages it follows).  Host logic plus one copy
// kernel: a call's expert copies (and the expert table) go host -> HBM in one
// launch on the side stream, the kernel reading the pinned host memory
// directly.  Expert-sized pieces moved that way reach the pinned-copy rate
// of large transfers (about 57 GB/s measured), where one runtime copy per
// 2 MB expert reaches about 44 GB/s.  If a host blob is not device-accessible
// the runtime copies are used instead.  The side stream is ordered against
// the compute stream with events.
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <numeric>
#include <vector>

#include "common.h"

namespace moe {
moe_status tier_fail(moe_status st, const char* fmt, ...);
}

struct TierCopy {  // one piece: bytes [0, n16 * 16) of src -> dst
  const uint4* src;
  uint4* dst;
};

struct moe_tier {
  int L = 0, E = 0, R = 0, S = 0;
  size_t eb = 0;
  std::vector<const void*> host_blob;   // [L*E]
  std::vector<moe_expert_ref> scales;   // [L*E]
  uint8_t* pool = nullptr;              // L*R resident slots, then S staging slots
  std::vector<int32_t> slot_of;         // [L*E] resident slot (0..R-1) or -1
  std::vector<int32_t> resident;        // [L*R] expert in slot or -1
  hipStream_t copy = nullptr;
  hipEvent_t ev_active = nullptr, ev_copies = nullptr;
  int32_t* h_active = nullptr;          // pinned [E + 1]: active list, n_active
  moe_expert_ref* h_table = nullptr;    // pinned [E]
  std::vector<uint32_t> h_hist;
  // Copy kernel: device addresses of the host blobs (empty: runtime copies),
  // pinned job list [max(S, R)], its and the table's device addresses.
  std::vector<const void*> dev_blob;
  TierCopy* h_jobs = nullptr;
  const TierCopy* d_jobs = nullptr;
  const moe_expert_ref* d_h_table = nullptr;
  moe_tier_stats st{};
};

namespace {

uint8_t* slot_ptr(moe_tier* t, int layer, int slot) {
  return t->pool + ((size_t)layer * t->R + slot) * t->eb;
}
uint8_t* stage_ptr(moe_tier* t, int s) { return t->pool + ((size_t)t->L * t->R + s) * t->eb; }

moe_status hip_err(const char* where, hipError_t e) {
  return moe::tier_fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr int kCopyWG = 8;  // workgroups per expert piece

// blockIdx.y < n_jobs: a contiguous 1/gridDim.x slice of piece blockIdx.y
// (n16 16-byte chunks; pieces are 256-byte aligned); blockIdx.y == n_jobs:
// the table (t4 32-bit words: a moe_expert_ref array is 8-byte aligned), by
// workgroup 0 of that row.
__global__ __launch_bounds__(256) void k_tier_copy(const TierCopy* __restrict__ jobs, int n_jobs,
                                                   size_t n16, const uint32_t* __restrict__ tsrc,
                                                   uint32_t* __restrict__ tdst, int t4) {
  if ((int)blockIdx.y == n_jobs) {
    if (blockIdx.x == 0)
      for (int i = threadIdx.x; i < t4; i += 256) tdst[i] = tsrc[i];
    return;
  }
  const TierCopy j = jobs[blockIdx.y];
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b = (size_t)blockIdx.x * per;
  const size_t e = b + per < n16 ? b + per : n16;
  for (size_t i = b + threadIdx.x; i < e; i += 256) j.dst[i] = j.src[i];
}

// The n jobs in h_jobs (and, with table_dev, the table) host -> HBM on the
// copy stream: one kernel, or runtime copies when the blobs are not
// device-accessible.
hipError_t tier_copies(moe_tier* t, int n, moe_expert_ref* table_dev) {
  if (!t->dev_blob.empty()) {
    if (n == 0 && !table_dev) return hipSuccess;
    hipLaunchKernelGGL(k_tier_copy, dim3(kCopyWG, (unsigned)(n + (table_dev ? 1 : 0))), dim3(256), 0,
                       t->copy, t->d_jobs, n, t->eb / 16, (const uint32_t*)t->d_h_table,
                       (uint32_t*)table_dev, (int)(sizeof(moe_expert_ref) * t->E / 4));
    return hipGetLastError();
  }
  hipError_t e;
  for (int i = 0; i < n; ++i)
    if ((e = hipMemcpyAsync(t->h_jobs[i].dst, t->h_jobs[i].src, t->eb, hipMemcpyHostToDevice,
                            t->copy)) != hipSuccess)
      return e;
  if (table_dev)
    return hipMemcpyAsync(table_dev, t->h_table, sizeof(moe_expert_ref) * t->E,
                          hipMemcpyHostToDevice, t->copy);
  return hipSuccess;
}

}  // namespace

extern "C" {

moe_status moe_tier_create(const moe_tier_desc* d, moe_tier** out) {
  const char* W = "moe_tier_create";
  if (!d || !out) return moe::tier_fail(MOE_ERR_INVALID_ARG, "%s: NULL argument", W);
  *out = nullptr;
  if (d->L < 1 || d->E < 1 || d->E > 1024 || d->resident_per_layer < 0 ||
      d->resident_per_layer > d->E || d->staging_slots < 1 || d->staging_slots > d->E ||
      d->expert_bytes == 0 || d->expert_bytes % moe::kAlign != 0)
    return moe::tier_fail(MOE_ERR_INVALID_ARG, "%s: L=%d E=%d R=%d S=%d expert_bytes=%zu", W,
                          d->L, d->E, d->resident_per_layer, d->staging_slots, d->expert_bytes);
  if (!d->host_blobs || !d->scales || !d->hbm_pool)
    return moe::tier_fail(MOE_ERR_INVALID_ARG, "%s: host_blobs, scales or hbm_pool is NULL", W);
  if ((uintptr_t)d->hbm_pool % moe::kAlign != 0)
    return moe::tier_fail(MOE_ERR_INVALID_ARG, "%s: hbm_pool not 256-byte aligned", W);
  const size_t need = ((size_t)d->L * d->resident_per_layer + d->staging_slots) * d->expert_bytes;
  if (d->hbm_pool_bytes < need)
    return moe::tier_fail(MOE_ERR_BUDGET,
                          "%s: HBM pool of %zu bytes < %zu needed for %d layers x %d resident + "
                          "%d staging experts",
                          W, d->hbm_pool_bytes, need, d->L, d->resident_per_layer, d->staging_slots);
  const size_t n = (size_t)d->L * d->E;
  for (size_t i = 0; i < n; ++i)
    if (!d->host_blobs[i]) return moe::tier_fail(MOE_ERR_INVALID_ARG, "%s: host_blobs[%zu] is NULL", W, i);

  moe_tier* t = new (std::nothrow) moe_tier();
  if (!t) return moe::tier_fail(MOE_ERR_HOST_ALLOC, "%s: out of host memory", W);
  t->L = d->L; t->E = d->E; t->R = d->resident_per_layer; t->S = d->staging_slots;
  t->eb = d->expert_bytes;
  t->host_blob.assign(d->host_blobs, d->host_blobs + n);
  t->scales.assign(d->scales, d->scales + n);
  t->pool = (uint8_t*)d->hbm_pool;
  t->slot_of.assign(n, -1);
  t->resident.assign((size_t)t->L * t->R, -1);
  t->h_hist.resize(t->E);
  t->copy = d->copy_stream;
  hipError_t e;
  const int nj = std::max(t->S, t->R);
  if ((e = hipEventCreateWithFlags(&t->ev_active, hipEventDisableTiming)) != hipSuccess ||
      (e = hipEventCreateWithFlags(&t->ev_copies, hipEventDisableTiming)) != hipSuccess ||
      (e = hipHostMalloc((void**)&t->h_active, sizeof(int32_t) * (t->E + 1), hipHostMallocDefault)) != hipSuccess ||
      (e = hipHostMalloc((void**)&t->h_table, sizeof(moe_expert_ref) * t->E, hipHostMallocDefault)) != hipSuccess ||
      (e = hipHostMalloc((void**)&t->h_jobs, sizeof(TierCopy) * std::max(nj, 1), hipHostMallocDefault)) != hipSuccess) {
    moe_tier_destroy(t);
    return hip_err(W, e);
  }
  // The copy kernel needs every host blob (and the tier's own pinned job list
  // and table) mapped for the device; otherwise the runtime copies are used.
  void *dj = nullptr, *dt = nullptr;
  bool mapped = hipHostGetDevicePointer(&dj, t->h_jobs, 0) == hipSuccess && dj &&
                hipHostGetDevicePointer(&dt, t->h_table, 0) == hipSuccess && dt;
  if (mapped) {
    t->dev_blob.resize(n);
    for (size_t i = 0; i < n && mapped; ++i) {
      hipPointerAttribute_t a;
      mapped = hipPointerGetAttributes(&a, t->host_blob[i]) == hipSuccess &&
               a.type == hipMemoryTypeHost && a.devicePointer != nullptr &&
               (uintptr_t)a.devicePointer % 16 == 0;
      if (mapped) t->dev_blob[i] = a.devicePointer;
    }
  }
  if (!mapped) {
    t->dev_blob.clear();
    (void)hipGetLastError();  // clear a failed query's error state
  }
  t->d_jobs = (const TierCopy*)dj;
  t->d_h_table = (const moe_expert_ref*)dt;
  *out = t;
  return MOE_OK;
}

moe_status moe_tier_prepare(moe_tier* t, int32_t layer, const moe_buckets* b,
                            moe_expert_ref* table_dev, hipStream_t compute) {
  const char* W = "moe_tier_prepare";
  if (!t || !b || !table_dev) return moe::tier_fail(MOE_ERR_INVALID_ARG, "%s: NULL argument", W);
  if (layer < 0 || layer >= t->L) return moe::tier_fail(MOE_ERR_INVALID_ARG, "%s: layer %d", W, layer);
  if (b->E != t->E) return moe::tier_fail(MOE_ERR_INVALID_ARG, "%s: buckets carved for E=%d", W, b->E);
  hipError_t e;
  // 1. the active list of this step -> host (the one synchronization)
  if ((e = hipMemcpyAsync(t->h_active, b->active, sizeof(int32_t) * t->E, hipMemcpyDeviceToHost, compute)) != hipSuccess ||
      (e = hipMemcpyAsync(t->h_active + t->E, b->n_active, sizeof(int32_t), hipMemcpyDeviceToHost, compute)) != hipSuccess ||
      (e = hipEventRecord(t->ev_active, compute)) != hipSuccess ||
      (e = hipEventSynchronize(t->ev_active)) != hipSuccess)
    return hip_err(W, e);
  const int na = t->h_active[t->E];
  if (na < 0 || na > t->E) return moe::tier_fail(MOE_ERR_INVALID_ARG, "%s: corrupt active count %d", W, na);
  // 2. table: resident experts point at their slot; misses get a staging slot
  const size_t base = (size_t)layer * t->E;
  for (int x = 0; x < t->E; ++x) {
    moe_expert_ref r = t->scales[base + x];
    const int sl = t->slot_of[base + x];
    r.blob = sl >= 0 ? slot_ptr(t, layer, sl) : nullptr;
    r.reserved = 0;
    t->h_table[x] = r;
  }
  int used = 0;
  for (int i = 0; i < na; ++i) {
    const int x = t->h_active[i];
    if (x < 0 || x >= t->E) return moe::tier_fail(MOE_ERR_INVALID_ARG, "%s: corrupt active expert %d", W, x);
    if (t->slot_of[base + x] >= 0) { t->st.hits++; continue; }
    if (used >= t->S)
      return moe::tier_fail(MOE_ERR_BUDGET, "%s: %d misses exceed the %d staging slots", W, used + 1, t->S);
    uint8_t* dst = stage_ptr(t, used);
    t->h_jobs[used].src = (const uint4*)(t->dev_blob.empty() ? t->host_blob[base + x] : t->dev_blob[base + x]);
    t->h_jobs[used].dst = (uint4*)dst;
    ++used;
    t->h_table[x].blob = dst;
    t->st.misses++;
    t->st.h2d_bytes += t->eb;
  }
  // 3. the copies and the table; the compute stream waits for all of it
  if ((e = tier_copies(t, used, table_dev)) != hipSuccess ||
      (e = hipEventRecord(t->ev_copies, t->copy)) != hipSuccess ||
      (e = hipStreamWaitEvent(compute, t->ev_copies, 0)) != hipSuccess)
    return hip_err(W, e);
  // The pinned table and job list are rewritten at the next prepare only
  // after that call's event wait, which follows this layer's experts (and
  // hence these copies).
  t->st.prepares++;
  return MOE_OK;
}

moe_status moe_tier_rebalance(moe_tier* t, int32_t layer, const uint32_t* hist_dev,
                              hipStream_t compute) {
  const char* W = "moe_tier_rebalance";
  if (!t || !hist_dev) return moe::tier_fail(MOE_ERR_INVALID_ARG, "%s: NULL argument", W);
  if (layer < 0 || layer >= t->L) return moe::tier_fail(MOE_ERR_INVALID_ARG, "%s: layer %d", W, layer);
  hipError_t e;
  if ((e = hipMemcpyAsync(t->h_hist.data(), hist_dev, sizeof(uint32_t) * t->E, hipMemcpyDeviceToHost, compute)) != hipSuccess ||
      (e = hipStreamSynchronize(compute)) != hipSuccess)
    return hip_err(W, e);
  // The copy stream may still be writing this layer's previous staging; all
  // kernels that read resident slots have finished (compute is synchronized).
  if ((e = hipStreamSynchronize(t->copy)) != hipSuccess) return hip_err(W, e);
  std::vector<int> order(t->E);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int a, int c) {
    return t->h_hist[a] > t->h_hist[c];  // stable: ties keep the lower index first
  });
  const size_t base = (size_t)layer * t->E;
  std::vector<char> want(t->E, 0);
  for (int i = 0; i < t->R; ++i) want[order[i]] = 1;
  int32_t* res = t->resident.data() + (size_t)layer * t->R;
  for (int s = 0; s < t->R; ++s)  // evict residents that fell out of the top R
    if (res[s] >= 0 && !want[res[s]]) { t->slot_of[base + res[s]] = -1; res[s] = -1; }
  int free_slot = 0, njobs = 0;
  for (int i = 0; i < t->R; ++i) {
    const int x = order[i];
    if (t->slot_of[base + x] >= 0) continue;
    while (res[free_slot] >= 0) ++free_slot;
    t->h_jobs[njobs].src = (const uint4*)(t->dev_blob.empty() ? t->host_blob[base + x] : t->dev_blob[base + x]);
    t->h_jobs[njobs].dst = (uint4*)slot_ptr(t, layer, free_slot);
    ++njobs;
    res[free_slot] = x;
    t->slot_of[base + x] = free_slot;
    t->st.promotions++;
    t->st.h2d_bytes += t->eb;
  }
  if ((e = tier_copies(t, njobs, nullptr)) != hipSuccess ||
      (e = hipEventRecord(t->ev_copies, t->copy)) != hipSuccess ||
      (e = hipStreamWaitEvent(compute, t->ev_copies, 0)) != hipSuccess)
    return hip_err(W, e);
  t->st.rebalances++;
  return MOE_OK;
}

moe_status moe_tier_stats_get(const moe_tier* t, moe_tier_stats* out, int32_t layer,
                              int32_t* resident_out) {
  if (!t || !out) return moe::tier_fail(MOE_ERR_INVALID_ARG, "moe_tier_stats_get: NULL argument");
  *out = t->st;
  if (resident_out) {
    if (layer < 0 || layer >= t->L)
      return moe::tier_fail(MOE_ERR_INVALID_ARG, "moe_tier_stats_get: layer %d", layer);
    memcpy(resident_out, t->resident.data() + (size_t)layer * t->R, sizeof(int32_t) * t->R);
  }
  return MOE_OK;
}

void moe_tier_destroy(moe_tier* t) {
  if (!t) return;
  if (t->ev_active) (void)hipEventDestroy(t->ev_active);
  if (t->ev_copies) (void)hipEventDestroy(t->ev_copies);
  if (t->h_active) (void)hipHostFree(t->h_active);
  if (t->h_table) (void)hipHostFree(t->h_table);
  if (t->h_jobs) (void)hipHostFree(t->h_jobs);
  delete t;
}

}  // extern "C"
