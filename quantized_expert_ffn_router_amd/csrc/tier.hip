// tier.hip -- optional cold-expert tier: experts that do not fit the HBM
// budget stay in pinned host RAM and are copied in on demand; the most-used
// experts of each layer keep resident slots (see the moe_tier_* declarations
// for the contract and the pages it follows).  Host code only: HIP runtime
// copies on a side stream ordered against the compute stream with events.
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <numeric>
#include <vector>

#include "common.h"

namespace moe {
moe_status tier_fail(moe_status st, const char* fmt, ...);
}

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
  if ((e = hipEventCreateWithFlags(&t->ev_active, hipEventDisableTiming)) != hipSuccess ||
      (e = hipEventCreateWithFlags(&t->ev_copies, hipEventDisableTiming)) != hipSuccess ||
      (e = hipHostMalloc((void**)&t->h_active, sizeof(int32_t) * (t->E + 1), hipHostMallocDefault)) != hipSuccess ||
      (e = hipHostMalloc((void**)&t->h_table, sizeof(moe_expert_ref) * t->E, hipHostMallocDefault)) != hipSuccess) {
    moe_tier_destroy(t);
    return hip_err(W, e);
  }
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
    uint8_t* dst = stage_ptr(t, used++);
    if ((e = hipMemcpyAsync(dst, t->host_blob[base + x], t->eb, hipMemcpyHostToDevice, t->copy)) != hipSuccess)
      return hip_err(W, e);
    t->h_table[x].blob = dst;
    t->st.misses++;
    t->st.h2d_bytes += t->eb;
  }
  // 3. the table after the copies; the compute stream waits for all of it
  if ((e = hipMemcpyAsync(table_dev, t->h_table, sizeof(moe_expert_ref) * t->E, hipMemcpyHostToDevice, t->copy)) != hipSuccess ||
      (e = hipEventRecord(t->ev_copies, t->copy)) != hipSuccess ||
      (e = hipStreamWaitEvent(compute, t->ev_copies, 0)) != hipSuccess)
    return hip_err(W, e);
  // The pinned table is rewritten at the next prepare only after that call's
  // event wait, which follows this layer's experts (and hence these copies).
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
  int free_slot = 0;
  for (int i = 0; i < t->R; ++i) {
    const int x = order[i];
    if (t->slot_of[base + x] >= 0) continue;
    while (res[free_slot] >= 0) ++free_slot;
    if ((e = hipMemcpyAsync(slot_ptr(t, layer, free_slot), t->host_blob[base + x], t->eb,
                            hipMemcpyHostToDevice, t->copy)) != hipSuccess)
      return hip_err(W, e);
    res[free_slot] = x;
    t->slot_of[base + x] = free_slot;
    t->st.promotions++;
    t->st.h2d_bytes += t->eb;
  }
  if ((e = hipEventRecord(t->ev_copies, t->copy)) != hipSuccess ||
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
  delete t;
}

}  // extern "C"
