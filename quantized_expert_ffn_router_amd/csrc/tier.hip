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
//
// The asynchronous prepare does the same on the device, with no host round
// trip: a planning kernel reads the step's active list and a device copy of
// the layer's base table (resident experts -> their slots), assigns staging
// slots to the misses and writes the table and the copy jobs; the copy kernel
// then runs on the compute stream itself.
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
  // Asynchronous prepare (device memory, allocated at create when the blobs
  // are mapped): base tables [L*E] (blob = resident slot or NULL), blob
  // sources [L*E], job list [S] with its count, and hit/miss counters.
  moe_expert_ref* d_base = nullptr;
  const uint4** d_src = nullptr;
  TierCopy* d_ajobs = nullptr;
  int32_t* d_anjobs = nullptr;
  unsigned long long* d_counts = nullptr;  // [0] hits, [1] misses
  moe_expert_ref* h_row = nullptr;         // pinned [E]: base row staging for rebalance
  uint64_t async_prepares = 0;
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

// Asynchronous prepare, one workgroup: table_dev = the layer's base row, then
// each active expert without a resident slot (in active-list order) gets
// staging slot j, a copy job and its table entry.  Counters: hits, misses.
__global__ __launch_bounds__(1024) void k_tier_plan(
    const moe_expert_ref* __restrict__ base, const uint4* const* __restrict__ src,
    const int32_t* __restrict__ active, const int32_t* __restrict__ n_active, int E,
    uint8_t* __restrict__ staging, size_t eb, moe_expert_ref* __restrict__ table,
    TierCopy* __restrict__ jobs, int32_t* __restrict__ n_jobs,
    unsigned long long* __restrict__ counts) {
  __shared__ int miss_rank[1024];
  const int tid = threadIdx.x;
  const int na = *n_active;
  for (int x = tid; x < E; x += blockDim.x) table[x] = base[x];
  // misses among the first na active entries, ranked by a block-wide scan
  const int x = tid < na ? active[tid] : -1;
  const int miss = (x >= 0 && base[x].blob == nullptr) ? 1 : 0;
  miss_rank[tid] = miss;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
    const int v = tid >= off ? miss_rank[tid - off] : 0;
    __syncthreads();
    miss_rank[tid] += v;
    __syncthreads();
  }
  // (the scan's barriers also order the base-row writes before the patches)
  if (miss) {
    const int j = miss_rank[tid] - 1;
    uint8_t* dst = staging + (size_t)j * eb;
    table[x].blob = dst;
    jobs[j] = TierCopy{src[x], (uint4*)dst};
  }
  if (tid == 0) {
    const int n_miss = miss_rank[1023];
    *n_jobs = n_miss;
    counts[0] += (unsigned long long)(na - n_miss);
    counts[1] += (unsigned long long)n_miss;
  }
}

// Copy kernel of the asynchronous prepare: rows blockIdx.y >= *n_jobs exit.
__global__ __launch_bounds__(256) void k_tier_copy_async(const TierCopy* __restrict__ jobs,
                                                         const int32_t* __restrict__ n_jobs,
                                                         size_t n16) {
  if ((int)blockIdx.y >= *n_jobs) return;
  const TierCopy j = jobs[blockIdx.y];
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b = (size_t)blockIdx.x * per;
  const size_t e = b + per < n16 ? b + per : n16;
  for (size_t i = b + threadIdx.x; i < e; i += 256) j.dst[i] = j.src[i];
}

// The layer's base row: resident experts -> their slot, the others NULL.
void fill_base_row(moe_tier* t, int layer, moe_expert_ref* row) {
  const size_t base = (size_t)layer * t->E;
  for (int x = 0; x < t->E; ++x) {
    moe_expert_ref r = t->scales[base + x];
    const int sl = t->slot_of[base + x];
    r.blob = sl >= 0 ? slot_ptr(t, layer, sl) : nullptr;
    r.reserved = 0;
    row[x] = r;
  }
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
  if (mapped) {  // device state of the asynchronous prepare
    const size_t nb = sizeof(moe_expert_ref) * n;
    std::vector<moe_expert_ref> b0(n);
    for (int l = 0; l < t->L; ++l) fill_base_row(t, l, b0.data() + (size_t)l * t->E);
    if ((e = hipMalloc((void**)&t->d_base, nb)) != hipSuccess ||
        (e = hipMalloc((void**)&t->d_src, sizeof(void*) * n)) != hipSuccess ||
        (e = hipMalloc((void**)&t->d_ajobs, sizeof(TierCopy) * t->S)) != hipSuccess ||
        (e = hipMalloc((void**)&t->d_anjobs, sizeof(int32_t))) != hipSuccess ||
        (e = hipMalloc((void**)&t->d_counts, 2 * sizeof(unsigned long long))) != hipSuccess ||
        (e = hipHostMalloc((void**)&t->h_row, sizeof(moe_expert_ref) * t->E, hipHostMallocDefault)) != hipSuccess ||
        (e = hipMemcpy(t->d_base, b0.data(), nb, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(t->d_src, t->dev_blob.data(), sizeof(void*) * n, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemset(t->d_counts, 0, 2 * sizeof(unsigned long long))) != hipSuccess ||
        (e = hipDeviceSynchronize()) != hipSuccess) {
      moe_tier_destroy(t);
      return hip_err(W, e);
    }
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
  fill_base_row(t, layer, t->h_table);
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

moe_status moe_tier_prepare_async(moe_tier* t, int32_t layer, const moe_buckets* b,
                                  moe_expert_ref* table_dev, hipStream_t compute) {
  const char* W = "moe_tier_prepare_async";
  if (!t || !b || !table_dev) return moe::tier_fail(MOE_ERR_INVALID_ARG, "%s: NULL argument", W);
  if (layer < 0 || layer >= t->L) return moe::tier_fail(MOE_ERR_INVALID_ARG, "%s: layer %d", W, layer);
  if (b->E != t->E) return moe::tier_fail(MOE_ERR_INVALID_ARG, "%s: buckets carved for E=%d", W, b->E);
  if (!t->d_base)
    return moe::tier_fail(MOE_ERR_UNSUPPORTED, "%s: host blobs are not mapped for the device", W);
  const int64_t max_active = std::min<int64_t>(t->E, b->T_max * b->k);
  if (max_active > t->S)
    return moe::tier_fail(MOE_ERR_BUDGET,
                          "%s: %lld possible misses per step (T_max * k) exceed the %d staging slots",
                          W, (long long)max_active, t->S);
  if (max_active == 0) return MOE_OK;
  const size_t base = (size_t)layer * t->E;
  hipLaunchKernelGGL(k_tier_plan, dim3(1), dim3(1024), 0, compute, t->d_base + base,
                     t->d_src + base, b->active, b->n_active, t->E, stage_ptr(t, 0), t->eb,
                     table_dev, t->d_ajobs, t->d_anjobs, t->d_counts);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) {
    hipLaunchKernelGGL(k_tier_copy_async, dim3(kCopyWG, (unsigned)max_active), dim3(256), 0,
                       compute, t->d_ajobs, t->d_anjobs, t->eb / 16);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return hip_err(W, e);
  t->async_prepares++;
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
  if (t->d_base) {  // the asynchronous prepare's copy of this layer's base row
    // h_row is free: the previous rebalance's copy of it finished before
    // this call synchronized the compute stream.
    fill_base_row(t, layer, t->h_row);
    if ((e = hipMemcpyAsync(t->d_base + base, t->h_row, sizeof(moe_expert_ref) * t->E,
                            hipMemcpyHostToDevice, compute)) != hipSuccess)
      return hip_err(W, e);
  }
  t->st.rebalances++;
  return MOE_OK;
}

moe_status moe_tier_stats_get(const moe_tier* t, moe_tier_stats* out, int32_t layer,
                              int32_t* resident_out) {
  if (!t || !out) return moe::tier_fail(MOE_ERR_INVALID_ARG, "moe_tier_stats_get: NULL argument");
  *out = t->st;
  if (t->d_counts && t->async_prepares) {  // counters of the asynchronous prepares
    unsigned long long c[2];
    hipError_t e = hipMemcpy(c, t->d_counts, sizeof(c), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_err("moe_tier_stats_get", e);
    out->hits += c[0];
    out->misses += c[1];
    out->h2d_bytes += c[1] * t->eb;
    out->prepares += t->async_prepares;
  }
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
  if (t->h_row) (void)hipHostFree(t->h_row);
  if (t->d_base) (void)hipFree(t->d_base);
  if (t->d_src) (void)hipFree((void*)t->d_src);
  if (t->d_ajobs) (void)hipFree(t->d_ajobs);
  if (t->d_anjobs) (void)hipFree(t->d_anjobs);
  if (t->d_counts) (void)hipFree(t->d_counts);
  delete t;
}

}  // extern "C"
