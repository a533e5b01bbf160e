// bucket.hip -- token-to-expert bucketing and the usage histogram.
//
// Bucketing is a stable counting sort of the A = T*k assignments a = t*k + j
// by expert: counts, exclusive offsets, the assignments of each expert in
// ascending a, the inverse permutation and the list of active experts.  The
// order never depends on the timing of atomics: atomics only count, and every
// position is a prefix count (block base + earlier waves + rank among the
// equal-expert lanes of a wavefront, found with ballots).
//
// Large A: three kernels (per-block counts, one-block scan, per-block stable
// scatter).  A <= kChunk: one kernel does all three inside a workgroup.
#include "common.h"

namespace moe {

namespace {

constexpr int kWaves = 16;
constexpr int kPerWave = 256;
constexpr int kChunk = kWaves * kPerWave;  // assignments per block
constexpr int kThreads = kWaves * 64;

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
}

// Lanes of the wavefront holding the same key (valid lanes only).
__device__ __forceinline__ uint64_t match_key(int key, bool valid, int nbits) {
  uint64_t peers = ballot64(valid);
  for (int b = 0; b < nbits; ++b) {
    bool bit = (key >> b) & 1;
    uint64_t m = ballot64(valid && bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

// Block-wide exclusive scan of one value per thread (kThreads threads).
__device__ int block_exclusive_scan(int v, int* sm_waves, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) sm_waves[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int w = (lane < kWaves) ? sm_waves[lane] : 0;
    int wi = w;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int o = __shfl_up(wi, off);
      if (lane >= off) wi += o;
    }
    if (lane < kWaves) sm_waves[lane] = wi - w;
    if (lane == kWaves - 1) sm_waves[kWaves] = wi;
  }
  __syncthreads();
  int res = sm_waves[wave] + incl - v;
  *total = sm_waves[kWaves];
  __syncthreads();
  return res;
}

// Per-wave counts of one block's chunk into cur[w][e] (wave-private rows, no
// atomics: the highest lane of each equal-expert group adds the group size).
__device__ void count_chunk(const int32_t* __restrict__ idx, int64_t a0, int64_t A, int nbits,
                            uint16_t* cur, int E) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint16_t* mycur = cur + wave * E;
  for (int r = 0; r < kPerWave / 64; ++r) {
    int64_t a = a0 + (int64_t)wave * kPerWave + r * 64 + lane;
    bool valid = a < A;
    int e = valid ? idx[a] : 0;
    uint64_t peers = match_key(e, valid, nbits);
    if (valid && (peers >> lane) == 1ull) mycur[e] = (uint16_t)(mycur[e] + __popcll(peers));
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// cur[w][e] (counts) -> exclusive prefix over waves, block-relative.
__device__ void scan_waves(uint16_t* cur, int E) {
  for (int e = threadIdx.x; e < E; e += kThreads) {
    int run = 0;
    for (int w = 0; w < kWaves; ++w) {
      int c = cur[w * E + e];
      cur[w * E + e] = (uint16_t)run;
      run += c;
    }
  }
}

// Stable scatter of one block's chunk: position of assignment a of expert e
// handled by wave w = ebase[e] + cur[w][e] + (rank among earlier lanes with e).
__device__ void scatter_chunk(const int32_t* __restrict__ idx, int64_t a0, int64_t A, int E,
                              int nbits, uint16_t* cur, const int* ebase,
                              int32_t* __restrict__ sorted, int32_t* __restrict__ pos) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint16_t* mycur = cur + wave * E;
  for (int r = 0; r < kPerWave / 64; ++r) {
    int64_t a = a0 + (int64_t)wave * kPerWave + r * 64 + lane;
    bool valid = a < A;
    int e = valid ? idx[a] : 0;
    uint64_t peers = match_key(e, valid, nbits);
    int rank = __popcll(peers & lanemask_lt());
    int rel = valid ? (int)mycur[e] : 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (valid && (peers >> lane) == 1ull) mycur[e] = (uint16_t)(rel + __popcll(peers));
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (valid) {
      int p = ebase[e] + rel + rank;
      sorted[p] = (int32_t)a;
      pos[a] = p;
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_bucket_count(const int32_t* __restrict__ idx,
                                                           int64_t A, int E,
                                                           uint32_t* __restrict__ blockcnt) {
  __shared__ uint32_t c[1024];
  for (int e = threadIdx.x; e < E; e += kThreads) c[e] = 0;
  __syncthreads();
  int64_t a0 = (int64_t)blockIdx.x * kChunk;
  int64_t a1 = min(A, a0 + kChunk);
  for (int64_t a = a0 + threadIdx.x; a < a1; a += kThreads) atomicAdd(&c[idx[a]], 1u);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) blockcnt[(size_t)blockIdx.x * E + e] = c[e];
}

// Totals per expert, offsets, active list and per-block bases.
__global__ __launch_bounds__(kThreads) void k_bucket_scan(const uint32_t* __restrict__ blockcnt,
                                                          int nb, int E,
                                                          uint32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ active,
                                                          int32_t* __restrict__ n_active,
                                                          int32_t* __restrict__ base) {
  __shared__ int sm[kWaves + 1];
  const int e = threadIdx.x;
  // Both passes over the blocks are unrolled so that 8 loads are in flight
  // per round trip.
  int tot = 0;
  if (e < E) {
#pragma unroll 8
    for (int b = 0; b < nb; ++b) tot += (int)blockcnt[(size_t)b * E + e];
  }
  int total, nact;
  int off = block_exclusive_scan(tot, sm, &total);
  int apos = block_exclusive_scan((e < E && tot > 0) ? 1 : 0, sm, &nact);
  if (e < E) {
    counts[e] = (uint32_t)tot;
    offsets[e] = off;
    if (tot > 0) active[apos] = e;
    int run = off;
#pragma unroll 8
    for (int b = 0; b < nb; ++b) {
      base[(size_t)b * E + e] = run;
      run += (int)blockcnt[(size_t)b * E + e];
    }
  }
  if (e == 0) {
    offsets[E] = total;
    *n_active = nact;
  }
}

__global__ __launch_bounds__(kThreads) void k_bucket_scatter(const int32_t* __restrict__ idx,
                                                             int64_t A, int E, int nbits,
                                                             const int32_t* __restrict__ base,
                                                             int32_t* __restrict__ sorted,
                                                             int32_t* __restrict__ pos) {
  __shared__ uint16_t cur[kWaves * 1024];
  __shared__ int ebase[1024];
  for (int i = threadIdx.x; i < kWaves * E; i += kThreads) cur[i] = 0;
  for (int e = threadIdx.x; e < E; e += kThreads) ebase[e] = base[(size_t)blockIdx.x * E + e];
  __syncthreads();
  const int64_t a0 = (int64_t)blockIdx.x * kChunk;
  count_chunk(idx, a0, A, nbits, cur, E);
  __syncthreads();
  scan_waves(cur, E);
  __syncthreads();
  scatter_chunk(idx, a0, A, E, nbits, cur, ebase, sorted, pos);
}

// A <= kChunk: everything in one workgroup.
__global__ __launch_bounds__(kThreads) void k_bucket_single(const int32_t* __restrict__ idx,
                                                            int64_t A, int E, int nbits,
                                                            uint32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ active,
                                                            int32_t* __restrict__ n_active,
                                                            int32_t* __restrict__ sorted,
                                                            int32_t* __restrict__ pos) {
  __shared__ uint16_t cur[kWaves * 1024];
  __shared__ int ebase[1024];
  __shared__ int sm[kWaves + 1];
  for (int i = threadIdx.x; i < kWaves * E; i += kThreads) cur[i] = 0;
  __syncthreads();
  count_chunk(idx, 0, A, nbits, cur, E);
  __syncthreads();
  const int e = threadIdx.x;
  int tot = 0;
  if (e < E)
    for (int w = 0; w < kWaves; ++w) tot += cur[w * E + e];
  int total, nact;
  int off = block_exclusive_scan(tot, sm, &total);
  int apos = block_exclusive_scan((e < E && tot > 0) ? 1 : 0, sm, &nact);
  if (e < E) {
    counts[e] = (uint32_t)tot;
    offsets[e] = off;
    ebase[e] = off;
    if (tot > 0) active[apos] = e;
  }
  if (e == 0) {
    offsets[E] = total;
    *n_active = nact;
  }
  __syncthreads();
  scan_waves(cur, E);
  __syncthreads();
  scatter_chunk(idx, 0, A, E, nbits, cur, ebase, sorted, pos);
}

// A <= 64 * kWaveRounds: one wavefront does everything (decode-size steps).
constexpr int kWaveRounds = 4;

__global__ __launch_bounds__(64) void k_bucket_wave(const int32_t* __restrict__ idx, int A,
                                                    int E, int nbits,
                                                    uint32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ active,
                                                    int32_t* __restrict__ n_active,
                                                    int32_t* __restrict__ sorted,
                                                    int32_t* __restrict__ pos) {
  __shared__ int cnt[1024];
  __shared__ int cur[1024];
  const int lane = threadIdx.x;
  int key[kWaveRounds];
#pragma unroll
  for (int r = 0; r < kWaveRounds; ++r) {
    const int a = r * 64 + lane;
    key[r] = (a < A) ? idx[a] : 0;
  }
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint64_t peers[kWaveRounds];
#pragma unroll
  for (int r = 0; r < kWaveRounds; ++r) {
    const bool valid = r * 64 + lane < A;
    peers[r] = match_key(key[r], valid, nbits);
    if (valid && (peers[r] >> lane) == 1ull) cnt[key[r]] += __popcll(peers[r]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  // Exclusive scans over experts: lane owns experts [lane*per, lane*per+per).
  const int per = (E + 63) / 64;
  const int e0 = lane * per;
  int s_cnt = 0, s_act = 0;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < E) { s_cnt += cnt[e]; s_act += cnt[e] > 0; }
  }
  int inc_cnt = s_cnt, inc_act = s_act;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int oc = __shfl_up(inc_cnt, off), oa = __shfl_up(inc_act, off);
    if (lane >= off) { inc_cnt += oc; inc_act += oa; }
  }
  int run = inc_cnt - s_cnt, arun = inc_act - s_act;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < E) {
      const int c = cnt[e];
      counts[e] = (uint32_t)c;
      offsets[e] = run;
      cur[e] = run;
      if (c > 0) active[arun++] = e;
      run += c;
    }
  }
  if (lane == 63) { offsets[E] = inc_cnt; *n_active = inc_act; }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int r = 0; r < kWaveRounds; ++r) {
    const int a = r * 64 + lane;
    const bool valid = a < A;
    const int rank = __popcll(peers[r] & lanemask_lt());
    const int base = valid ? cur[key[r]] : 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (valid && (peers[r] >> lane) == 1ull) cur[key[r]] = base + __popcll(peers[r]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (valid) {
      sorted[base + rank] = a;
      pos[a] = base + rank;
    }
  }
}

__global__ void k_hist(const uint32_t* __restrict__ counts, int E, uint32_t* __restrict__ hist,
                       int ds, int us) {
  int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < E) {
    uint32_t h = hist[e];
    hist[e] = h - (h >> ds) + (counts[e] << us);
  }
}

int key_bits(int E) {
  int b = 0;
  while ((1 << b) < E) ++b;
  return b;
}

}  // namespace

size_t bucket_ws_bytes(int E, int64_t A) {
  int64_t nb = (A + kChunk - 1) / kChunk;
  if (nb <= 1) return 0;
  return align_up((size_t)nb * E * sizeof(uint32_t)) * 2;
}

hipError_t launch_bucket(const int32_t* idx, int64_t A, int E, const moe_buckets* b, void* ws,
                         hipStream_t s) {
  const int nbits = key_bits(E);
  int64_t nb = (A + kChunk - 1) / kChunk;
  if (A <= 64 * kWaveRounds) {
    hipLaunchKernelGGL(k_bucket_wave, dim3(1), dim3(64), 0, s, idx, (int)A, E, nbits, b->counts,
                       b->offsets, b->active, b->n_active, b->sorted_asg, b->asg_pos);
    return hipGetLastError();
  }
  if (nb <= 1) {
    hipLaunchKernelGGL(k_bucket_single, dim3(1), dim3(kThreads), 0, s, idx, A, E, nbits,
                       b->counts, b->offsets, b->active, b->n_active, b->sorted_asg, b->asg_pos);
    return hipGetLastError();
  }
  uint32_t* blockcnt = (uint32_t*)ws;
  int32_t* base = (int32_t*)((char*)ws + align_up((size_t)nb * E * sizeof(uint32_t)));
  hipLaunchKernelGGL(k_bucket_count, dim3((unsigned)nb), dim3(kThreads), 0, s, idx, A, E,
                     blockcnt);
  hipLaunchKernelGGL(k_bucket_scan, dim3(1), dim3(kThreads), 0, s, blockcnt, (int)nb, E,
                     b->counts, b->offsets, b->active, b->n_active, base);
  hipLaunchKernelGGL(k_bucket_scatter, dim3((unsigned)nb), dim3(kThreads), 0, s, idx, A, E,
                     nbits, base, b->sorted_asg, b->asg_pos);
  return hipGetLastError();
}

hipError_t launch_hist(const uint32_t* counts, int E, uint32_t* hist, int ds, int us,
                       hipStream_t s) {
  hipLaunchKernelGGL(k_hist, dim3((E + 255) / 256), dim3(256), 0, s, counts, E, hist, ds, us);
  return hipGetLastError();
}

}  // namespace moe
