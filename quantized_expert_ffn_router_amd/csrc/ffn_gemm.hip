// ffn_gemm.hip -- expert FFNs for prefill-sized batches: grouped GEMM on
// MFMA with the block-quantized weights dequantized into LDS.
//
// With thousands of tokens the routed experts (NVFP4; Q6_K in the DQ6_K
// packs: basalt.jgulfo.com, "Models" and "Quick start") are a real dense
// contraction per expert: the m_e tokens routed to expert e (rows of x in
// bucket order) times the expert's weights.  One launch covers all experts:
//   - tiles: (expert, 128 token rows) x (128 output columns); the tile list is
//     built on the device from the bucket counts (no host round trip), and the
//     grid is sized for the worst case -- workgroups past the list exit;
//   - tile order is XCD-aware: consecutive workgroup ids go to different XCDs
//     (8), so logical tiles are laid out XCD-major and the column tiles of one
//     token block share that XCD's L2 for the re-read token rows;
//   - per K step of 128: the A tile (gathered bf16 token rows, or the bf16 h
//     rows of the down projection) is copied to LDS; each wave reads its B
//     fragments from the packed weight blob (one 16-byte granule per lane and
//     column tile, see "B fragments") and dequantizes them in registers,
//     exactly to bf16 (E2M1 x E4M3 has at most 6 significant bits; Q6_K
//     d*sc*(q-32) has up to 24 and is rounded to bf16 -- see the design
//     notes); the next K step's global data is loaded into registers while
//     the MFMAs of this one run;
//   - 4 waves, each a 64 x 64 sub-tile = 4 x 4 v_mfma_f32_16x16x32_bf16 tiles
//     with fp32 accumulation;
//   - gate/up: the 128 B columns are 64 gate rows and the same 64 up rows of
//     the weights, so each lane holds matching g and u values and the SwiGLU
//     epilogue h = silu(g*ts_g) * (u*ts_u) runs in registers; h is stored as
//     bf16.  Down: y = acc * ts_d in bf16 or fp32.
#include <type_traits>

#include "gemv_common.h"

namespace moe {

namespace {

typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));
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
  if (e == 1023) *n_tiles = pre[1023];
}

// Logical tile of this workgroup with an XCD-major layout of the grid.
__device__ __forceinline__ int logical_tile(int total) {
  const int w = blockIdx.x;
  const int per = total / 8;  // total is a multiple of 8
  return (w & 7) * per + (w >> 3);
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
#else
__device__ uint4 gl16(const uint8_t* p);
__device__ uint2 gl8(const uint8_t* p);
__device__ uint32_t gl2(const uint8_t* p);
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

// Sub-step s: 8 exact bf16 values (E2M1 x E4M3 has at most 6 significant bits).
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

struct FragQ6k {
  uint4 lo;     // 32 low nibbles: word s = sub-step s
  uint2 hi;     // 32 x 2 high bits: 16 bits per sub-step
  uint32_t sc;  // the two int8 sub-scales of the granule (low 16 bits)
  uint32_t d;   // fp16 superblock scale
};

__device__ __forceinline__ void load_frag_q6k(FragQ6k& f, const uint8_t* ql, const uint8_t* qh,
                                              const uint8_t* sc, const uint8_t* dd, int N, int n,
                                              int step) {
  const int grp = (threadIdx.x & 63) >> 4;
  const int c = 4 * step + grp, sb = c >> 3;
  f.lo = gl16(ql + ((size_t)c * N + n) * 16);
  f.hi = gl8(qh + ((size_t)(c >> 1) * N + n) * 16 + 8 * (c & 1));
  f.sc = gl2(sc + ((size_t)sb * N + n) * 16 + 2 * (c & 7));
  f.d = gl2(dd + ((size_t)sb * N + n) * 2);
}

template <int S>
__device__ __forceinline__ v8bf_t dequant_frag_q6k(const FragQ6k& f) {
  const float s = f16_to_f32((uint16_t)f.d) * (float)(int8_t)((f.sc >> (8 * (S >> 1))) & 0xffu);
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

// ---------------------------------------------------------------- main loop
// WG = 8 waves; tile = 128 rows x 8*NC*16 columns; wave w owns all 128 rows
// and column tiles cols(w, j), j < NC (NC = 2: 64 accumulators per lane, so
// four waves fit per SIMD and hide each other's LDS and barrier waits).  K
// runs in steps of 128.
//   - A (bf16 rows) lives in LDS as 256-byte rows whose 16-byte chunks are
//     XOR-swizzled (chunk c of row r at position c ^ (r & 15)), so the
//     fragment reads (16 rows, one chunk) hit distinct banks.  The load unit
//     copies it global -> LDS itself (global_load_lds_dwordx4: lane i of a
//     wave writes LDS slot i, so lane i fetches the chunk that belongs in
//     slot i); two buffers, loads one step ahead, and before the barrier the
//     wave waits until only the step's weight loads are still in flight.
//   - B fragments go global -> registers, one step ahead, and are
//     dequantized right before their MFMAs.
constexpr int GBM = 128, GBK = 128;
constexpr int ARB = GBK;  // bf16 per LDS row (no padding: swizzled)

__device__ __forceinline__ int aswz(int r, int c) { return r * ARB + 8 * (c ^ (r & 15)); }

// GU: column tiles j < NC/2 read planes (p0, p1) and the rest (p2, p3) --
// the gate and up matrices of one expert; otherwise (p0..p3) are the planes of
// one matrix (NVFP4 codes, scales; Q6_K ql, qh, sc, d).
struct ARows {
  const uint16_t* base;  // x or h
  uint32_t off[4];       // element offsets of rows 16w + 4k + lane/16 (k < 4, w < 8)
};

// s_waitcnt vmcnt(n) (gfx9 encoding; expcnt and lgkmcnt not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int FMT, int NC, bool GU, typename ColFn>
__device__ __forceinline__ void gemm_main(const ARows& arow, int K, int N,
                                          const uint8_t* p0, const uint8_t* p1, const uint8_t* p2,
                                          const uint8_t* p3, ColFn col_of, uint16_t* As,
                                          v4f_t (*acc)[NC]) {
  typedef typename std::conditional<FMT == MOE_FMT_NVFP4, FragNvfp4, FragQ6k>::type Frag;
  constexpr int kBLoads = NC * ((FMT == MOE_FMT_NVFP4) ? 2 : 4);  // weight loads per step
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  Frag bnext[NC];

  // Rows 16w + 4k + lane/16, slot lane%16 of row r holds chunk (lane%16) ^ (r & 15).
  auto load_a = [&](int k0, int buf) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 16 * wave + 4 * k + (lane >> 4);
      const int c = (lane & 15) ^ (r & 15);
      const uint16_t* src = arow.base + arow.off[k] + k0 + 8 * c;
      __builtin_amdgcn_global_load_lds(
          (const void*)src,
          (void __attribute__((address_space(3)))*)(As + buf * GBM * ARB + (16 * wave + 4 * k) * ARB),
          16, 0, 0);
    }
  };
  auto load_b = [&](int step) {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int n = col_of(j) + (lane & 15);
      if constexpr (GU) {
        if (j < NC / 2) load_frag(bnext[j], p0, p1, N, n, step);
        else load_frag(bnext[j], p2, p3, N, n, step);
      } else if constexpr (FMT == MOE_FMT_NVFP4) {
        load_frag(bnext[j], p0, p1, N, n, step);
      } else {
        load_frag_q6k(bnext[j], p0, p1, p2, p3, N, n, step);
      }
    }
  };

  load_a(0, 0);
  __builtin_amdgcn_sched_barrier(0);
  load_b(0);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<kBLoads>();  // step 0's rows are in LDS (its weight loads may still fly)
  __syncthreads();
  const int nsteps = K / GBK;
  const int r = lane & 15, cq = 4 * (lane >> 4);
  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    Frag bcur[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) bcur[j] = bnext[j];
    const bool more = st + 1 < nsteps;
    if (more) {
      load_a((st + 1) * GBK, buf ^ 1);  // the buffer step st-1 read
      __builtin_amdgcn_sched_barrier(0);
      load_b(st + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    const uint16_t* Ab = As + buf * GBM * ARB;
    auto sub = [&](auto S_) {
      constexpr int S = decltype(S_)::value;
      v8bf_t bf[NC];
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        if constexpr (FMT == MOE_FMT_NVFP4) bf[j] = dequant_frag<S>(bcur[j]);
        else bf[j] = dequant_frag_q6k<S>(bcur[j]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const v8bf_t af = *reinterpret_cast<const v8bf_t*>(Ab + aswz(16 * i + r, cq + S));
#pragma unroll
        for (int j = 0; j < NC; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[j], acc[i][j], 0, 0, 0);
      }
    };
    sub(std::integral_constant<int, 0>{});
    sub(std::integral_constant<int, 1>{});
    sub(std::integral_constant<int, 2>{});
    sub(std::integral_constant<int, 3>{});
    __builtin_amdgcn_sched_barrier(0);
    if (more) wait_vmcnt<kBLoads>();  // step st+1's rows are in LDS
    __syncthreads();
  }
}

// ------------------------------------------------------------------ gate/up
// Tile columns: 128 consecutive rows n0.. of gate and the same rows of up;
// wave w takes gate columns n0 + 32w .. +32 (tiles j = 0, 1) and the matching
// up columns (tiles j = 2, 3).

__global__ __launch_bounds__(kThreads, 2) void k_gemm_gateup_nvfp4(
    const uint16_t* __restrict__ x, int H, int I, int ktop,
    const moe_expert_ref* __restrict__ experts, size_t off_gq, size_t off_gs, size_t off_uq,
    size_t off_us, const int32_t* __restrict__ offsets, const uint32_t* __restrict__ counts,
    const int32_t* __restrict__ sorted_asg, const int2* __restrict__ tiles,
    const int* __restrict__ n_tiles, int grid_tiles, uint16_t* __restrict__ hout) {
  __shared__ __align__(16) uint16_t As[2 * GBM * ARB];
  const int NT = I / 128;
  const int L = logical_tile(grid_tiles);
  const int mtile = L / NT, ntile = L - mtile * NT;
  if (mtile >= *n_tiles) return;
  const int2 te = tiles[mtile];
  const int e = te.x, m0 = te.y;
  const int m_e = (int)counts[e];
  const int base = offsets[e];
  const moe_expert_ref ref = experts[e];
  const uint8_t* blob = (const uint8_t*)ref.blob;
  const int n0 = ntile * 128;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  ARows arow;
  arow.base = x;
#pragma unroll
  for (int k = 0; k < 4; ++k) {  // rows past m_e read a valid row, never stored
    const int row = m0 + 16 * (tid >> 6) + 4 * k + ((tid & 63) >> 4);
    arow.off[k] = (uint32_t)(sorted_asg[base + (row < m_e ? row : 0)] / ktop) * (uint32_t)H;
  }
  v4f_t acc[8][2];  // column tile 0: gate rows cb..; 1: the same rows of up
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int cb = n0 + 16 * wave;
  gemm_main<MOE_FMT_NVFP4, 2, true>(arow, H, I, blob + off_gq, blob + off_gs, blob + off_uq,
                                    blob + off_us, [&](int) { return cb; }, As, acc);

  const float tg = ref.ts_gate, tu = ref.ts_up;
  const int col = cb + (lane & 15);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = m0 + 16 * i + 4 * (lane >> 4) + q;
      if (row < m_e) {
        const float g = acc[i][0][q] * tg, u = acc[i][1][q] * tu;
        hout[(size_t)(base + row) * I + col] = f32_to_bf16_rne(g / (1.0f + expf(-g)) * u);
      }
    }
  }
}

// ------------------------------------------------------------------ down
// Tile columns: 256 consecutive rows of the down weights (output features);
// wave w takes columns n0 + 64w .. +64 (4 tiles).

template <int FMT, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 2) void k_gemm_down(
    const uint16_t* __restrict__ h, int H, int I, const moe_expert_ref* __restrict__ experts,
    size_t off_a, size_t off_b, size_t off_c, size_t off_d, const int32_t* __restrict__ offsets,
    const uint32_t* __restrict__ counts, const int2* __restrict__ tiles,
    const int* __restrict__ n_tiles, int grid_tiles, void* __restrict__ y) {
  __shared__ __align__(16) uint16_t As[2 * GBM * ARB];
  const int NT = H / 256;
  const int L = logical_tile(grid_tiles);
  const int mtile = L / NT, ntile = L - mtile * NT;
  if (mtile >= *n_tiles) return;
  const int2 te = tiles[mtile];
  const int e = te.x, m0 = te.y;
  const int m_e = (int)counts[e];
  const int base = offsets[e];
  const moe_expert_ref ref = experts[e];
  const uint8_t* blob = (const uint8_t*)ref.blob;
  const int n0 = ntile * 256;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  ARows arow;
  arow.base = h;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int row = m0 + 16 * (tid >> 6) + 4 * k + ((tid & 63) >> 4);
    arow.off[k] = (uint32_t)(base + (row < m_e ? row : 0)) * (uint32_t)I;
  }
  v4f_t acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int cb = n0 + 32 * wave;
  gemm_main<FMT, 2, false>(arow, I, H, blob + off_a, blob + off_b, blob + off_c, blob + off_d,
                    [&](int j) { return cb + 16 * j; }, As, acc);

  const float ts = (FMT == MOE_FMT_NVFP4) ? ref.ts_down : 1.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = cb + 16 * j + (lane & 15);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = m0 + 16 * i + 4 * (lane >> 4) + q;
        if (row < m_e) {
          const float v = acc[i][j][q] * ts;
          if (OUT_BF16) reinterpret_cast<uint16_t*>(y)[(size_t)(base + row) * H + col] = f32_to_bf16_rne(v);
          else reinterpret_cast<float*>(y)[(size_t)(base + row) * H + col] = v;
        }
      }
    }
  }
}

}  // namespace

size_t gemm_tiles_bytes(int E, int64_t A) {
  return align_up((size_t)(A / BM + E + 1) * sizeof(int2)) + align_up(sizeof(int));
}

// Grouped-GEMM expert FFN.  ws_h: bf16 [A][I]; ws_tiles: gemm_tiles_bytes().
hipError_t launch_gemm_ffn(const moe_layer_desc* L, const uint16_t* x, int64_t T,
                           const moe_buckets* b, uint16_t* hbuf, void* tiles_ws, void* y,
                           int y_dtype, hipStream_t s) {
  const BlobLayout lay = blob_layout(L->H, L->I, L->fmt_down);
  const int64_t A = T * L->k;
  int2* tiles = (int2*)tiles_ws;
  int* n_tiles = (int*)((char*)tiles_ws + align_up((size_t)(A / BM + L->E + 1) * sizeof(int2)));
  hipLaunchKernelGGL(k_build_tiles, dim3(1), dim3(1024), 0, s, b->counts, L->E, BM, tiles, n_tiles);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int max_mtiles = (int)(A / BM) + L->E;
  {
    const int NT = L->I / 128;
    int total = max_mtiles * NT;
    total = (total + 7) / 8 * 8;
    hipLaunchKernelGGL(k_gemm_gateup_nvfp4, dim3((unsigned)total), dim3(kThreads), 0, s, x, L->H,
                       L->I, L->k, L->experts, lay.gate_q, lay.gate_s, lay.up_q, lay.up_s,
                       b->offsets, b->counts, b->sorted_asg, tiles, n_tiles, total, hbuf);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  {
    const int NT = L->H / 256;
    int total = max_mtiles * NT;
    total = (total + 7) / 8 * 8;
    const bool bf = (y_dtype == MOE_DTYPE_BF16);
    if (L->fmt_down == MOE_FMT_NVFP4) {
      if (bf)
        hipLaunchKernelGGL((k_gemm_down<MOE_FMT_NVFP4, true>), dim3((unsigned)total), dim3(kThreads), 0, s,
                           hbuf, L->H, L->I, L->experts, lay.down_q, lay.down_s, (size_t)0, (size_t)0,
                           b->offsets, b->counts, tiles, n_tiles, total, y);
      else
        hipLaunchKernelGGL((k_gemm_down<MOE_FMT_NVFP4, false>), dim3((unsigned)total), dim3(kThreads), 0, s,
                           hbuf, L->H, L->I, L->experts, lay.down_q, lay.down_s, (size_t)0, (size_t)0,
                           b->offsets, b->counts, tiles, n_tiles, total, y);
    } else {
      if (bf)
        hipLaunchKernelGGL((k_gemm_down<MOE_FMT_Q6K, true>), dim3((unsigned)total), dim3(kThreads), 0, s,
                           hbuf, L->H, L->I, L->experts, lay.down_ql, lay.down_qh, lay.down_sc,
                           lay.down_d, b->offsets, b->counts, tiles, n_tiles, total, y);
      else
        hipLaunchKernelGGL((k_gemm_down<MOE_FMT_Q6K, false>), dim3((unsigned)total), dim3(kThreads), 0, s,
                           hbuf, L->H, L->I, L->experts, lay.down_ql, lay.down_qh, lay.down_sc,
                           lay.down_d, b->offsets, b->counts, tiles, n_tiles, total, y);
    }
    err = hipGetLastError();
  }
  return err;
}

}  // namespace moe
