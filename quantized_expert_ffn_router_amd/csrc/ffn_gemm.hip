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
//   - per K step of 64: the A tile (gathered bf16 token rows, or the bf16 h
//     rows of the down projection) is copied to LDS; the B tile is read from
//     the packed weight blob, dequantized exactly to bf16 (E2M1 x E4M3 has at
//     most 6 significant bits, Q6_K d*sc*(q-32) at most 24 and is rounded to
//     bf16 -- see the design notes) and written to LDS; the next K step's
//     global data is loaded into registers while the MFMAs of this one run;
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
constexpr int kThreads = 256;

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
// Lane l of a wave feeds column n0 + l%16 of a 16-column MFMA tile with the
// 8 K-elements k0 + 8*(l/16) .. +8 of a 32-element K step.  In the packed
// blob those 8 codes are one dword of the row's 16-byte granule, so a
// wave-wide load of 16 granules (256 contiguous bytes) covers the fragment.

struct FragNvfp4 {
  uint32_t code;   // 8 E2M1 codes
  uint32_t scale;  // E4M3 scale byte of this lane's 16-block (low byte)
};

__device__ __forceinline__ void load_frag(FragNvfp4& f, const uint8_t* q, const uint8_t* sc, int N,
                                          int n, int k32) {
  const int lane = threadIdx.x & 63;
  f.code = *(const __attribute__((address_space(1))) uint32_t*)(uintptr_t)(
      q + ((size_t)(k32 >> 5) * N + n) * 16 + 4 * (lane >> 4));
  const int blk = ((k32 & 127) >> 4) + (lane >> 5);  // 16-block within the 128-group
  f.scale = *(const __attribute__((address_space(1))) uint8_t*)(uintptr_t)(
      sc + ((size_t)(k32 >> 7) * N + n) * 8 + blk);
}

__device__ __forceinline__ v8bf_t dequant_frag(const FragNvfp4& f) {
  const float s = e4m3x2<false>(f.scale).x;
  float w[8];
  e2m1x8_f32(f.code, w);
  v8bf_t r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const v2bf_t b = to_v2bf(w[2 * p] * s, w[2 * p + 1] * s);
    r[2 * p] = b[0];
    r[2 * p + 1] = b[1];
  }
  return r;
}

struct FragQ6k {
  uint32_t lo;    // 8 low nibbles
  uint32_t hi;    // 8 x 2 high bits (low 16 bits)
  uint32_t sc;    // int8 sub-scale (low byte)
  uint32_t d;     // fp16 superblock scale
};

__device__ __forceinline__ void load_frag_q6k(FragQ6k& f, const uint8_t* ql, const uint8_t* qh,
                                              const uint8_t* sc, const uint8_t* dd, int N, int n,
                                              int k32) {
  typedef __attribute__((address_space(1))) uint32_t g32;
  typedef __attribute__((address_space(1))) uint16_t g16;
  typedef __attribute__((address_space(1))) uint8_t g8;
  const int lane = threadIdx.x & 63;
  const int c = k32 >> 5, sb = k32 >> 8;
  f.lo = *(const g32*)(uintptr_t)(ql + ((size_t)c * N + n) * 16 + 4 * (lane >> 4));
  f.hi = *(const g16*)(uintptr_t)(qh + ((size_t)(c >> 1) * N + n) * 16 + 8 * (c & 1) + 2 * (lane >> 4));
  f.sc = *(const g8*)(uintptr_t)(sc + ((size_t)sb * N + n) * 16 + 2 * (c & 7) + (lane >> 5));
  f.d = *(const g16*)(uintptr_t)(dd + ((size_t)sb * N + n) * 2);
}

__device__ __forceinline__ v8bf_t dequant_frag_q6k(const FragQ6k& f) {
  const float s = f16_to_f32((uint16_t)f.d) * (float)(int8_t)(f.sc & 0xffu);
  v8bf_t r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t byte = (f.lo >> (8 * p)) & 0xffu;
    const uint32_t hb = (f.hi >> (4 * p)) & 0xfu;
    const int q0 = (int)((byte & 15u) | ((hb & 3u) << 4));
    const int q1 = (int)((byte >> 4) | ((hb >> 2) << 4));
    const v2bf_t b = to_v2bf((float)(q0 - 32) * s, (float)(q1 - 32) * s);
    r[2 * p] = b[0];
    r[2 * p + 1] = b[1];
  }
  return r;
}

// ---------------------------------------------------------------- main loop
// WG = 4 waves; tile = 128 rows x 4*NC*16 columns; wave w owns all 128 rows
// and column tiles cols(w, j), j < NC.  A (bf16 rows) is double-buffered in
// LDS with one barrier per K step of 64; B fragments go global -> registers,
// prefetched one K step ahead and dequantized right before their MFMAs.
constexpr int GBM = 128, GBK = 64, GLDA = GBK + 8;

// GU: column tiles j < NC/2 read planes (p0, p1) and the rest (p2, p3) --
// the gate and up matrices of one expert; otherwise (p0..p3) are the planes of
// one matrix (NVFP4 codes, scales; Q6_K ql, qh, sc, d).
struct ARows {
  const uint16_t* r[4];  // this thread's 4 A rows (passed by value: no scratch)
};

template <int FMT, int NC, bool GU, typename ColFn>
__device__ __forceinline__ void gemm_main(ARows arow, int K, int N,
                                          const uint8_t* p0, const uint8_t* p1, const uint8_t* p2,
                                          const uint8_t* p3, ColFn col_of, uint16_t* As,
                                          v4f_t (*acc)[NC]) {
  typedef typename std::conditional<FMT == MOE_FMT_NVFP4, FragNvfp4, FragQ6k>::type Frag;
  const int tid = threadIdx.x, lane = tid & 63;
  const int ar = tid >> 3, ac = tid & 7;  // A loader: rows ar + 32*j, 16-byte chunk ac
  uint4 a0, a1, a2, a3;  // named (not an array) so they stay in registers
  Frag bnext[2][NC];

  auto load_a = [&](int k0) {
    a0 = *reinterpret_cast<const uint4*>(arow.r[0] + k0 + 8 * ac);
    a1 = *reinterpret_cast<const uint4*>(arow.r[1] + k0 + 8 * ac);
    a2 = *reinterpret_cast<const uint4*>(arow.r[2] + k0 + 8 * ac);
    a3 = *reinterpret_cast<const uint4*>(arow.r[3] + k0 + 8 * ac);
  };
  auto store_a = [&](int buf) {
    uint16_t* d = As + buf * GBM * GLDA + ar * GLDA + 8 * ac;
    *reinterpret_cast<uint4*>(d) = a0;
    *reinterpret_cast<uint4*>(d + 32 * GLDA) = a1;
    *reinterpret_cast<uint4*>(d + 64 * GLDA) = a2;
    *reinterpret_cast<uint4*>(d + 96 * GLDA) = a3;
  };
  auto load_b = [&](int k0) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const int n = col_of(j) + (lane & 15);
        if constexpr (GU) {
          if (j < NC / 2) load_frag(bnext[s][j], p0, p1, N, n, k0 + 32 * s);
          else load_frag(bnext[s][j], p2, p3, N, n, k0 + 32 * s);
        } else if constexpr (FMT == MOE_FMT_NVFP4) {
          load_frag(bnext[s][j], p0, p1, N, n, k0 + 32 * s);
        } else {
          load_frag_q6k(bnext[s][j], p0, p1, p2, p3, N, n, k0 + 32 * s);
        }
      }
  };

  load_a(0);
  load_b(0);
  store_a(0);
  __syncthreads();
  const int nsteps = K / GBK;
  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    // Dequantize this step's B fragments, then prefetch the next step.
    v8bf_t bf[2][NC];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        if constexpr (FMT == MOE_FMT_NVFP4) bf[s][j] = dequant_frag(bnext[s][j]);
        else bf[s][j] = dequant_frag_q6k(bnext[s][j]);
      }
    if (st + 1 < nsteps) {
      load_a((st + 1) * GBK);
      load_b((st + 1) * GBK);
    }
    const uint16_t* Ab = As + buf * GBM * GLDA;
    const int r = lane & 15, kq = (lane >> 4) * 8;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const v8bf_t af = *reinterpret_cast<const v8bf_t*>(Ab + (16 * i + r) * GLDA + 32 * s + kq);
#pragma unroll
        for (int j = 0; j < NC; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[s][j], acc[i][j], 0, 0, 0);
      }
    }
    if (st + 1 < nsteps) store_a(buf ^ 1);
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
  __shared__ __align__(16) uint16_t As[2 * GBM * GLDA];
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
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = m0 + (tid >> 3) + 32 * j;  // rows past m_e read a valid row, never stored
    arow.r[j] = x + (size_t)(sorted_asg[base + (row < m_e ? row : 0)] / ktop) * H;
  }
  v4f_t acc[8][4];  // column tiles 0, 1: gate; 2, 3: the same columns of up
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int cb = n0 + 32 * wave;
  gemm_main<MOE_FMT_NVFP4, 4, true>(arow, H, I, blob + off_gq, blob + off_gs, blob + off_uq,
                                    blob + off_us, [&](int j) { return cb + 16 * (j & 1); }, As,
                                    acc);

  const float tg = ref.ts_gate, tu = ref.ts_up;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = cb + 16 * j + (lane & 15);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = m0 + 16 * i + 4 * (lane >> 4) + q;
        if (row < m_e) {
          const float g = acc[i][j][q] * tg, u = acc[i][j + 2][q] * tu;
          hout[(size_t)(base + row) * I + col] = f32_to_bf16_rne(g / (1.0f + expf(-g)) * u);
        }
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
  __shared__ __align__(16) uint16_t As[2 * GBM * GLDA];
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
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = m0 + (tid >> 3) + 32 * j;
    arow.r[j] = h + (size_t)(base + (row < m_e ? row : 0)) * I;
  }
  v4f_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int cb = n0 + 64 * wave;
  gemm_main<FMT, 4, false>(arow, I, H, blob + off_a, blob + off_b, blob + off_c, blob + off_d,
                    [&](int j) { return cb + 16 * j; }, As, acc);

  const float ts = (FMT == MOE_FMT_NVFP4) ? ref.ts_down : 1.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
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
