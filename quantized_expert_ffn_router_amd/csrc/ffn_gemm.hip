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
#include "gemv_common.h"

namespace moe {

namespace {

typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

constexpr int BM = 128;       // token rows per tile
constexpr int BN = 128;       // output columns per tile (gate/up: 64 + 64)
constexpr int BK = 64;        // K per step
constexpr int LDA = BK + 8;   // padded LDS row (bf16 elements)
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

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, to_v2bf(a, b));
}

// 32 NVFP4 elements (one 16-byte code granule) with their two E4M3 scales ->
// 16 packed bf16 pairs (exact).
__device__ __forceinline__ void dequant32_nvfp4(const uint4& c, uint32_t s2, uint32_t* o) {
  const v2f_t sp = e4m3x2<false>(s2);
  const float s0 = sp.x, s1 = sp.y;
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float f[8];
    e2m1x8_f32(w[q], f);
    const float s = (q < 2) ? s0 : s1;
#pragma unroll
    for (int p = 0; p < 4; ++p) o[4 * q + p] = pack_bf16x2(f[2 * p] * s, f[2 * p + 1] * s);
  }
}

// 32 Q6_K elements: low nibbles (16 bytes), high bits (8 bytes), the two
// int8 sub-scales and d -> 16 packed bf16 pairs (d*sc*(q-32) rounded to bf16).
__device__ __forceinline__ void dequant32_q6k(const uint4& ql, const uint2& qh, uint32_t sc2,
                                              float d, uint32_t* o) {
  const float s0 = d * (float)(int8_t)(sc2 & 0xffu);
  const float s1 = d * (float)(int8_t)((sc2 >> 8) & 0xffu);
  const uint32_t lw[4] = {ql.x, ql.y, ql.z, ql.w};
  const uint32_t hw[2] = {qh.x, qh.y};
#pragma unroll
  for (int p = 0; p < 16; ++p) {  // elements 2p, 2p+1
    const uint32_t byte = (lw[p >> 2] >> (8 * (p & 3))) & 0xffu;
    const uint32_t hb = (hw[p >> 3] >> (4 * (p & 7))) & 0xfu;
    const int q0 = (int)((byte & 15u) | ((hb & 3u) << 4));
    const int q1 = (int)((byte >> 4) | ((hb >> 2) << 4));
    const float s = (p < 8) ? s0 : s1;
    o[p] = pack_bf16x2((float)(q0 - 32) * s, (float)(q1 - 32) * s);
  }
}

// Logical tile of this workgroup with an XCD-major layout of the grid.
__device__ __forceinline__ int logical_tile(int total) {
  const int w = blockIdx.x;
  const int per = total / 8;  // total is a multiple of 8
  return (w & 7) * per + (w >> 3);
}

// MFMA over one K step of LDS tiles for this wave's 64 x 64 sub-tile:
// A rows [a0, a0+64), B rows b_rows[0..3] (16 each).
__device__ __forceinline__ void mma_step(const uint16_t* As, const uint16_t* Bs, int a0,
                                         const int* b0, v4f_t (*acc)[4]) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, kq = (lane >> 4) * 8;
#pragma unroll
  for (int kk = 0; kk < BK; kk += 32) {
    v8bf_t af[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      af[i] = *reinterpret_cast<const v8bf_t*>(As + (a0 + 16 * i + r) * LDA + kk + kq);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bf[j] = *reinterpret_cast<const v8bf_t*>(Bs + (b0[j] + r) * LDA + kk + kq);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
  }
}

// ------------------------------------------------------------------ gate/up

__global__ __launch_bounds__(kThreads, 2) void k_gemm_gateup_nvfp4(
    const uint16_t* __restrict__ x, int H, int I, int ktop,
    const moe_expert_ref* __restrict__ experts, size_t off_gq, size_t off_gs, size_t off_uq,
    size_t off_us, const int32_t* __restrict__ offsets, const uint32_t* __restrict__ counts,
    const int32_t* __restrict__ sorted_asg, const int2* __restrict__ tiles,
    const int* __restrict__ n_tiles, int grid_tiles, uint16_t* __restrict__ hout) {
  __shared__ __align__(16) uint16_t As[BM * LDA];
  __shared__ __align__(16) uint16_t Bs[BN * LDA];
  const int NT = I / 64;  // column tiles (64 gate + 64 up columns each)
  const int L = logical_tile(grid_tiles);
  const int mtile = L / NT, ntile = L - mtile * NT;
  if (mtile >= *n_tiles) return;
  const int2 te = tiles[mtile];
  const int e = te.x, m0 = te.y;
  const int m_e = (int)counts[e];
  const int base = offsets[e];
  const moe_expert_ref ref = experts[e];
  const uint8_t* blob = (const uint8_t*)ref.blob;
  const int n0 = ntile * 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  // A loader: thread -> rows ar + 32*j (j < 4), 16-byte chunk ac of the K step.
  const int ar = tid >> 3, ac = tid & 7;
  const uint16_t* arow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = m0 + ar + 32 * j;
    const int tok = sorted_asg[base + (row < m_e ? row : 0)] / ktop;
    arow[j] = x + (size_t)tok * H;
  }
  // B loader: thread -> B row br (0..63 gate, 64..127 up), 32-element half bh.
  const int br = tid >> 1, bh = tid & 1;
  const int wrow = n0 + (br & 63);
  const uint8_t* bq = blob + (br < 64 ? off_gq : off_uq);
  const uint8_t* bs = blob + (br < 64 ? off_gs : off_us);

  uint4 a_reg[4], b_reg;
  uint32_t s_reg;
  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j)  // rows past m_e read a valid row; their outputs are never stored
      a_reg[j] = *reinterpret_cast<const uint4*>(arow[j] + k0 + 8 * ac);
    const int c = k0 / 32 + bh;  // 32-element code granule
    b_reg = ld16(bq + ((size_t)c * I + wrow) * 16);
    const uint2 sg = ld8(bs + ((size_t)(k0 / 128) * I + wrow) * 8);
    const int sb = ((k0 & 127) / 16) + 2 * bh;  // first of the two 16-blocks
    const uint32_t sw = (sb < 4) ? sg.x : sg.y;
    s_reg = (sw >> (8 * (sb & 3))) & 0xffffu;
  };
  auto lstore = [&]() {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<uint4*>(As + (ar + 32 * j) * LDA + 8 * ac) = a_reg[j];
    uint32_t o[16];
    dequant32_nvfp4(b_reg, s_reg, o);
    uint4* dst = reinterpret_cast<uint4*>(Bs + br * LDA + 32 * bh);
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    dst[2] = make_uint4(o[8], o[9], o[10], o[11]);
    dst[3] = make_uint4(o[12], o[13], o[14], o[15]);
  };

  v4f_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int wm = wave >> 1, wn = wave & 1;
  const int a0 = wm * 64;
  const int b0[4] = {wn * 32, wn * 32 + 16, 64 + wn * 32, 64 + wn * 32 + 16};  // g, g, u, u

  gload(0);
  for (int k0 = 0; k0 < H; k0 += BK) {
    __syncthreads();
    lstore();
    __syncthreads();
    if (k0 + BK < H) gload(k0 + BK);
    mma_step(As, Bs, a0, b0, acc);
  }

  // SwiGLU epilogue: lane holds rows 4*(lane/16)+i, column lane%16 of each tile.
  const float tg = ref.ts_gate, tu = ref.ts_up;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 32 + 16 * j + (lane & 15);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = m0 + a0 + 16 * i + 4 * (lane >> 4) + q;
        if (row < m_e) {
          const float g = acc[i][j][q] * tg, u = acc[i][j + 2][q] * tu;
          hout[(size_t)(base + row) * I + col] = f32_to_bf16_rne(g / (1.0f + expf(-g)) * u);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ down

template <int FMT, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 2) void k_gemm_down(
    const uint16_t* __restrict__ h, int H, int I, const moe_expert_ref* __restrict__ experts,
    size_t off_a, size_t off_b, size_t off_c, size_t off_d, const int32_t* __restrict__ offsets,
    const uint32_t* __restrict__ counts, const int2* __restrict__ tiles,
    const int* __restrict__ n_tiles, int grid_tiles, void* __restrict__ y) {
  __shared__ __align__(16) uint16_t As[BM * LDA];
  __shared__ __align__(16) uint16_t Bs[BN * LDA];
  const int NT = H / BN;
  const int L = logical_tile(grid_tiles);
  const int mtile = L / NT, ntile = L - mtile * NT;
  if (mtile >= *n_tiles) return;
  const int2 te = tiles[mtile];
  const int e = te.x, m0 = te.y;
  const int m_e = (int)counts[e];
  const int base = offsets[e];
  const moe_expert_ref ref = experts[e];
  const uint8_t* blob = (const uint8_t*)ref.blob;
  const int n0 = ntile * BN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  const int ar = tid >> 3, ac = tid & 7;
  const uint16_t* arow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = m0 + ar + 32 * j;
    arow[j] = h + (size_t)(base + (row < m_e ? row : 0)) * I;
  }
  const int br = tid >> 1, bh = tid & 1;
  const int wrow = n0 + br;

  uint4 a_reg[4], b_reg;
  uint2 qh_reg;
  uint32_t s_reg, d_reg;
  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j)  // rows past m_e read a valid row; their outputs are never stored
      a_reg[j] = *reinterpret_cast<const uint4*>(arow[j] + k0 + 8 * ac);
    const int c = k0 / 32 + bh;
    b_reg = ld16(blob + off_a + ((size_t)c * H + wrow) * 16);
    if (FMT == MOE_FMT_NVFP4) {
      const uint2 sg = ld8(blob + off_b + ((size_t)(k0 / 128) * H + wrow) * 8);
      const int sb = ((k0 & 127) / 16) + 2 * bh;
      const uint32_t sw = (sb < 4) ? sg.x : sg.y;
      s_reg = (sw >> (8 * (sb & 3))) & 0xffffu;
    } else {
      // high bits: granule c/2 holds 64 elements; this 32-element chunk is its half c&1
      qh_reg = ld8(blob + off_b + ((size_t)(c >> 1) * H + wrow) * 16 + 8 * (c & 1));
      const int sb = c >> 3;                  // superblock
      const int j0 = (c & 7) * 2;             // first 16-element sub-block of the chunk
      s_reg = (uint32_t)ld2(blob + off_c + ((size_t)sb * H + wrow) * 16 + j0);
      d_reg = ld2(blob + off_d + ((size_t)sb * H + wrow) * 2);
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<uint4*>(As + (ar + 32 * j) * LDA + 8 * ac) = a_reg[j];
    uint32_t o[16];
    if (FMT == MOE_FMT_NVFP4) dequant32_nvfp4(b_reg, s_reg, o);
    else dequant32_q6k(b_reg, qh_reg, s_reg, f16_to_f32((uint16_t)d_reg), o);
    uint4* dst = reinterpret_cast<uint4*>(Bs + br * LDA + 32 * bh);
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    dst[2] = make_uint4(o[8], o[9], o[10], o[11]);
    dst[3] = make_uint4(o[12], o[13], o[14], o[15]);
  };

  v4f_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int wm = wave >> 1, wn = wave & 1;
  const int a0 = wm * 64;
  const int b0[4] = {wn * 64, wn * 64 + 16, wn * 64 + 32, wn * 64 + 48};

  gload(0);
  for (int k0 = 0; k0 < I; k0 += BK) {
    __syncthreads();
    lstore();
    __syncthreads();
    if (k0 + BK < I) gload(k0 + BK);
    mma_step(As, Bs, a0, b0, acc);
  }

  const float ts = (FMT == MOE_FMT_NVFP4) ? ref.ts_down : 1.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 64 + 16 * j + (lane & 15);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = m0 + a0 + 16 * i + 4 * (lane >> 4) + q;
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
    const int NT = L->I / 64;
    int total = max_mtiles * NT;
    total = (total + 7) / 8 * 8;
    hipLaunchKernelGGL(k_gemm_gateup_nvfp4, dim3((unsigned)total), dim3(kThreads), 0, s, x, L->H,
                       L->I, L->k, L->experts, lay.gate_q, lay.gate_s, lay.up_q, lay.up_s,
                       b->offsets, b->counts, b->sorted_asg, tiles, n_tiles, total, hbuf);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  {
    const int NT = L->H / BN;
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
