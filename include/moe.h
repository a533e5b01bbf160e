/*
 * moe.h -- C ABI of libmoe, a single-GPU (MI355X / gfx950) implementation of
 * the mixture-of-experts layer of a Basalt-style local inference engine:
 * router logits, softmax top-k gating, token-to-expert bucketing, block-
 * quantized (NVFP4, Q6_K-style, Q8_0, IQ3-style) SwiGLU expert FFNs with the dequantization
 * fused into the matmuls, the gate-weighted combine, and the per-step expert
 * usage histogram that decides which experts stay resident.
 *
 * What the pages fix, and where:
 *   - each token uses a few experts chosen from many; the busiest experts stay
 *     in GPU memory and the rest may live in system RAM and be streamed on
 *     demand -- basalt.jgulfo.com, section "Expert tiers"; aiopssre.com
 *     ("What Basalt changes in a Blackwell local inference stack"), section
 *     "Experts can move without becoming free";
 *   - routed experts are NVIDIA NVFP4, packs also carry GGUF Q6_K tensors --
 *     basalt.jgulfo.com, sections "Models", "Quick start" and the engine notes
 *     under "All the numbers";
 *   - 1 to 8 concurrent request slots, so decode batches of 1..8 tokens --
 *     aiopssre.com, section "Concurrency divides context unless you pay for
 *     more cache"; devotd.net (en), section "--parallel slots and KV cache
 *     allocation";
 *   - Q8_0 is the 8-bit GGUF format the pages measure quality against and
 *     keep for Basalt's dense projections -- basalt.jgulfo.com, "All the
 *     numbers" (the quality table and the engine notes); here it is offered
 *     as a down-projection format of the experts;
 *   - community packs run IQ3 GGUF files -- basalt.jgulfo.com, "Community";
 *     their grids are not on the pages, so MOE_FMT_IQ3G keeps the IQ3
 *     structure (grid indices per 4 weights, sign bits, small scales) with a
 *     grid defined here (below), offered as a down-projection format;
 *   - the pages' packs also carry IQ1_M tensors (basalt.jgulfo.com,
 *     "Models"), a codebook format of under two bits per weight whose grid
 *     the pages do not give either, so MOE_FMT_IQ1G keeps that structure
 *     (a ternary grid vector per 8 weights, small scales) with a grid
 *     defined here (below), offered as a down-projection format.
 * The pages give no formula.  The arithmetic below is the plainest reading;
 * each entry point states it.
 *
 * Conventions (all entry points):
 *   - Pointers are DEVICE pointers unless marked "host".  Every buffer is
 *     owned by the caller; the library allocates nothing per call and frees
 *     nothing it was given.
 *   - Calls are asynchronous and ordered on the given stream.  T == 0 returns
 *     MOE_OK without launching anything.
 *   - Arguments are validated on the host before any launch; an invalid or
 *     unsupported argument returns an error status and launches nothing (no
 *     clamping, no truncation).  A failed launch returns MOE_ERR_HIP.  The
 *     message of the last failure on the calling thread is moe_last_error().
 *     Device-side faults surface at the caller's next synchronization.
 *   - Calls on different streams may run concurrently if they write
 *     different buffers.
 *   - bf16 values are passed as uint16_t bit patterns.
 *
 * Supported shapes: 1 <= k <= min(E, 64), E <= 1024, H % 128 == 0,
 * 128 <= H <= 8192, I % 128 == 0 (NVFP4, Q8_0) or I % 256 == 0 (Q6_K, IQ3G, IQ1G),
 * I <= 8192.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 2

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,  /* null pointer, negative size, k > E, ... */
  MOE_ERR_UNSUPPORTED = -2,  /* shape or format outside the supported set */
  MOE_ERR_WORKSPACE = -3,    /* workspace or bucket buffer too small */
  MOE_ERR_BUDGET = -4,       /* tier: HBM budget below the working set */
  MOE_ERR_HIP = -5,          /* a HIP runtime call or launch failed */
  MOE_ERR_HOST_ALLOC = -6    /* tier: host metadata allocation failed */
} moe_status;

/* Weight formats. */
#define MOE_FMT_NVFP4 1  /* E2M1 codes, E4M3 scale per 16 along K, fp32 per-tensor scale */
#define MOE_FMT_Q6K 2    /* 256-element superblocks: 16 x int8 sub-scales, fp16 scale, 6-bit codes */
#define MOE_FMT_Q8_0 3   /* 32-element blocks: fp16 scale, 32 int8 codes (down projection only) */
#define MOE_FMT_IQ3G 4   /* 256-element superblocks: fp16 scale, 4-bit odd multipliers per 32,
                            8-bit grid index per 4, sign bits (down projection only) */
#define MOE_FMT_IQ1G 5   /* 256-element superblocks: fp16 scale, 4-bit odd multipliers per 32,
                            10-bit ternary grid index per 8 (down projection only) */

/* Element types of the expert-output buffer y. */
#define MOE_DTYPE_F32 0
#define MOE_DTYPE_BF16 1

/* Library version of this header (MOE_ABI_VERSION). */
int moe_abi_version(void);

/* Expert-FFN kernel family (moe_layer_desc.ffn_mode, read by each
 * moe_expert_ffn call; there is no process-wide state):
 *   MOE_FFN_AUTO -- dequant-fused GEMV for decode-sized batches, MFMA grouped
 *                   GEMM once experts average >= 16 tokens (default);
 *   MOE_FFN_GEMV / MOE_FFN_GEMM -- force one family (any size; results agree
 *                   within the stated tolerance).  The grouped GEMM needs
 *                   H % 256 == 0, T*H < 2^32 and T*k*I < 2^32; AUTO uses the
 *                   GEMV otherwise, and a forced GEMM call fails with
 *                   MOE_ERR_UNSUPPORTED.
 * Any other value is rejected with MOE_ERR_INVALID_ARG by every call that
 * takes the layer. */
#define MOE_FFN_AUTO 0
#define MOE_FFN_GEMV 1
#define MOE_FFN_GEMM 2

/* Message of the last failing call on this thread ("" if none).  Host
 * string owned by the library, valid until the next failing call. */
const char* moe_last_error(void);

/* ------------------------------------------------------------------------ */
/* Expert weights                                                            */
/* ------------------------------------------------------------------------ */

/*
 * Canonical input layouts (what moe_pack_experts reads):
 *   NVFP4 matrix W[N][K]: codes u8 [N][K/2], element k of row n in nibble
 *     (k & 1) of byte k/2 (even element low); E2M1 code: bit 3 sign, bits 2..1
 *     exponent (bias 1), bit 0 mantissa.  scales u8 [N][K/16]: E4M3 (fn) scale
 *     of elements 16b..16b+15.  One fp32 per-tensor scale ts.
 *     w[n][k] = e2m1(code) * e4m3(scale) * ts.
 *   Q6_K-style matrix W[N][K]: row n is K/256 superblocks of 210 bytes:
 *     ql[128] (low 4 bits of element i: nibble i&1 of byte i/2), qh[64]
 *     (high 2 bits of element i: bits 2*(i&3) of byte i/4), sc int8[16]
 *     (sub-block i/16), d fp16 little-endian[2];
 *     w = d * sc[i/16] * (q - 32), q = low | high << 4 in 0..63.
 *   Q8_0 matrix W[N][K]: row n is K/32 blocks of 34 bytes: d fp16
 *     little-endian[2], then the int8 codes q[32] of elements 32b..32b+31;
 *     w = d * q.
 *   IQ3G matrix W[N][K] (3.19 bits per weight): row n is K/256 superblocks of
 *     102 bytes: d fp16 little-endian[2]; s[4], the 4-bit multiplier s_j of
 *     sub-block j (elements 32j..32j+31) in byte j/2 (low nibble for even j);
 *     idx[64], the grid entry of elements 4g..4g+3; sgn[32], bit i%8 of byte
 *     i/8 set when element i is negative;
 *     w = d * (2 s_j + 1) * grid[idx[i/4]][i%4] * (sgn ? -1 : 1),
 *     grid = the 256 smallest vectors of four positive odd integers <= 15,
 *     ordered by squared norm, then lexicographically (entry 0 = (1,1,1,1);
 *     every magnitude is at most 9).
 *   IQ1G matrix W[N][K] (1.44 bits per weight): row n is K/256 superblocks of
 *     46 bytes: d fp16 little-endian[2]; s[4], the 4-bit multiplier s_j of
 *     sub-block j (elements 32j..32j+31) in byte j/2 (low nibble for even j);
 *     qs[32], the low 8 bits of the grid entry of elements 8g..8g+7; qh[8],
 *     its high 2 bits at bits 2(g%4), 2(g%4)+1 of byte g/4;
 *     w = d * (2 s_j + 1) * grid[idx[i/8]][i%8],
 *     grid = the 1024 vectors of eight values in {-1, 0, +1} with the fewest
 *     nonzero values, ordered by that count, then lexicographically
 *     (-1 < 0 < +1, value 0 the most significant; entry 0 = all zero).
 *   Gate and up are [I][H] (K = H); down is [H][I] (K = I).
 *
 * The GPU kernels read a packed "blob" per expert (a device-friendly
 * re-arrangement of the same bytes, 16-byte granules transposed so that one
 * wavefront load covers consecutive rows).  moe_expert_blob_bytes gives its
 * size; moe_pack_experts writes it.  With Q6_K, Q8_0, IQ3G or IQ1G down weights the blob
 * ends with a 256-byte section holding one int32 computed by the pack from
 * the expert's block scales: the power of two by which the grouped GEMM
 * scales that expert's fp16 down weights (so none can overflow fp16, for any
 * scales; the product is scaled back in fp32).
 */

/* One entry of the device-resident expert table (24 bytes). */
typedef struct moe_expert_ref {
  const void* blob;   /* device pointer to the packed expert (256-byte aligned) */
  float ts_gate;      /* NVFP4 per-tensor scales */
  float ts_up;
  float ts_down;      /* ignored when the down projection is Q6_K, Q8_0, IQ3G or IQ1G */
  uint32_t reserved;  /* 0 (not read by the library) */
} moe_expert_ref;

/* Bytes of one packed expert blob (a multiple of 256); 0 if unsupported. */
size_t moe_expert_blob_bytes(int32_t H, int32_t I, int32_t fmt_gate_up, int32_t fmt_down);

/* Pack E experts from the canonical layouts (device arrays stacked over
 * experts: gate_q [E][I][H/2], gate_s [E][I][H/16], up likewise, down_q
 * [E][H][I/2] and down_s [E][H][I/16] for NVFP4, down_q [E][H][I/256*210]
 * for Q6_K, [E][H][I/32*34] for Q8_0, [E][H][I/256*102] for IQ3G or
 * [E][H][I/256*46] for IQ1G, down_s == NULL for those four) into
 * E blobs at blobs + e * blob_stride.
 * blob_stride >= moe_expert_blob_bytes(...) and a multiple of 256. */
moe_status moe_pack_experts(int32_t E, int32_t H, int32_t I, int32_t fmt_gate_up,
                            int32_t fmt_down, const uint8_t* gate_q, const uint8_t* gate_s,
                            const uint8_t* up_q, const uint8_t* up_s, const uint8_t* down_q,
                            const uint8_t* down_s, void* blobs, size_t blob_stride,
                            hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Layer description and bucket buffers                                      */
/* ------------------------------------------------------------------------ */

/* Host struct holding device pointers; read during each call only. */
typedef struct moe_layer_desc {
  int32_t E;            /* experts */
  int32_t k;            /* experts per token */
  int32_t H;            /* hidden size */
  int32_t I;            /* expert intermediate size */
  int32_t fmt_gate_up;  /* MOE_FMT_NVFP4 */
  int32_t fmt_down;     /* MOE_FMT_NVFP4, MOE_FMT_Q6K, MOE_FMT_Q8_0, MOE_FMT_IQ3G or MOE_FMT_IQ1G */
  int32_t renormalize;  /* 1: softmax renormalised over the selected k; 0: full softmax */
  int32_t ffn_mode;     /* MOE_FFN_AUTO (0), MOE_FFN_GEMV or MOE_FFN_GEMM */
  const moe_expert_ref* experts;  /* device [E] */
  const float* w_router;          /* device fp32 [E][H] */
  const float* router_bias;       /* device fp32 [E], or NULL (no bias) */
} moe_layer_desc;

/* Per-step bucket results (device pointers into one caller buffer). */
typedef struct moe_buckets {
  uint32_t* counts;     /* [E]   assignments per expert */
  int32_t* offsets;     /* [E+1] exclusive prefix sum of counts */
  int32_t* sorted_asg;  /* [T*k] assignments a = t*k + j ordered by (expert, a) */
  int32_t* asg_pos;     /* [T*k] position of assignment a in sorted_asg */
  int32_t* active;      /* [E]   experts with counts > 0, ascending (first n_active) */
  int32_t* n_active;    /* [1] */
  int64_t T_max;        /* capacity in tokens */
  int32_t E;
  int32_t k;
} moe_buckets;

/* Bytes needed for the bucket buffers of (E, T_max, k). */
size_t moe_buckets_bytes(int32_t E, int64_t T_max, int32_t k);

/* Point the fields of *out into the caller's device buffer buf (bytes long,
 * 256-byte aligned).  Host-only bookkeeping: launches nothing. */
moe_status moe_buckets_carve(void* buf, size_t bytes, int32_t E, int64_t T_max, int32_t k,
                             moe_buckets* out);

/* Device workspace bytes for moe_bucket and moe_expert_ffn on up to T_max
 * tokens of layer L (covers both calls; one buffer may serve both). */
size_t moe_workspace_bytes(const moe_layer_desc* L, int64_t T_max);

/* ------------------------------------------------------------------------ */
/* The layer's steps                                                         */
/* ------------------------------------------------------------------------ */

/* Router and top-k gating.  The pages' model routes every token to a small
 * subset of its many experts (basalt.jgulfo.com, "Expert tiers"; aiopssre.com,
 * "Experts can move without becoming free"); how the subset is scored is not
 * given, so this is the plainest reading: a linear router, top-k on its
 * logits, softmax weights.
 *   logits[t][e] = fp32( sum_h x[t][h] * w_router[e][h] + bias[e] ), the sum
 *     taken in double precision in one fixed order -- 64 interleaved partial
 *     sums (partial j adds h = j, j+64, ... ascending), combined pairwise
 *     p[j] += p[j+w] for w = 32, 16, ..., 1, then the bias -- and rounded to
 *     fp32 once, so the logits (and hence the selected experts) are
 *     reproducible bit for bit.
 *   topk_idx[t][0..k) = the k experts first in the order (logit desc, expert
 *     index asc): ties go to the lower index.
 *   topk_w[t][j] = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0) (renormalize=1),
 *     or the full softmax probability of expert idx[t][j] (renormalize=0).
 * x: bf16 [T][H]; logits: fp32 [T][E]; topk_idx: int32 [T][k];
 * topk_w: fp32 [T][k].  All caller-allocated. */
moe_status moe_route(const moe_layer_desc* L, const uint16_t* x, int64_t T, float* logits,
                     int32_t* topk_idx, float* topk_w, hipStream_t stream);

/* Token-to-expert bucketing: a stable counting sort of the T*k assignments by
 * expert (deterministic; no dependence on atomic ordering), so that each
 * selected expert runs once per step over all the tokens that chose it and
 * experts nobody chose are not touched (the sparse selection of
 * basalt.jgulfo.com, "Expert tiers").  Fills every
 * field of *b for this step.  b->T_max >= T, b->E == L->E, b->k == L->k.
 * ws: device workspace of at least moe_workspace_bytes(L, T) bytes. */
moe_status moe_bucket(const moe_layer_desc* L, const int32_t* topk_idx, int64_t T,
                      const moe_buckets* b, void* ws, size_t ws_bytes, hipStream_t stream);

/* Gating step in one call: moe_route, then moe_bucket, then (when hist is
 * not NULL) moe_expert_hist, with the same arguments and the same results
 * bit for bit.  For E <= 256, T <= 64 and T*k <= 256 (decode-sized steps) top-k,
 * bucketing and the histogram update run as one single-workgroup kernel
 * after the router logits, two launches instead of four.
 * hist: uint32 [E] or NULL; shifts as for moe_expert_hist (checked only when
 * hist is not NULL).  ws: as for moe_bucket. */
moe_status moe_route_bucket(const moe_layer_desc* L, const uint16_t* x, int64_t T,
                            float* logits, int32_t* topk_idx, float* topk_w, const moe_buckets* b,
                            void* ws, size_t ws_bytes, uint32_t* hist, int32_t decay_shift,
                            int32_t unit_shift, hipStream_t stream);

/* Expert FFNs with fused dequantization (SwiGLU).  The routed experts are
 * stored block-quantized -- NVFP4 in the pages' packs, with GGUF Q6_K tensors
 * in the DQ6_K packs (basalt.jgulfo.com, "Models" and "Quick start"); the
 * weights are decoded inside the matmuls, never materialised:
 *   for each assignment a of expert e (token t = a / k), at sorted position
 *   p = b->asg_pos[a]:
 *     g = x[t] . dq(Wg_e)^T,  u = x[t] . dq(Wu_e)^T,  h = silu(g) * u,
 *     y[p] = h . dq(Wd_e)^T,  silu(z) = z / (1 + exp(-z)),
 *   accumulated in fp32.  y: [T*k][H] of y_dtype (MOE_DTYPE_F32 or _BF16),
 *   rows in sorted order.  Decode-sized batches run as dequant-fused GEMV;
 *   larger ones as an MFMA grouped GEMM over experts, which multiplies an
 *   fp16 copy of x scaled per token row by a power of two (exact for every
 *   value above 2^-29 of the row's largest magnitude).  h between the two
 *   projections is rounded to 16 bits (bf16 in the GEMV; scaled fp16 in the
 *   GEMM, redone in bf16 if it would overflow).  The GEMM rounds Q6_K and
 *   Q8_0 down weights once to fp16 after scaling each expert's weights by a
 *   power of two fixed at pack time (see the blob), so any scales are in
 *   range; the GEMV decodes them exactly.
 * ws: at least moe_workspace_bytes(L, T) bytes. */
moe_status moe_expert_ffn(const moe_layer_desc* L, const uint16_t* x, int64_t T,
                          const moe_buckets* b, void* y, int32_t y_dtype, void* ws,
                          size_t ws_bytes, hipStream_t stream);

/* moe_expert_ffn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, kernels and results (bit for bit) as moe_expert_ffn,
 * with the workspace taken from a static buffer inside the library instead
 * of a caller argument.  The caller still passes x, the buckets and y.
 *   - The buffer is MOE_NOALLOC_WORKSPACE_BYTES (32 MiB) per GPU, part of the
 *     library's code object: each GPU the library runs on holds it until the
 *     process ends.  Its device address is looked up on the first call made
 *     with that device current; the call itself allocates nothing (no
 *     hipMalloc, no hipFree, no allocating library routine).
 *   - A call whose workspace (moe_workspace_bytes covers it) would exceed the
 *     buffer returns MOE_ERR_WORKSPACE before any launch.  At the decode
 *     layer's shape (E 128, k 8, H 2048, I 768) that is above about 2,000
 *     tokens.
 *   - Every call on one GPU shares that GPU's buffer, which keeps the last
 *     call's contents (nothing in it needs to start at zero): calls that
 *     overlap on one GPU -- on different streams, or from different threads --
 *     race and must not be issued.  Calls on different GPUs do not interact. */
#define MOE_NOALLOC_WORKSPACE_BYTES ((size_t)32 << 20)
moe_status moe_expert_ffn_noalloc(const moe_layer_desc* L, const uint16_t* x, int64_t T,
                                  const moe_buckets* b, void* y, int32_t y_dtype,
                                  hipStream_t stream);

/* moe_route_bucket followed by moe_expert_ffn (the layer's routing and its
 * routed experts: basalt.jgulfo.com, "Expert tiers"), with the same arguments
 * and the same outputs bit for bit (logits, top-k, buckets, histogram, y).  For
 * batches of up to 4 tokens (with E <= 256, the GEMV family, NVFP4 gate/up
 * with H <= 2048) it takes one launch fewer: every
 * workgroup of the gate/up kernel repeats the batch's top-k and bucketing
 * in its own LDS from the router logits and finds its expert there, and one
 * of them writes the gating outputs.  Otherwise it makes the two calls.
 * ws: at least moe_workspace_bytes(L, T) bytes (serves both steps). */
moe_status moe_route_ffn(const moe_layer_desc* L, const uint16_t* x, int64_t T, float* logits,
                         int32_t* topk_idx, float* topk_w, const moe_buckets* b, uint32_t* hist,
                         int32_t decay_shift, int32_t unit_shift, void* y, int32_t y_dtype,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* The whole layer step: moe_route_ffn then moe_combine (same arguments,
 * routing outputs, buckets and histogram bit for bit; out within the bf16
 * rounding of the combine).  For decode batches of 2 to 8 tokens on the
 * GEMV family the down projection and the combine run as one kernel that
 * writes out straight from h: y is then not written (the caller still
 * passes it, for the other sizes), and out sums each token's k gate-weighted
 * expert rows in a fixed order (slots j = w mod 8 for each w, then w
 * ascending) -- the mixture of the experts a token uses (basalt.jgulfo.com,
 * "Expert tiers").  residual: bf16 [T][H] or NULL; out: bf16 [T][H] (may
 * alias residual).  ws: at least moe_workspace_bytes(L, T) bytes. */
moe_status moe_layer_forward(const moe_layer_desc* L, const uint16_t* x, int64_t T,
                             const uint16_t* residual, uint16_t* out, float* logits,
                             int32_t* topk_idx, float* topk_w, const moe_buckets* b,
                             uint32_t* hist, int32_t decay_shift, int32_t unit_shift, void* y,
                             int32_t y_dtype, void* ws, size_t ws_bytes, hipStream_t stream);

/* Gate-weighted combine: each token's output is its selected experts'
 * outputs weighted by the gates (the mixture the pages' model computes from
 * the few experts a token uses: basalt.jgulfo.com, "Expert tiers"), written
 * as a gather so that the result does not depend on scheduling:
 *   out[t] = bf16_rne( residual[t] + sum_{j=0..k-1} topk_w[t][j] * y[asg_pos[t*k+j]] ),
 *   in fp32 with j ascending.  residual: bf16 [T][H] or NULL; out: bf16 [T][H]
 *   (may alias residual). */
moe_status moe_combine(const moe_layer_desc* L, const void* y, int32_t y_dtype,
                       const moe_buckets* b, const float* topk_w, int64_t T,
                       const uint16_t* residual, uint16_t* out, hipStream_t stream);

/* Expert-usage histogram deciding residency: the pages keep the most-routed
 * experts in GPU memory and let the placement follow usage as the
 * conversation changes (basalt.jgulfo.com, "Expert tiers" and the FAQ).  The
 * running count is this reading: an exponentially decaying integer count,
 * unsigned 32-bit arithmetic:
 *   hist[e] = hist[e] - (hist[e] >> decay_shift) + (counts[e] << unit_shift).
 * hist: uint32 [E], read and written.  0 <= decay_shift, unit_shift < 32. */
moe_status moe_expert_hist(const moe_layer_desc* L, const moe_buckets* b, uint32_t* hist,
                           int32_t decay_shift, int32_t unit_shift, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Optional cold-expert tier: pinned host RAM -> HBM slots                   */
/* ------------------------------------------------------------------------ */
/*
 * Experts that do not fit the GPU memory budget stay in system RAM and are
 * copied in when a token routes to them (aiopssre.com, "Experts can move
 * without becoming free"); the most-routed experts are the ones kept in GPU
 * memory, with system RAM as the last tier (basalt.jgulfo.com, "Expert
 * tiers"); the resident set follows the usage histogram, so it moves as usage
 * changes (basalt.jgulfo.com, FAQ).  One GPU only: no peer-GPU tier.
 *
 * Per layer l: R resident slots (experts chosen by moe_tier_rebalance) in the
 * caller's HBM pool, plus S staging slots shared by all layers.  Before the
 * experts of layer l run, moe_tier_prepare copies the step's active list to
 * the host (the one host synchronization per layer), copies every active
 * expert that is not resident from pinned host memory into a staging slot on
 * the copy stream, writes the layer's device expert table (moe_expert_ref [E])
 * and makes the compute stream wait for those copies.  moe_expert_ffn then
 * reads every expert through that table, so a tiered step computes exactly
 * (bit for bit) what the same step computes with every expert resident.
 * Entries of inactive, non-resident experts are set to blob = NULL.
 *
 * Copies: when every host blob is mapped for the device (hipHostMalloc
 * memory is), one kernel on the copy stream moves a call's experts and the
 * table, reading the pinned memory directly (expert-sized pieces then move at
 * the large-transfer rate); otherwise one runtime copy per expert is issued.
 *
 * Ownership: host blobs (pinned, e.g. hipHostMalloc), the HBM pool, the
 * device tables and both streams belong to the caller and must outlive the
 * tier.  The tier owns host metadata, a few pinned bytes for the active
 * list, the table staging and the copy list, two events and the device state
 * of moe_tier_prepare_async (allocated at create, freed by destroy).  A tier
 * is not thread-safe.
 */
typedef struct moe_tier_desc {
  int32_t L;                      /* layers */
  int32_t E;                      /* experts per layer */
  int32_t resident_per_layer;     /* R (0 <= R <= E) */
  int32_t staging_slots;          /* S: most misses one layer step may have (<= E) */
  size_t expert_bytes;            /* moe_expert_blob_bytes(...) of every expert */
  const void* const* host_blobs;  /* host array [L*E]: pinned host address of blob (l, e) */
  const moe_expert_ref* scales;   /* host array [L*E]: ts_gate/ts_up/ts_down of (l, e); blob ignored */
  void* hbm_pool;                 /* device, 256-aligned, >= (L*R + S) * expert_bytes */
  size_t hbm_pool_bytes;
  hipStream_t copy_stream;        /* side stream for the H2D copies */
} moe_tier_desc;

typedef struct moe_tier_stats {
  uint64_t hits;          /* active experts found resident */
  uint64_t misses;        /* active experts copied from host */
  uint64_t h2d_bytes;     /* bytes copied host -> HBM (misses and promotions) */
  uint64_t promotions;    /* experts moved into a resident slot by rebalance */
  uint64_t prepares;
  uint64_t rebalances;
} moe_tier_stats;

typedef struct moe_tier moe_tier;

/* Validates (budget: MOE_ERR_BUDGET if the pool is below (L*R + S) slots)
 * and creates the tier with no expert resident. */
moe_status moe_tier_create(const moe_tier_desc* desc, moe_tier** out);

/* After moe_bucket of layer `layer` on `compute`: stage this step's missing
 * experts and fill table_dev (device moe_expert_ref [E]).  Blocks the host
 * until the active list of this step is known (one event wait).  Returns
 * MOE_ERR_BUDGET if the step has more misses than staging slots. */
moe_status moe_tier_prepare(moe_tier* t, int32_t layer, const moe_buckets* b,
                            moe_expert_ref* table_dev, hipStream_t compute);

/* The same on the device, with no host synchronization: two launches on
 * `compute`, a planning kernel (reads the step's active list and the tier's
 * device copy of the layer's resident slots, assigns the misses staging slots
 * in active-list order, writes table_dev and the copy list) and the copy
 * kernel, which reads the pinned host blobs directly.  So a caller can
 * enqueue many layers ahead, or capture them in a graph (with
 * moe_tier_rebalance, which synchronizes, outside it).  Results equal those
 * of moe_tier_prepare bit for bit.  The tier's device state (base tables,
 * blob addresses, copy list, counters: about 36 bytes per expert of every
 * layer) is allocated once by moe_tier_create, when the host blobs are mapped
 * for the device; otherwise this call returns MOE_ERR_UNSUPPORTED.  Staging
 * must hold every possible miss: MOE_ERR_BUDGET, before any launch, if
 * min(E, b->T_max * b->k) > S.  Hit and miss counts are kept on the device and
 * added by moe_tier_stats_get (synchronize `compute` before reading them).
 * This call and moe_tier_prepare share the staging slots: do not interleave
 * them on different streams. */
moe_status moe_tier_prepare_async(moe_tier* t, int32_t layer, const moe_buckets* b,
                                  moe_expert_ref* table_dev, hipStream_t compute);

/* Make the R most used experts of `layer` (hist_dev: device uint32 [E], as
 * updated by moe_expert_hist; ties to the lower index) resident, copying the
 * newcomers into freed slots.  Synchronizes `compute` (reads the histogram). */
moe_status moe_tier_rebalance(moe_tier* t, int32_t layer, const uint32_t* hist_dev,
                              hipStream_t compute);

/* Host copy of the counters; resident expert list of a layer (host int32 [R],
 * -1 for an empty slot) when resident_out is not NULL. */
moe_status moe_tier_stats_get(const moe_tier* t, moe_tier_stats* out, int32_t layer,
                              int32_t* resident_out);

/* Releases host metadata and events (not the caller's buffers). */
void moe_tier_destroy(moe_tier* t);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
