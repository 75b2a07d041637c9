/*
 * mla.h — C ABI of the MI355X (gfx950) Multi-head Latent Attention decode library (libmla.so).
 *
 * One decode step of one attention layer, over a cache that stores per token only the joint
 * KV latent c^KV (d_c values) followed by the decoupled, already-rotated rotary key k^R
 * (d_h^R values): "DeepSeek-V2 from Scratch: Multi-head Latent Attention and DeepSeekMoE",
 * section 4.5 (what gets cached) and section 6 (the complete algorithm, boxed quantities).
 * W^UK is absorbed into the query and W^UV into the output (same page, sections 5.1-5.3), so
 * attention runs against the latents directly and the full keys/values are never formed.
 *
 * A full step is:  mla_absorb_q -> mla_rope -> mla_decode_attn -> mla_combine -> mla_absorb_out
 * (or, fused: mla_absorb_q -> mla_rope -> mla_decode_attn -> mla_combine_absorb_out)
 * (chunked prefill: mla_prefill_tables, then the same five calls over the pseudo-sequences;
 *  pre-combined absorption: mla_precombine once, then mla_absorb_q_pre / mla_absorb_out_pre in
 *  place of mla_absorb_q / mla_absorb_out; naive-form chunked prefill: mla_absorb_q_naive ->
 *  mla_rope -> mla_prefill_naive_attn -> mla_output_proj)
 *
 * Conventions shared by every entry point
 *  - Pointers are DEVICE pointers unless the comment says host. Tensors and workspaces must be
 *    16-byte aligned (kernels use vector accesses); int32 arrays (lengths, block tables), the fp8
 *    scales and lse need 4 bytes. The caller owns every buffer (inputs, outputs, workspaces);
 *    the library never allocates, frees or keeps per-call state.
 *  - Every call only enqueues work on `stream` (may be NULL = the default stream) and returns.
 *    Nothing synchronises. Work is ordered with the caller's other work on that stream.
 *  - Arguments are validated on the host before anything is enqueued. On an error nothing is
 *    launched, the call returns a non-zero mla_status and mla_last_error() describes it
 *    (thread-local text). A failed launch returns MLA_E_HIP.
 *  - Device-resident values (sequence lengths, block tables) are the caller's contract: lengths
 *    must satisfy 1 <= seq_lens[b] <= capacity and block-table entries must name pages of the pool.
 *  - Weights are row-major [out, in] so that y = W x, as the pages write them:
 *      W_dq [d_cq, d]         W_uq [n_h*d_h, d_cq]   W_qr [n_h*d_r, d_cq]
 *      W_dkv [d_c, d]         W_kr [d_r, d]
 *      W_uk [n_h*d_h, d_c]    W_uv [n_h*d_h, d_c]    W_o [d, n_h*d_h]
 *    Head i owns rows [i*d_h, (i+1)*d_h) of W_uq/W_uk/W_uv, rows [i*d_r, (i+1)*d_r) of W_qr and
 *    columns [i*d_h, (i+1)*d_h) of W_o.
 *  - Activations passed between calls are float32, row-major:
 *      q_lat [B, n_h, d_c]   absorbed content query (W^UK_i)^T q^C_i
 *      q_pe  [B, n_h, d_r]   rotary query (raw after mla_absorb_q, rotated after mla_rope)
 *      kv_new [B, d_c + d_r] current token's [c^KV | k^R] (k^R raw, then rotated by mla_rope)
 *      o_lat [B, n_h, d_c]   attention-weighted latent sum per head;  lse [B, n_h] natural log
 *      u     [B, d]          layer output
 *  - Positions are 0-based: the current token of sequence b sits at position seq_lens[b]-1,
 *    cache row j holds position j, and attention covers rows 0..seq_lens[b]-1 inclusive.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

#if defined(__GNUC__)
#define MLA_API __attribute__((visibility("default")))
#else
#define MLA_API
#endif

typedef enum {
  MLA_F32 = 0,       /* IEEE binary32 */
  MLA_F16 = 1,       /* IEEE binary16 */
  MLA_BF16 = 2,      /* bfloat16 */
  MLA_FP8_E4M3 = 3,  /* OCP e4m3 (max 448, no inf) codes + one float32 scale per cached token;
                        cache storage only */
  MLA_FP6_E2M3 = 4   /* OCP FP6 E2M3 codes (max 7.5, no inf / NaN) packed 6 bits each, as a
                        little-endian bit stream per row (code j at bits 6j..6j+5), + one float32
                        scale per cached token; cache storage only */
} mla_dtype;

typedef enum {
  MLA_OK = 0,
  MLA_E_ARG = 1,          /* invalid argument (null pointer, bad size, inconsistent dims) */
  MLA_E_UNSUPPORTED = 2,  /* valid but not implemented (dtype/dims combination) */
  MLA_E_WORKSPACE = 3,    /* workspace missing or smaller than the *_workspace_bytes query */
  MLA_E_HIP = 4           /* a HIP runtime call or kernel launch failed */
} mla_status;

/* Model dimensions (the pages' notation). rope_base: rotary frequency base (10000 on the
 * pages' configs). sm_scale <= 0 selects 1/sqrt(d_h + d_r), the scale of "DeepSeek-V2 from
 * Scratch" section 4.4. Requirements: all dims > 0, d_r even, d_c and d_r multiples of 8.
 *
 * Long-context extension of the decoupled RoPE (the DeepSeek-V2 review page, "4. Pre-Training":
 * YaRN applied to k^R to extend the context from 4K to 128K; the page gives no formula, so the
 * YaRN method is taken as published, with its parameters supplied here). yarn_factor <= 1 turns
 * it off (plain RoPE). With yarn_factor s > 1, pair m's frequency theta_m = rope_base^(-2m/d_r)
 * becomes
 *     theta'_m = (1 - g) * theta_m / s + g * theta_m,
 *     r = yarn_orig_len * theta_m / (2 pi)   (turns of pair m over the original context),
 *     g = 0 for r < yarn_alpha, 1 for r > yarn_beta, (r - yarn_alpha) / (yarn_beta - yarn_alpha)
 *         in between,
 * for q^R and k^R alike, and the default score scale (sm_scale <= 0) is multiplied by
 * (0.1 ln s + 1)^2, the method's attention temperature. */
typedef struct {
  int32_t d, n_h, d_h, d_c, d_cq, d_r;
  double rope_base;
  float sm_scale;
  float yarn_factor;      /* s; <= 1: off */
  int32_t yarn_orig_len;  /* original context length (tokens), >= 1 when s > 1 */
  float yarn_alpha;       /* ramp start (turns), >= 0 */
  float yarn_beta;        /* ramp end (turns), > yarn_alpha */
} mla_dims;

/* Latent cache of one layer. Row width is d_c + d_r elements: [c^KV | k^R].
 *  contiguous (page_size == 0): rows is [B, t_cap, d_c + d_r]; token j of sequence b at
 *      rows + (b * t_cap + j) * (d_c + d_r).
 *  paged (page_size > 0): rows is a pool [num_pages, page_size, d_c + d_r]; token j of sequence
 *      b lives in page block_table[b * max_pages + j / page_size], slot j % page_size.
 *      block_table is device int32 [B, max_pages]; unused entries may hold -1.
 *  dtype MLA_FP8_E4M3: rows holds uint8 codes and scales holds one float32 per row with the
 *      same indexing (scales[(b * t_cap + j)] or scales[page * page_size + slot]); value =
 *      code * scale. The scale is amax / 448 of the row (1 for an all-zero row).
 *  dtype MLA_FP6_E2M3: rows are (d_c + d_r) * 6 / 8 bytes (the packed codes; 432 bytes at
 *      d_c + d_r = 576) with the same row indexing; scales as for fp8, amax / 7.5 of the row.
 *  scales must be NULL for the other dtypes.
 * The struct itself is read on the host during the call; it need not outlive the call. */
typedef struct {
  void* rows;
  float* scales;
  int32_t dtype;          /* mla_dtype */
  int32_t page_size;      /* 0 = contiguous */
  int64_t t_cap;          /* contiguous: rows per sequence; paged: max_pages * page_size */
  const int32_t* block_table;
  int32_t max_pages;
  int32_t num_pages;
} mla_cache;

/* ---------------------------------------------------------------------------------------------
 * mla_absorb_q — query pathway with W^UK absorbed, plus the current token's KV projection.
 * "DeepSeek-V2 from Scratch" section 4.1 (c^Q = W^DQ h, q^C = W^UQ c^Q, raw q^R = W^QR c^Q),
 * section 2.1 (c^KV = W^DKV h), section 4.2 (raw k^R = W^KR h) and section 5.1
 * (absorbed query q~_i = (W^UK_i)^T q^C_i, one matrix-vector product per head).
 *   h: [B, d] in `wdtype`; weights in `wdtype` (F32, F16 or BF16).
 *   workspace: device scratch of at least mla_absorb_q_workspace_bytes(dims, B) bytes.
 *   Outputs (float32): q_lat [B, n_h, d_c], q_pe [B, n_h, d_r] (NOT yet rotated),
 *   kv_new [B, d_c + d_r] (k^R part NOT yet rotated). */
MLA_API size_t mla_absorb_q_workspace_bytes(const mla_dims* dims, int32_t B);
MLA_API mla_status mla_absorb_q(const mla_dims* dims, int32_t B, int32_t wdtype, const void* h,
                        const void* W_dq, const void* W_uq, const void* W_qr, const void* W_uk,
                        const void* W_dkv, const void* W_kr, void* workspace, size_t ws_bytes,
                        float* q_lat, float* q_pe, float* kv_new, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * mla_rope — decoupled rotary embedding and cache append.
 * "DeepSeek-V2 from Scratch" section 3.1 (a position-dependent rotation whose query-key dot
 * product depends only on the offset), sections 4.1-4.2 (q^R per head, one k^R shared by all
 * heads) and section 4.5 (k^R is cached already rotated). Pairs (x[2m], x[2m+1]) are rotated by
 * angle pos * theta_m, theta_m = rope_base^(-2m/d_r) (or its YaRN form, see mla_dims), computed
 * in float64.
 *   seq_lens: device int32 [B]; pos_b = seq_lens[b] - 1.
 *   q_pe [B, n_h, d_r] and the k^R part of kv_new [B, d_c + d_r] are rotated IN PLACE.
 *   cache: if non-NULL, row [c^KV | k^R] of each sequence is written to slot pos_b, rounded to
 *   the cache dtype (RNE; fp8 / fp6: per-token scale amax/448 or amax/7.5 and saturating RNE
 *   codes).
 *   A sequence with seq_lens[b] == 0 (outside the contract) is left alone: its q_pe and kv_new
 *   rows are not rotated and nothing is written to the cache. */
MLA_API mla_status mla_rope(const mla_dims* dims, int32_t B, const int32_t* seq_lens, float* q_pe,
                    float* kv_new, const mla_cache* cache, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * mla_decode_attn — attention of the absorbed query against the cached latents.
 * "DeepSeek-V2 from Scratch" section 4.4 (score = q^C.k^C + q^R.k^R over sqrt(d_h + d_r)),
 * section 5.1 (q^C.k^C = q~.c^KV) and section 5.3 (steps 2-3: dot with every cached latent,
 * softmax-weighted sum of latents). Per head i and cached row j:
 *     s_ij = (q_lat_i . c_j + q_pe_i . k^R_j) * sm_scale
 * and the result is the softmax-weighted latent sum plus its log-sum-exp.
 * The batch's tokens (sum of seq_lens) are cut into `num_splits` contiguous ranges of equal
 * length (0 = the library's choice: one per compute unit at n_h = 128, d_c = 512, d_r = 64, two
 * per compute unit otherwise; at most 1024); each range is one workgroup, and a sequence
 * is split where ranges cut it. Each (range, sequence) piece writes a partial result into the
 * workspace: its normalised latent sum and log-sum-exp per head; mla_combine merges them. At most
 * num_splits + B - 1 pieces exist. The partial latent sums are float32, except on the MFMA path
 * (n_h = 128, d_c = 512, d_r = 64 with a bf16 or fp8 cache) where each (piece, head) row is kept
 * as float16 after scaling by a power of two that brings its largest magnitude into [0.5, 1):
 * a relative rounding of at most 2^-11 per element, below the bf16 rounding of the operands.
 *   q_lat [B, n_h, d_c], q_pe [B, n_h, d_r] (rotated): float32.
 *   seq_lens: device int32 [B] (including the current token, already appended).
 *   workspace: at least mla_decode_workspace_bytes(dims, B, num_splits) bytes. At the MFMA
 *   shape it also holds the query in the fp8 kernel's form (per head: scaled by a power of two
 *   and split into two e4m3 parts), written by this call before the attention kernel reads it. */
MLA_API size_t mla_decode_workspace_bytes(const mla_dims* dims, int32_t B, int32_t num_splits);
MLA_API mla_status mla_decode_attn(const mla_dims* dims, int32_t B, const float* q_lat, const float* q_pe,
                           const mla_cache* cache, const int32_t* seq_lens, int32_t num_splits,
                           void* workspace, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * mla_combine — merge the split-sequence partial results of mla_decode_attn.
 * Regroups the softmax sum of "DeepSeek-V2 from Scratch" section 4.4 over the pieces of each
 * sequence: with piece lse_s and normalised partial o_s, M = max_s lse_s, w_s = exp(lse_s - M),
 *     o_lat = sum_s w_s o_s / sum_s w_s,   lse = M + log(sum_s w_s).
 * Deterministic (fixed order, no atomics). Must be called with the same dims, B, num_splits,
 * seq_lens and workspace as the preceding mla_decode_attn.
 *   Outputs: o_lat [B, n_h, d_c] float32, lse [B, n_h] float32 (lse may be NULL). */
MLA_API mla_status mla_combine(const mla_dims* dims, int32_t B, int32_t num_splits, const int32_t* seq_lens,
                       const void* workspace, size_t ws_bytes, float* o_lat, float* lse,
                       hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * mla_absorb_out — value up-projection after the weighted sum, then the output projection.
 * "DeepSeek-V2 from Scratch" section 5.2 (o_i = W^UV_i sum_j a_j c_j) and sections 1/6
 * (u = W^O [o_1; ...; o_nh]), applied in that two-step order.
 *   o_lat [B, n_h, d_c] float32; W_uv, W_o in `wdtype`; u [B, d] float32.
 *   workspace: at least mla_absorb_out_workspace_bytes(dims, B) bytes.
 * The per-head outputs o_i stay float32 between the two products, except for bf16 weights at
 * B >= 256 rows (the batches of a chunked prefill), where they are rounded to bf16 so that the
 * W^O product runs on bf16 activations. */
MLA_API size_t mla_absorb_out_workspace_bytes(const mla_dims* dims, int32_t B);
MLA_API mla_status mla_absorb_out(const mla_dims* dims, int32_t B, int32_t wdtype, const float* o_lat,
                          const void* W_uv, const void* W_o, void* workspace, size_t ws_bytes,
                          float* u, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * mla_absorb_out_noalloc — mla_absorb_out for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. Same inputs,
 * output, kernels and result as mla_absorb_out, but no workspace argument: the W^UV output and
 * the K-split partial sums live in a library-owned static device array of
 * MLA_NOALLOC_SCRATCH_BYTES bytes per GPU (each GPU the library runs on holds it until the process
 * ends). The call allocates and frees nothing.
 *   Rejects (MLA_E_WORKSPACE, nothing launched) a B whose mla_absorb_out_workspace_bytes(dims, B)
 *   exceeds MLA_NOALLOC_SCRATCH_BYTES (at the DeepSeek-V2 shape: any B above 255; from 256 columns
 *   on, W^O takes the wide-product kernel, whose K-split partials outgrow the array).
 *   Every call on one GPU uses that GPU's one array: calls that overlap on the same GPU (other
 *   streams, other threads) race and must be ordered by the caller. */
#define MLA_NOALLOC_SCRATCH_BYTES (32u << 20)
MLA_API mla_status mla_absorb_out_noalloc(const mla_dims* dims, int32_t B, int32_t wdtype, const float* o_lat,
                                  const void* W_uv, const void* W_o, float* u, hipStream_t stream);

/* mla_combine_absorb_out — mla_combine followed by mla_absorb_out in one call, with the merge of
 * the pieces fused into the per-head W^UV product: for each head i and sequence b the pieces'
 * partials are merged ("DeepSeek-V2 from Scratch" section 4.4, the softmax regrouped) and
 * multiplied by W^UV_i (section 5.2) without writing o_lat, then u = W^O [o_1; ...; o_nh]
 * (section 6), with the per-head outputs o_i rounded to bf16 between the two products (the
 * two-call path keeps them in float32). Same results as the two calls up to that rounding.
 *   dec_workspace: the workspace mla_decode_attn filled (same B and num_splits);
 *   workspace: mla_absorb_out_workspace_bytes(dims, B) bytes; u [B, d] float32;
 *   lse: optional [B, n_h] float32 (NULL to skip), as mla_combine writes it.
 * Kernels exist for bf16 weights with d_h = 128, d_c = 512, d_r = 64 (and the MFMA GEMM shapes);
 * other cases return MLA_E_UNSUPPORTED and the caller uses mla_combine + mla_absorb_out. */
MLA_API mla_status mla_combine_absorb_out(const mla_dims* dims, int32_t B, int32_t wdtype, int32_t num_splits,
                                  const void* dec_workspace, size_t dec_ws_bytes, const void* W_uv,
                                  const void* W_o, void* workspace, size_t ws_bytes, float* u, float* lse,
                                  hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * mla_prefill_tables — chunked prefill through the decode calls.
 * "DeepSeek-V2 from Scratch" section 6 gives attention for token t over positions 0..t. A chunk
 * of C new tokens per sequence (positions p0[b] .. p0[b] + C - 1) is run as a batch of B * C
 * causal pseudo-sequences: pseudo-sequence b * C + t is token t of sequence b's chunk, with length
 * p0[b] + t + 1 and sequence b's pages. With these tables, the five calls of a decode step over
 * B * C pseudo-sequences (h rows ordered the same way) append every chunk token's row at its
 * position and give each token its causal attention output, exactly as C decode steps in turn.
 *   cache: the paged cache (page_size > 0; its block_table is [B, max_pages] device int32).
 *   p0: device int32 [B], rows already in the cache per sequence; p0[b] + C <= max_pages *
 *       page_size and the pages covering those positions assigned (caller's contract).
 *   seq_lens_out: device int32 [B * C]; block_table_out: device int32 [B * C, max_pages]. */
MLA_API mla_status mla_prefill_tables(const mla_cache* cache, int32_t B, int32_t C, const int32_t* p0,
                              int32_t* seq_lens_out, int32_t* block_table_out, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Pre-combined absorption — the alternative form of the two absorbed projections.
 * "DeepSeek-V2 from Scratch" section 5.1 merges W^UQ_i and W^UK_i into one matrix
 * W~^Q_i = (W^UK_i)^T W^UQ_i (d_c x d_cq) that maps c^Q straight to the absorbed query, and
 * section 5.2 merges W^UV_i and W^O_i into W~^O_i = W^O_i W^UV_i (d x d_c) that maps the
 * attention-weighted latent straight to the output. The results equal the two-step form up to
 * rounding; the weight bytes differ (at the DeepSeek-V2 shape W~^Q is 3x and W~^O 3.6x the bytes
 * of the factors they replace, at the running model's shape W~^Q is smaller).
 *
 * mla_precombine — build the stacked matrices once from the factors (float32 accumulation, one
 * rounding to wdtype):
 *   Wq_pre [n_h*d_c, d_cq]: row i*d_c + c is column c of (W^UK_i)^T W^UQ_i, i.e.
 *       Wq_pre[i*d_c + c][k] = sum_e W_uk[i*d_h + e][c] * W_uq[i*d_h + e][k];
 *   Wo_pre [d, n_h*d_c]:    Wo_pre[m][i*d_c + c] = sum_e W_o[m][i*d_h + e] * W_uv[i*d_h + e][c].
 * Either output may be NULL (then it is not built, and its factors may be NULL). Outputs are in
 * wdtype and caller-owned. */
MLA_API mla_status mla_precombine(const mla_dims* dims, int32_t wdtype, const void* W_uq, const void* W_uk,
                          const void* W_uv, const void* W_o, void* Wq_pre, void* Wo_pre, hipStream_t stream);

/* mla_absorb_q_pre — mla_absorb_q with W~^Q: q_lat = Wq_pre c^Q in one product (W_uq and W_uk
 * are not read). Same outputs, layouts and workspace size (mla_absorb_q_workspace_bytes). */
MLA_API mla_status mla_absorb_q_pre(const mla_dims* dims, int32_t B, int32_t wdtype, const void* h,
                            const void* W_dq, const void* Wq_pre, const void* W_qr, const void* W_dkv,
                            const void* W_kr, void* workspace, size_t ws_bytes, float* q_lat,
                            float* q_pe, float* kv_new, hipStream_t stream);

/* mla_absorb_out_pre — u = Wo_pre [o_lat_1; ...; o_lat_nh] in one product (the two-step
 * mla_absorb_out with W~^O). o_lat [B, n_h, d_c] float32; u [B, d] float32. The workspace
 * (K-split partial sums) needs mla_absorb_out_pre_workspace_bytes(dims, B) bytes, which may be
 * 0 (then workspace may be NULL). */
MLA_API size_t mla_absorb_out_pre_workspace_bytes(const mla_dims* dims, int32_t B);
MLA_API mla_status mla_absorb_out_pre(const mla_dims* dims, int32_t B, int32_t wdtype, const float* o_lat,
                              const void* Wo_pre, void* workspace, size_t ws_bytes, float* u,
                              hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Naive-form chunked prefill — the other execution path for a chunk of many query tokens.
 * "DeepSeek-V2/V3: The Two Bills Behind MLA and MoE" (section "The First Bill") names two ways to
 * run MLA: one that expands the keys and values, one that absorbs the up-projections. Here the
 * cache stays latent either way; this path expands, per call, the keys and values of every
 * context token of the chunk's sequences ("DeepSeek-V2 from Scratch" section 2.2:
 * k^C_{j,i} = W^UK_i c^KV_j, v_{j,i} = W^UV_i c^KV_j; section 4.2: k_{j,i} = [k^C_{j,i}; k^R_j]) and
 * runs attention per head on them (section 4.4) with the un-absorbed query
 * q_{t,i} = [q^C_{t,i}; q^R_{t,i}]. Outputs equal those of the absorbed path up to rounding
 * (section 5 of the same page: absorption is exact). Per (query, key) pair this form costs
 * 2 n_h (d_h + d_r + d_h) flop against 2 n_h (d_c + d_r + d_c) absorbed, plus 4 n_h d_h d_c flop to
 * expand each context token once per call: it wins for long chunks (the compute-bound regime).
 *
 * A chunk is:  mla_prefill_tables -> mla_absorb_q_naive -> mla_rope (the tables' lengths and
 * view of the cache, as for the absorbed chunk) -> mla_prefill_naive_attn -> mla_output_proj.
 * Kernels exist for d_h = 128, d_c = 512, d_r = 64 with the MFMA GEMM shapes (d and d_cq multiples
 * of 256, n_h d_h a multiple of 256), bfloat16 weights and a bfloat16 cache; other cases return
 * MLA_E_UNSUPPORTED.
 *
 * mla_absorb_q_naive — mla_absorb_q without the W^UK step: writes q_c [B, n_h, d_h] float32 (the
 * content query q^C_{t,i}) in place of q_lat; q_pe and kv_new as mla_absorb_q (raw rotary parts).
 * Workspace: mla_absorb_q_workspace_bytes(dims, B). W_uk is not read. */
MLA_API mla_status mla_absorb_q_naive(const mla_dims* dims, int32_t B, int32_t wdtype, const void* h,
                              const void* W_dq, const void* W_uq, const void* W_qr, const void* W_dkv,
                              const void* W_kr, void* workspace, size_t ws_bytes, float* q_c, float* q_pe,
                              float* kv_new, hipStream_t stream);

/* mla_prefill_naive_attn — causal attention of a C-token chunk per sequence over its expanded
 * context. Token t of sequence b (row b * C + t of q_c / q_pe / o, position p0[b] + t) attends to
 * cache rows 0 .. p0[b] + t, which must already hold the chunk's rows (mla_rope appends them).
 *   q_c [B * C, n_h, d_h], q_pe [B * C, n_h, d_r] (rotated) float32; o [B * C, n_h, d_h] bfloat16
 *   (o_{t,i} of the page's section 4.4, before W^O, rounded to nearest even);
 *   cache: the sequences' own cache (block table [B, max_pages] when paged), bfloat16 rows;
 *   p0: device int32 [B]; max_ctx (host): bound on every p0[b] + C, at most the cache capacity.
 *   Keys beyond max_ctx are not read (a caller error leaves such outputs unspecified).
 * Workspace (mla_prefill_naive_workspace_bytes(dims, B, max_ctx)): the gathered latent rows
 * [B, max_ctx, d_c + d_r] and the expanded K^C and V [B * max_ctx, n_h d_h], all bfloat16. */
MLA_API size_t mla_prefill_naive_workspace_bytes(const mla_dims* dims, int32_t B, int32_t max_ctx);
MLA_API mla_status mla_prefill_naive_attn(const mla_dims* dims, int32_t B, int32_t C, int32_t wdtype,
                                  const float* q_c, const float* q_pe, const mla_cache* cache,
                                  const int32_t* p0, int32_t max_ctx, const void* W_uk, const void* W_uv,
                                  void* workspace, size_t ws_bytes, void* o, hipStream_t stream);

/* mla_output_proj — u = W^O [o_1; ...; o_nh] ("DeepSeek-V2 from Scratch" section 1, the output
 * projection) for N rows of per-head outputs o [N, n_h * d_h] of type odtype (MLA_F32, or MLA_BF16
 * as mla_prefill_naive_attn writes it); u [N, d] float32. A float32 o keeps ~16 significant bits
 * on the MFMA path (bf16 hi + lo halves). The workspace (K-split partial sums) needs
 * mla_output_proj_workspace_bytes(dims, N) bytes, which may be 0 (then workspace may be NULL). */
MLA_API size_t mla_output_proj_workspace_bytes(const mla_dims* dims, int32_t N);
MLA_API mla_status mla_output_proj(const mla_dims* dims, int32_t N, int32_t wdtype, int32_t odtype,
                           const void* o, const void* W_o, void* workspace, size_t ws_bytes, float* u,
                           hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * mla_cache_store — write given rows into a cache (prefix fill; not part of a decode step).
 * Rows of sequence b, j < n_rows[b], are read from src + (b * src_stride + j) * (d_c + d_r)
 * (float32) and stored at position j exactly as mla_rope stores its appended row (same
 * rounding / same fp8 scale rule). n_rows: device int32 [B]; n_rows[b] <= capacity.
 * max_rows (host) bounds every n_rows[b] and sizes the launch. */
MLA_API mla_status mla_cache_store(const mla_dims* dims, const mla_cache* cache, int32_t B,
                           const int32_t* n_rows, int32_t max_rows, const float* src,
                           int64_t src_stride, hipStream_t stream);

/*
 * mla_stream_read — measurement helper, not a step of the path: a plain read-only streaming
 * kernel over `bytes` bytes at `src`, the HBM read ceiling that the latent-cache read of
 * mla_decode_attn is reported against. Every 16-byte word is loaded once and
 * folded into an XOR; word k of sink (k < the launch's workgroup count, at most
 * MLA_STREAM_SINK_WORDS) receives the XOR of the 32-bit words its workgroup read, so the XOR of
 * all sink words written equals the XOR of every 32-bit word of the buffer.
 * src: device, 16-byte aligned, bytes a multiple of 16 (> 0). sink: device uint32
 * [MLA_STREAM_SINK_WORDS], zero it first when comparing the XOR. Returns MLA_E_ARG otherwise.
 */
#define MLA_STREAM_SINK_WORDS 4096
MLA_API mla_status mla_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

/* Status text, and the last error message of the calling thread ("" if none). */
MLA_API const char* mla_status_str(mla_status s);
MLA_API const char* mla_last_error(void);
/* Library version string (host). */
MLA_API const char* mla_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MLA_H_ */
