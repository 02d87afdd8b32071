/*
 * gtq.h -- C ABI of libgtq: Block-GTQ packed mixed-rate TQ-MSE KV cache and
 * attention over it, for AMD Instinct MI355X (gfx950).
 *
 * The operations follow the Block-GTQ page ("Block-GTQ: RoPE-Block Rate
 * Allocation for KV-Cache Quantization", abstract) and the TurboQuant pipeline
 * diagram (hsthanb4.github.io kvcache_quant_tutorial_2026, 01_turboquant_pipeline,
 * "paper" column):
 *   - keys are split into the 64 two-coordinate RoPE frequency blocks of a
 *     128-dim head; each block gets its own bit width (abstract, 2nd sentence);
 *   - the width comes from largest-marginal-gain allocation of a label-free
 *     query-key energy score weighted by codec rate penalties (3rd, 4th sentence);
 *   - blocks of equal rate form a group; each group of a key, and the whole value
 *     vector, is a TurboQuant-MSE vector: norm, random rotation, per-coordinate
 *     Lloyd-Max scalar quantization, bit packing (5th sentence; diagram boxes
 *     "random rotation", "per-coordinate MSE scalar quantization");
 *   - attention reads the packed cache directly and never builds a decoded
 *     fp16 K/V cache (5th sentence).
 *
 * Conventions for every call:
 *   - head_dim is 128 (64 RoPE blocks); other sizes return GTQ_EUNSUPPORTED.
 *   - "host" pointers are read during the call only; the library copies what it
 *     keeps. "device" pointers are caller-owned GPU memory (e.g. torch tensors).
 *   - Calls that take a hip_stream enqueue asynchronous GPU work on that stream
 *     (NULL = the default stream) and return before it finishes. They allocate no
 *     device memory; scratch memory comes from a caller-provided workspace.
 *   - Every call validates its arguments on the host before enqueuing anything.
 *     On failure it returns a nonzero gtq_status, enqueues nothing, and
 *     gtq_last_error() returns a message (per thread) describing the failure.
 *   - Device-side slot/length overruns that the host cannot see (slot values in
 *     device arrays) are skipped by the kernels and counted; see
 *     gtq_plan_overflow_count.
 */
#ifndef GTQ_H_
#define GTQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t gtq_status;
enum {
  GTQ_OK = 0,
  GTQ_EINVAL = 1,        /* bad argument (null pointer, out-of-range value)     */
  GTQ_EUNSUPPORTED = 2,  /* valid but not supported (head_dim != 128, capacity > 2^25) */
  GTQ_ENOMEM = 3,        /* host or device allocation failed (plan creation)   */
  GTQ_EDEVICE = 4,       /* HIP runtime or kernel launch error                  */
  GTQ_ECAPACITY = 5      /* cache or workspace too small for the request        */
};

enum { GTQ_ROPE_HALF = 0,        /* block j = coordinates (j, j + 64)          */
       GTQ_ROPE_INTERLEAVED = 1  /* block j = coordinates (2j, 2j + 1)         */ };

#define GTQ_HEAD_DIM 128
#define GTQ_BLOCKS 64
#define GTQ_MAX_GROUPS 4
#define GTQ_KNORM_STRIDE 4  /* floats per token of K norms (one per group, padded) */
#define GTQ_VBLOCK 8        /* tokens per V code block                          */
#define GTQ_SEQ_ALIGN 32    /* cache capacity must be a multiple of this        */

/* Message of the last failing call on this thread ("" if none). Never NULL. */
const char* gtq_last_error(void);

/* ---------------------------------------------------------------- host math */

/* Rate penalties: d_out[b] for b = 0..b_max (b_max <= 4) is the mean squared error
 * of the b-bit Lloyd-Max quantizer of a unit Gaussian (d_out[0] = 1). These are the
 * "codec-dependent rate penalties" of the abstract (3rd sentence) for TQ-MSE.
 * Errors: EINVAL if d_out is NULL or b_max outside [1, 4]. */
gtq_status gtq_rate_distortion(int32_t b_max, double* d_out);

/* The stored codebook of rate `bits` (1..4): centroids[2^bits] ascending (the
 * Lloyd-Max centroids of N(0,1), rounded to binary16 and returned as float) and
 * thresholds[2^bits - 1] (midpoints; a value >= t_k is above threshold k). A group of
 * dimension d quantizes sqrt(d) * Pi * x / ||x|| against these. Either output may be
 * NULL. Errors: EINVAL if bits outside [1, 4]. */
gtq_status gtq_codebook(int32_t bits, float* centroids, float* thresholds);

/* Largest-marginal-gain rate allocation for one (layer, KV head)
 * (abstract, 3rd and 4th sentence).
 *   q_cal [n_q][head_dim] host fp32: pre-RoPE calibration queries of all the query
 *         heads that share this KV head, flattened;
 *   k_cal [n_k][head_dim] host fp32: pre-RoPE calibration keys.
 * Energy score s_j = mean_q ||q_j||^2 * mean_k ||k_j||^2 per RoPE block j (fp64).
 * Starting from b_j = b_min, one bit at a time goes to the block with the largest
 * s_j * (D(b_j) - D(b_j + 1)) among blocks with b_j < b_max (ties: smallest j) until
 * sum_j b_j == budget. Outputs: rates_out[64] (required), scores_out[64] and
 * proxy_out (= sum_j s_j D(b_j)) optional.
 * Errors: EINVAL for NULL inputs, n_q/n_k < 1, bad rope_layout, b_min/b_max outside
 * 1 <= b_min <= b_max <= 4, budget outside [64 b_min, 64 b_max];
 * EUNSUPPORTED if head_dim != 128. */
gtq_status gtq_alloc_rates(const float* q_cal, int64_t n_q, const float* k_cal, int64_t n_k,
                           int32_t head_dim, int32_t rope_layout, int32_t b_min, int32_t b_max,
                           int32_t budget, uint8_t* rates_out, double* scores_out,
                           double* proxy_out);

/* Group layout of one head's packed key record, derived from its 64 block rates.
 * Groups are the distinct rates in ascending order; inside a group, blocks ascend
 * and each contributes its two coordinates (abstract, 5th sentence). The key record
 * is one little-endian bit stream: code i of group g occupies bits
 * [bit_offset[g] + i*rate[g], ... + rate[g]); bit p is bit (p % 32) of u32 word p/32. */
typedef struct gtq_head_layout {
  int32_t n_groups;                 /* distinct rates present (1..4)                 */
  int32_t rate[GTQ_MAX_GROUPS];     /* ascending                                    */
  int32_t dim[GTQ_MAX_GROUPS];      /* 2 * number of blocks at that rate             */
  int32_t bit_offset[GTQ_MAX_GROUPS];
  int32_t rot_offset[GTQ_MAX_GROUPS]; /* float offset of the group's rotation inside
                                         this head's slice of gtq_plan_desc.k_rot   */
  int32_t k_words;                  /* u32 words of one token's key record          */
  int32_t coord[GTQ_HEAD_DIM];      /* head coordinate of each record position      */
  int32_t v_hadamard;               /* gtq_plan_layout only: 1 when the head's value
                                       rotation is H_128 diag(s) / sqrt(128) for a sign
                                       vector s (Sylvester H, entries exactly
                                       +-fp32(1/sqrt(128))): the library then applies
                                       it as a fast Walsh-Hadamard transform where it
                                       can ("TurboQuant" diagram, rotate box: random
                                       rotation or Hadamard)                          */
} gtq_head_layout;

/* Computes the layout from rates[64] (each in [1, 4]). Host only.
 * Errors: EINVAL for NULL pointers, rates outside [1,4], bad rope_layout. */
gtq_status gtq_head_layout_from_rates(const uint8_t* rates, int32_t rope_layout,
                                      gtq_head_layout* out);

/* ---------------------------------------------------------------- plans */

enum {
  GTQ_PLAN_HOST_ONLY = 1,     /* build and validate on the host, no device copy           */
  GTQ_PLAN_NORM_CORRECT = 2,  /* norm-corrected variant ("TurboQuant: paper algorithm
                                 and vLLM engineering" diagram, vLLM column, NC box): the
                                 stored norm of every key group and of the value is
                                 nu * sqrt(d) / ||C[code]|| (fp64, rounded to fp32), so
                                 that the decoded vector keeps the input's norm; codes and
                                 the attention are unchanged                               */
  GTQ_PLAN_QJL = 4            /* 1-bit QJL residual sketch of the keys (TurboQuant-prod;
                                 "TurboQuant: paper algorithm and vLLM engineering"
                                 diagram, paper column, residual and QJL boxes): each key
                                 record goes on after its MSE words with sign(S r) for the
                                 residual r = k - k_hat (128 bits, 4 words; a zero
                                 projection counts as +) and gamma = ||r|| (fp64, stored
                                 as fp32 bits, 1 word); the attention logit adds
                                 gamma sqrt(pi/2) / 128 * sum_j (S q)_j sign_j. Needs
                                 desc.qjl and k_budget <= 176 (records of at most 16
                                 words); a prod key at b bits is k_budget = 64 (b - 1).
                                 Decode only (gtq_prefill_attn returns EUNSUPPORTED); chunk
                                 appends run through the per-token kernel.                 */
};

typedef struct gtq_plan_desc {
  int32_t n_layers, n_kv_heads, n_q_heads; /* n_q_heads a multiple of n_kv_heads      */
  int32_t head_dim;                        /* 128                                     */
  int32_t rope_layout;                     /* GTQ_ROPE_HALF | GTQ_ROPE_INTERLEAVED     */
  int32_t k_budget;                        /* sum_j b_j of every head (128 = K2, 192 = K3) */
  int32_t v_bits;                          /* 1..4, values are one 128-dim group       */
  int32_t flags;                           /* GTQ_PLAN_HOST_ONLY | _NORM_CORRECT | _QJL */
  const uint8_t* k_rates; /* host [n_layers][n_kv_heads][64], each head summing to k_budget */
  const float* k_rot;     /* host: for l, h, groups in ascending rate: the group's d x d
                             rotation, row-major fp32, concatenated (each head's slice is
                             sum_g d_g^2 floats)                                     */
  const float* v_rot;     /* host [n_layers][n_kv_heads][128][128] row-major fp32      */
  const float* qjl;       /* host [n_layers][n_kv_heads][128][128] row-major fp32, the
                             sketch matrices S (entries N(0,1)) of GTQ_PLAN_QJL; else
                             NULL                                                    */
} gtq_plan_desc;

typedef struct gtq_plan gtq_plan;

/* Builds a plan: group layouts, codebooks, decode tables; copies the rotations and
 * uploads everything to the current HIP device (unless GTQ_PLAN_HOST_ONLY). The pages
 * have no passage for this step as a call of its own; what it sets up is the grouping of
 * equal-rate blocks ("Block-GTQ" abstract, 5th sentence) and the rotate / per-coordinate
 * quantizer pair of each group ("TurboQuant: paper algorithm and vLLM engineering"
 * diagram, paper column, rotate and scalar-MSE boxes). The plan
 * is immutable afterwards and may be used from several streams at once.
 * Errors: EINVAL (NULL, counts < 1, rates outside [1,4] or not summing to k_budget,
 * k_budget not a multiple of 16, v_bits outside [1,4], bad flags/layout, GTQ_PLAN_QJL
 * without the qjl matrices or the matrices without the flag);
 * EUNSUPPORTED (head_dim != 128; GTQ_PLAN_QJL with k_budget > 176); ENOMEM; EDEVICE (no
 * device / upload failed). */
gtq_status gtq_plan_create(const gtq_plan_desc* desc, gtq_plan** out);
/* Frees the plan (host and device copies). Synchronizes the device. NULL is a no-op. */
gtq_status gtq_plan_destroy(gtq_plan* plan);
gtq_status gtq_plan_layout(const gtq_plan* plan, int32_t layer, int32_t kv_head,
                           gtq_head_layout* out);
/* Number of device-side overruns (slot >= capacity, seq >= batch, an absent page) skipped by append
 * kernels since the plan was created. Synchronizes the device. */
gtq_status gtq_plan_overflow_count(const gtq_plan* plan, int64_t* out);

/* ---------------------------------------------------------------- caches */

/* One layer's packed cache, device memory owned by the caller:
 *   k_codes [batch][n_kv_heads][capacity][k_words]   u32, token-major key records
 *   k_norms [batch][n_kv_heads][capacity][4]          fp32, one norm per key group
 *   v_codes [batch][n_kv_heads][capacity/8][32*v_bits] u32: blocks of 8 tokens; inside
 *           a block, coordinate c (in the value rotation's basis) owns bits
 *           [8*v_bits*c, 8*v_bits*(c+1)) and token j of the block the v_bits at
 *           8*v_bits*c + v_bits*j (little-endian u32 words)
 *   v_norms [batch][n_kv_heads][capacity]            fp32
 * capacity is a multiple of 32 and at most 2^25 (calls on a larger cache return
 * GTQ_EUNSUPPORTED).
 *
 * Paged layout (block_table non-NULL), for serving ("Block-GTQ" abstract, 9th sentence,
 * reports packed serving; the block-table organisation is this library's): the four
 * buffers are a pool
 * of n_pages pages of page_tokens tokens, each page laid out like a contiguous cache
 * with batch = n_pages and capacity = page_tokens (size it with gtq_cache_bytes(plan,
 * n_pages, page_tokens)). Position p of sequence b lives in pool page
 * block_table[b * table_stride + p / page_tokens] (device int32) at p % page_tokens.
 * capacity is then the per-sequence limit (at most table_stride * page_tokens);
 * page_tokens is a multiple of 32 in [32, 2^25]. Table entries outside [0, n_pages):
 * appends there are skipped and counted (gtq_plan_overflow_count) and reads return
 * zero codes and norms, so every page that covers a visible position must be valid.
 * With block_table NULL the last three fields are ignored. */
typedef struct gtq_cache_view {
  uint32_t* k_codes;
  float* k_norms;
  uint32_t* v_codes;
  float* v_norms;
  int32_t batch;
  int64_t capacity;
  const int32_t* block_table;
  int32_t page_tokens;
  int32_t n_pages;
  int32_t table_stride;
} gtq_cache_view;

typedef struct gtq_cache_sizes {
  size_t k_codes_bytes, k_norms_bytes, v_codes_bytes, v_norms_bytes;
  int32_t k_words, v_words_per_block;
  /* code bits per token and KV head ("logical bits", abstract 7th sentence) and the
     bytes per token and KV head including norms */
  int32_t logical_bits_per_token;
  int32_t bytes_per_token;
} gtq_cache_sizes;

/* Byte sizes of one layer's cache. Errors: EINVAL (NULL, batch < 1, capacity < 1 or
 * not a multiple of 32). */
gtq_status gtq_cache_bytes(const gtq_plan* plan, int32_t batch, int64_t capacity,
                           gtq_cache_sizes* out);

/* ---------------------------------------------------------------- append */

/* Fused rotate + quantize + pack of n_tok new tokens into layer `layer`'s cache
 * (TurboQuant diagram, "paper" column: input -> rotation -> scalar MSE quantization).
 *   k, v     device [n_tok][n_kv_heads][128] fp32, post-RoPE keys, values;
 *   seq_idx  device [n_tok] int32: sequence (batch row) of each token;
 *   slot     device [n_tok] int64: position of each token in its sequence.
 * Per token and KV head: for each key group, nu = ||x_g|| (accumulated in fp64,
 * stored fp32), z = sqrt(d_g) * Pi_g * x_g / nu, code_i = #{k : z_i >= t_k}; same for
 * the value vector with Pi_V and v_bits. A zero vector stores norm 0 and codes
 * 2^(b-1). Tokens with seq_idx outside [0, batch) or slot outside [0, capacity) are
 * skipped and counted (gtq_plan_overflow_count). Two tokens of one call must not
 * target the same (sequence, slot).
 * Errors: EINVAL (NULL, layer out of range, host-only plan, n_tok < 0). */
gtq_status gtq_quantize_append(const gtq_plan* plan, int32_t layer, const gtq_cache_view* cache,
                               const float* k, const float* v, const int32_t* seq_idx,
                               const int64_t* slot, int64_t n_tok, void* hip_stream);

/* Same for n_tok consecutive tokens of one sequence at slots pos0 .. pos0+n_tok-1
 * (a prompt chunk); k, v device [n_tok][n_kv_heads][128]. Writes whole value blocks
 * without atomics where the chunk covers them.
 * Errors: EINVAL (as above, seq outside [0, batch)); ECAPACITY if
 * pos0 + n_tok > capacity. */
gtq_status gtq_quantize_append_chunk(const gtq_plan* plan, int32_t layer,
                                     const gtq_cache_view* cache, const float* k,
                                     const float* v, int32_t seq, int64_t pos0,
                                     int64_t n_tok, void* hip_stream);

/* ---------------------------------------------------------------- attention */

/* Workspace bytes that gtq_decode_attn needs for `batch` sequences of at most
 * max_len cached tokens with split parameter `chunk` (0 = automatic; else a multiple
 * of 32 giving at most 256 splits of max_len). The partials phase runs G workgroups
 * that share the batch's 32-token blocks (of every tile of up to 8 query rows of one
 * sequence and KV head) equally: G = the device's compute units for chunk 0, else
 * tiles x ceil(max_len / chunk). The workspace holds the rotated queries (8 KB per
 * tile) and the split-K partials (m, l, acc[128] of 8 rows per piece of a tile that
 * one workgroup runs, G + tiles - 1 at most, plus one per tile for a window split) and
 * 16 bytes per tile that tell the merge where the tile's pieces are; its contents need
 * no initialisation.
 * Calls that share a workspace must be ordered on one stream. */
gtq_status gtq_decode_workspace_bytes(const gtq_plan* plan, int32_t batch, int64_t max_len,
                                      int32_t chunk, size_t* out);

/* Decode attention of one new query per sequence over the packed cache, without a
 * decoded K/V cache (abstract, 5th sentence).
 *   q        device [batch][n_q_heads][128] fp32, post-RoPE; query head h reads KV
 *            head h / (n_q_heads / n_kv_heads);
 *   seq_len  device [batch] int32: cached tokens of each sequence (all visible;
 *            values are clamped to [0, min(max_len, capacity)]);
 *   max_len  host: an upper bound of seq_len (sizes the split grid);
 *   out      device [batch][n_q_heads][128] fp32;
 *   logits   optional device [batch][n_q_heads][max_len] fp32 (scale * q . k_hat for
 *            every visible token; entries >= seq_len untouched), for tests.
 * Logit of token n, query head h: scale * sum_g nu_{n,g} / sqrt(d_g) *
 * sum_{i in g} (Pi_g q_g)_i C_{b_g}[code_{n,i}]; softmax over n < seq_len; output
 * Pi_V^T sum_n p_n nu^V_n C_{b_V}[vcode_n] / sqrt(128). Split-K over the pieces of
 * the workgroups' equal shares of blocks (gtq_decode_attn_partials; see
 * gtq_decode_workspace_bytes) followed by a log-sum-exp merge and the inverse value
 * rotation (gtq_decode_attn_merge). A sequence with seq_len 0 gets a zero output.
 * Errors: EINVAL (NULL, layer, scale not finite, chunk not a multiple of 32 or more than
 * 256 splits, host-only plan, max_len < 0); ECAPACITY (workspace too small,
 * max_len > capacity). */
gtq_status gtq_decode_attn(const gtq_plan* plan, int32_t layer, const gtq_cache_view* cache,
                           const float* q, const int32_t* seq_len, int64_t max_len,
                           float softmax_scale, int32_t chunk, float* out, float* logits,
                           void* workspace, size_t ws_bytes, void* hip_stream);

/* gtq_decode_attn for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same computation
 * and arguments without the workspace, which is a device array of 16 MiB inside the
 * library instead (one copy per device, held until the process ends; its address is
 * taken when a plan is created on that device). Calls no allocating routine. The plan's
 * device must be current. Every call on a device shares that one array: calls that
 * overlap on a device (other streams, other threads) race and give wrong results; calls
 * ordered on one stream are safe. The array needs no initialisation (each call writes
 * what it reads). Errors: those of gtq_decode_attn; ECAPACITY when the workspace that
 * gtq_decode_workspace_bytes gives for (batch, max_len, chunk) exceeds 16 MiB (e.g.
 * more than about 900 tiles of 8 query rows at the automatic split on 256 compute
 * units); EINVAL when the plan's device is not current. */
gtq_status gtq_decode_attn_static(const gtq_plan* plan, int32_t layer, const gtq_cache_view* cache,
                                  const float* q, const int32_t* seq_len, int64_t max_len,
                                  float softmax_scale, int32_t chunk, float* out, float* logits,
                                  void* hip_stream);

/* The three phases of gtq_decode_attn, for callers that interleave other work between
 * them or time them separately; all three take the same (cache, max_len, chunk) and
 * workspace, ordered on one stream.
 * gtq_decode_rotate_queries: r_g = Pi_g q_g for every key group of every query row
 *   (the query side of the logit above), scaled by softmax_scale * log2(e) / sqrt(d_g),
 *   stored in the workspace as the operand the partials phase reads. Errors as for
 *   gtq_decode_attn.
 * gtq_decode_attn_partials: per query row and piece, the running maximum m (base 2),
 *   the sum l of 2^(logit*log2(e) - m) and the accumulator of p * nu_V * C[vcode] in
 *   the value rotation's basis, into the workspace (needs the rotated queries; the
 *   merge must see the same seq_len, max_len and chunk).
 * gtq_decode_attn_merge: combines the splits and writes `out`. */
gtq_status gtq_decode_rotate_queries(const gtq_plan* plan, int32_t layer, const gtq_cache_view* cache,
                                     const float* q, int64_t max_len, float softmax_scale, int32_t chunk,
                                     void* workspace, size_t ws_bytes, void* hip_stream);
gtq_status gtq_decode_attn_partials(const gtq_plan* plan, int32_t layer, const gtq_cache_view* cache,
                                    const int32_t* seq_len, int64_t max_len, int32_t chunk, float* logits,
                                    void* workspace, size_t ws_bytes, void* hip_stream);
gtq_status gtq_decode_attn_merge(const gtq_plan* plan, int32_t layer, const gtq_cache_view* cache,
                                 const int32_t* seq_len, int64_t max_len, int32_t chunk, float* out,
                                 const void* workspace, size_t ws_bytes, void* hip_stream);

/* One decode step of a layer in three launches (the serving hot path): each sequence b
 * appends its new token (k_new, v_new: device [batch][n_kv_heads][128] fp32, post-RoPE)
 * at slot seq_len[b] - 1, then attends with its query to all seq_len[b] cached tokens.
 * gtq_decode_prepare runs the append and the query rotation in one launch (they
 * share no data); gtq_decode_step is prepare + partials + merge. seq_len counts the new
 * token; a sequence with seq_len[b] < 1 or > capacity appends nothing (counted by
 * gtq_plan_overflow_count) and, with seq_len 0, gets a zero output. Arguments and errors
 * otherwise as for gtq_quantize_append and gtq_decode_attn. */
gtq_status gtq_decode_prepare(const gtq_plan* plan, int32_t layer, const gtq_cache_view* cache,
                              const float* k_new, const float* v_new, const float* q, const int32_t* seq_len,
                              int64_t max_len, float softmax_scale, int32_t chunk, void* workspace,
                              size_t ws_bytes, void* hip_stream);
gtq_status gtq_decode_step(const gtq_plan* plan, int32_t layer, const gtq_cache_view* cache,
                           const float* k_new, const float* v_new, const float* q, const int32_t* seq_len,
                           int64_t max_len, float softmax_scale, int32_t chunk, float* out, void* workspace,
                           size_t ws_bytes, void* hip_stream);

/* Workspace bytes for gtq_prefill_attn on a chunk of n_tok queries whose last
 * position is pos0 + n_tok - 1 (no initialisation needed). */
gtq_status gtq_prefill_workspace_bytes(const gtq_plan* plan, int64_t pos0, int64_t n_tok,
                                       int32_t chunk, size_t* out);

/* Causal attention of a prompt chunk over the packed cache of sequence `seq`. No passage
 * of the pages describes prefill; it is the attention over packed caches of the
 * "Block-GTQ" abstract (5th sentence) applied to the query rows of a prompt chunk, each
 * seeing the cached positions up to its own:
 * q device [n_tok][n_q_heads][128] fp32 (post-RoPE) at positions pos0 .. pos0+n_tok-1;
 * the chunk's own keys/values must already be appended (gtq_quantize_append_chunk).
 * Query t sees cached positions 0 .. pos0 + t. out device [n_tok][n_q_heads][128].
 * Errors: as gtq_decode_attn; ECAPACITY if pos0 + n_tok > capacity; EUNSUPPORTED for a
 * GTQ_PLAN_QJL plan. */
gtq_status gtq_prefill_attn(const gtq_plan* plan, int32_t layer, const gtq_cache_view* cache,
                            const float* q, int32_t seq, int64_t pos0, int64_t n_tok,
                            float softmax_scale, int32_t chunk, float* out, void* workspace,
                            size_t ws_bytes, void* hip_stream);

/* ---------------------------------------------------------------- fp16 window */

/* fp16 sink and recent-token buffers beside the packed cache ("Block-GTQ" abstract,
 * 8th sentence, names them as the variant its K3V2 result does without): positions
 * p < n_sink and p >= seq_len - n_recent of a sequence attend through binary16 copies
 * of their key and value (round to nearest even), every other position through the
 * packed cache. Device buffers, caller-owned, one set per layer:
 *   k_sink   [batch][n_kv_heads][sink_slots][128]      binary16, token-major
 *   v_sink   [batch][n_kv_heads][sink_slots / 8][128][8] binary16: blocks of 8 tokens,
 *            coordinate-major inside a block (slot s: block s / 8, lane s % 8)
 *   k_recent [batch][n_kv_heads][n_recent][128]        ring: position p at slot p % n_recent
 *   v_recent [batch][n_kv_heads][n_recent / 8][128][8] the same ring, V block layout
 * with sink_slots = n_sink rounded up to a multiple of 32. n_sink in [0, 256];
 * n_recent a multiple of 32 in [0, 8192]. Slots that no token has filled may hold
 * anything: the kernels never read their values into a result. */
typedef struct {
  uint16_t* k_sink;
  uint16_t* v_sink;
  uint16_t* k_recent;
  uint16_t* v_recent;
  int32_t batch;
  int32_t n_sink;
  int32_t n_recent;
} gtq_window_view;

/* Copy tokens into the fp16 buffers: token t (k, v device [n_tok][n_kv_heads][128]
 * fp32) of sequence seq_idx[t] at position pos[t] (device int32 / int64) goes to sink
 * slot pos when pos < n_sink, else to recent slot pos % n_recent (nowhere if
 * n_recent is 0). Tokens of one call that map to the same slot race: pass each slot
 * at most once per call (for a prompt, its sink positions and its last n_recent
 * positions). The packed cache is filled separately (gtq_quantize_append), for every
 * position. Tokens with seq_idx outside [0, batch) or pos < 0 are skipped and
 * counted (gtq_plan_overflow_count). Errors: EINVAL (NULL, layer, window sizes,
 * host-only plan). */
gtq_status gtq_window_append(const gtq_plan* plan, int32_t layer, const gtq_window_view* window,
                             const float* k, const float* v, const int32_t* seq_idx, const int64_t* pos,
                             int64_t n_tok, void* hip_stream);

/* Workspace bytes of gtq_decode_attn_window: gtq_decode_workspace_bytes plus one more
 * partial per query row (the fp16 window's). */
gtq_status gtq_decode_window_workspace_bytes(const gtq_plan* plan, int32_t batch, int64_t max_len,
                                             int32_t chunk, size_t* out);

/* gtq_decode_attn with the fp16 window: for sequence b of length L = seq_len[b] the
 * packed partials cover positions [n_sink, max(n_sink, L - n_recent)); the fp16
 * positions (sink p < min(n_sink, L), recent p >= max(n_sink, L - n_recent)) form one
 * more split computed in the original basis and carried into the rotated value basis
 * before the merge. logits (optional) get every visible position's logit, packed or
 * fp16. window->batch must equal cache->batch. Errors: as gtq_decode_attn, plus EINVAL
 * for window sizes. */
gtq_status gtq_decode_attn_window(const gtq_plan* plan, int32_t layer, const gtq_cache_view* cache,
                                  const gtq_window_view* window, const float* q, const int32_t* seq_len,
                                  int64_t max_len, float softmax_scale, int32_t chunk, float* out,
                                  float* logits, void* workspace, size_t ws_bytes, void* hip_stream);

/* One decode step with the fp16 window in three launches: every sequence b of length
 * L = seq_len[b] >= 1 appends its newest token (k_new, v_new device
 * [batch][n_kv_heads][128] fp32) at position L - 1 to the packed cache and to the fp16
 * buffers, then attends as gtq_decode_attn_window with seq_len. The same results as
 * gtq_quantize_append (slot L - 1) + gtq_window_append (pos L - 1) +
 * gtq_decode_attn_window; the window append and the window split share a workgroup
 * (the append of the step's token to the fp16 buffers and the first use of it), the packed
 * append and the query rotation share the first launch ("Block-GTQ" abstract, 8th
 * sentence, for the buffers). A sequence with seq_len 0 appends nothing (counted once, as
 * in gtq_decode_step). Workspace: gtq_decode_window_workspace_bytes. Errors: as
 * gtq_decode_attn_window; EUNSUPPORTED with more than 8 query heads per KV head. */
gtq_status gtq_decode_step_window(const gtq_plan* plan, int32_t layer, const gtq_cache_view* cache,
                                  const gtq_window_view* window, const float* k_new, const float* v_new,
                                  const float* q, const int32_t* seq_len, int64_t max_len, float softmax_scale,
                                  int32_t chunk, float* out, void* workspace, size_t ws_bytes, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* GTQ_H_ */
