/*
 * pkv.h — C ABI of libpkv, attention over a paged KV cache on AMD MI355X (gfx950).
 *
 * Objects (the names the pages and the vLLM attention metadata use):
 *   q             bf16 [num_tokens, num_q_heads, head_dim]; the new tokens of every request,
 *                 concatenated request after request (batched prefill: Tencent Cloud
 *                 article on vLLM inference acceleration, batched-prefill paragraph).
 *   k_cache       bf16 [num_blocks, num_kv_heads, 16, head_dim] for 16-token blocks: physical
 *                 key blocks, token-major (a key is one contiguous row).
 *   v_cache       bf16 [num_blocks, num_kv_heads, head_dim, 16]: physical value blocks,
 *                 dim-major (16 tokens of one dimension are contiguous).
 *                 A block of bs = 16 R tokens (R = 2, 4, 8 or 16: blocks of 32 to 256 tokens;
 *                 "11. vLLM principles", section 11.2 names blocks of 16 or 256 tokens) is R
 *                 consecutive such 16-token tiles: k_cache
 *                 [num_blocks, R, num_kv_heads, 16, head_dim], v_cache
 *                 [num_blocks, R, num_kv_heads, head_dim, 16].  Either way slot s (below) is
 *                 row s % 16 of 16-token tile s / 16 of the pool.
 *                 Token p of a request lives in physical block block_tables[r][p / bs] at
 *                 offset p % bs ("11. vLLM principles", section 11.2 PagedAttention).
 *   block_tables  int32 [num_seqs, bt_stride]; logical block -> physical block per request.
 *                 Rows may share physical blocks (shared, read-only prefix; same section).
 *   query_start_loc int32 [num_seqs + 1]; request r owns tokens [qsl[r], qsl[r+1]).
 *   context_lens  int32 [num_seqs]; tokens of request r already cached before this step
 *                 (earlier chunks, or a prefix-cache hit: Tencent Cloud article, chunked
 *                 prefill and prefix caching sections).
 *   seq_lens      int32 [num_seqs]; keys visible after this step = context_lens + query len.
 *   slot_mapping  int64 [num_tokens]; flat pool slot (physical_block * bs + offset) of every
 *                 new token; a negative slot means "do not write".
 *
 * Attention: token i of request r sits at position p = context_lens[r] + i and attends to
 * keys 0..p of its own request (its own key included), with scale 1/sqrt(head_dim) unless
 * pkv_shape.scale > 0.  q head h reads kv head h / (num_q_heads / num_kv_heads).
 * LSE outputs are natural-log log-sum-exp of the scaled scores, fp32.
 *
 * Conventions for every entry point:
 *   - all tensor pointers are device pointers owned by the caller, except the h_* arguments
 *     of pkv_plan_varlen which are host pointers; the library keeps no pointer after return;
 *   - work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and is
 *     asynchronous; no entry point synchronises the device or allocates device memory;
 *   - return 0 on success or a negative PKV_E* code; on error nothing was enqueued and
 *     pkv_last_error() (thread-local) describes the failure;
 *   - device-resident metadata is trusted: block ids must lie in [0, num_blocks), and the
 *     device copies must agree with the host copies given to pkv_plan_varlen.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_OK 0
#define PKV_EINVAL (-1)     /* null pointer, unsupported shape, inconsistent metadata */
#define PKV_EWORKSPACE (-2) /* workspace too small for the plan */
#define PKV_EPREFIX (-3)    /* cascade prefix length not a multiple of block_size */
#define PKV_EHIP (-4)       /* the HIP runtime reported an error (launch or copy) */

#define PKV_DTYPE_BF16 0
#define PKV_DTYPE_F32 1

/* Static shape of one attention layer's cache.  Supported: head_dim 64 or 128,
 * block_size 16, 32, 64, 128 or 256, num_q_heads / num_kv_heads in {1, 2, 4, 8}. */
typedef struct pkv_shape {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t num_blocks; /* physical blocks in each pool */
  int32_t bt_stride;  /* int32 elements between consecutive block-table rows */
  float scale;        /* softmax scale; <= 0 selects 1/sqrt(head_dim) */
} pkv_shape;

/* Host-side summary of a varlen plan, filled by pkv_plan_varlen and read by
 * pkv_paged_attention_varlen.  Plain data; the work list itself lives in the workspace. */
typedef struct pkv_varlen_plan {
  int32_t num_seqs;
  int32_t num_tokens;
  int32_t num_items;       /* work items (each is launched once per kv head) */
  int32_t num_prefill_items;
  int32_t num_decode_items;
  int32_t num_partials;    /* split-KV partial states per q head */
  int32_t blocks_per_split; /* most 16-token blocks per split of a decode row: a row of n
                              blocks is cut into ceil(n / blocks_per_split) splits of that size,
                              except that a last split under a quarter of it is evened out with
                              the one before (short rows choose their own, usually longer,
                              split) */
  int32_t has_splits;
  int64_t workspace_used;  /* bytes of the workspace the plan occupies */
  int32_t head_dim, num_q_heads, num_kv_heads, block_size; /* shape the plan was made for */
  int32_t tile_rows;       /* packed (token, q head) rows per prefill tile: 128 or 256 */
  int32_t num_short_items; /* items of rows of 2 .. 32 / G query tokens (short items) */
  int32_t decode_waves;    /* waves per workgroup of decode items launched on their own: 4, or 1
                              when every decode item has at most 64 16-token blocks, G >= 8 and
                              there are at least 4096 (item, kv head) workgroups */
} pkv_varlen_plan;

/* Size in bytes of a workspace that fits any plan with at most these sizes. */
size_t pkv_varlen_workspace_size(int32_t num_seqs, int32_t num_tokens, int32_t max_seq_len,
                                 const pkv_shape* shape);

/* a1 — slot mapping [Tencent Cloud article, chunked prefill / prefix caching sections, and
 * "11. vLLM principles" section 11.2]: for token i of request r at position
 * p = context_lens[r] + i, slot = block_tables[r][p / bs] * bs + p % bs.
 * Writes slot_mapping[num_tokens] (int64).  query_start_loc holds num_seqs + 1 ascending
 * entries (requests with no new token are allowed); token t belongs to the request r with
 * query_start_loc[r] <= t < query_start_loc[r + 1].  A token whose logical block index is
 * >= bt_stride, or whose position is negative, gets slot -1 (so does a token that no request
 * owns, which only a malformed query_start_loc produces).  num_tokens == 0 is a no-op. */
int pkv_compute_slot_mapping(int64_t* slot_mapping, const int32_t* block_tables,
                             const int32_t* query_start_loc, const int32_t* context_lens,
                             int32_t num_seqs, int32_t num_tokens, const pkv_shape* shape,
                             void* stream);

/* a2 — KV caching [2048ai.net vLLM V1 article, "KV Caching"]: copies the bits of k[t] and
 * v[t] (bf16 [num_tokens, num_kv_heads, head_dim]) into the pools at slot_mapping[t]
 * (keys token-major [num_blocks, Hkv, bs, D]; values dim-major [num_blocks, Hkv, D, bs]).
 * Negative slots and slots >= num_blocks * block_size are skipped.  Bit-exact copy. */
int pkv_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                          const int64_t* slot_mapping, int32_t num_tokens,
                          const pkv_shape* shape, void* stream);

/* a1 + a2 in one launch, for callers that do not need the slots separately: computes every
 * new token's slot from block_tables / query_start_loc / context_lens exactly as
 * pkv_compute_slot_mapping does, stores the token's K and V there as pkv_reshape_and_cache
 * does, and also writes the slots to slot_mapping when it is not NULL. */
int pkv_append_kv(int64_t* slot_mapping, const void* k, const void* v, void* k_cache,
                  void* v_cache, const int32_t* block_tables, const int32_t* query_start_loc,
                  const int32_t* context_lens, int32_t num_seqs, int32_t num_tokens,
                  const pkv_shape* shape, void* stream);

/* Copy-on-write of shared blocks ["11. vLLM principles", section 11.2: requests with a common
 * prefix point their block tables at the same physical blocks]: for each of num_pairs pairs
 * {src, dst} in block_pairs (device int32 [num_pairs, 2]), copies physical block src to dst in
 * both pools, every kv head, bit for bit, so that a request can take a private copy of a
 * shared block before writing into it.  Pairs naming a block outside [0, num_blocks), or
 * src == dst, are skipped.  No destination may also appear as another pair's source or
 * destination (the copies run concurrently).  num_pairs == 0 is a no-op. */
int pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs, int32_t num_pairs,
                    const pkv_shape* shape, void* stream);

/* ---- FP8 (e4m3) KV cache ------------------------------------------------------------------
 * Storing the KV cache in a low-precision float format such as FP8 cuts its size and speeds up
 * attention, above all for long contexts [2048ai.net vLLM V1 article, quantisation section].
 * Format: OCP FP8 E4M3 ("e4m3fn": bias 7, subnormals, no infinities, 0x7f / 0xff NaN, largest
 * finite value 448), one byte per element, pools in the same layouts as the bf16 pools
 * (k_cache uint8 [num_blocks, Hkv, bs, D], v_cache uint8 [num_blocks, Hkv, D, bs]).
 * Scales: k_scale and v_scale are device fp32 [num_blocks, num_kv_heads], owned by the caller:
 * a code stored in block b (of block_size tokens), kv head g means code_value * scale[b][g] (a
 * per-head or per-tensor scale is the case of equal entries).  The scales of a block must be set before any token is
 * written into it and stay fixed while the block holds tokens.
 * Quantisation of a bf16 value x: y = x * (1 / scale) in fp32, clamped to [-448, 448], rounded
 * to the nearest code with ties to even; NaN stores 0x7f.  Attention over fp8 pools equals
 * attention over the dequantised keys and values. */

/* a2 for fp8 pools: quantises k[t], v[t] (bf16 [num_tokens, Hkv, D]) under the scales of the
 * block that slot_mapping[t] falls in and stores the codes there.  Slots are skipped as in
 * pkv_reshape_and_cache.  Bit-exact against the definition above. */
int pkv_reshape_and_cache_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                              const float* k_scale, const float* v_scale,
                              const int64_t* slot_mapping, int32_t num_tokens,
                              const pkv_shape* shape, void* stream);

/* a1 + a2 for fp8 pools, in one launch (as pkv_append_kv, quantising as
 * pkv_reshape_and_cache_fp8). */
int pkv_append_kv_fp8(int64_t* slot_mapping, const void* k, const void* v, void* k_cache,
                      void* v_cache, const float* k_scale, const float* v_scale,
                      const int32_t* block_tables, const int32_t* query_start_loc,
                      const int32_t* context_lens, int32_t num_seqs, int32_t num_tokens,
                      const pkv_shape* shape, void* stream);

/* pkv_copy_blocks for fp8 pools: also copies the blocks' scales (k_scale[src][*] ->
 * k_scale[dst][*], v_scale alike). */
int pkv_copy_blocks_fp8(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                        const int32_t* block_pairs, int32_t num_pairs, const pkv_shape* shape,
                        void* stream);

/* Builds the work list of one varlen attention call from host copies of the metadata:
 * validates seq_lens[r] == context_lens[r] + (qsl[r+1] - qsl[r]) and every length, cuts
 * query-length-1 rows into split-KV decode items and longer rows into prefill tiles of
 * 128 or 256 packed (token, q head) rows (256 once the batch holds at least 2048 prefill
 * rows), orders them heaviest first, and enqueues a host-to-device copy of the list into
 * `workspace` on `stream`.  Fills *plan.  The workspace must stay untouched until the
 * attention call that uses the plan has run.  The copy goes through a ring of 32 pinned host
 * buffers of 256 KB per device and calling thread, allocated on the thread's first plan on the
 * device (a plan of more than 8192 work items grows its buffer once); the call waits only when
 * 32 earlier uploads of the thread have not yet been read by the device. */
int pkv_plan_varlen(pkv_varlen_plan* plan, void* workspace, size_t workspace_bytes,
                    const int32_t* h_query_start_loc, const int32_t* h_context_lens,
                    const int32_t* h_seq_lens, int32_t num_seqs, int32_t num_tokens,
                    const pkv_shape* shape, void* stream);

/* The same planning into host memory only (no device work): writes up to `max_items`
 * work items of 8 int32 each {seq, kind (0 decode, 1 prefill, 2 short), q_begin, q_count
 * (prefill and short: tokens; decode: splits of the row), kv_begin, kv_end, partial_base,
 * split} into `items`.  For inspection and tests. */
int pkv_plan_varlen_host(pkv_varlen_plan* plan, int32_t* items, int32_t max_items,
                         const int32_t* h_query_start_loc, const int32_t* h_context_lens,
                         const int32_t* h_seq_lens, int32_t num_seqs, int32_t num_tokens,
                         const pkv_shape* shape);

/* a3/a4/a5 — paged attention over a mixed continuous batch [Tencent Cloud article,
 * continuous batching, chunked prefill and prefix caching sections; "11. vLLM principles"
 * section 11.3, prefill vs decode]: decode rows (one query token; VALU path with split-KV) and
 * chunked-prefill / prefix-hit rows (MFMA tiles with the causal mask offset by context_lens).
 * Launches, by plan: a batch of decode rows and 128-row prefill tiles is one kernel; a batch
 * with 256-row prefill tiles (at least 2048 packed prefill rows) runs them in one kernel and
 * its decode rows in a second; rows of 2 .. 32 / G tokens (short items) add one more kernel;
 * a split-KV reduce follows when any row was split.
 * out: [num_tokens, num_q_heads, head_dim], bf16 or fp32 (out_dtype); lse: nullable fp32
 * [num_tokens, num_q_heads].  The pools must already hold this step's new keys/values
 * (pkv_reshape_and_cache first).  `plan` must come from pkv_plan_varlen with the same
 * metadata, shape and workspace. */
int pkv_paged_attention_varlen(void* out, int32_t out_dtype, float* lse, const void* q,
                               const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* query_start_loc,
                               const int32_t* context_lens, const int32_t* seq_lens,
                               int32_t num_seqs, int32_t num_tokens, const pkv_shape* shape,
                               const pkv_varlen_plan* plan, void* workspace,
                               size_t workspace_bytes, void* stream);

/* a3/a4/a5 over fp8 pools: as pkv_paged_attention_varlen (same plan and workspace), reading
 * e4m3 codes with their per-(block, kv head) scales.  Every path converts codes to bf16
 * exactly (prefill tiles stage the exact codes in LDS) and applies the key scale to the
 * block's scores and the value scale to its probabilities, in fp32. */
int pkv_paged_attention_varlen_fp8(void* out, int32_t out_dtype, float* lse, const void* q,
                                   const void* k_cache, const void* v_cache, const float* k_scale,
                                   const float* v_scale, const int32_t* block_tables,
                                   const int32_t* query_start_loc, const int32_t* context_lens,
                                   const int32_t* seq_lens, int32_t num_seqs, int32_t num_tokens,
                                   const pkv_shape* shape, const pkv_varlen_plan* plan,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* ---- Graph-capturable decode step (f4) -----------------------------------------------------
 * Recording a step once and replaying it saves the per-launch CPU cost; the recording needs
 * fixed shapes, so batches are padded up to a few bucketed sizes (1, 2, 4, ..., 512) ["11. vLLM
 * principles", section 11.5].  pkv_paged_attention_decode is the decode part of
 * pkv_paged_attention_varlen for batches of one query token per row, with no host plan: its
 * launches depend only on (num_seqs, max_seq_len, shape), and block_tables, query_start_loc,
 * seq_lens and q are read on the device.  So a step captured once in a HIP graph (this call,
 * after pkv_append_kv) replays correctly for any new metadata written into the same buffers,
 * as long as every seq_lens[r] <= max_seq_len.  Rows are cut into splits of a fixed key count
 * chosen from (num_seqs, max_seq_len); splits past a row's end contribute nothing.  A padded row
 * with seq_lens[r] == 0 gets output 0 and lse -inf. */

/* Workspace bytes for pkv_paged_attention_decode(_fp8) with these sizes (0 if none needed). */
size_t pkv_decode_workspace_size(int32_t num_seqs, int32_t max_seq_len, const pkv_shape* shape);

/* Decode attention (a3) for num_seqs rows of one query token each: token query_start_loc[r] of
 * q attends to keys 0..seq_lens[r]-1 of row r.  One token per row means query_start_loc must be
 * 0, 1, ..., num_seqs (row r's token is token r; split rows' partial states are indexed by it),
 * so q, out and lse have num_seqs rows: out bf16 or fp32 [num_seqs, Hq, D], lse nullable fp32
 * [num_seqs, Hq].  Errors as pkv_paged_attention_varlen. */
int pkv_paged_attention_decode(void* out, int32_t out_dtype, float* lse, const void* q,
                               const void* k_cache, const void* v_cache, const int32_t* block_tables,
                               const int32_t* query_start_loc, const int32_t* seq_lens,
                               int32_t num_seqs, int32_t max_seq_len, const pkv_shape* shape,
                               void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): pkv_paged_attention_decode with no workspace.  The
 * split-KV partial states go to a device scratch array of PKV_DECODE_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends; the call allocates nothing.
 * Same arguments, layouts, results (bit for bit) and errors as pkv_paged_attention_decode,
 * plus PKV_EWORKSPACE when the batch's partial states exceed the scratch
 * (pkv_decode_workspace_size(num_seqs, max_seq_len, shape) > PKV_DECODE_SCRATCH_BYTES; e.g.
 * 512 rows of 32 q heads at D 128 up to 8192 keys fit).  Every call on one GPU shares that
 * GPU's scratch: calls that may overlap on one GPU (other streams, other threads) race and
 * must be serialised by the caller.  Not timed by pkv_timing_begin. */
#define PKV_DECODE_SCRATCH_BYTES ((size_t)32 << 20)
int pkv_paged_attention_decode_noalloc(void* out, int32_t out_dtype, float* lse, const void* q,
                                       const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, const int32_t* query_start_loc,
                                       const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                                       const pkv_shape* shape, void* stream);

/* The same over fp8 (e4m3) pools with per-(block, kv head) scales. */
int pkv_paged_attention_decode_fp8(void* out, int32_t out_dtype, float* lse, const void* q,
                                   const void* k_cache, const void* v_cache, const float* k_scale,
                                   const float* v_scale, const int32_t* block_tables,
                                   const int32_t* query_start_loc, const int32_t* seq_lens,
                                   int32_t num_seqs, int32_t max_seq_len, const pkv_shape* shape,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes for pkv_cascade_prefix_attention with these sizes. */
size_t pkv_cascade_workspace_size(int32_t num_tokens, int32_t prefix_len, const pkv_shape* shape);

/* a6 — cascade inference, shared-prefix pass [2048ai.net vLLM V1 article, "Cascade
 * Inference"]: the attention state of every query token over the prefix keys
 * 0..prefix_len-1 named by prefix_block_table (int32 [prefix_len / block_size]); no mask
 * (every query lies after the prefix).  Writes out_prefix fp32 [num_tokens, num_q_heads,
 * head_dim] and lse_prefix fp32 [num_tokens, num_q_heads].  prefix_len must be a positive
 * multiple of block_size (PKV_EPREFIX otherwise).  The workspace holds per-segment
 * partial states when the prefix is cut into segments. */
int pkv_cascade_prefix_attention(float* out_prefix, float* lse_prefix, const void* q,
                                 const void* k_cache, const void* v_cache,
                                 const int32_t* prefix_block_table, int32_t prefix_len,
                                 int32_t num_tokens, const pkv_shape* shape, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* a6 over fp8 pools: as pkv_cascade_prefix_attention (same workspace size), the prefix keys
 * and values read as e4m3 codes times their per-(block, kv head) scales. */
int pkv_cascade_prefix_attention_fp8(float* out_prefix, float* lse_prefix, const void* q,
                                     const void* k_cache, const void* v_cache,
                                     const float* k_scale, const float* v_scale,
                                     const int32_t* prefix_block_table, int32_t prefix_len,
                                     int32_t num_tokens, const pkv_shape* shape, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* a8 — merge of two attention states over disjoint key sets [2048ai.net vLLM V1 article,
 * "Cascade Inference", the associative and commutative merge operator]:
 * out = (e^lse_a o_a + e^lse_b o_b) / (e^lse_a + e^lse_b), lse_out = ln(e^lse_a + e^lse_b),
 * computed shifted by max(lse_a, lse_b); (0, -inf) is the identity.  out is bf16 or fp32
 * [num_tokens, num_heads, head_dim]; lse_out nullable.  head_dim must be a multiple of 4. */
int pkv_merge_attn_states(void* out, int32_t out_dtype, float* lse_out, const float* out_a,
                          const float* lse_a, const float* out_b, const float* lse_b,
                          int32_t num_tokens, int32_t num_heads, int32_t head_dim, void* stream);

/* Launch timing (measurement aid, per calling thread): after pkv_timing_begin(), the attention
 * kernels launched by pkv_paged_attention_varlen(_fp8), pkv_paged_attention_decode(_fp8) and
 * pkv_cascade_prefix_attention(_fp8) are bracketed by two HIP events recorded on their stream
 * (the split-KV / segment reduce falls outside them; a varlen call whose plan needs more than
 * one attention kernel counts as one launch).  pkv_timing_end() stops recording, waits for the
 * last event and returns the summed kernel milliseconds and the number of launches.  Creates
 * HIP events on first use; not for graph capture. */
int pkv_timing_begin(void);
int pkv_timing_end(double* total_ms, int32_t* launches);

/* Per-launch milliseconds of the window the last pkv_timing_end() closed, in launch order:
 * copies up to `capacity` of them into ms_each (host memory) and returns how many there were
 * (negative PKV_E* code on a bad buffer). */
int pkv_timing_durations(double* ms_each, int32_t capacity);

/* Thread-local description of the last error returned on this thread ("" if none). */
const char* pkv_last_error(void);

/* Library version string. */
const char* pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
