// Internal declarations shared by the host front end (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Tokens per 16-token tile, the unit every kernel addresses.  A cache block of 16 R tokens
// (block_size 16, 32, 64, 128 or 256) is R consecutive tiles, so "block" below means such a tile.
constexpr int kBlockSize = 16;
constexpr int kKvTile = 64;          // keys per MFMA KV tile (4 cache blocks)
constexpr int kTileRows = 128;       // packed (token, q head) rows of a varlen prefill tile
constexpr int kWideTileRows = 256;   // rows of a wide tile (prefill-heavy batches, cascade)
constexpr int kPrefillRowsForWideTiles = 2048;  // packed prefill rows from which wide tiles pay
constexpr int kMinBlocksPerSplit = 16;
// Short multi-token rows (at most kSplitRowsMax packed (token, q head) rows, such as
// speculative-verify rows) over a long context are cut into key splits of kPrefillSplitKeys
// keys, so that no workgroup walks a whole long context alone.
constexpr int kSplitRowsMax = 64;
constexpr int kPrefillSplitKeys = 1024;

// kShort: a row of 2 .. kShortRowsMax / G query tokens run like a decode item (key splits, one
// workgroup per split) with its packed rows as MFMA columns.
enum ItemKind : int32_t { kDecode = 0, kPrefill = 1, kShort = 2 };
constexpr int kShortRowsMax = 32;

// One unit of work of the varlen kernel; it is run once per kv head.
struct WorkItem {
  int32_t seq;           // request index
  int32_t kind;          // ItemKind
  int32_t q_begin;       // first query token of the tile, relative to the request
  int32_t q_count;       // prefill: query tokens in the tile; decode: splits of the row
  int32_t kv_begin;      // first key (token index) of this item
  int32_t kv_end;        // one past the last key
  int32_t partial_base;  // -1: write the output; decode: partial row base of the request, the
                         // item writes row partial_base + split; prefill: the partial row of the
                         // tile's first token for this split, token t writes partial_base + t
  int32_t split;         // split index within the request (or tile)
};
static_assert(sizeof(WorkItem) == 32, "work item layout");

struct VarlenArgs {
  const uint16_t* q;
  const void* k_cache;     // bf16 pools, or fp8 (e4m3) pools for the *_fp8 launchers
  const void* v_cache;
  const float* k_scale;    // fp8 pools: scale per (physical block, kv head); else unused
  const float* v_scale;
  const int32_t* block_tables;
  const int32_t* query_start_loc;
  const int32_t* context_lens;
  const int32_t* seq_lens;
  void* out;
  float* lse;
  int32_t out_f32;
  const WorkItem* items;
  int32_t num_items;
  float* part_o;    // [num_partials * Hq, D]
  float* part_lse;  // [num_partials * Hq]
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t bt_stride;
  int32_t bt_shift;  // log2(block_size / 16): a block is 1 << bt_shift 16-token tiles
  float scale_log2;  // softmax scale * log2(e)
};

struct CascadeArgs {
  const uint16_t* q;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* prefix_bt;
  int32_t prefix_len;
  int32_t num_tokens;
  int32_t num_segments;
  int32_t seg_len;     // keys per segment (multiple of the KV tile)
  int32_t num_tiles;   // query tiles per kv head
  float* out;          // final fp32 output when num_segments == 1
  float* lse;
  float* part_o;       // [num_segments, T, Hq, D] when num_segments > 1
  float* part_lse;     // [num_segments, T, Hq]
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t bt_shift;  // log2(block_size / 16)
  float scale_log2;
};

// Split-KV reduce: row (token, head) merges `count` partial states.
struct ReduceArgs {
  const float* part_o;
  const float* part_lse;
  const int32_t* token_split;  // per token {first partial row, count, row stride}; nullptr: uniform layout
  int32_t uniform_count;       // uniform layout: partial row of split s = (s * T + token)
  int32_t num_tokens;
  int32_t num_q_heads;
  void* out;
  int32_t out_f32;
  float* lse;
};

// Launchers (defined in the .hip files); return the hipError_t of the launch.
// bs_log2 = log2(block_size); slots are flat token indices, so a slot's 16-token tile is
// slot / 16 whatever the block size.
hipError_t launch_slot_mapping(int64_t* slot_mapping, const int32_t* block_tables,
                               const int32_t* qsl, const int32_t* ctx, int32_t num_seqs,
                               int32_t num_tokens, int32_t bt_stride, int32_t bs_log2,
                               hipStream_t stream);
hipError_t launch_append_kv(int64_t* slot_mapping, const uint16_t* k, const uint16_t* v,
                            uint16_t* k_cache, uint16_t* v_cache, const int32_t* block_tables,
                            const int32_t* qsl, const int32_t* ctx, int32_t num_seqs,
                            int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                            int32_t bt_stride, int64_t num_slots, int32_t bs_log2,
                            hipStream_t stream);
hipError_t launch_reshape_and_cache(const uint16_t* k, const uint16_t* v, uint16_t* k_cache,
                                    uint16_t* v_cache, const int64_t* slots, int32_t num_tokens,
                                    int32_t num_kv_heads, int32_t head_dim, int64_t num_slots,
                                    hipStream_t stream);
hipError_t launch_append_kv_fp8(int64_t* slot_mapping, const uint16_t* k, const uint16_t* v,
                                uint8_t* k_cache, uint8_t* v_cache, const float* k_scale,
                                const float* v_scale, const int32_t* block_tables, const int32_t* qsl,
                                const int32_t* ctx, int32_t num_seqs, int32_t num_tokens,
                                int32_t num_kv_heads, int32_t head_dim, int32_t bt_stride,
                                int64_t num_slots, int32_t bs_log2, hipStream_t stream);
hipError_t launch_reshape_and_cache_fp8(const uint16_t* k, const uint16_t* v, uint8_t* k_cache,
                                        uint8_t* v_cache, const float* k_scale, const float* v_scale,
                                        const int64_t* slots, int32_t num_tokens, int32_t num_kv_heads,
                                        int32_t head_dim, int64_t num_slots, int32_t bs_log2,
                                        hipStream_t stream);
// Copies whole blocks of both pools (elem_bytes per element: 2 for bf16, 1 for fp8) and, when
// k_scale / v_scale are given, their per-(block, kv head) scales.
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                              const int32_t* pairs, int32_t num_pairs, int32_t num_blocks,
                              int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                              int32_t elem_bytes, hipStream_t stream);
// Launches the attention kernels of a varlen plan whose items list n_prefill prefill tiles of
// tile_rows rows first, then n_decode decode items, then n_short short items; decode items in a
// launch of their own run decode_waves (4, or 1) waves per workgroup.
hipError_t launch_varlen(const VarlenArgs& a, int head_dim, int group, int n_prefill, int n_decode,
                         int n_short, int tile_rows, int decode_waves, hipStream_t stream);
hipError_t launch_cascade(const CascadeArgs& a, int head_dim, int group, hipStream_t stream);
// The same over fp8 (e4m3) pools with per-(block, kv head) scales (attention.hip built with
// PKV_KV_FP8=1).
hipError_t launch_varlen_fp8(const VarlenArgs& a, int head_dim, int group, int n_prefill,
                             int n_decode, int n_short, int tile_rows, int decode_waves,
                             hipStream_t stream);
hipError_t launch_cascade_fp8(const CascadeArgs& a, int head_dim, int group, hipStream_t stream);
// Decode batch (one query token per row) split into `splits` key ranges of split_keys keys per
// row, with the split computed on the device (graph-capturable); num_tokens = rows of the
// partial layout (split * num_tokens + token).
hipError_t launch_decode_graph(const VarlenArgs& a, int head_dim, int group, int num_seqs, int splits,
                               int split_keys, int num_tokens, hipStream_t stream);
hipError_t launch_decode_graph_fp8(const VarlenArgs& a, int head_dim, int group, int num_seqs,
                                   int splits, int split_keys, int num_tokens, hipStream_t stream);
hipError_t launch_reduce(const ReduceArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_merge(void* out, int32_t out_f32, float* lse_out, const float* oa,
                        const float* la, const float* ob, const float* lb, int64_t rows,
                        int32_t head_dim, hipStream_t stream);

}  // namespace pkv
