// C-ABI front end of libpkv: argument validation, the varlen work plan, and kernel dispatch.
// Every entry point is declared (with the passage of the pages it follows) in include/pkv.h.
#include "pkv.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "internal.h"

namespace {

thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int ok() {
  g_error.clear();
  return PKV_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(PKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int check_shape(const pkv_shape* s) {
  if (!s) return fail(PKV_EINVAL, "shape is null");
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(PKV_EINVAL, "head_dim %d unsupported (64 or 128)", s->head_dim);
  if (s->block_size != 16 && s->block_size != 32 && s->block_size != 64 && s->block_size != 128 &&
      s->block_size != 256)
    return fail(PKV_EINVAL, "block_size %d unsupported (16, 32, 64, 128 or 256)", s->block_size);
  if (s->num_q_heads <= 0 || s->num_kv_heads <= 0 || s->num_q_heads % s->num_kv_heads)
    return fail(PKV_EINVAL, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                s->num_q_heads, s->num_kv_heads);
  const int G = s->num_q_heads / s->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(PKV_EINVAL, "q heads per kv head %d unsupported (1, 2, 4, 8)", G);
  if (s->num_blocks <= 0) return fail(PKV_EINVAL, "num_blocks must be positive");
  if ((int64_t)s->num_blocks * (s->block_size / pkv::kBlockSize) > INT32_MAX)
    return fail(PKV_EINVAL, "num_blocks %d too large: 16-token tile ids must fit int32", s->num_blocks);
  if (s->bt_stride <= 0) return fail(PKV_EINVAL, "bt_stride must be positive");
  return PKV_OK;
}

// log2(block_size) and log2(block_size / 16) of a checked shape (block_size a power of two).
int32_t bs_log2(const pkv_shape* s) { return __builtin_ctz((unsigned)s->block_size); }
int32_t bt_shift(const pkv_shape* s) { return bs_log2(s) - 4; }

float scale_log2(const pkv_shape* s) {
  const double sc = s->scale > 0 ? (double)s->scale : 1.0 / std::sqrt((double)s->head_dim);
  return (float)(sc * 1.4426950408889634);  // log2(e)
}

// ---------------------------------------------------------------------------------------
// Workspace layout of a varlen plan.
// ---------------------------------------------------------------------------------------
struct VarlenLayout {
  size_t items_off, split_off, plse_off, po_off, total;
};

VarlenLayout varlen_layout(int64_t items, int64_t tokens, int64_t partials, int64_t Hq, int64_t D) {
  VarlenLayout L;
  L.items_off = 0;
  L.split_off = align256(L.items_off + (size_t)items * sizeof(pkv::WorkItem));
  L.plse_off = align256(L.split_off + (size_t)tokens * 3 * sizeof(int32_t));
  L.po_off = align256(L.plse_off + (size_t)partials * Hq * sizeof(float));
  L.total = align256(L.po_off + (size_t)partials * Hq * D * sizeof(float));
  return L;
}

// Workgroups the decode split size aims for (about two and a half rounds of the decode
// workgroups 256 CUs hold; 1024, 4096 and 8192 measured slower on the bench batch).
constexpr int64_t kDecodeTargetWorkgroups = 2048;

struct Plan {
  std::vector<pkv::WorkItem> items;
  std::vector<int32_t> token_split;  // per token {first partial row, count, row stride}
  int32_t num_partials = 0;
  int32_t bps = 0;
  int32_t tile_rows = pkv::kTileRows;
  int32_t n_prefill = 0, n_decode = 0, n_short = 0;
  int32_t decode_waves = 4;
};

// First block of key split k (0 <= k <= splits) of a row of nblk blocks cut into splits of at
// most bps blocks: full splits of bps blocks, except that a last split under bps / 4 blocks is
// evened out with the one before it, so that no item is a sliver (a row of 1030 keys with 64-block
// splits is two items of 33 and 32 blocks, not 64 and 1).  Splits keep their order; the last one
// ends at nblk.
int32_t split_start(int32_t nblk, int32_t bps, int32_t splits, int32_t k) {
  if (k >= splits) return nblk;
  const int32_t rem = nblk - (splits - 1) * bps;
  if (splits > 1 && rem < bps / 4 && k == splits - 1) return (splits - 2) * bps + (bps + rem + 1) / 2;
  return k * bps;
}

constexpr int64_t kOneWaveDecodeItems = 4096;  // decode workgroups from which one-wave ones pay

int build_plan(Plan& P, const int32_t* qsl, const int32_t* ctx, const int32_t* seq,
               int32_t num_seqs, int32_t num_tokens, const pkv_shape* s) {
  if (num_seqs < 0 || num_tokens < 0) return fail(PKV_EINVAL, "negative num_seqs/num_tokens");
  if (num_seqs > 0 && (!qsl || !ctx || !seq)) return fail(PKV_EINVAL, "null host metadata");
  if (num_seqs == 0 && num_tokens != 0) return fail(PKV_EINVAL, "tokens without sequences");
  if (num_seqs > 0) {
    if (qsl[0] != 0) return fail(PKV_EINVAL, "query_start_loc[0] must be 0");
    if (qsl[num_seqs] != num_tokens)
      return fail(PKV_EINVAL, "query_start_loc[num_seqs]=%d != num_tokens=%d", qsl[num_seqs],
                  num_tokens);
  }
  const int G = s->num_q_heads / s->num_kv_heads;
  for (int r = 0; r < num_seqs; ++r) {
    const int32_t ql = qsl[r + 1] - qsl[r];
    if (ql < 0) return fail(PKV_EINVAL, "query_start_loc not ascending at %d", r);
    if (ctx[r] < 0) return fail(PKV_EINVAL, "context_lens[%d] negative", r);
    if ((int64_t)seq[r] != (int64_t)ctx[r] + ql)
      return fail(PKV_EINVAL, "seq_lens[%d]=%d != context_lens %d + query len %d", r, seq[r],
                  ctx[r], ql);
    if (ceil_div(seq[r], s->block_size) > s->bt_stride)
      return fail(PKV_EINVAL, "seq_lens[%d]=%d needs more than bt_stride=%d blocks", r, seq[r],
                  s->bt_stride);
    if (ceil_div(seq[r], s->block_size) > s->num_blocks && ql > 0)
      return fail(PKV_EINVAL, "seq_lens[%d]=%d needs more blocks than the pool has", r, seq[r]);
  }
  // Split size for decode rows: the smallest power of two (>= kMinBlocksPerSplit, <= 256
  // blocks, i.e. at most 64 per wave, which the decode kernel relies on) whose item count
  // times Hkv stays within the target workgroup count.
  // Prefill tiles hold 256 packed (token, q head) rows (wide tiles) when the batch has enough
  // rows in requests long enough to fill them, else 128.
  int64_t wide_rows = 0;
  for (int r = 0; r < num_seqs; ++r) {
    const int64_t rows = (int64_t)(qsl[r + 1] - qsl[r]) * G;
    if (qsl[r + 1] - qsl[r] > 1 && rows >= pkv::kWideTileRows) wide_rows += rows;
  }
  P.tile_rows = wide_rows >= pkv::kPrefillRowsForWideTiles ? pkv::kWideTileRows : pkv::kTileRows;
  const int tok_per_tile = P.tile_rows / G;
  // Rows of 2 .. kShortRowsMax / G tokens run as short items, split by keys like decode rows
  // but with a split size of their own: a short split writes ql partial rows and pays the
  // item's setup and wave merge, so fewer, longer splits run faster (measured on rows of
  // 1 + 4 tokens: 256-block splits 121 us, 64-block 134 us, 16-block 174 us) as long as the
  // short items still give every CU a workgroup.  Their size is the largest power of two
  // (kMinBlocksPerSplit .. 256 blocks) whose item count times Hkv reaches 256.
  auto is_short = [&](int32_t ql) { return ql > 1 && (int64_t)ql * G <= pkv::kShortRowsMax; };
  auto count_items = [&](bool shorts, int split) {
    int64_t n = 0;
    for (int r = 0; r < num_seqs; ++r) {
      const int32_t ql = qsl[r + 1] - qsl[r];
      if (shorts ? is_short(ql) : ql == 1) n += ceil_div(ceil_div(seq[r], pkv::kBlockSize), split);
    }
    return n;
  };
  int bps_short = 256;
  while (bps_short > pkv::kMinBlocksPerSplit && count_items(true, bps_short) * s->num_kv_heads < 256) bps_short /= 2;
  const int64_t short_wgs = count_items(true, bps_short) * s->num_kv_heads;
  int bps = pkv::kMinBlocksPerSplit;
  for (; bps < 256; bps *= 2)
    if (count_items(false, bps) * s->num_kv_heads + short_wgs <= kDecodeTargetWorkgroups) break;
  P.bps = bps;
  P.items.clear();
  P.token_split.assign((size_t)num_tokens * 3, 0);
  for (int32_t t = 0; t < num_tokens; ++t) {
    P.token_split[3 * t] = -1;
    P.token_split[3 * t + 1] = 1;
    P.token_split[3 * t + 2] = 1;
  }
  std::vector<pkv::WorkItem> pre, dec, shrt;
  int32_t partials = 0;
  for (int r = 0; r < num_seqs; ++r) {
    const int32_t ql = qsl[r + 1] - qsl[r];
    if (ql == 0) continue;
    if (ql == 1) {
      const int32_t nblk = (int32_t)ceil_div(seq[r], pkv::kBlockSize);
      const int32_t splits = (int32_t)ceil_div(nblk, bps);
      const int32_t t = qsl[r];
      if (splits > 1) {
        P.token_split[3 * t] = partials;
        P.token_split[3 * t + 1] = splits;
      }
      for (int32_t sidx = 0; sidx < splits; ++sidx) {
        pkv::WorkItem it;
        it.seq = r;
        it.kind = pkv::kDecode;
        it.q_begin = 0;
        it.q_count = splits;
        it.kv_begin = split_start(nblk, bps, splits, sidx) * pkv::kBlockSize;
        it.kv_end = std::min<int32_t>(seq[r], split_start(nblk, bps, splits, sidx + 1) * pkv::kBlockSize);
        it.partial_base = splits > 1 ? partials : -1;
        it.split = sidx;
        dec.push_back(it);
      }
      if (splits > 1) partials += splits;
    } else if (is_short(ql)) {
      // Token t of split s writes partial row base + s * ql + t; the reduce merges the splits
      // of each token (stride ql).
      const int32_t nblk = (int32_t)ceil_div(seq[r], pkv::kBlockSize);
      const int32_t splits = (int32_t)ceil_div(nblk, bps_short);
      if (splits > 1) {
        for (int32_t i = 0; i < ql; ++i) {
          const int32_t t = qsl[r] + i;
          P.token_split[3 * t] = partials + i;
          P.token_split[3 * t + 1] = splits;
          P.token_split[3 * t + 2] = ql;
        }
      }
      for (int32_t sidx = 0; sidx < splits; ++sidx) {
        pkv::WorkItem it;
        it.seq = r;
        it.kind = pkv::kShort;
        it.q_begin = 0;
        it.q_count = ql;
        it.kv_begin = split_start(nblk, bps_short, splits, sidx) * pkv::kBlockSize;
        it.kv_end = std::min<int32_t>(seq[r], split_start(nblk, bps_short, splits, sidx + 1) * pkv::kBlockSize);
        it.partial_base = splits > 1 ? partials + sidx * ql : -1;
        it.split = sidx;
        shrt.push_back(it);
      }
      if (splits > 1) partials += splits * ql;
    } else {
      const int32_t tiles = (int32_t)ceil_div(ql, tok_per_tile);
      // A short row over a long context (one 128-row tile of at most kSplitRowsMax rows) is
      // cut into key splits: token t of split s writes partial row base + s * ql + t, and the
      // reduce merges the splits of each token (stride ql).
      const bool cut = P.tile_rows == pkv::kTileRows && (int64_t)ql * G <= pkv::kSplitRowsMax &&
                       seq[r] > pkv::kPrefillSplitKeys;
      if (cut) {
        const int32_t splits = (int32_t)ceil_div(seq[r], pkv::kPrefillSplitKeys);
        for (int32_t i = 0; i < ql; ++i) {
          const int32_t t = qsl[r] + i;
          P.token_split[3 * t] = partials + i;
          P.token_split[3 * t + 1] = splits;
          P.token_split[3 * t + 2] = ql;
        }
        for (int32_t sidx = 0; sidx < splits; ++sidx) {
          pkv::WorkItem it;
          it.seq = r;
          it.kind = pkv::kPrefill;
          it.q_begin = 0;
          it.q_count = ql;
          it.kv_begin = sidx * pkv::kPrefillSplitKeys;
          it.kv_end = std::min<int32_t>(seq[r], (sidx + 1) * pkv::kPrefillSplitKeys);
          it.partial_base = partials + sidx * ql;
          it.split = sidx;
          pre.push_back(it);
        }
        partials += splits * ql;
        continue;
      }
      for (int32_t i = 0; i < tiles; ++i) {
        pkv::WorkItem it;
        it.seq = r;
        it.kind = pkv::kPrefill;
        it.q_begin = i * tok_per_tile;
        it.q_count = std::min<int32_t>(tok_per_tile, ql - it.q_begin);
        it.kv_begin = 0;
        it.kv_end = std::min<int32_t>(seq[r], ctx[r] + it.q_begin + it.q_count);
        it.partial_base = -1;
        it.split = 0;
        pre.push_back(it);
      }
    }
  }
  // Heaviest first: prefill tiles by (rows x keys), then decode items by key count.
  std::stable_sort(pre.begin(), pre.end(), [](const pkv::WorkItem& x, const pkv::WorkItem& y) {
    return (int64_t)x.q_count * (x.kv_end - x.kv_begin) > (int64_t)y.q_count * (y.kv_end - y.kv_begin);
  });
  auto by_keys = [](const pkv::WorkItem& x, const pkv::WorkItem& y) {
    return (x.kv_end - x.kv_begin) > (y.kv_end - y.kv_begin);
  };
  std::stable_sort(dec.begin(), dec.end(), by_keys);
  std::stable_sort(shrt.begin(), shrt.end(), by_keys);
  P.items = pre;
  P.items.insert(P.items.end(), dec.begin(), dec.end());
  P.items.insert(P.items.end(), shrt.begin(), shrt.end());
  P.n_short = (int32_t)shrt.size();
  P.num_partials = partials;
  P.n_prefill = (int32_t)pre.size();
  P.n_decode = (int32_t)dec.size();
  // Decode items in a launch of their own (no 128-row tiles beside them) run one wave per
  // workgroup when every item fits one wave (one block id per lane: at most 64 blocks), q heads
  // share a kv head eight at a time, and there are at least kOneWaveDecodeItems of them (two
  // rounds of the one-wave workgroups the chip holds at two waves per SIMD).  Short rows cut
  // from a long shared prefix (a cascade's suffix pass) are the case: the 4-wave item's start
  // and cross-wave merge are then a large part of its time.
  int32_t max_blocks = 0;
  for (const pkv::WorkItem& it : dec)
    max_blocks = std::max<int32_t>(max_blocks, (int32_t)ceil_div(it.kv_end, pkv::kBlockSize) -
                                                   it.kv_begin / pkv::kBlockSize);
  const bool decode_alone = P.n_prefill == 0 || P.tile_rows == pkv::kWideTileRows;
  P.decode_waves = decode_alone && G >= 8 && max_blocks <= 64 &&
                           (int64_t)P.n_decode * s->num_kv_heads >= kOneWaveDecodeItems
                       ? 1
                       : 4;
  return PKV_OK;
}

void fill_plan_struct(pkv_varlen_plan* out, const Plan& P, int32_t num_seqs, int32_t num_tokens,
                      const pkv_shape* s) {
  out->num_seqs = num_seqs;
  out->num_tokens = num_tokens;
  out->num_items = (int32_t)P.items.size();
  out->num_prefill_items = P.n_prefill;
  out->num_decode_items = P.n_decode;
  out->num_short_items = P.n_short;
  out->num_partials = P.num_partials;
  out->blocks_per_split = P.bps;
  out->has_splits = P.num_partials > 0;
  out->head_dim = s->head_dim;
  out->num_q_heads = s->num_q_heads;
  out->num_kv_heads = s->num_kv_heads;
  out->block_size = s->block_size;
  out->tile_rows = P.tile_rows;
  out->decode_waves = P.decode_waves;
  const VarlenLayout L =
      varlen_layout(out->num_items, num_tokens, P.num_partials, s->num_q_heads, s->head_dim);
  out->workspace_used = (int64_t)L.total;
}

// Pinned host staging for the plan upload: a ring of kStagingSlots buffers per device and thread,
// so a buffer is only refilled after the copy that last read it has completed.  The whole ring
// (kStagingSlots x kStagingSlotBytes of pinned memory) is allocated on the first upload of a
// thread on a device; after that an upload allocates nothing unless a plan is larger than a slot
// (more than kStagingSlotBytes / 32 work items), when that slot grows once.  An upload waits
// only when the host has enqueued kStagingSlots uploads that the device has not yet read.
struct StagingSlot {
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  bool pending = false;
};
constexpr int kStagingSlots = 32;
constexpr size_t kStagingSlotBytes = size_t(256) << 10;
struct StagingRing {
  StagingSlot slot[kStagingSlots];
  int next = 0;
  bool ready = false;
};
thread_local std::unordered_map<int, StagingRing> g_rings;

int grow_slot(StagingSlot& sl, size_t bytes) {
  if (sl.host) (void)hipHostFree(sl.host);
  sl.host = nullptr;
  sl.cap = 0;
  hipError_t e = hipHostMalloc(&sl.host, bytes, hipHostMallocDefault);
  if (e != hipSuccess) return hip_fail(e, "hipHostMalloc(staging)");
  sl.cap = bytes;
  return PKV_OK;
}

int stage_and_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return PKV_OK;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  StagingRing& ring = g_rings[dev];
  if (!ring.ready) {
    for (StagingSlot& s0 : ring.slot) {
      if (int rc = grow_slot(s0, kStagingSlotBytes)) return rc;
      e = hipEventCreateWithFlags(&s0.ev, hipEventDisableTiming);
      if (e != hipSuccess) return hip_fail(e, "hipEventCreate(staging)");
    }
    ring.ready = true;
  }
  StagingSlot& sl = ring.slot[ring.next];
  ring.next = (ring.next + 1) % kStagingSlots;
  if (sl.pending) {
    // The copy that last read this buffer was enqueued kStagingSlots uploads ago.
    e = hipEventSynchronize(sl.ev);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize(staging)");
    sl.pending = false;
  }
  if (sl.cap < bytes)
    if (int rc = grow_slot(sl, bytes)) return rc;
  std::memcpy(sl.host, src, bytes);
  e = hipMemcpyAsync(dst, sl.host, bytes, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(plan)");
  e = hipEventRecord(sl.ev, stream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord(staging)");
  sl.pending = true;
  return PKV_OK;
}

// Launch timing of the varlen attention kernel: while enabled (per thread), every varlen launch
// is bracketed by a pair of HIP events recorded on the caller's stream immediately before and
// after the kernel (the split-KV reduce is outside the pair).
struct LaunchTiming {
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pool;
  size_t used = 0;
  std::vector<double> last;  // per-launch milliseconds of the window pkv_timing_end closed
};
thread_local LaunchTiming g_timing;

int timing_mark(hipStream_t stream, bool before) {
  if (!g_timing.on) return PKV_OK;
  if (before) {
    if (g_timing.used == g_timing.pool.size()) {
      hipEvent_t a, b;
      hipError_t e = hipEventCreate(&a);
      if (e != hipSuccess) return hip_fail(e, "hipEventCreate(timing)");
      e = hipEventCreate(&b);
      if (e != hipSuccess) return hip_fail(e, "hipEventCreate(timing)");
      g_timing.pool.emplace_back(a, b);
    }
    hipError_t e = hipEventRecord(g_timing.pool[g_timing.used].first, stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord(timing)");
  } else {
    hipError_t e = hipEventRecord(g_timing.pool[g_timing.used].second, stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord(timing)");
    ++g_timing.used;
  }
  return PKV_OK;
}

// Cascade segmenting: enough (tile, segment) workgroups to give every CU one 8-wave workgroup,
// with segments of at least 1024 keys, rounded to whole KV tiles.
struct CascadeSplit {
  int32_t tiles, segs, seg_len;
};
CascadeSplit cascade_split(int32_t num_tokens, int32_t prefix_len, const pkv_shape* s) {
  const int G = s->num_q_heads / s->num_kv_heads;
  CascadeSplit c;
  c.tiles = (int32_t)ceil_div(num_tokens, pkv::kWideTileRows / G);
  const int64_t wgs = std::max<int64_t>(1, (int64_t)c.tiles * s->num_kv_heads);
  const int64_t want = ceil_div(256, wgs);  // one wide-tile workgroup per CU
  const int64_t max_segs = std::max<int64_t>(1, prefix_len / 1024);
  int64_t segs = std::max<int64_t>(1, std::min(want, max_segs));
  int64_t seg_len = ceil_div(ceil_div(prefix_len, segs), pkv::kKvTile) * pkv::kKvTile;
  segs = ceil_div(prefix_len, seg_len);
  c.segs = (int32_t)segs;
  c.seg_len = (int32_t)seg_len;
  return c;
}

size_t cascade_bytes(const CascadeSplit& c, int32_t num_tokens, const pkv_shape* s) {
  if (c.segs <= 1) return 0;
  const size_t rows = (size_t)c.segs * num_tokens * s->num_q_heads;
  return align256(rows * sizeof(float)) + align256(rows * s->head_dim * sizeof(float));
}

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_error.c_str(); }

const char* pkv_version(void) { return "pkv 0.1 (gfx950)"; }

int pkv_timing_begin(void) {
  g_timing.on = true;
  g_timing.used = 0;
  return ok();
}

int pkv_timing_end(double* total_ms, int32_t* launches) {
  if (!total_ms || !launches) return fail(PKV_EINVAL, "null pointer argument");
  g_timing.on = false;
  double sum = 0.0;
  g_timing.last.clear();
  for (size_t i = 0; i < g_timing.used; ++i) {
    hipError_t e = hipEventSynchronize(g_timing.pool[i].second);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize(timing)");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, g_timing.pool[i].first, g_timing.pool[i].second);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime(timing)");
    sum += ms;
    g_timing.last.push_back(ms);
  }
  *total_ms = sum;
  *launches = (int32_t)g_timing.used;
  g_timing.used = 0;
  return ok();
}

int pkv_timing_durations(double* ms_each, int32_t capacity) {
  if (capacity < 0 || (capacity > 0 && !ms_each)) return fail(PKV_EINVAL, "bad duration buffer");
  const size_t n = std::min<size_t>((size_t)capacity, g_timing.last.size());
  for (size_t i = 0; i < n; ++i) ms_each[i] = g_timing.last[i];
  g_error.clear();
  return (int)g_timing.last.size();
}

size_t pkv_varlen_workspace_size(int32_t num_seqs, int32_t num_tokens, int32_t max_seq_len,
                                 const pkv_shape* shape) {
  if (check_shape(shape) != PKV_OK || num_seqs < 0 || num_tokens < 0 || max_seq_len < 0) return 0;
  const int G = shape->num_q_heads / shape->num_kv_heads;
  const int64_t per_row = ceil_div(ceil_div(max_seq_len, pkv::kBlockSize), pkv::kMinBlocksPerSplit);
  // Key splits of short multi-token rows: at most kSplitRowsMax / G tokens per such row.
  const int64_t cut_splits = ceil_div(max_seq_len, pkv::kPrefillSplitKeys);
  const int64_t cut_tokens = std::min<int64_t>(num_tokens, (int64_t)num_seqs * std::max(1, pkv::kSplitRowsMax / G));
  const int64_t items = ceil_div((int64_t)num_tokens * G, 128) + num_seqs +
                        (int64_t)num_seqs * std::max<int64_t>(1, per_row) + (int64_t)num_seqs * cut_splits;
  const int64_t short_tokens = std::min<int64_t>(num_tokens, (int64_t)num_seqs * std::max(1, pkv::kShortRowsMax / G));
  const int64_t partials = (int64_t)num_seqs * std::max<int64_t>(1, per_row) + cut_tokens * cut_splits +
                           short_tokens * std::max<int64_t>(1, per_row);
  return varlen_layout(items, num_tokens, partials, shape->num_q_heads, shape->head_dim).total;
}

int pkv_compute_slot_mapping(int64_t* slot_mapping, const int32_t* block_tables,
                             const int32_t* query_start_loc, const int32_t* context_lens,
                             int32_t num_seqs, int32_t num_tokens, const pkv_shape* shape,
                             void* stream) {
  if (int rc = check_shape(shape)) return rc;
  if (num_tokens < 0 || num_seqs < 0) return fail(PKV_EINVAL, "negative sizes");
  if (num_tokens == 0) return ok();
  if (num_seqs == 0) return fail(PKV_EINVAL, "tokens without sequences");
  if (!slot_mapping || !block_tables || !query_start_loc || !context_lens)
    return fail(PKV_EINVAL, "null pointer argument");
  hipError_t e = pkv::launch_slot_mapping(slot_mapping, block_tables, query_start_loc,
                                          context_lens, num_seqs, num_tokens, shape->bt_stride,
                                          bs_log2(shape), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "slot_mapping launch");
  return ok();
}

int pkv_append_kv(int64_t* slot_mapping, const void* k, const void* v, void* k_cache,
                  void* v_cache, const int32_t* block_tables, const int32_t* query_start_loc,
                  const int32_t* context_lens, int32_t num_seqs, int32_t num_tokens,
                  const pkv_shape* shape, void* stream) {
  if (int rc = check_shape(shape)) return rc;
  if (num_tokens < 0 || num_seqs < 0) return fail(PKV_EINVAL, "negative sizes");
  if (num_tokens == 0) return ok();
  if (num_seqs == 0) return fail(PKV_EINVAL, "tokens without sequences");
  if (!k || !v || !k_cache || !v_cache || !block_tables || !query_start_loc || !context_lens)
    return fail(PKV_EINVAL, "null pointer argument");
  const int64_t num_slots = (int64_t)shape->num_blocks * shape->block_size;
  hipError_t e = pkv::launch_append_kv(
      slot_mapping, static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
      static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), block_tables,
      query_start_loc, context_lens, num_seqs, num_tokens, shape->num_kv_heads, shape->head_dim,
      shape->bt_stride, num_slots, bs_log2(shape), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "append_kv launch");
  return ok();
}

int pkv_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                          const int64_t* slot_mapping, int32_t num_tokens,
                          const pkv_shape* shape, void* stream) {
  if (int rc = check_shape(shape)) return rc;
  if (num_tokens < 0) return fail(PKV_EINVAL, "negative num_tokens");
  if (num_tokens == 0) return ok();
  if (!k || !v || !k_cache || !v_cache || !slot_mapping)
    return fail(PKV_EINVAL, "null pointer argument");
  const int64_t num_slots = (int64_t)shape->num_blocks * shape->block_size;
  hipError_t e = pkv::launch_reshape_and_cache(
      static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
      static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), slot_mapping, num_tokens,
      shape->num_kv_heads, shape->head_dim, num_slots, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "reshape_and_cache launch");
  return ok();
}

int pkv_append_kv_fp8(int64_t* slot_mapping, const void* k, const void* v, void* k_cache,
                      void* v_cache, const float* k_scale, const float* v_scale,
                      const int32_t* block_tables, const int32_t* query_start_loc,
                      const int32_t* context_lens, int32_t num_seqs, int32_t num_tokens,
                      const pkv_shape* shape, void* stream) {
  if (int rc = check_shape(shape)) return rc;
  if (num_tokens < 0 || num_seqs < 0) return fail(PKV_EINVAL, "negative sizes");
  if (num_tokens == 0) return ok();
  if (num_seqs == 0) return fail(PKV_EINVAL, "tokens without sequences");
  if (!k || !v || !k_cache || !v_cache || !k_scale || !v_scale || !block_tables ||
      !query_start_loc || !context_lens)
    return fail(PKV_EINVAL, "null pointer argument");
  const int64_t num_slots = (int64_t)shape->num_blocks * shape->block_size;
  hipError_t e = pkv::launch_append_kv_fp8(
      slot_mapping, static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
      static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache), k_scale, v_scale, block_tables,
      query_start_loc, context_lens, num_seqs, num_tokens, shape->num_kv_heads, shape->head_dim,
      shape->bt_stride, num_slots, bs_log2(shape), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "append_kv_fp8 launch");
  return ok();
}

int pkv_reshape_and_cache_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                              const float* k_scale, const float* v_scale,
                              const int64_t* slot_mapping, int32_t num_tokens,
                              const pkv_shape* shape, void* stream) {
  if (int rc = check_shape(shape)) return rc;
  if (num_tokens < 0) return fail(PKV_EINVAL, "negative num_tokens");
  if (num_tokens == 0) return ok();
  if (!k || !v || !k_cache || !v_cache || !k_scale || !v_scale || !slot_mapping)
    return fail(PKV_EINVAL, "null pointer argument");
  const int64_t num_slots = (int64_t)shape->num_blocks * shape->block_size;
  hipError_t e = pkv::launch_reshape_and_cache_fp8(
      static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), static_cast<uint8_t*>(k_cache),
      static_cast<uint8_t*>(v_cache), k_scale, v_scale, slot_mapping, num_tokens, shape->num_kv_heads,
      shape->head_dim, num_slots, bs_log2(shape), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "reshape_and_cache_fp8 launch");
  return ok();
}

int pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs, int32_t num_pairs,
                    const pkv_shape* shape, void* stream) {
  if (int rc = check_shape(shape)) return rc;
  if (num_pairs < 0) return fail(PKV_EINVAL, "negative num_pairs");
  if (num_pairs == 0) return ok();
  if (!k_cache || !v_cache || !block_pairs) return fail(PKV_EINVAL, "null pointer argument");
  hipError_t e = pkv::launch_copy_blocks(k_cache, v_cache, nullptr, nullptr, block_pairs, num_pairs,
                                         shape->num_blocks, shape->block_size, shape->num_kv_heads,
                                         shape->head_dim, 2, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "copy_blocks launch");
  return ok();
}

int pkv_copy_blocks_fp8(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                        const int32_t* block_pairs, int32_t num_pairs, const pkv_shape* shape,
                        void* stream) {
  if (int rc = check_shape(shape)) return rc;
  if (num_pairs < 0) return fail(PKV_EINVAL, "negative num_pairs");
  if (num_pairs == 0) return ok();
  if (!k_cache || !v_cache || !k_scale || !v_scale || !block_pairs)
    return fail(PKV_EINVAL, "null pointer argument");
  hipError_t e = pkv::launch_copy_blocks(k_cache, v_cache, k_scale, v_scale, block_pairs, num_pairs,
                                         shape->num_blocks, shape->block_size, shape->num_kv_heads,
                                         shape->head_dim, 1, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "copy_blocks launch");
  return ok();
}

int pkv_plan_varlen_host(pkv_varlen_plan* plan, int32_t* items, int32_t max_items,
                         const int32_t* h_query_start_loc, const int32_t* h_context_lens,
                         const int32_t* h_seq_lens, int32_t num_seqs, int32_t num_tokens,
                         const pkv_shape* shape) {
  if (int rc = check_shape(shape)) return rc;
  if (!plan) return fail(PKV_EINVAL, "plan is null");
  Plan P;
  if (int rc = build_plan(P, h_query_start_loc, h_context_lens, h_seq_lens, num_seqs, num_tokens,
                          shape))
    return rc;
  fill_plan_struct(plan, P, num_seqs, num_tokens, shape);
  if (items) {
    if ((int64_t)P.items.size() > max_items)
      return fail(PKV_EWORKSPACE, "plan has %zu items, buffer holds %d", P.items.size(), max_items);
    std::memcpy(items, P.items.data(), P.items.size() * sizeof(pkv::WorkItem));
  }
  return ok();
}

int pkv_plan_varlen(pkv_varlen_plan* plan, void* workspace, size_t workspace_bytes,
                    const int32_t* h_query_start_loc, const int32_t* h_context_lens,
                    const int32_t* h_seq_lens, int32_t num_seqs, int32_t num_tokens,
                    const pkv_shape* shape, void* stream) {
  if (int rc = check_shape(shape)) return rc;
  if (!plan) return fail(PKV_EINVAL, "plan is null");
  thread_local Plan P;
  if (int rc = build_plan(P, h_query_start_loc, h_context_lens, h_seq_lens, num_seqs, num_tokens,
                          shape))
    return rc;
  fill_plan_struct(plan, P, num_seqs, num_tokens, shape);
  if (plan->num_items == 0) return ok();
  if (!workspace) return fail(PKV_EINVAL, "workspace is null");
  if ((size_t)plan->workspace_used > workspace_bytes)
    return fail(PKV_EWORKSPACE, "plan needs %lld workspace bytes, got %zu",
                (long long)plan->workspace_used, workspace_bytes);
  const VarlenLayout L =
      varlen_layout(plan->num_items, num_tokens, P.num_partials, shape->num_q_heads, shape->head_dim);
  // One upload: the items followed (at split_off) by the per-token split table.
  thread_local std::vector<char> host;
  const size_t bytes = P.num_partials > 0 ? L.split_off + P.token_split.size() * sizeof(int32_t)
                                          : P.items.size() * sizeof(pkv::WorkItem);
  host.assign(bytes, 0);
  std::memcpy(host.data(), P.items.data(), P.items.size() * sizeof(pkv::WorkItem));
  if (P.num_partials > 0)
    std::memcpy(host.data() + L.split_off, P.token_split.data(),
                P.token_split.size() * sizeof(int32_t));
  if (int rc = stage_and_copy(workspace, host.data(), bytes, (hipStream_t)stream)) return rc;
  return ok();
}

static int varlen_impl(void* out, int32_t out_dtype, float* lse, const void* q,
                       const void* k_cache, const void* v_cache, const float* k_scale,
                       const float* v_scale, bool fp8, const int32_t* block_tables,
                       const int32_t* query_start_loc, const int32_t* context_lens,
                       const int32_t* seq_lens, int32_t num_seqs, int32_t num_tokens,
                       const pkv_shape* shape, const pkv_varlen_plan* plan, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (int rc = check_shape(shape)) return rc;
  if (!plan) return fail(PKV_EINVAL, "plan is null");
  if (out_dtype != PKV_DTYPE_BF16 && out_dtype != PKV_DTYPE_F32)
    return fail(PKV_EINVAL, "out_dtype %d unsupported", out_dtype);
  if (plan->num_seqs != num_seqs || plan->num_tokens != num_tokens ||
      plan->head_dim != shape->head_dim || plan->num_q_heads != shape->num_q_heads ||
      plan->num_kv_heads != shape->num_kv_heads)
    return fail(PKV_EINVAL, "plan was made for different metadata or shape");
  if (plan->decode_waves != 1 && plan->decode_waves != 4)
    return fail(PKV_EINVAL, "plan decode_waves %d invalid (1 or 4)", plan->decode_waves);
  if (num_tokens == 0 || plan->num_items == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !query_start_loc || !context_lens ||
      !seq_lens || !workspace || (fp8 && (!k_scale || !v_scale)))
    return fail(PKV_EINVAL, "null pointer argument");
  if ((size_t)plan->workspace_used > workspace_bytes)
    return fail(PKV_EWORKSPACE, "plan needs %lld workspace bytes, got %zu",
                (long long)plan->workspace_used, workspace_bytes);
  const VarlenLayout L = varlen_layout(plan->num_items, num_tokens, plan->num_partials,
                                       shape->num_q_heads, shape->head_dim);
  char* ws = static_cast<char*>(workspace);
  pkv::VarlenArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_tables = block_tables;
  a.query_start_loc = query_start_loc;
  a.context_lens = context_lens;
  a.seq_lens = seq_lens;
  a.out = out;
  a.lse = lse;
  a.out_f32 = out_dtype == PKV_DTYPE_F32;
  a.items = reinterpret_cast<const pkv::WorkItem*>(ws + L.items_off);
  a.num_items = plan->num_items;
  a.part_o = reinterpret_cast<float*>(ws + L.po_off);
  a.part_lse = reinterpret_cast<float*>(ws + L.plse_off);
  a.num_q_heads = shape->num_q_heads;
  a.num_kv_heads = shape->num_kv_heads;
  a.bt_stride = shape->bt_stride;
  a.bt_shift = bt_shift(shape);
  a.scale_log2 = scale_log2(shape);
  const int G = shape->num_q_heads / shape->num_kv_heads;
  if (int rc = timing_mark((hipStream_t)stream, true)) return rc;
  hipError_t e = (fp8 ? pkv::launch_varlen_fp8 : pkv::launch_varlen)(
      a, shape->head_dim, G, plan->num_prefill_items, plan->num_decode_items, plan->num_short_items,
      plan->tile_rows, plan->decode_waves, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "varlen attention launch");
  if (int rc = timing_mark((hipStream_t)stream, false)) return rc;
  if (plan->num_partials > 0) {
    pkv::ReduceArgs ra;
    ra.part_o = a.part_o;
    ra.part_lse = a.part_lse;
    ra.token_split = reinterpret_cast<const int32_t*>(ws + L.split_off);
    ra.uniform_count = 0;
    ra.num_tokens = num_tokens;
    ra.num_q_heads = shape->num_q_heads;
    ra.out = out;
    ra.out_f32 = a.out_f32;
    ra.lse = lse;
    e = pkv::launch_reduce(ra, shape->head_dim, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "split-KV reduce launch");
  }
  return ok();
}

int pkv_paged_attention_varlen(void* out, int32_t out_dtype, float* lse, const void* q,
                               const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* query_start_loc,
                               const int32_t* context_lens, const int32_t* seq_lens,
                               int32_t num_seqs, int32_t num_tokens, const pkv_shape* shape,
                               const pkv_varlen_plan* plan, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return varlen_impl(out, out_dtype, lse, q, k_cache, v_cache, nullptr, nullptr, false,
                     block_tables, query_start_loc, context_lens, seq_lens, num_seqs, num_tokens,
                     shape, plan, workspace, workspace_bytes, stream);
}

int pkv_paged_attention_varlen_fp8(void* out, int32_t out_dtype, float* lse, const void* q,
                                   const void* k_cache, const void* v_cache, const float* k_scale,
                                   const float* v_scale, const int32_t* block_tables,
                                   const int32_t* query_start_loc, const int32_t* context_lens,
                                   const int32_t* seq_lens, int32_t num_seqs, int32_t num_tokens,
                                   const pkv_shape* shape, const pkv_varlen_plan* plan,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return varlen_impl(out, out_dtype, lse, q, k_cache, v_cache, k_scale, v_scale, true,
                     block_tables, query_start_loc, context_lens, seq_lens, num_seqs, num_tokens,
                     shape, plan, workspace, workspace_bytes, stream);
}

// Device scratch of pkv_paged_attention_decode_noalloc: the split-KV partial states live in this
// file-scope array instead of a caller workspace.  In host code `scratch` is only the host-side
// handle of the symbol; its device address (one copy per GPU) comes from hipGetSymbolAddress,
// taken once per device on the entry point's first call there with that device current.
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

std::mutex g_scratch_mu;
std::unordered_map<int, void*> g_scratch_ptr;  // device ordinal -> device address of `scratch`

static int scratch_address(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    it = g_scratch_ptr.emplace(dev, p).first;
  }
  *ptr = it->second;
  return PKV_OK;
}

// Work split of a graph-capturable decode batch: the split size the varlen planner would pick
// if every row had max_seq_len keys (a power of two of 16 to 256 blocks of 16 keys), and the
// number of splits of the longest row.
struct DecodeSplit {
  int32_t splits, split_keys;
};
static DecodeSplit decode_split(int32_t num_seqs, int32_t max_seq_len, const pkv_shape* s) {
  const int64_t blocks = ceil_div(std::max(max_seq_len, 1), pkv::kBlockSize);
  int64_t bps = pkv::kMinBlocksPerSplit;
  while (bps < 256 && (int64_t)num_seqs * ceil_div(blocks, bps) * s->num_kv_heads > kDecodeTargetWorkgroups) bps *= 2;
  DecodeSplit d;
  d.split_keys = (int32_t)(bps * pkv::kBlockSize);
  d.splits = (int32_t)ceil_div(std::max(max_seq_len, 1), d.split_keys);
  return d;
}

static size_t decode_bytes(int32_t num_seqs, const DecodeSplit& d, const pkv_shape* s) {
  if (d.splits <= 1) return 0;
  const size_t rows = (size_t)d.splits * num_seqs * s->num_q_heads;
  return align256(rows * sizeof(float)) + align256(rows * s->head_dim * sizeof(float));
}

size_t pkv_decode_workspace_size(int32_t num_seqs, int32_t max_seq_len, const pkv_shape* shape) {
  if (check_shape(shape) != PKV_OK || num_seqs < 0 || max_seq_len < 0) return 0;
  return decode_bytes(num_seqs, decode_split(num_seqs, max_seq_len, shape), shape);
}

// use_scratch: the partial states go to the device scratch array (no workspace, no timing
// events); the call then allocates nothing.
static int decode_impl(void* out, int32_t out_dtype, float* lse, const void* q, const void* k_cache,
                       const void* v_cache, const float* k_scale, const float* v_scale, bool fp8,
                       const int32_t* block_tables, const int32_t* query_start_loc,
                       const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                       const pkv_shape* shape, void* workspace, size_t workspace_bytes,
                       void* stream, bool use_scratch = false) {
  if (int rc = check_shape(shape)) return rc;
  if (out_dtype != PKV_DTYPE_BF16 && out_dtype != PKV_DTYPE_F32)
    return fail(PKV_EINVAL, "out_dtype %d unsupported", out_dtype);
  if (num_seqs < 0 || max_seq_len < 0) return fail(PKV_EINVAL, "negative sizes");
  if (ceil_div(max_seq_len, shape->block_size) > shape->bt_stride)
    return fail(PKV_EINVAL, "max_seq_len %d needs more than bt_stride=%d blocks", max_seq_len,
                shape->bt_stride);
  if (num_seqs == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !query_start_loc || !seq_lens ||
      (fp8 && (!k_scale || !v_scale)))
    return fail(PKV_EINVAL, "null pointer argument");
  const DecodeSplit d = decode_split(num_seqs, max_seq_len, shape);
  const size_t need = decode_bytes(num_seqs, d, shape);
  if (use_scratch) {
    if (need > kDecodeScratchBytes)
      return fail(PKV_EWORKSPACE,
                  "decode of %d rows up to %d keys needs %zu bytes of partial states, more than the %zu-byte "
                  "device scratch of the allocation-free entry point",
                  num_seqs, max_seq_len, need, kDecodeScratchBytes);
    if (need > 0) {
      if (int rc = scratch_address(&workspace)) return rc;
      workspace_bytes = kDecodeScratchBytes;
    }
  }
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PKV_EWORKSPACE, "decode needs %zu workspace bytes, got %zu", need, workspace_bytes);
  pkv::VarlenArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_tables = block_tables;
  a.query_start_loc = query_start_loc;
  a.context_lens = nullptr;
  a.seq_lens = seq_lens;
  a.out = out;
  a.lse = lse;
  a.out_f32 = out_dtype == PKV_DTYPE_F32;
  a.items = nullptr;
  a.num_items = 0;
  const size_t rows = (size_t)d.splits * num_seqs * shape->num_q_heads;
  a.part_lse = need ? static_cast<float*>(workspace) : nullptr;
  a.part_o = need ? reinterpret_cast<float*>(static_cast<char*>(workspace) + align256(rows * sizeof(float)))
                  : nullptr;
  a.num_q_heads = shape->num_q_heads;
  a.num_kv_heads = shape->num_kv_heads;
  a.bt_stride = shape->bt_stride;
  a.bt_shift = bt_shift(shape);
  a.scale_log2 = scale_log2(shape);
  const int G = shape->num_q_heads / shape->num_kv_heads;
  if (!use_scratch)
    if (int rc = timing_mark((hipStream_t)stream, true)) return rc;
  hipError_t e = (fp8 ? pkv::launch_decode_graph_fp8 : pkv::launch_decode_graph)(
      a, shape->head_dim, G, num_seqs, d.splits, d.split_keys, num_seqs, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  if (!use_scratch)
    if (int rc = timing_mark((hipStream_t)stream, false)) return rc;
  if (d.splits > 1) {
    pkv::ReduceArgs ra;
    ra.part_o = a.part_o;
    ra.part_lse = a.part_lse;
    ra.token_split = nullptr;
    ra.uniform_count = d.splits;
    ra.num_tokens = num_seqs;
    ra.num_q_heads = shape->num_q_heads;
    ra.out = out;
    ra.out_f32 = a.out_f32;
    ra.lse = lse;
    e = pkv::launch_reduce(ra, shape->head_dim, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "decode split reduce launch");
  }
  return ok();
}

int pkv_paged_attention_decode(void* out, int32_t out_dtype, float* lse, const void* q,
                               const void* k_cache, const void* v_cache, const int32_t* block_tables,
                               const int32_t* query_start_loc, const int32_t* seq_lens,
                               int32_t num_seqs, int32_t max_seq_len, const pkv_shape* shape,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(out, out_dtype, lse, q, k_cache, v_cache, nullptr, nullptr, false, block_tables,
                     query_start_loc, seq_lens, num_seqs, max_seq_len, shape, workspace,
                     workspace_bytes, stream);
}

int pkv_paged_attention_decode_noalloc(void* out, int32_t out_dtype, float* lse, const void* q,
                                       const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, const int32_t* query_start_loc,
                                       const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                                       const pkv_shape* shape, void* stream) {
  return decode_impl(out, out_dtype, lse, q, k_cache, v_cache, nullptr, nullptr, false, block_tables,
                     query_start_loc, seq_lens, num_seqs, max_seq_len, shape, nullptr, 0, stream,
                     /*use_scratch=*/true);
}

int pkv_paged_attention_decode_fp8(void* out, int32_t out_dtype, float* lse, const void* q,
                                   const void* k_cache, const void* v_cache, const float* k_scale,
                                   const float* v_scale, const int32_t* block_tables,
                                   const int32_t* query_start_loc, const int32_t* seq_lens,
                                   int32_t num_seqs, int32_t max_seq_len, const pkv_shape* shape,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(out, out_dtype, lse, q, k_cache, v_cache, k_scale, v_scale, true, block_tables,
                     query_start_loc, seq_lens, num_seqs, max_seq_len, shape, workspace,
                     workspace_bytes, stream);
}

size_t pkv_cascade_workspace_size(int32_t num_tokens, int32_t prefix_len, const pkv_shape* shape) {
  if (check_shape(shape) != PKV_OK || num_tokens < 0 || prefix_len <= 0) return 0;
  return cascade_bytes(cascade_split(num_tokens, prefix_len, shape), num_tokens, shape);
}

static int cascade_impl(float* out_prefix, float* lse_prefix, const void* q, const void* k_cache,
                        const void* v_cache, const float* k_scale, const float* v_scale, bool fp8,
                        const int32_t* prefix_block_table, int32_t prefix_len, int32_t num_tokens,
                        const pkv_shape* shape, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (int rc = check_shape(shape)) return rc;
  if (prefix_len <= 0 || prefix_len % shape->block_size)
    return fail(PKV_EPREFIX, "prefix_len %d must be a positive multiple of block_size %d",
                prefix_len, shape->block_size);
  if (prefix_len / shape->block_size > shape->num_blocks)
    return fail(PKV_EINVAL, "prefix needs more blocks than the pool has");
  if (num_tokens < 0) return fail(PKV_EINVAL, "negative num_tokens");
  if (num_tokens == 0) return ok();
  if (!out_prefix || !lse_prefix || !q || !k_cache || !v_cache || !prefix_block_table ||
      (fp8 && (!k_scale || !v_scale)))
    return fail(PKV_EINVAL, "null pointer argument");
  const CascadeSplit cs = cascade_split(num_tokens, prefix_len, shape);
  const size_t need = cascade_bytes(cs, num_tokens, shape);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PKV_EWORKSPACE, "cascade needs %zu workspace bytes, got %zu", need, workspace_bytes);
  pkv::CascadeArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.prefix_bt = prefix_block_table;
  a.prefix_len = prefix_len;
  a.num_tokens = num_tokens;
  a.num_segments = cs.segs;
  a.seg_len = cs.seg_len;
  a.num_tiles = cs.tiles;
  a.out = out_prefix;
  a.lse = lse_prefix;
  const size_t rows = (size_t)cs.segs * num_tokens * shape->num_q_heads;
  a.part_lse = static_cast<float*>(workspace);
  a.part_o = cs.segs > 1
                 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + align256(rows * sizeof(float)))
                 : nullptr;
  a.num_q_heads = shape->num_q_heads;
  a.num_kv_heads = shape->num_kv_heads;
  a.bt_shift = bt_shift(shape);
  a.scale_log2 = scale_log2(shape);
  const int G = shape->num_q_heads / shape->num_kv_heads;
  if (int rc = timing_mark((hipStream_t)stream, true)) return rc;
  hipError_t e = (fp8 ? pkv::launch_cascade_fp8 : pkv::launch_cascade)(a, shape->head_dim, G,
                                                                       (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "cascade prefix launch");
  if (int rc = timing_mark((hipStream_t)stream, false)) return rc;
  if (cs.segs > 1) {
    pkv::ReduceArgs ra;
    ra.part_o = a.part_o;
    ra.part_lse = a.part_lse;
    ra.token_split = nullptr;
    ra.uniform_count = cs.segs;
    ra.num_tokens = num_tokens;
    ra.num_q_heads = shape->num_q_heads;
    ra.out = out_prefix;
    ra.out_f32 = 1;
    ra.lse = lse_prefix;
    e = pkv::launch_reduce(ra, shape->head_dim, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "cascade segment reduce launch");
  }
  return ok();
}

int pkv_cascade_prefix_attention(float* out_prefix, float* lse_prefix, const void* q,
                                 const void* k_cache, const void* v_cache,
                                 const int32_t* prefix_block_table, int32_t prefix_len,
                                 int32_t num_tokens, const pkv_shape* shape, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return cascade_impl(out_prefix, lse_prefix, q, k_cache, v_cache, nullptr, nullptr, false,
                      prefix_block_table, prefix_len, num_tokens, shape, workspace,
                      workspace_bytes, stream);
}

int pkv_cascade_prefix_attention_fp8(float* out_prefix, float* lse_prefix, const void* q,
                                     const void* k_cache, const void* v_cache,
                                     const float* k_scale, const float* v_scale,
                                     const int32_t* prefix_block_table, int32_t prefix_len,
                                     int32_t num_tokens, const pkv_shape* shape, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return cascade_impl(out_prefix, lse_prefix, q, k_cache, v_cache, k_scale, v_scale, true,
                      prefix_block_table, prefix_len, num_tokens, shape, workspace,
                      workspace_bytes, stream);
}

int pkv_merge_attn_states(void* out, int32_t out_dtype, float* lse_out, const float* out_a,
                          const float* lse_a, const float* out_b, const float* lse_b,
                          int32_t num_tokens, int32_t num_heads, int32_t head_dim, void* stream) {
  if (out_dtype != PKV_DTYPE_BF16 && out_dtype != PKV_DTYPE_F32)
    return fail(PKV_EINVAL, "out_dtype %d unsupported", out_dtype);
  if (num_tokens < 0 || num_heads <= 0 || head_dim <= 0 || head_dim % 4)
    return fail(PKV_EINVAL, "bad sizes (tokens %d, heads %d, head_dim %d)", num_tokens, num_heads,
                head_dim);
  if (num_tokens == 0) return ok();
  if (!out || !out_a || !lse_a || !out_b || !lse_b) return fail(PKV_EINVAL, "null pointer argument");
  hipError_t e = pkv::launch_merge(out, out_dtype == PKV_DTYPE_F32, lse_out, out_a, lse_a, out_b,
                                   lse_b, (int64_t)num_tokens * num_heads, head_dim,
                                   (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return ok();
}

}  // extern "C"
