// Slot mapping and the paged cache write.
//
// Paging ["11. vLLM principles", section 11.2 PagedAttention]: the cache is cut into blocks of
// 16 tokens; a request's block table maps logical block p / 16 to a physical block anywhere in
// the pool.  New tokens follow the cached ones [Tencent Cloud article on vLLM inference
// acceleration, chunked prefill and prefix caching sections], so token i of request r is at
// position context_lens[r] + i.  KV caching [2048ai.net vLLM V1 article, "KV Caching"] stores
// each new token's K and V at its slot.
#include "internal.h"

namespace pkv {
namespace {

constexpr int kCacheThreads = 256;
constexpr int kRunMax = kCacheThreads + 1;  // tokens a workgroup's run of threads can touch

// Owner and position of every token of a workgroup's run [t0, t0 + n) of new tokens, into LDS.
// query_start_loc holds num_seqs + 1 ascending entries; the owner of token t is the request r
// with qsl[r] <= t < qsl[r + 1] (requests with no new token own nothing) and the token's
// position is context_lens[r] + t - qsl[r].  A binary search per thread would chain about
// log2(num_seqs) dependent loads before the block table could be read; here the workgroup
// finds the owners together in one round of loads (two when num_seqs exceeds the workgroup):
//   * beyond blockDim requests, a coarse round samples qsl every S = ceil(num_seqs / blockDim)
//     requests and narrows the candidates to [last sample <= t0, first sample past the run);
//   * then thread j takes candidates lo + j, lo + j + blockDim, ..., loads qsl[r], qsl[r + 1]
//     and context_lens[r] together and writes r and the position for each token of the run
//     that r owns.
// Tokens nobody claims (a malformed qsl) keep owner -1.  Every thread of the workgroup must
// call this.
__device__ void find_owners(const int32_t* __restrict__ qsl, const int32_t* __restrict__ ctx,
                            int32_t num_seqs, int64_t t0, int32_t n, int32_t* s_owner,
                            int32_t* s_pos, int32_t* s_range) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int64_t t_end = t0 + n;  // one past the run's last token
  for (int i = tid; i < n; i += nt) s_owner[i] = -1;
  if (tid == 0) {
    s_range[0] = 0;
    s_range[1] = num_seqs;
  }
  // Every reset above happens before any thread records an owner below: a request's tokens can
  // lie in entries another wave resets.
  __syncthreads();
  int32_t lo = 0, hi = num_seqs;
  if (num_seqs > nt) {
    const int32_t S = (num_seqs + nt - 1) / nt;
    const int64_t r = (int64_t)tid * S;
    if (r < num_seqs) {
      const int32_t a = qsl[r];
      if (a <= t0) atomicMax(&s_range[0], (int32_t)r);
      if (a >= t_end) atomicMin(&s_range[1], (int32_t)r);
    }
    __syncthreads();
    lo = s_range[0];
    hi = s_range[1];
  }
  for (int64_t r = (int64_t)lo + tid; r < hi; r += nt) {
    const int32_t a = qsl[r], b = qsl[r + 1], c = ctx[r];
    const int64_t from = a > t0 ? a : t0, to = b < t_end ? b : t_end;
    for (int64_t t = from; t < to; ++t) {
      s_owner[t - t0] = (int32_t)r;
      s_pos[t - t0] = c + (int32_t)(t - a);
    }
  }
  __syncthreads();
}

// The run of tokens touched by this workgroup when thread gid handles token gid / per_token.
__device__ __forceinline__ void token_run(int64_t per_token, int32_t num_tokens, int64_t& t0, int32_t& n) {
  const int64_t g0 = (int64_t)blockIdx.x * blockDim.x;
  t0 = g0 / per_token;
  int64_t t1 = (g0 + blockDim.x - 1) / per_token;  // last token (inclusive)
  if (t1 > num_tokens - 1) t1 = num_tokens - 1;
  n = (int32_t)(t1 - t0 + 1);
}

// Slot of a token from its owner and position, or -1 (no owner, negative position, or a
// position past the block table's width).
__device__ __forceinline__ int64_t slot_of(const int32_t* __restrict__ bt, int32_t owner, int32_t pos,
                                           int32_t bt_stride, int32_t bs_log2) {
  if (owner < 0 || pos < 0) return -1;
  const int32_t logical = pos >> bs_log2;
  if (logical >= bt_stride) return -1;
  return ((int64_t)bt[(int64_t)owner * bt_stride + logical] << bs_log2) + (pos & ((1 << bs_log2) - 1));
}

// One thread per new token.
__global__ void __launch_bounds__(kCacheThreads)
slot_mapping_kernel(int64_t* __restrict__ slots, const int32_t* __restrict__ bt,
                    const int32_t* __restrict__ qsl, const int32_t* __restrict__ ctx, int32_t num_seqs,
                    int32_t num_tokens, int32_t bt_stride, int32_t bs_log2) {
  __shared__ int32_t s_owner[kRunMax], s_pos[kRunMax], s_range[2];
  int64_t t0;
  int32_t n;
  token_run(1, num_tokens, t0, n);
  find_owners(qsl, ctx, num_seqs, t0, n, s_owner, s_pos, s_range);
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= num_tokens) return;
  slots[t] = slot_of(bt, s_owner[t - t0], s_pos[t - t0], bt_stride, bs_log2);
}

// One thread per 16-byte chunk (8 bf16) of one token's K and V for one kv head.  A slot names
// (block, offset).  A block of 16 R tokens (R = 1, 2, ..., 16) is R consecutive 16-token tiles, so
// slot / 16 is the token's 16-token tile in the pool and slot % 16 its row there, whatever the
// block size.  The key pool is [tiles, Hkv, 16, D]: the token's key is one 16-byte store.  The
// value pool is [tiles, Hkv, D, 16] (dim-major, so attention can read 16-token rows of one
// dimension): the token's 8 values go to 8 rows, 2 bytes each.
__global__ void reshape_and_cache_kernel(const uint4* __restrict__ k, const uint4* __restrict__ v,
                                         uint4* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
                                         const int64_t* __restrict__ slots, int32_t num_tokens,
                                         int32_t num_kv_heads, int32_t chunks_per_head,
                                         int64_t num_slots) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_token = (int64_t)num_kv_heads * chunks_per_head;
  const int64_t t = gid / per_token;
  if (t >= num_tokens) return;
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t within = gid - t * per_token;
  const int64_t h = within / chunks_per_head;
  const int64_t c = within - h * chunks_per_head;
  const int64_t blk = slot / kBlockSize;
  const int64_t off = slot - blk * kBlockSize;
  const int64_t tile = blk * num_kv_heads + h;  // (block, head) tile index
  k_cache[(tile * kBlockSize + off) * chunks_per_head + c] = k[gid];
  const uint4 x = v[gid];
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint16_t* vt = v_cache + (tile * chunks_per_head * 8 + c * 8) * kBlockSize + off;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    vt[(2 * e) * kBlockSize] = (uint16_t)(w[e] & 0xffffu);
    vt[(2 * e + 1) * kBlockSize] = (uint16_t)(w[e] >> 16);
  }
}

// Slot mapping and cache write in one launch: one thread per 16-byte chunk of one token's K
// and V for one kv head.  The chunk loads are issued first; the workgroup finds its tokens'
// owners meanwhile (find_owners), then each thread reads its token's block table entry and
// stores the chunk; the (head 0, chunk 0) thread also records the slot when slot_mapping is
// given.
__global__ void __launch_bounds__(kCacheThreads)
append_kv_kernel(int64_t* __restrict__ slot_out, const uint4* __restrict__ k, const uint4* __restrict__ v,
                 uint4* __restrict__ k_cache, uint16_t* __restrict__ v_cache, const int32_t* __restrict__ bt,
                 const int32_t* __restrict__ qsl, const int32_t* __restrict__ ctx, int32_t num_seqs,
                 int32_t num_tokens, int32_t num_kv_heads, int32_t chunks_per_head, int32_t bt_stride,
                 int64_t num_slots, int32_t bs_log2) {
  __shared__ int32_t s_owner[kRunMax], s_pos[kRunMax], s_range[2];
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_token = (int64_t)num_kv_heads * chunks_per_head;
  const int64_t t = gid / per_token;
  const bool live = t < num_tokens;
  uint4 kx = {}, vx = {};
  if (live) {
    kx = k[gid];
    vx = v[gid];
  }
  int64_t t0;
  int32_t n;
  token_run(per_token, num_tokens, t0, n);
  find_owners(qsl, ctx, num_seqs, t0, n, s_owner, s_pos, s_range);
  if (!live) return;
  const int64_t slot = slot_of(bt, s_owner[t - t0], s_pos[t - t0], bt_stride, bs_log2);
  const int64_t within = gid - t * per_token;
  if (slot_out && within == 0) slot_out[t] = slot;
  if (slot < 0 || slot >= num_slots) return;
  const int64_t h = within / chunks_per_head;
  const int64_t c = within - h * chunks_per_head;
  const int64_t blk = slot / kBlockSize;
  const int64_t off = slot - blk * kBlockSize;
  const int64_t tile = blk * num_kv_heads + h;
  k_cache[(tile * kBlockSize + off) * chunks_per_head + c] = kx;
  const uint32_t w[4] = {vx.x, vx.y, vx.z, vx.w};
  uint16_t* vt = v_cache + (tile * chunks_per_head * 8 + c * 8) * kBlockSize + off;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    vt[(2 * e) * kBlockSize] = (uint16_t)(w[e] & 0xffffu);
    vt[(2 * e + 1) * kBlockSize] = (uint16_t)(w[e] >> 16);
  }
}


// ------------------------------------------------------------------------------------------
// FP8 (OCP E4M3FN) cache write.  Storing the cache in a low-precision float format shrinks it and
// speeds up attention [2048ai.net vLLM V1 article, quantisation section].  Every (physical block,
// kv head) tile of each pool has its own fp32 scale (k_scale / v_scale, [num_blocks, Hkv]): a
// stored code means code_value * scale.  A token's bf16 value x becomes
// y = x * (1 / scale) in fp32, clamped to +-448 (the largest finite code; the conversion
// instruction itself turns larger values into NaN instead of saturating), then rounded to the
// nearest code, ties to even, by v_cvt_pk_fp8_f32.  A NaN input stores the NaN code 0x7f.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ float fp8_clamp(float y) {
  return fabsf(y) > 448.f ? copysignf(448.f, y) : y;
}

// The 8 bf16 values of chunk x as 8 e4m3 codes (byte e = value e).  NaN inputs get the code
// 0x7f written explicitly, whatever code the conversion instruction gives a NaN.
__device__ __forceinline__ uint2 quantize8(const uint4 x, float inv) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t out[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float f[4];
    uint32_t nan_bytes = 0;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      f[2 * e] = __uint_as_float(w[2 * h + e] << 16) * inv;
      f[2 * e + 1] = __uint_as_float(w[2 * h + e] & 0xffff0000u) * inv;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (f[e] != f[e]) nan_bytes |= 0xffu << (8 * e);
      f[e] = fp8_clamp(f[e]);
    }
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);  // bytes 0, 1
    r = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], r, true);       // bytes 2, 3
    out[h] = ((uint32_t)r & ~nan_bytes) | (0x7f7f7f7fu & nan_bytes);
  }
  return make_uint2(out[0], out[1]);
}

// Store chunk c (8 values) of token slot `slot`, kv head h, into the fp8 pools: 8 key bytes in the
// token's row, 8 value bytes down 8 rows of the dim-major value tile.
__device__ __forceinline__ void store_fp8_chunk(const uint4 kx, const uint4 vx, uint2* __restrict__ k_cache,
                                                uint8_t* __restrict__ v_cache,
                                                const float* __restrict__ k_scale,
                                                const float* __restrict__ v_scale, int64_t slot,
                                                int64_t h, int64_t c, int32_t num_kv_heads,
                                                int32_t chunks_per_head, int32_t bs_log2) {
  const int64_t blk = slot / kBlockSize;  // 16-token tile
  const int64_t off = slot - blk * kBlockSize;
  const int64_t tile = blk * num_kv_heads + h;
  const int64_t sidx = (slot >> bs_log2) * num_kv_heads + h;  // scales: per (block, kv head)
  const float kinv = 1.0f / k_scale[sidx];
  const float vinv = 1.0f / v_scale[sidx];
  k_cache[(tile * kBlockSize + off) * chunks_per_head + c] = quantize8(kx, kinv);
  const uint2 vq = quantize8(vx, vinv);
  uint8_t* vt = v_cache + (tile * chunks_per_head * 8 + c * 8) * kBlockSize + off;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    vt[e * kBlockSize] = (uint8_t)(vq.x >> (8 * e));
    vt[(4 + e) * kBlockSize] = (uint8_t)(vq.y >> (8 * e));
  }
}

// As reshape_and_cache_kernel, quantising into fp8 pools.
__global__ void reshape_and_cache_fp8_kernel(const uint4* __restrict__ k, const uint4* __restrict__ v,
                                             uint2* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
                                             const float* __restrict__ k_scale,
                                             const float* __restrict__ v_scale,
                                             const int64_t* __restrict__ slots, int32_t num_tokens,
                                             int32_t num_kv_heads, int32_t chunks_per_head,
                                             int64_t num_slots, int32_t bs_log2) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_token = (int64_t)num_kv_heads * chunks_per_head;
  const int64_t t = gid / per_token;
  if (t >= num_tokens) return;
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t within = gid - t * per_token;
  const int64_t h = within / chunks_per_head;
  store_fp8_chunk(k[gid], v[gid], k_cache, v_cache, k_scale, v_scale, slot, h, within - h * chunks_per_head,
                  num_kv_heads, chunks_per_head, bs_log2);
}

// As append_kv_kernel, quantising into fp8 pools.
__global__ void __launch_bounds__(kCacheThreads)
append_kv_fp8_kernel(int64_t* __restrict__ slot_out, const uint4* __restrict__ k, const uint4* __restrict__ v,
                     uint2* __restrict__ k_cache, uint8_t* __restrict__ v_cache, const float* __restrict__ k_scale,
                     const float* __restrict__ v_scale, const int32_t* __restrict__ bt,
                     const int32_t* __restrict__ qsl, const int32_t* __restrict__ ctx, int32_t num_seqs,
                     int32_t num_tokens, int32_t num_kv_heads, int32_t chunks_per_head, int32_t bt_stride,
                     int64_t num_slots, int32_t bs_log2) {
  __shared__ int32_t s_owner[kRunMax], s_pos[kRunMax], s_range[2];
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_token = (int64_t)num_kv_heads * chunks_per_head;
  const int64_t t = gid / per_token;
  const bool live = t < num_tokens;
  uint4 kx = {}, vx = {};
  if (live) {
    kx = k[gid];
    vx = v[gid];
  }
  int64_t t0;
  int32_t n;
  token_run(per_token, num_tokens, t0, n);
  find_owners(qsl, ctx, num_seqs, t0, n, s_owner, s_pos, s_range);
  if (!live) return;
  const int64_t slot = slot_of(bt, s_owner[t - t0], s_pos[t - t0], bt_stride, bs_log2);
  const int64_t within = gid - t * per_token;
  if (slot_out && within == 0) slot_out[t] = slot;
  if (slot < 0 || slot >= num_slots) return;
  const int64_t h = within / chunks_per_head;
  store_fp8_chunk(kx, vx, k_cache, v_cache, k_scale, v_scale, slot, h, within - h * chunks_per_head,
                  num_kv_heads, chunks_per_head, bs_log2);
}

// Copy-on-write support ["11. vLLM principles", section 11.2: requests that share a prefix
// point their block tables at the same physical blocks]: before one of them writes into a
// shared block, the block is copied to a fresh one.  Workgroup (pair, pool) copies the whole
// physical block src -> dst of one pool (K for pool 0, V for pool 1; every kv head), 16 bytes
// per thread and step, and, for fp8 pools, the block's per-kv-head scales of that pool.  Pairs
// naming a block outside [0, num_blocks) are skipped.
__global__ void copy_blocks_kernel(uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
                                   float* __restrict__ k_scale, float* __restrict__ v_scale,
                                   const int32_t* __restrict__ pairs, int32_t num_blocks,
                                   int32_t num_kv_heads, int64_t chunks_per_block) {
  const int32_t p = blockIdx.x;
  const int32_t src = pairs[2 * p];
  const int32_t dst = pairs[2 * p + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
  uint4* pool = blockIdx.y == 0 ? k_cache : v_cache;
  const uint4* from = pool + (int64_t)src * chunks_per_block;
  uint4* to = pool + (int64_t)dst * chunks_per_block;
  for (int64_t c = threadIdx.x; c < chunks_per_block; c += blockDim.x) to[c] = from[c];
  float* scale = blockIdx.y == 0 ? k_scale : v_scale;
  if (scale && (int)threadIdx.x < num_kv_heads)
    scale[(int64_t)dst * num_kv_heads + threadIdx.x] = scale[(int64_t)src * num_kv_heads + threadIdx.x];
}

}  // namespace

hipError_t launch_append_kv(int64_t* slot_mapping, const uint16_t* k, const uint16_t* v,
                            uint16_t* k_cache, uint16_t* v_cache, const int32_t* block_tables,
                            const int32_t* qsl, const int32_t* ctx, int32_t num_seqs,
                            int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                            int32_t bt_stride, int64_t num_slots, int32_t bs_log2,
                            hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int32_t chunks = head_dim / 8;
  const int64_t total = (int64_t)num_tokens * num_kv_heads * chunks;
  const int threads = kCacheThreads;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(append_kv_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     slot_mapping, reinterpret_cast<const uint4*>(k),
                     reinterpret_cast<const uint4*>(v), reinterpret_cast<uint4*>(k_cache), v_cache,
                     block_tables, qsl, ctx, num_seqs, num_tokens, num_kv_heads, chunks, bt_stride,
                     num_slots, bs_log2);
  return hipGetLastError();
}

hipError_t launch_append_kv_fp8(int64_t* slot_mapping, const uint16_t* k, const uint16_t* v,
                                uint8_t* k_cache, uint8_t* v_cache, const float* k_scale,
                                const float* v_scale, const int32_t* block_tables, const int32_t* qsl,
                                const int32_t* ctx, int32_t num_seqs, int32_t num_tokens,
                                int32_t num_kv_heads, int32_t head_dim, int32_t bt_stride,
                                int64_t num_slots, int32_t bs_log2, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int32_t chunks = head_dim / 8;
  const int64_t total = (int64_t)num_tokens * num_kv_heads * chunks;
  const int threads = kCacheThreads;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(append_kv_fp8_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, slot_mapping,
                     reinterpret_cast<const uint4*>(k), reinterpret_cast<const uint4*>(v),
                     reinterpret_cast<uint2*>(k_cache), v_cache, k_scale, v_scale, block_tables, qsl, ctx,
                     num_seqs, num_tokens, num_kv_heads, chunks, bt_stride, num_slots, bs_log2);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache_fp8(const uint16_t* k, const uint16_t* v, uint8_t* k_cache,
                                        uint8_t* v_cache, const float* k_scale, const float* v_scale,
                                        const int64_t* slots, int32_t num_tokens, int32_t num_kv_heads,
                                        int32_t head_dim, int64_t num_slots, int32_t bs_log2,
                                        hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int32_t chunks = head_dim / 8;
  const int64_t total = (int64_t)num_tokens * num_kv_heads * chunks;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(reshape_and_cache_fp8_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     reinterpret_cast<const uint4*>(k), reinterpret_cast<const uint4*>(v),
                     reinterpret_cast<uint2*>(k_cache), v_cache, k_scale, v_scale, slots, num_tokens,
                     num_kv_heads, chunks, num_slots, bs_log2);
  return hipGetLastError();
}

hipError_t launch_slot_mapping(int64_t* slot_mapping, const int32_t* block_tables,
                               const int32_t* qsl, const int32_t* ctx, int32_t num_seqs,
                               int32_t num_tokens, int32_t bt_stride, int32_t bs_log2,
                               hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int threads = kCacheThreads;
  const int blocks = (num_tokens + threads - 1) / threads;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(blocks), dim3(threads), 0, stream, slot_mapping,
                     block_tables, qsl, ctx, num_seqs, num_tokens, bt_stride, bs_log2);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const uint16_t* k, const uint16_t* v, uint16_t* k_cache,
                                    uint16_t* v_cache, const int64_t* slots, int32_t num_tokens,
                                    int32_t num_kv_heads, int32_t head_dim, int64_t num_slots,
                                    hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int32_t chunks = head_dim / 8;
  const int64_t total = (int64_t)num_tokens * num_kv_heads * chunks;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     reinterpret_cast<const uint4*>(k), reinterpret_cast<const uint4*>(v),
                     reinterpret_cast<uint4*>(k_cache), v_cache, slots,
                     num_tokens, num_kv_heads, chunks, num_slots);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                              const int32_t* pairs, int32_t num_pairs, int32_t num_blocks,
                              int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                              int32_t elem_bytes, hipStream_t stream) {
  if (num_pairs == 0) return hipSuccess;
  const int64_t chunks = (int64_t)num_kv_heads * block_size * head_dim * elem_bytes / 16;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)num_pairs, 2), dim3(256), 0, stream,
                     reinterpret_cast<uint4*>(k_cache), reinterpret_cast<uint4*>(v_cache), k_scale,
                     v_scale, pairs, num_blocks, num_kv_heads, chunks);
  return hipGetLastError();
}

}  // namespace pkv
