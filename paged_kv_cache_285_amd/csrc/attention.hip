// Attention over a paged KV cache for a mixed continuous batch, on CDNA4 (gfx950).
//
// What is computed ["11. vLLM principles", sections 11.2 and 11.3; Tencent Cloud article on
// vLLM inference acceleration, continuous batching, chunked prefill and prefix caching
// sections; 2048ai.net vLLM V1 article, "Cascade Inference"]: for token i of request r at
// position p = context_lens[r] + i and q head h, softmax(scale * q . k_j) over keys
// j = 0..p of the request, read through its block table, weighting the values v_j.
//
// Kernel design (MI355X-first, not a translation of any printed kernel):
//  * varlen_kernel: one launch serves the batch's decode items and 128-row prefill tiles.  The
//    host plan lists work items; each is run once per kv head (grid = items * Hkv, kv head
//    fastest so that all tiles of one kv head fall on the same XCD under round-robin dispatch
//    and share its L2).  Each workgroup branches uniformly on the item kind:
//      - decode item (query length 1): VALU path.  4 waves stream disjoint 16-token blocks of
//        the item's key range straight from HBM with 16-byte coalesced loads (one wave load
//        covers 1 KB of a 4 KB block tile), software-pipelined one block ahead.  All G q heads
//        of the kv head share every K/V byte.  Q.K: 8 lanes per key with v_dot2_f32_bf16 and
//        a DPP transpose-reduce; a wave-uniform, lazily raised running max; P.V on the
//        dim-major value tile with v_dot2_f32_bf16 against bf16 p pairs.  Waves are merged
//        with the (o, lse) merge in LDS; long rows are cut into split-KV items whose partial
//        states reduce_kernel merges.  A decode-only batch uses a specialisation with no
//        prefill branch and a tighter register budget, with one-wave workgroups when the plan
//        asks for them (many short items at G = 8).
//      - prefill tile (query length > 1): 32 packed (token, q head) rows per wave (4 or 8
//        waves) x 64-key tiles on bf16 MFMA 32x32x16.  S^T = K Q^T puts one query per lane
//        column so the row max and row sum stay inside a lane (plus one cross-half exchange);
//        O^T = V^T P^T feeds P from the S^T accumulator registers.  K tiles are staged in LDS
//        row-major, V^T tiles key-permuted so every MFMA operand is one conflict-free 16-byte
//        read, both double-buffered; the causal mask (offset by the cached length) is only
//        evaluated on tiles that straddle the diagonal or the sequence end.
//    A batch with enough prompt rows runs its prefill tiles as 256-row tiles of 8 waves in
//    prefill_wide_kernel and its decode items in a varlen launch of their own; rows of
//    2 .. 32/G tokens (speculative verification) run as short items in short_kernel, a launch
//    of its own.
//  * cascade_kernel: the shared-prefix pass, the same 8-wave MFMA tile with no mask over the
//    prefix block table, cut into key segments when there are too few query tiles to fill
//    the chip; the segment states are merged afterwards.
//  * reduce_kernel: merges split-KV / segment partial states into the final output.
//
// FP8 KV cache [2048ai.net vLLM V1 article, quantisation section]: this file is compiled twice.
// With PKV_KV_FP8=1 every kernel reads e4m3 pools (one byte per element, the same layouts) with
// one fp32 scale per (physical block, kv head).  Cache chunks of 8 elements are then 8-byte
// loads, so every path moves half the bytes.  Codes become bf16 exactly (every e4m3 value is a
// bf16 value), and the scales are applied per cache block where they cost nothing in precision:
// the key scale to the block's scores (in fp32) and the value scale to the block's p before
// p is rounded for P.V.  The MFMA tiles stage the exact codes into LDS (same layout as bf16
// pools) and pass each tile's 4 block scales of both pools through a small LDS slot array.
#include "internal.h"

#ifndef PKV_KV_FP8
#define PKV_KV_FP8 0
#endif

#include <algorithm>
#include <type_traits>

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;

// Waves per SIMD the decode-only kernel is register-budgeted for (by q heads per kv head).
#ifndef PKV_DECODE_WAVES_G8
#define PKV_DECODE_WAVES_G8 2
#endif
#ifndef PKV_DECODE_WAVES
#define PKV_DECODE_WAVES 3
#endif

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         c, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte load with the streaming (non-temporal) cache policy: for K/V bytes read once.
#ifndef PKV_DECODE_NT
#define PKV_DECODE_NT 1
#endif
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
#if PKV_DECODE_NT
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
#else
  return *p;
#endif
}

__device__ __forceinline__ uint2 ld_stream(const uint2* p) {
#if PKV_DECODE_NT
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v[0], v[1]);
#else
  return *p;
#endif
}

__device__ __forceinline__ uint32_t ld_stream(const uint32_t* p) {
#if PKV_DECODE_NT
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

// Cache chunk of 8 elements: 16 bytes of bf16, or 8 bytes of e4m3 codes.
template <bool FP8>
using Chunk = std::conditional_t<FP8, uint2, uint4>;
template <bool FP8>
using ChunkV = std::conditional_t<FP8, u32x2, u32x4>;

// Two e4m3 codes (bytes 0-1, or 2-3 when HI) as a packed bf16 pair, exactly (every e4m3 value is
// a bf16 value): one v_cvt_scalef32_pk_bf16_fp8 with scale 1.  That instruction only applies
// the power of two of its scale operand, so the per-block scales are applied separately.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// 8 e4m3 codes -> 8 bf16 (16 bytes), exact.
__device__ __forceinline__ uint4 widen8(uint2 c) {
  return make_uint4(fp8x2_to_bf16x2<false>(c.x), fp8x2_to_bf16x2<true>(c.x), fp8x2_to_bf16x2<false>(c.y),
                    fp8x2_to_bf16x2<true>(c.y));
}
__device__ __forceinline__ uint4 widen8(uint4 c) { return c; }
__device__ __forceinline__ u32x4 widen8(u32x2 c) {
  return u32x4{fp8x2_to_bf16x2<false>(c[0]), fp8x2_to_bf16x2<true>(c[0]), fp8x2_to_bf16x2<false>(c[1]),
               fp8x2_to_bf16x2<true>(c[1])};
}
__device__ __forceinline__ u32x4 widen8(u32x4 c) { return c; }

// Physical 16-token tile of logical tile j of a request.  A block of 16 << L tokens is 1 << L
// consecutive 16-token tiles (L = 0 for 16-token blocks, ..., 4 for 256-token blocks), so the tile
// is (block_tables[j >> L] << L) + the low L bits of j.
template <typename IntPtr>
__device__ __forceinline__ int tile_of(IntPtr bt, int j, int L) {
  return (bt[j >> L] << L) + (j & ((1 << L) - 1));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LANES (8 or 16) lanes; every lane of a group gets the same bits.
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f32<0x141>(x);  // row_half_mirror: pairs the two quads of each 8-lane half
  if constexpr (LANES == 16) x += dpp_f32<0x140>(x);  // row_mirror: pairs the two halves
  return x;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Merge state (m2, l2, r2, o2) into (m, l, r, o); m in log2 units of scaled scores, l the fp32
// sum of p, r the sum of the bf16-rounded weights that o accumulated.
template <int N>
__device__ __forceinline__ void merge_state(float& m, float& l, float& r, float (&o)[N], float m2, float l2,
                                            float r2, const float (&o2)[N]) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  const float f1 = fast_exp2(m - mn), f2 = fast_exp2(m2 - mn);
  l = l * f1 + l2 * f2;
  r = r * f1 + r2 * f2;
#pragma unroll
  for (int e = 0; e < N; ++e) o[e] = o[e] * f1 + o2[e] * f2;
  m = mn;
}

// Store 8 consecutive output values of one (token, head) row at element offset `off`.
__device__ __forceinline__ void store8(void* out, int out_f32, int64_t off, const float (&v)[8]) {
  if (out_f32) {
    float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + off);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    uint4 w;
    w.x = pack_bf16x2(v[0], v[1]);
    w.y = pack_bf16x2(v[2], v[3]);
    w.z = pack_bf16x2(v[4], v[5]);
    w.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + off) = w;
  }
}

// ------------------------------------------------------------------------------------------
// Decode item: one query token, G q heads sharing kv head g, keys [kv_begin, kv_end).
//
// Each wave streams whole 16-token blocks (4 KB of K, 4 KB of V^T at D=128).
//  * Q.K: 8 lanes per key; lane group a (= lane / 8) takes tokens a and a+8, lane c (= lane % 8)
//    the dims 8c + 64k.  Partial dot products (v_dot2_f32_bf16) for the 2 tokens x G heads are
//    reduced over the 8 lanes by a transpose-reduce: three DPP exchange stages that halve the
//    values each lane keeps, so every lane ends with distinct, fully reduced scores
//    (score n = 2*head + token-of-pair, lane c keeps n = c*NK .. c*NK+NK-1) and the softmax
//    exponentials are not repeated across lanes.
//  * softmax: the running maximum per head is wave-uniform and only raised when a score
//    exceeds it by more than kLazy (log2 units), so p = exp2(s - m) <= 2^kLazy and the
//    rescale of the accumulators is rare; the block's p go to LDS as bf16.
//  * P.V on the dim-major value tile: lane l holds rows l/2 + 32i of V^T for the token half
//    l%2 (8 tokens = 4 packed pairs) and accumulates with v_dot2_f32_bf16 against the packed
//    (p_t, p_t+1) pairs read back from LDS.
// ------------------------------------------------------------------------------------------
constexpr float kLazy = 8.0f;

template <int N, int CTRL, int BIT>
__device__ __forceinline__ void transpose_stage(const float (&in)[N], float (&out)[N / 2], int c) {
  const bool up = (c >> BIT) & 1;
#pragma unroll
  for (int k = 0; k < N / 2; ++k) {
    const float keep = up ? in[k + N / 2] : in[k];
    const float send = up ? in[k] : in[k + N / 2];
    out[k] = keep + dpp_f32<CTRL>(send);
  }
}

template <int D, int G, int NW>
struct DecodeSmem {
  static constexpr int O_FLOATS = NW * G * D;                 // per-wave output states
  static constexpr int ML_FLOATS = 3 * NW * G;                // per-wave m, l and r
  static constexpr int SCR_BYTES = G * 16 * 4 + G * 16 * 2;   // per-wave scores + bf16 p
  static constexpr int BYTES = (O_FLOATS + ML_FLOATS) * 4 + NW * SCR_BYTES;
};

// Merges the NW per-wave states of a decode item (unnormalised o [NW][G][D], running max m
// (log2 units), row sum l and rounded-weight sum r [NW][G] in LDS) and stores the output
// (o / r) and LSE (from l), or the item's split-KV partial state.
template <int D, int G, int NW>
__device__ __forceinline__ void decode_merge(const VarlenArgs& a, const WorkItem& it, int g, int token,
                                             char* smem_raw) {
  constexpr int CH = D / 8;
  using SM = DecodeSmem<D, G, NW>;
  const float* s_o = reinterpret_cast<const float*>(smem_raw);
  const float* s_m = s_o + SM::O_FLOATS;
  const float* s_l = s_m + NW * G;
  const float* s_r = s_l + NW * G;
  const int Hq = a.num_q_heads;
  __syncthreads();
  for (int t = threadIdx.x; t < G * CH; t += 64 * NW) {
    const int hh = t / CH, cc = t % CH;
    float mm = -INFINITY, ll = 0.f, rr = 0.f, oo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) oo[e] = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float* src = s_o + (w * G + hh) * D + cc * 8;
      float o2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o2[e] = src[e];
      merge_state<8>(mm, ll, rr, oo, s_m[w * G + hh], s_l[w * G + hh], s_r[w * G + hh], o2);
    }
    const float inv = (rr > 0.f) ? 1.f / rr : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) oo[e] *= inv;
    const float lse = (ll > 0.f) ? (mm + __log2f(ll)) * kLn2 : -INFINITY;
    const int head = g * G + hh;
    if (it.partial_base < 0) {
      store8(a.out, a.out_f32, ((int64_t)token * Hq + head) * D + cc * 8, oo);
      if (a.lse && cc == 0) a.lse[(int64_t)token * Hq + head] = lse;
    } else {
      const int64_t prow = (int64_t)(it.partial_base + it.split) * Hq + head;
      store8(a.part_o, 1, prow * D + cc * 8, oo);
      if (cc == 0) a.part_lse[prow] = lse;
    }
  }
}

template <int D, int G, int NW, bool FP8, int DEPTH>
__device__ void decode_item(const VarlenArgs& a, const WorkItem& it, int g, char* smem_raw) {
  constexpr int CH = D / 8;    // 16-byte chunks per key row
  constexpr int CPT = D / 64;  // chunks of one key a lane holds
  constexpr int RPL = D / 32;  // V^T rows a lane holds
  constexpr int NV = 2 * G;    // scores per lane before the reduction
  constexpr int NS = NV >= 8 ? 3 : (NV == 4 ? 2 : 1);  // transpose stages (rest: plain adds)
  constexpr int NK = NV >= 8 ? NV / 8 : 1;            // scores per lane after the reduction
  constexpr int DUP = 3 - NS;                          // low lane bits holding duplicates
  using SM = DecodeSmem<D, G, NW>;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int grp = lane >> 3;
  const int c = lane & 7;
  const int r = it.seq;
  const int token = a.query_start_loc[r] + it.q_begin;
  const int kv_end = it.kv_end;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const float sl = a.scale_log2;

  // Scores this lane owns after the reduction: index n = 2*hh + tsel, token grp + 8*tsel.
  const int n0 = (c >> DUP) * NK;
  const int my_hh = n0 >> 1;  // the same head for both scores when NK == 2
  const bool owner = (c & ((1 << DUP) - 1)) == 0;

  // fp8 pools with D = 128: a key row is 128 bytes, so lane c reads dims 16c .. 16c+15 of its
  // tokens with one 16-byte load (8 lanes cover the row, a wave load covers whole cache lines);
  // otherwise lane c holds dims 8c + 64k.  The query chunks follow the same dims.
  constexpr bool WIDEK = FP8 && CPT == 2;
  uint4 qv[G][CPT];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int k = 0; k < CPT; ++k)
      qv[hh][k] = reinterpret_cast<const uint4*>(a.q + ((int64_t)token * Hq + g * G + hh) * D)[WIDEK ? 2 * c + k : c + 8 * k];

  float m[G];        // wave-uniform running max per head (log2 units of scaled scores)
  float o[G][RPL];   // P.V accumulators: head hh, V^T row (lane >> 1) + 32 i, token half
  float l_own = 0.f; // sum of p over the scores this lane owns (head my_hh), for the LSE
  float r_own = 0.f; // sum of the bf16-rounded weights P.V applies to them, for the output
  float m_own = -INFINITY;
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = -INFINITY;
#pragma unroll
    for (int i = 0; i < RPL; ++i) o[hh][i] = 0.f;
  }

  char* scr = smem_raw + (SM::O_FLOATS + SM::ML_FLOATS) * 4 + wave * SM::SCR_BYTES;
  float* sbuf = reinterpret_cast<float*>(scr);                  // [G][16] scaled scores
  uint16_t* pbuf = reinterpret_cast<uint16_t*>(scr + G * 64);   // [G][16] bf16 p

  const int32_t* bt = a.block_tables + (int64_t)r * a.bt_stride;
  const int b_begin = it.kv_begin / kBlockSize;
  const int b_end = (kv_end + kBlockSize - 1) / kBlockSize;
  using C8 = Chunk<FP8>;
  const int64_t tile_stride = (int64_t)kBlockSize * CH;  // chunks per (block, head) tile
  const int64_t blk_stride = (int64_t)Hkv * tile_stride;
  const C8* kb = reinterpret_cast<const C8*>(a.k_cache) + (int64_t)g * tile_stride;
  const C8* vb = reinterpret_cast<const C8*>(a.v_cache) + (int64_t)g * tile_stride;
  const int th = lane & 1;  // token half of the V^T rows this lane holds

  // Blocks b_begin + wave + NW*k, k < nk (nk <= 64: a split has at most 256 blocks); their
  // physical ids are fetched once, one per lane, and read back with v_readlane.
  const int nb = b_end - b_begin;
  const int nk = nb > wave ? (nb - wave + NW - 1) / NW : 0;
  const int L = a.bt_shift;
  const int my_id = lane < nk ? tile_of(bt, b_begin + wave + NW * lane, L) : 0;
  // fp8 pools: the key and value scales of those blocks, likewise one per lane (issued before
  // the first K/V loads, so waiting for those data covers them).
  float my_ks = 1.f, my_vs = 1.f;
  if constexpr (FP8) {
    if (lane < nk) {
      my_ks = a.k_scale[(int64_t)(my_id >> L) * Hkv + g];
      my_vs = a.v_scale[(int64_t)(my_id >> L) * Hkv + g];
    }
  }
  const float my_rvs = FP8 ? 1.f / my_vs : 1.f;  // the rounded weight p * v_scale counts p

  constexpr int NKR = 2 * CPT;  // key chunks per lane per block
  auto load = [&](int k, C8 (&kr)[NKR], C8 (&vr)[RPL]) {
    const int64_t phys = __builtin_amdgcn_readlane(my_id, k);
    const C8* kp = kb + phys * blk_stride;
    const C8* vp = vb + phys * blk_stride;
    if constexpr (WIDEK) {
      const uint4* kp4 = reinterpret_cast<const uint4*>(kp);
#pragma unroll
      for (int ts = 0; ts < 2; ++ts) {
        const uint4 x = ld_stream(kp4 + (grp + 8 * ts) * (CH / 2) + c);
        kr[2 * ts] = C8{x.x, x.y};
        kr[2 * ts + 1] = C8{x.z, x.w};
      }
    } else {
#pragma unroll
      for (int ts = 0; ts < 2; ++ts)
#pragma unroll
        for (int cc = 0; cc < CPT; ++cc) kr[ts * CPT + cc] = ld_stream(kp + (grp + 8 * ts) * CH + c + 8 * cc);
    }
#pragma unroll
    for (int i = 0; i < RPL; ++i) vr[i] = ld_stream(vp + lane + 64 * i);
  };

  auto process = [&](int k, const C8 (&kc)[NKR], const C8 (&vc)[RPL]) {
    const int t0 = (b_begin + wave + NW * k) * kBlockSize;
    const int nvalid = kv_end - t0;  // < 16 only in the last block
    uint4 kr[NKR], vr[RPL];
#pragma unroll
    for (int i = 0; i < NKR; ++i) kr[i] = widen8(kc[i]);
#pragma unroll
    for (int i = 0; i < RPL; ++i) vr[i] = widen8(vc[i]);
    float slb = sl, vsb = 1.f, rvsb = 1.f;  // this block's score scale and value scale
    if constexpr (FP8) {
      slb = sl * __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_ks), k));
      vsb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_vs), k));
      rvsb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_rvs), k));
    }
    // Q.K partial dot products: v[2*hh + ts].
    float v[NV];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int ts = 0; ts < 2; ++ts) {
        float acc = 0.f;
#pragma unroll
        for (int cc = 0; cc < CPT; ++cc) {
          const uint4 kk = kr[ts * CPT + cc];
          acc = dot2(qv[hh][cc].x, kk.x, acc);
          acc = dot2(qv[hh][cc].y, kk.y, acc);
          acc = dot2(qv[hh][cc].z, kk.z, acc);
          acc = dot2(qv[hh][cc].w, kk.w, acc);
        }
        v[2 * hh + ts] = acc;
      }
    // Transpose-reduce over the 8 lanes of the group (partners 7-c, c^2, c^1).
    float sc[NK];
    if constexpr (NV == 16) {
      float s1[8], s2[4];
      transpose_stage<16, 0x141, 2>(v, s1, c);
      transpose_stage<8, 0x4E, 1>(s1, s2, c);
      transpose_stage<4, 0xB1, 0>(s2, sc, c);
    } else if constexpr (NV == 8) {
      float s1[4], s2[2];
      transpose_stage<8, 0x141, 2>(v, s1, c);
      transpose_stage<4, 0x4E, 1>(s1, s2, c);
      transpose_stage<2, 0xB1, 0>(s2, sc, c);
    } else if constexpr (NV == 4) {
      float s1[2];
      transpose_stage<4, 0x141, 2>(v, s1, c);
      transpose_stage<2, 0x4E, 1>(s1, sc, c);
      sc[0] += dpp_f32<0xB1>(sc[0]);
    } else {
      transpose_stage<2, 0x141, 2>(v, sc, c);
      sc[0] += dpp_f32<0x4E>(sc[0]);
      sc[0] += dpp_f32<0xB1>(sc[0]);
    }
    int tok[NK];
    bool over = false;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      tok[kk] = grp + 8 * ((n0 + kk) & 1);
      sc[kk] = (tok[kk] < nvalid) ? sc[kk] * slb : -INFINITY;
      over |= sc[kk] > m_own + kLazy;
    }
    if (__ballot(over) != 0) {
      // Raise the running max to this block's max (rare after the first block).
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) sbuf[my_hh * 16 + tok[kk]] = sc[kk];
      __builtin_amdgcn_wave_barrier();  // LDS ops of one wave run in order; keep them so
      const float4* row = reinterpret_cast<const float4*>(sbuf + my_hh * 16);
      float bm = -INFINITY;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 x = row[q4];
        bm = fmaxf(fmaxf(bm, fmaxf(x.x, x.y)), fmaxf(x.z, x.w));
      }
      const float mn_own = fmaxf(m_own, bm);
      const float f_own = fast_exp2(m_own - ((mn_own == -INFINITY) ? 0.f : mn_own));
      l_own *= f_own;
      r_own *= f_own;
      m_own = mn_own;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        // lane hh * (8 / G) owns head hh
        const float mn = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_own), hh * (8 / G)));
        const float alpha = fast_exp2(m[hh] - ((mn == -INFINITY) ? 0.f : mn));
#pragma unroll
        for (int i = 0; i < RPL; ++i) o[hh][i] *= alpha;
        m[hh] = mn;
      }
    }
    const float mref = (m_own == -INFINITY) ? 0.f : m_own;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const float p = fast_exp2(sc[kk] - mref);
      const __bf16 pw = (__bf16)(FP8 ? p * vsb : p);
      if (owner) {
        l_own += p;
        r_own += FP8 ? (float)pw * rvsb : (float)pw;
      }
      pbuf[my_hh * 16 + tok[kk]] = __builtin_bit_cast(uint16_t, pw);
    }
    if (nvalid < kBlockSize) {
      // Zero the V^T entries of tokens past the end (the cache may hold NaN there).
      uint32_t msk[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = 8 * th + 2 * u;
        msk[u] = (t < nvalid ? 0x0000ffffu : 0u) | (t + 1 < nvalid ? 0xffff0000u : 0u);
      }
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        vr[i].x &= msk[0];
        vr[i].y &= msk[1];
        vr[i].z &= msk[2];
        vr[i].w &= msk[3];
      }
    }
    // P.V: packed (p_t, p_t+1) pairs of this lane's token half, for every head.
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const uint4 pp = *reinterpret_cast<const uint4*>(pbuf + hh * 16 + 8 * th);
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        float acc = o[hh][i];
        acc = dot2(pp.x, vr[i].x, acc);
        acc = dot2(pp.y, vr[i].y, acc);
        acc = dot2(pp.z, vr[i].z, acc);
        acc = dot2(pp.w, vr[i].w, acc);
        o[hh][i] = acc;
      }
    }
  };

  // Software pipeline: the next block's loads are in flight while the current one computes.
  // The steady-state loads are unconditional so the compiler's wait counts only ever wait
  // for the block about to be used (a conditional load would make it wait for both).  DEPTH
  // blocks stay in flight per wave: 2 for fp8 blocks (half the bytes), else 1.
  if constexpr (DEPTH == 2) {
    if (nk > 0) {
      C8 k0[NKR], v0[RPL], k1[NKR], v1[RPL], k2[NKR], v2[RPL];
      load(0, k0, v0);
      if (nk > 1) load(1, k1, v1);
      int k = 0;
      for (; k + 4 < nk; k += 3) {  // sets 0, 1 hold blocks k, k + 1
        load(k + 2, k2, v2);
        process(k, k0, v0);
        load(k + 3, k0, v0);
        process(k + 1, k1, v1);
        load(k + 4, k1, v1);
        process(k + 2, k2, v2);
      }
      // 1 to 4 blocks left; k and (when present) k + 1 are loaded.
      if (k + 2 < nk) load(k + 2, k2, v2);
      process(k, k0, v0);
      if (k + 1 < nk) {
        if (k + 3 < nk) load(k + 3, k0, v0);
        process(k + 1, k1, v1);
        if (k + 2 < nk) process(k + 2, k2, v2);
        if (k + 3 < nk) process(k + 3, k0, v0);
      }
    }
  } else if (nk > 0) {
    C8 ka[NKR], va[RPL], kn[NKR], vn[RPL];
    load(0, ka, va);
    int k = 0;
    for (; k + 2 < nk; k += 2) {
      load(k + 1, kn, vn);
      process(k, ka, va);
      load(k + 2, ka, va);
      process(k + 1, kn, vn);
    }
    if (k + 1 < nk) {
      load(k + 1, kn, vn);
      process(k, ka, va);
      process(k + 1, kn, vn);
    } else {
      process(k, ka, va);
    }
  }

  // Wave epilogue: add the two token halves, sum l over the lanes owning each head.
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int i = 0; i < RPL; ++i) o[hh][i] += dpp_f32<0xB1>(o[hh][i]);
  float lsum = owner ? l_own : 0.f;
  float rsum = owner ? r_own : 0.f;
  if constexpr (G <= 4) lsum += __shfl_xor(lsum, 1), rsum += __shfl_xor(rsum, 1);
  if constexpr (G <= 2) lsum += __shfl_xor(lsum, 2), rsum += __shfl_xor(rsum, 2);
  if constexpr (G <= 1) lsum += __shfl_xor(lsum, 4), rsum += __shfl_xor(rsum, 4);
  lsum += __shfl_xor(lsum, 8);
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  rsum += __shfl_xor(rsum, 8);
  rsum += __shfl_xor(rsum, 16);
  rsum += __shfl_xor(rsum, 32);

  float* s_o = reinterpret_cast<float*>(smem_raw);  // [NW][G][D]
  float* s_m = s_o + SM::O_FLOATS;                   // [NW][G]
  float* s_l = s_m + NW * G;                         // [NW][G]
  float* s_r = s_l + NW * G;                         // [NW][G]
  if (th == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int i = 0; i < RPL; ++i) s_o[(wave * G + hh) * D + (lane >> 1) + 32 * i] = o[hh][i];
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const int src = hh * (8 / G);
    const float lh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lsum), src));
    const float rh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rsum), src));
    if (lane == 0) {
      s_m[wave * G + hh] = m[hh];
      s_l[wave * G + hh] = lh;
      s_r[wave * G + hh] = rh;
    }
  }
  decode_merge<D, G, NW>(a, it, g, token, smem_raw);
}

// ------------------------------------------------------------------------------------------
// Short item: a row of a few query tokens (at most 32 packed (token, q head) rows, such as a
// speculative-verify row of 1 + k tokens) over a key range, on the matrix cores, with the
// decode item's work split (whole 16-key blocks per wave, block ids and scales fetched once per
// lane) and two blocks in flight per wave.  The packed rows are the columns
// of two 16-column groups:
//  * S^T = K Q^T per group: v_mfma_f32_16x16x32_bf16 over D/32 K-steps.  A = the block's 16
//    key rows: lane (i = lane % 16, q = lane / 16) holds dims 32s + 8q .. +7 of key i, one
//    16-byte load (8 bytes of fp8).  B = Q^T: lane (n, q) holds the same dims of column n.
//  * The 16x16 result gives lane (n, q) keys 4q .. 4q+3 of column n, so the causal mask and
//    the softmax are lane-local apart from the rare raise of a column's running max (a 4-lane
//    reduction), and those 4 p are exactly the B operand (keys 4q .. 4q+3, column n) of
//  * O^T += V^T P^T per group: v_mfma_f32_16x16x16_bf16 per 16 dims.  A = V^T: lane (d, q)
//    holds keys 4q .. 4q+3 of dim 16 dg + d, one 8-byte load (4 of fp8) shared by both groups.
// The waves' states are merged in LDS: each wave writes its sums, rescaled to the common max, to
// a slot of its own, and the slots are added in wave order (the result does not depend on
// timing).
// ------------------------------------------------------------------------------------------
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// 4 e4m3 codes -> 4 bf16 (exact); 4 bf16 pass through.
__device__ __forceinline__ uint2 widen4(uint32_t c) {
  return make_uint2(fp8x2_to_bf16x2<false>(c), fp8x2_to_bf16x2<true>(c));
}
__device__ __forceinline__ uint2 widen4(uint2 c) { return c; }

// LDS of a short item: the packed query rows (bf16, pitch QP) while the blocks stream, then, from
// the same bytes on, one slot of output sums per wave (fp32, pitch DP); the per-wave m, l and r
// after them.
template <int D, int NW>
struct ShortSmem {
  static constexpr int COLS = 32;
  static constexpr int DP = D + 4;  // row pitch (floats): 16 columns' float4 stores hit distinct banks
  static constexpr int QP = D + 8;  // query row pitch (bf16): conflict-free 16-byte operand reads
  static_assert(COLS * QP * 2 <= COLS * DP * 4, "query rows fit the first output slot");
  static constexpr int BYTES = (NW * COLS * DP + 3 * NW * COLS) * 4;
  static_assert(BYTES <= 160 * 1024, "fits the LDS of a CU");
};

// Waves of a short item's workgroup: one workgroup fills a CU at two waves per SIMD, so the
// items (longest first) are taken by CUs as they free up.
#ifndef PKV_SHORT_WAVES
#define PKV_SHORT_WAVES 8
#endif
constexpr int kShortWaves = PKV_SHORT_WAVES;

// bf16 pair (1, 1): v_dot2 against it sums a packed pair of bf16 weights exactly in fp32.
constexpr uint32_t kBf16OnePair = 0x3f803f80u;

template <int D, int G, int NW, bool FP8>
__device__ void short_item(const VarlenArgs& a, const WorkItem& it, int g, char* smem_raw) {
  constexpr int CH = D / 8;   // 8-element chunks per key row
  constexpr int KS = D / 32;  // K-steps of S^T
  constexpr int DG = D / 16;  // 16-dim groups of O^T
  constexpr int NC = 2;       // column groups
  using SM = ShortSmem<D, NW>;
  using KC = Chunk<FP8>;                                  // 8 key elements
  using VC = std::conditional_t<FP8, uint32_t, uint2>;  // 4 value elements

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15;
  const int q = lane >> 4;
  const int r = it.seq;
  const int ntok = it.q_count;
  const int tok0 = a.query_start_loc[r] + it.q_begin;
  const int pos0 = a.context_lens[r] + it.q_begin;  // position of the row's first token
  const int kv_end = it.kv_end;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int ncols = ntok * G;  // <= 32
  const float sl = a.scale_log2;

  // The packed query rows go to LDS once (zeros for padding columns); the Q^T operands of every
  // block are read back from there, which keeps 32 VGPRs free for the blocks in flight.
  uint16_t* sq = reinterpret_cast<uint16_t*>(smem_raw);
  for (int idx = threadIdx.x; idx < SM::COLS * CH; idx += 64 * NW) {
    const int n = idx / CH, cc = idx % CH;
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    if (n < ncols)
      x = reinterpret_cast<const uint4*>(a.q + ((int64_t)(tok0 + n / G) * Hq + g * G + n % G) * D)[cc];
    *reinterpret_cast<uint4*>(sq + n * SM::QP + 8 * cc) = x;
  }
  int qpos[NC];
#pragma unroll
  for (int cg = 0; cg < NC; ++cg) qpos[cg] = pos0 + min(16 * cg + n16, ncols - 1) / G;
  __syncthreads();
  floatx4 o[NC][DG];
  float m[NC], lsum[NC], rsum[NC];  // running max; fp32 sum of p (LSE); sum of rounded weights (output)
#pragma unroll
  for (int cg = 0; cg < NC; ++cg) {
    m[cg] = -INFINITY;
    lsum[cg] = 0.f;
    rsum[cg] = 0.f;
#pragma unroll
    for (int d = 0; d < DG; ++d) o[cg][d] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  const int32_t* bt = a.block_tables + (int64_t)r * a.bt_stride;
  const int b_begin = it.kv_begin / kBlockSize;
  const int b_end = (kv_end + kBlockSize - 1) / kBlockSize;
  const int nb = b_end - b_begin;
  const int nk = nb > wave ? (nb - wave + NW - 1) / NW : 0;
  const int L = a.bt_shift;
  const int my_id = lane < nk ? tile_of(bt, b_begin + wave + NW * lane, L) : 0;
  float my_ks = 1.f, my_vs = 1.f;
  if constexpr (FP8) {
    if (lane < nk) {
      my_ks = a.k_scale[(int64_t)(my_id >> L) * Hkv + g];
      my_vs = a.v_scale[(int64_t)(my_id >> L) * Hkv + g];
    }
  }
  const float my_rvs = FP8 ? 1.f / my_vs : 1.f;  // the rounded weight p * v_scale counts p
  const int64_t ktile = (int64_t)kBlockSize * CH;  // KC per (block, head) tile
  const int64_t vtile = (int64_t)4 * D;           // VC per (block, head) tile
  const KC* kb = reinterpret_cast<const KC*>(a.k_cache) + (int64_t)g * ktile;
  const VC* vb = reinterpret_cast<const VC*>(a.v_cache) + (int64_t)g * vtile;

  auto load = [&](int k, KC (&kr)[KS], VC (&vr)[DG]) __attribute__((always_inline)) {
    const int64_t phys = __builtin_amdgcn_readlane(my_id, k);
    const KC* kp = kb + phys * Hkv * ktile;
    const VC* vp = vb + phys * Hkv * vtile;
#pragma unroll
    for (int s = 0; s < KS; ++s) kr[s] = ld_stream(kp + n16 * CH + 4 * s + q);
#pragma unroll
    for (int d = 0; d < DG; ++d) vr[d] = ld_stream(vp + (16 * d + n16) * 4 + q);
  };

  auto process = [&](int k, const KC (&kr)[KS], const VC (&vr)[DG]) __attribute__((always_inline)) {
    const int t0 = (b_begin + wave + NW * k) * kBlockSize;  // first key of the block
    const int nvalid = kv_end - t0;                         // < 16 only in the last block
    float slb = sl, vsb = 1.f, rvsb = 1.f;
    if constexpr (FP8) {
      slb = sl * __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_ks), k));
      vsb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_vs), k));
      rvsb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_rvs), k));
    }
    uint2 vmask = make_uint2(0xffffffffu, 0xffffffffu);  // values of keys past the end -> 0
    if (nvalid < kBlockSize) {
      const int t = 4 * q;
      vmask.x = (t < nvalid ? 0x0000ffffu : 0u) | (t + 1 < nvalid ? 0xffff0000u : 0u);
      vmask.y = (t + 2 < nvalid ? 0x0000ffffu : 0u) | (t + 3 < nvalid ? 0xffff0000u : 0u);
    }
    // Keep the Q^T operand reads inside the loop (the compiler would otherwise hoist these
    // loop-invariant loads and hold them in registers again).
    asm volatile("" ::: "memory");
#pragma unroll
    for (int cg = 0; cg < NC; ++cg) {
      floatx4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 qop = *reinterpret_cast<const bf16x8*>(sq + (16 * cg + n16) * SM::QP + 32 * s + 8 * q);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, widen8(kr[s])), qop, sacc, 0,
                                                       0, 0);
      }
      float sc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = t0 + 4 * q + j;
        sc[j] = (4 * q + j < nvalid && key <= qpos[cg]) ? sacc[j] * slb : -INFINITY;
      }
      const float lm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      if (__ballot(lm > m[cg] + kLazy) != 0) {
        float cm = fmaxf(lm, __shfl_xor(lm, 16));
        cm = fmaxf(cm, __shfl_xor(cm, 32));
        const float mn = fmaxf(m[cg], cm);
        const float alpha = fast_exp2(m[cg] - ((mn == -INFINITY) ? 0.f : mn));
        lsum[cg] *= alpha;
        rsum[cg] *= alpha;
#pragma unroll
        for (int d = 0; d < DG; ++d) o[cg][d] *= alpha;
        m[cg] = mn;
      }
      const float mref = (m[cg] == -INFINITY) ? 0.f : m[cg];
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = fast_exp2(sc[j] - mref);
        lsum[cg] += p[j];
      }
      const uint2 pw = FP8 ? make_uint2(pack_bf16x2(p[0] * vsb, p[1] * vsb), pack_bf16x2(p[2] * vsb, p[3] * vsb))
                           : make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
      if constexpr (FP8)
        rsum[cg] = fmaf(dot2(pw.y, kBf16OnePair, dot2(pw.x, kBf16OnePair, 0.f)), rvsb, rsum[cg]);
      else
        rsum[cg] = dot2(pw.y, kBf16OnePair, dot2(pw.x, kBf16OnePair, rsum[cg]));
      const shortx4 pb = __builtin_bit_cast(shortx4, pw);
#pragma unroll
      for (int d = 0; d < DG; ++d) {
        uint2 v = widen4(vr[d]);  // converted per group: cheaper than holding both groups' operands
        v.x &= vmask.x;
        v.y &= vmask.y;
        o[cg][d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(shortx4, v), pb, o[cg][d], 0, 0, 0);
      }
    }
  };

  // Two blocks in flight per wave (three register sets), unconditional steady-state loads.
  if (nk > 0) {
    KC k0[KS], k1[KS], k2[KS];
    VC v0[DG], v1[DG], v2[DG];
    load(0, k0, v0);
    if (nk > 1) load(1, k1, v1);
    int k = 0;
    for (; k + 4 < nk; k += 3) {  // sets 0, 1 hold blocks k, k + 1
      load(k + 2, k2, v2);
      process(k, k0, v0);
      load(k + 3, k0, v0);
      process(k + 1, k1, v1);
      load(k + 4, k1, v1);
      process(k + 2, k2, v2);
    }
    if (k + 2 < nk) load(k + 2, k2, v2);
    process(k, k0, v0);
    if (k + 1 < nk) {
      if (k + 3 < nk) load(k + 3, k0, v0);
      process(k + 1, k1, v1);
      if (k + 2 < nk) process(k + 2, k2, v2);
      if (k + 3 < nk) process(k + 3, k0, v0);
    }
  }

  // Merge the waves: every wave publishes (m, l) per column; each lane rescales its o to the
  // columns' common max into an LDS slot of its wave; the store below adds the slots in wave
  // order (one barrier, rather than one per wave for a running sum).
  float* s_o = reinterpret_cast<float*>(smem_raw);  // [NW][COLS][DP], the first slot over the query rows
  float* s_m = s_o + NW * SM::COLS * SM::DP;         // [NW][COLS]
  float* s_l = s_m + NW * SM::COLS;                  // [NW][COLS]
  float* s_r = s_l + NW * SM::COLS;                  // [NW][COLS]
#pragma unroll
  for (int cg = 0; cg < NC; ++cg) {
    lsum[cg] += __shfl_xor(lsum[cg], 16);
    lsum[cg] += __shfl_xor(lsum[cg], 32);
    rsum[cg] += __shfl_xor(rsum[cg], 16);
    rsum[cg] += __shfl_xor(rsum[cg], 32);
    if (q == 0) {
      s_m[wave * SM::COLS + 16 * cg + n16] = m[cg];
      s_l[wave * SM::COLS + 16 * cg + n16] = lsum[cg];
      s_r[wave * SM::COLS + 16 * cg + n16] = rsum[cg];
    }
  }
  __syncthreads();
  float fac[NC];
#pragma unroll
  for (int cg = 0; cg < NC; ++cg) {
    const int n = 16 * cg + n16;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, s_m[w * SM::COLS + n]);
    fac[cg] = (mx == -INFINITY) ? 0.f : fast_exp2(m[cg] - mx);
  }
#pragma unroll
  for (int cg = 0; cg < NC; ++cg)
#pragma unroll
    for (int d = 0; d < DG; ++d)
      *reinterpret_cast<float4*>(s_o + (wave * SM::COLS + 16 * cg + n16) * SM::DP + 16 * d + 4 * q) =
          make_float4(o[cg][d][0] * fac[cg], o[cg][d][1] * fac[cg], o[cg][d][2] * fac[cg], o[cg][d][3] * fac[cg]);
  __syncthreads();
  // Store: thread per 8 output values of a valid column.
  for (int idx = threadIdx.x; idx < ncols * CH; idx += 64 * NW) {
    const int n = idx / CH, cc = idx % CH;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, s_m[w * SM::COLS + n]);
    float ll = 0.f, rr = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = fast_exp2(s_m[w * SM::COLS + n] - mx);
        ll += s_l[w * SM::COLS + n] * f;
        rr += s_r[w * SM::COLS + n] * f;
      }
    }
    const float inv = (rr > 0.f) ? 1.f / rr : 0.f;
    float oo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) oo[e] = s_o[n * SM::DP + 8 * cc + e];
#pragma unroll
    for (int w = 1; w < NW; ++w)
#pragma unroll
      for (int e = 0; e < 8; ++e) oo[e] += s_o[(w * SM::COLS + n) * SM::DP + 8 * cc + e];
#pragma unroll
    for (int e = 0; e < 8; ++e) oo[e] *= inv;
    const float lse = (ll > 0.f) ? (mx + __log2f(ll)) * kLn2 : -INFINITY;
    const int t = n / G, head = g * G + n % G;
    if (it.partial_base < 0) {
      store8(a.out, a.out_f32, ((int64_t)(tok0 + t) * Hq + head) * D + cc * 8, oo);
      if (a.lse && cc == 0) a.lse[(int64_t)(tok0 + t) * Hq + head] = lse;
    } else {
      const int64_t prow = (int64_t)(it.partial_base + t) * Hq + head;
      store8(a.part_o, 1, prow * D + cc * 8, oo);
      if (cc == 0) a.part_lse[prow] = lse;
    }
  }
}

// ------------------------------------------------------------------------------------------
// MFMA tile: 32*NW packed rows (32*NW/G tokens x G q heads of kv head g) over keys
// [kv_begin, kv_end).  Wave w owns rows 32w..32w+31; lane (n = lane % 32, h = lane / 32) owns
// query column n.  Rows beyond ntok tokens are padding (computed, never stored).  With 8 waves
// the 64-key K/V tile staged in LDS serves 256 rows, halving staging traffic per flop.
// ------------------------------------------------------------------------------------------
template <int D>
struct TileSmem {
  static constexpr int KP = D + 8;          // K row pitch (bf16): conflict-free 16-byte reads
  static constexpr int VP = kKvTile + 8;    // V^T row pitch (bf16)
  static constexpr int K_ELEMS = kKvTile * KP;
  static constexpr int V_ELEMS = D * VP;
  static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
  static constexpr int SC_OFF = 2 * BUF_ELEMS * 2;  // byte offset of the fp8 scale slots
  static constexpr int SC_SLOTS = 3;                // per tile: 4 key scales, then 4 value scales
  static constexpr int BYTES = SC_OFF + SC_SLOTS * 8 * 4;
};

// LDS of the pipelined 256-row tile: a ring of four K and four V tile buffers (same pitches
// as TileSmem), so that a tile is staged three steps (K) or one step (V) before its use and one
// barrier serves two steps, then eight fp8 scale slots.  143.6 KB at D = 128.
template <int D>
struct PipeSmem {
  using T = TileSmem<D>;
  static constexpr int NB = 4;                       // ring depth (power of two)
  static constexpr int V_OFF = NB * T::K_ELEMS;      // bf16 elements to the first V buffer
  static constexpr int SC_OFF = NB * T::BUF_ELEMS * 2;  // byte offset of the scale slots
  static constexpr int SC_SLOTS = 8;                 // per tile: 4 key scales, then 4 value scales
  static constexpr int BYTES = SC_OFF + SC_SLOTS * 8 * 4;
};

// The key and value scales of a tile's 4 cache blocks, read (uniformly) from scale slot `sc`.
struct TileScales {
  float k[4], v[4];
};
__device__ __forceinline__ TileScales read_scales(const float* sc) {
  const float4 a = *reinterpret_cast<const float4*>(sc);
  const float4 b = *reinterpret_cast<const float4*>(sc + 4);
  TileScales r;
  r.k[0] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.x)));
  r.k[1] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.y)));
  r.k[2] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.z)));
  r.k[3] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.w)));
  r.v[0] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(b.x)));
  r.v[1] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(b.y)));
  r.v[2] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(b.z)));
  r.v[3] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(b.w)));
  return r;
}

template <int D, int G, bool CAUSAL, int NW, bool FP8>
__device__ void mfma_tile(const uint16_t* __restrict__ q, int Hq, const void* __restrict__ k_cache,
                          const void* __restrict__ v_cache, const float* __restrict__ k_scale,
                          const float* __restrict__ v_scale, int Hkv, int g,
                          const int32_t* __restrict__ bt, int L, int tok0, int ntok, int pos0,
                          int kv_begin, int kv_end, float sl, void* out, int out_f32, float* lse_out,
                          int orow0, char* smem_raw) {
  using S = TileSmem<D>;
  constexpr int KSTEPS = D / 16;  // QK^T contraction steps
  constexpr int DT = D / 32;      // output d tiles
  constexpr int LPT = D / 8;      // lanes per key row when staging
  constexpr int KPI = 64 / LPT;   // key rows per wave load
  constexpr int NI = kBlockSize / KPI;  // loads per lane per block (K and V each)
  constexpr int CH = D / 8;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int n = lane & 31;
  const int h = lane >> 5;
  const int pr = wave * 32 + n;
  const int tq = pr / G;
  const int hh = pr % G;
  const bool row_valid = tq < ntok;
  const int qpos = row_valid ? pos0 + tq : 0x7fffffff;
  const bool wave_active = wave * 32 < ntok * G;  // wave-uniform

  uint16_t* smem = reinterpret_cast<uint16_t*>(smem_raw);

  // Q^T operand (B of S^T = K Q^T): lane holds dims 16s + 8h .. +7 of its query row.
  bf16x8 qb[KSTEPS];
  {
    const uint4* qrow =
        reinterpret_cast<const uint4*>(q + ((int64_t)(tok0 + (row_valid ? tq : 0)) * Hq + g * G + hh) * D);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      uint4 v = row_valid ? qrow[2 * s + h] : make_uint4(0u, 0u, 0u, 0u);
      qb[s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  floatx16 oacc[DT];
#pragma unroll
  for (int d = 0; d < DT; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[d][e] = 0.f;
  // Running max; fp32 sum of p (for the LSE); sum of the bf16-rounded weights P.V applies (for
  // the output, so that a row one key dominates comes out as that key's value).
  float m = -INFINITY, lsum = 0.f, rsum = 0.f;

  // Staging of the 64-key tile (4 cache blocks).  K rows are token-major: key
  // kk = KPI*i + lane/LPT, chunk lane%LPT.  The value pool is dim-major, so the V^T tile is a
  // plain copy: chunk lane + 64i is row (lane >> 1) + 32i, token half lane & 1.  With 4 waves,
  // wave w copies K and V of block w; with 8 waves, waves 0-3 copy K and waves 4-7 copy V, and
  // the loads run two tiles ahead of the compute (two register sets).  The loads are
  // unconditional (past the end they re-read the last block and are zeroed) so the compiler's
  // wait counts never wait for a later tile; block ids are scalar loads through the constant
  // address space, so they do not drain the vector-load counter either.
  constexpr int NIV = D / 32;
  static_assert(NI == NIV, "staging layout");
  constexpr bool SPLIT = NW == 8;
  constexpr int PD = SPLIT ? 2 : 1;           // prefetch distance in tiles
  constexpr int RS = SPLIT ? NI : 2 * NI;     // staging registers (uint4) per tile
  const int sblk = SPLIT ? (wave & 3) : wave;
  const bool does_k = !SPLIT || wave < 4;
  const bool does_v = !SPLIT || wave >= 4;
  const int sc = lane % LPT;
  const int sr = lane / LPT;
  using C8 = Chunk<FP8>;
  const int64_t tile_stride = (int64_t)kBlockSize * CH;  // chunks per (block, head) tile
  const int64_t blk_stride = (int64_t)Hkv * tile_stride;
  const C8* kbase = reinterpret_cast<const C8*>(k_cache) + (int64_t)g * tile_stride;
  const C8* vbase = reinterpret_cast<const C8*>(v_cache) + (int64_t)g * tile_stride;
  typedef __attribute__((address_space(4))) const int32_t cint32;
  typedef __attribute__((address_space(4))) const float cfloat;
  const cint32* cbt = (const cint32*)bt;
  const int last_blk = (kv_end - 1) / kBlockSize;
  C8 st[PD][RS];
  float ksc[PD], vsc[PD];  // fp8 pools: scales of the staged block
  float* scl = reinterpret_cast<float*>(smem_raw + S::SC_OFF);  // scale slot of buffer b: scl + 8b

  // Loads only: the masking of keys past the end happens at store time, so nothing here
  // waits for the data.  Returns how many of the block's keys are valid (<= 0: none).
  auto stage_load = [&](int tile, C8 (&r)[RS], float& ks, float& vs) -> int {
    const int lb = kv_begin / kBlockSize + 4 * tile + sblk;
    const int64_t phys = tile_of(cbt, min(lb, last_blk), L);
    const C8* kp = kbase + phys * blk_stride;
    const C8* vp = vbase + phys * blk_stride;
    if constexpr (FP8) {
      ks = ((const cfloat*)k_scale)[(phys >> L) * Hkv + g];
      vs = ((const cfloat*)v_scale)[(phys >> L) * Hkv + g];
    } else {
      ks = vs = 1.f;
    }
    if constexpr (SPLIT) {
      // One unconditional load stream per wave: K rows for waves 0-3, V^T chunks for 4-7.
#pragma unroll
      for (int i = 0; i < NI; ++i)
        r[i] = does_k ? kp[(KPI * i + sr) * CH + sc] : vp[lane + 64 * i];
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) r[i] = kp[(KPI * i + sr) * CH + sc];
#pragma unroll
      for (int i = 0; i < NIV; ++i) r[NI + i] = vp[lane + 64 * i];
    }
    return kv_end - lb * kBlockSize;
  };

  auto stage_store = [&](int buf, const C8 (&r)[RS], int nvalid, float kscale, float vscale) {
    uint16_t* ks = smem + buf * S::BUF_ELEMS;
    uint16_t* vs = ks + S::K_ELEMS;
    if constexpr (FP8) {
      if (lane == 0) {
        if (does_k) scl[8 * buf + sblk] = kscale;
        if (does_v) scl[8 * buf + 4 + sblk] = vscale;
      }
    }
    if (does_k) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int kk = KPI * i + sr;
        const uint4 x = (kk < nvalid) ? widen8(r[i]) : make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(ks + (sblk * kBlockSize + kk) * S::KP + sc * 8) = x;
      }
    }
    // Within each block the four 4-key groups are stored in the order 0, 2, 1, 3 (key t goes
    // to column 8*((t>>2)&1) + 4*(t>>3) + (t&3)), so the 8 keys one lane feeds a PV K-step
    // (t = 4h..4h+3 and 8+4h..8+4h+3) are one conflict-free 16-byte read.  Values of keys past
    // the end are zeroed (the cache may hold NaN there).
    if (does_v) {
      constexpr int vo = SPLIT ? 0 : NI;
      const int t = 8 * (lane & 1);
      uint32_t msk[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        msk[u] = (t + 2 * u < nvalid ? 0x0000ffffu : 0u) | (t + 2 * u + 1 < nvalid ? 0xffff0000u : 0u);
#pragma unroll
      for (int i = 0; i < NIV; ++i) {
        const int row = (lane >> 1) + 32 * i;
        uint16_t* dst = vs + row * S::VP + sblk * kBlockSize + 4 * (lane & 1);
        const uint4 x = widen8(r[vo + i]);
        *reinterpret_cast<uint2*>(dst) = make_uint2(x.x & msk[0], x.y & msk[1]);
        *reinterpret_cast<uint2*>(dst + 8) = make_uint2(x.z & msk[2], x.w & msk[3]);
      }
    }
  };

  const int ntiles = (kv_end - kv_begin + kKvTile - 1) / kKvTile;
  const int min_pos = pos0;  // first token of the tile has the smallest position

  int nv[PD];
  nv[0] = stage_load(0, st[0], ksc[0], vsc[0]);
  if constexpr (PD == 2) nv[1] = stage_load(1, st[1], ksc[1], vsc[1]);
  stage_store(0, st[0], nv[0], ksc[0], vsc[0]);
  __syncthreads();

  // One KV tile: prefetch tile t+PD into `ld`, compute tile t from LDS, then store tile t+1
  // (held in `sto`) into the other LDS buffer.
  auto body = [&](int t, C8 (&ld)[RS], int& nld, float& kld, float& vld, C8 (&sto)[RS], int& nsto,
                  float& ksto, float& vsto) {
    const int k0 = kv_begin + t * kKvTile;
    const int buf = t & 1;
    nld = stage_load(t + PD, ld, kld, vld);

    const uint16_t* ks = smem + buf * S::BUF_ELEMS;
    const uint16_t* vs = ks + S::K_ELEMS;

    // A wave whose 32 rows are all padding (a tile of a short row, such as a speculative-verify
    // row of 1 + k tokens) only helps stage the tiles.
    if (wave_active) {
      // S^T = K Q^T: two 32-key row tiles, their MFMA chains interleaved.
      floatx16 sacc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[mt][e] = 0.f;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const bf16x8 ka =
              *reinterpret_cast<const bf16x8*>(ks + (32 * mt + n) * S::KP + 16 * s + 8 * h);
          sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[s], sacc[mt], 0, 0, 0);
        }

      // Mask (raw scores): only tiles reaching past the first row's position or the sequence end.
      const bool need_mask = (k0 + kKvTile > kv_end) || (CAUSAL && k0 + kKvTile - 1 > min_pos);
      if (need_mask) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = k0 + 32 * mt + 8 * (e >> 2) + 4 * h + (e & 3);
            const bool vis = key < kv_end && (!CAUSAL || key <= qpos);
            sacc[mt][e] = vis ? sacc[mt][e] : -INFINITY;
          }
      }

      // Online softmax for this lane's query column.  The running max m (log2 units of scaled
      // scores) is only raised when a score exceeds it by more than kLazy, for every lane at
      // once, so the 64-register rescale of the output is rare; p stays <= 2^kLazy.  With fp8
      // pools, key block b of the tile (scores sacc[b >> 1][8 (b & 1) ..]) has score scale
      // sl * k_scale[b], and its p are multiplied by v_scale[b] before the P.V.
      float slk[4], svb[4], rsv[4];
      float mx = -INFINITY;
      if constexpr (FP8) {
        const TileScales tsc = read_scales(scl + 8 * buf);
        float mb[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int e = 0; e < 16; ++e) mb[2 * mt + (e >> 3)] = fmaxf(mb[2 * mt + (e >> 3)], sacc[mt][e]);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          slk[b] = sl * tsc.k[b];
          svb[b] = tsc.v[b];
          rsv[b] = __builtin_amdgcn_rcpf(tsc.v[b]);
          mx = fmaxf(mx, mb[b] * slk[b]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
      } else {
#pragma unroll
        for (int b = 0; b < 4; ++b) slk[b] = sl, svb[b] = 1.f, rsv[b] = 1.f;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[mt][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * sl;
      }
      if (__ballot(mx > m + kLazy) != 0) {
        const float mn = fmaxf(m, mx);
        const float alpha = fast_exp2(m - ((mn == -INFINITY) ? 0.f : mn));
        lsum *= alpha;
        rsum *= alpha;
#pragma unroll
        for (int d = 0; d < DT; ++d)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[d][e] *= alpha;
        m = mn;
      }
      const float mref = (m == -INFINITY) ? 0.f : m;

      // P^T operands: K-step ks covers keys 32*(ks/2) + 8*jj0 + 0..15, jj0 = 2*(ks%2).  Two row
      // sums: the fp32 sum of p gives the LSE (a sum of rounded p would cost ~1e-3 there), the
      // sum of the rounded weights (v_dot2 of each bf16 pair against (1, 1); fp8: divided by the
      // block's value scale) normalises the output.
      bf16x8 pb[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int mt = ks >> 1, b0 = 8 * (ks & 1);
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = fast_exp2(fmaf(sacc[mt][b0 + e], slk[ks], -mref));
          lsum += p;
          v[e] = (__bf16)(FP8 ? p * svb[ks] : p);
        }
        pb[ks] = v;
        const u32x4 w = __builtin_bit_cast(u32x4, v);
        float rb = FP8 ? 0.f : rsum;
#pragma unroll
        for (int u = 0; u < 4; ++u) rb = dot2(w[u], kBf16OnePair, rb);
        rsum = FP8 ? fmaf(rb, rsv[ks], rsum) : rb;
      }

      // O^T += V^T P^T.
#pragma unroll
      for (int d = 0; d < DT; ++d) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 xv = *reinterpret_cast<const bf16x8*>(vs + (32 * d + n) * S::VP + 16 * ks + 8 * h);
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xv, pb[ks], oacc[d], 0, 0, 0);
        }
      }
    }

    if (t + 1 < ntiles) stage_store(buf ^ 1, sto, nsto, ksto, vsto);
    __syncthreads();
  };

  int t = 0;
  for (; t + 1 < ntiles; t += 2) {
    body(t, st[0], nv[0], ksc[0], vsc[0], st[PD - 1], nv[PD - 1], ksc[PD - 1], vsc[PD - 1]);
    body(t + 1, st[PD - 1], nv[PD - 1], ksc[PD - 1], vsc[PD - 1], st[0], nv[0], ksc[0], vsc[0]);
  }
  if (t < ntiles) body(t, st[0], nv[0], ksc[0], vsc[0], st[PD - 1], nv[PD - 1], ksc[PD - 1], vsc[PD - 1]);

  lsum += __shfl_xor(lsum, 32);
  rsum += __shfl_xor(rsum, 32);
  if (!row_valid) return;
  const float inv = (rsum > 0.f) ? 1.f / rsum : 0.f;
  const int64_t orow = (int64_t)(orow0 + tq) * Hq + g * G + hh;
#pragma unroll
  for (int d = 0; d < DT; ++d) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int dim = 32 * d + 8 * jj + 4 * h;
      const float v0 = oacc[d][4 * jj] * inv, v1 = oacc[d][4 * jj + 1] * inv;
      const float v2 = oacc[d][4 * jj + 2] * inv, v3 = oacc[d][4 * jj + 3] * inv;
      if (out_f32) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + orow * D + dim) =
            make_float4(v0, v1, v2, v3);
      } else {
        uint2 w;
        w.x = pack_bf16x2(v0, v1);
        w.y = pack_bf16x2(v2, v3);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + orow * D + dim) = w;
      }
    }
  }
  if (lse_out && h == 0) lse_out[orow] = (lsum > 0.f) ? (m + __log2f(lsum)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------------------------------------
// Pipelined MFMA tile: 256 packed rows on 8 waves (32 rows per wave, two waves per SIMD).  The
// tile loop is software-pipelined so that one wave's instruction stream mixes matrix and vector
// work: step t issues the MFMAs of S^T(t+1) = K(t+1) Q^T and O^T += V(t-1)^T P^T(t-1) while the
// VALU computes the softmax of tile t (whose S^T the previous step produced).  Step t also
// loads K(t+3) and V(t+1) at its start and stores them into LDS at its end (waves 0-3 copy K,
// waves 4-7 copy V; a ring of four buffers each), with one barrier per two steps.  P^T is the
// S^T accumulator's p as they stand (a lane holds keys 4h..4h+3 and 8+4h..8+4h+3 of each 16-key
// step), and the value tile is staged with its 4-key groups in that order, so the V^T operand is
// one 16-byte read.  The softmax takes no tile maximum after the first tile (see pipe_step).
// ------------------------------------------------------------------------------------------
template <int D>
struct PipeRegs {
  static constexpr int KSTEPS = D / 16;
  static constexpr int DT = D / 32;
  bf16x8 qb[KSTEPS];    // Q^T operand: dims 16s + 8h .. +7 of the lane's query row
  floatx16 oacc[DT];    // O^T accumulators
  floatx16 sacc[2][2];  // two S^T sets (tile t and t+1), each two 32-key halves
  bf16x8 pb[4];         // P^T (four 16-key steps): tile t-1 until its P.V step, then tile t
  float m;             // running max (log2 units of scaled scores)
  float lr;            // sum of the bf16-rounded weights P.V applied: normalises the output and
                       // gives the LSE (within ln(1 + 2^-9) of the fp32 sum's, and consistent
                       // with the output when states are merged)
  int qpos;             // position of the lane's query row
};

// x of lane l ^ 32 (the other half of the wave).
__device__ __forceinline__ float other_half(float x, int h) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(h ? r[0] : r[1]);
}

// Masks the scores of S^T set SET for the tile starting at key k0: keys past kv_end and, for
// causal rows, keys after the row's position get -inf.
template <int D, int SET, bool CAUSAL>
__device__ __forceinline__ void pipe_mask(PipeRegs<D>& R, int h, int k0, int kv_end) {
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = k0 + 32 * mt + 8 * (e >> 2) + 4 * h + (e & 3);
      const bool vis = key < kv_end && (!CAUSAL || key <= R.qpos);
      R.sacc[SET][mt][e] = vis ? R.sacc[SET][mt][e] : -INFINITY;
    }
}

// O^T += V^T P^T over the V buffer `vb`, 16-key step ks.
template <int D>
__device__ __forceinline__ void pipe_pv_step(PipeRegs<D>& R, const uint16_t* __restrict__ vb, int n, int h, int ks) {
  using S = TileSmem<D>;
#pragma unroll
  for (int d = 0; d < D / 32; ++d) {
    const bf16x8 xv = *reinterpret_cast<const bf16x8*>(vb + (32 * d + n) * S::VP + 16 * ks + 8 * h);
    R.oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xv, R.pb[ks], R.oacc[d], 0, 0, 0);
  }
}

// Scores of the tile up to which p = exp2(s * scale - m) may grow before the tile is redone with
// its own maximum: a tile's rounded weights summing past 2^32 (or not finite).
constexpr float kPipeOverflow = 4294967296.0f;

// Softmax of S^T set CUR into P^T and the tile's row sums, all at once (the first tile, and a tile
// redone after an overflow): the running max becomes max(m, the tile's max), with the output and
// row sums rescaled when m was finite (they hold the tiles before this one).
template <int D, int CUR, bool FP8>
__device__ __forceinline__ void pipe_softmax_with_max(PipeRegs<D>& R, int h, const float (&slk)[4],
                                                      const float (&svb)[4], const float (&rsv)[4], float& tr) {
  float mx = -INFINITY;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    float mb = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) mb = fmaxf(mb, R.sacc[CUR][ks >> 1][8 * (ks & 1) + e]);
    mx = fmaxf(mx, mb * slk[ks]);
  }
  mx = fmaxf(mx, other_half(mx, h));
  const float mnew = fmaxf(R.m, mx);
  if (R.m != -INFINITY) {
    const float alpha = fast_exp2(R.m - mnew);
    R.lr *= alpha;
#pragma unroll
    for (int d = 0; d < D / 32; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) R.oacc[d][e] *= alpha;
  }
  R.m = mnew;
  const float mref = (mnew == -INFINITY) ? 0.f : mnew;
  tr = 0.f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4 w;
    float rb = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float p0 = fast_exp2(fmaf(R.sacc[CUR][ks >> 1][8 * (ks & 1) + 2 * u], slk[ks], -mref));
      const float p1 = fast_exp2(fmaf(R.sacc[CUR][ks >> 1][8 * (ks & 1) + 2 * u + 1], slk[ks], -mref));
      w[u] = FP8 ? pack_bf16x2(p0 * svb[ks], p1 * svb[ks]) : pack_bf16x2(p0, p1);
      rb = dot2(w[u], kBf16OnePair, rb);
    }
    tr = fmaf(rb, rsv[ks], tr);
    R.pb[ks] = __builtin_bit_cast(bf16x8, w);
  }
}

// One pipeline step.  CUR holds S^T(t) (already masked); the other set receives S^T(t+1) from
// K buffer `kb`; P^T holds tile t-1 for the P.V over V buffer `vb` and is overwritten, 16-key
// step by 16-key step after its last P.V use, with tile t.  The step is issued in a fixed
// order, one slot per MFMA: slot i reads the operand of MFMA i + 2 from LDS, issues MFMA i
// (first the P.V MFMAs, then the S MFMAs) and then a slice of the softmax of tile t, so that
// every MFMA runs under VALU work and its operand has been in flight for two MFMAs.
//
// The softmax of tile t uses the running max m as it stands: p = exp2(s * scale - m), in 16
// pieces of 4 keys (their bf16 pairs, the sum of the rounded weights as v_dot2 of each pair
// against (1, 1), and with LSE the fp32 sum of p).  No tile maximum is taken; a tile whose
// rounded weights sum past kPipeOverflow in some row (scores far above every earlier one) is
// redone with its maximum after the step, which keeps p finite and exact.  S^T's accumulator
// layout gives lane half h keys 4h..4h+3 and 8+4h..8+4h+3 of every 16-key step; those 8 p are the
// lane's P^T operand as they stand, and the value tile is staged with the same key order.
// FIRST (step 0, whose P.V is of the zeroed tile before the first): the slots carry no softmax
// work; tile 0's softmax runs after them, with its own maximum.
// Stage(i) runs after MFMA slot i: the staging of a later tile (LDS stores of the tile loaded in
// the previous step, then the loads of the next one) spread over the slots.
template <int D, int CUR, bool FP8, bool FIRST, typename Stage>
__device__ __forceinline__ void pipe_step(PipeRegs<D>& R, const uint16_t* __restrict__ kb,
                                          const uint16_t* __restrict__ vb, int n, int h, float sl,
                                          const TileScales& tsc, float& tr, Stage&& stage) {
  constexpr int NXT = 1 - CUR;
  constexpr int KSTEPS = D / 16;
  constexpr int DT = D / 32;
  constexpr int NPV = 4 * DT;           // P.V MFMAs (16-key step ks, d tile d: index DT*ks + d)
  constexpr int NM = NPV + 2 * KSTEPS;  // then S MFMAs (K-step s, key half mt: 2*s + mt)
  constexpr int PF = 2;                 // operand reads in flight
  constexpr int SPAN = NM - 2;          // slots over which the 16 exp pieces are spread
  using S = TileSmem<D>;
  const floatx16 zero = {};

  auto operand = [&](int i) __attribute__((always_inline)) -> bf16x8 {
    if (i < NPV) {
      const int ks = i / DT, d = i % DT;
      return *reinterpret_cast<const bf16x8*>(vb + (32 * d + n) * S::VP + 16 * ks + 8 * h);
    }
    const int j = i - NPV, s = j / 2, mt = j % 2;
    return *reinterpret_cast<const bf16x8*>(kb + (32 * mt + n) * S::KP + 16 * s + 8 * h);
  };

  // Score scale, p multiplier and rounded-weight divisor of key block b (16-key step b).
  float slk[4], svb[4], rsv[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    slk[b] = FP8 ? sl * tsc.k[b] : sl;
    svb[b] = FP8 ? tsc.v[b] : 1.f;
    rsv[b] = FP8 ? __builtin_amdgcn_rcpf(tsc.v[b]) : 1.f;
  }
  bf16x8 op[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) op[i] = operand(i);
  const float mref = R.m;
  uint32_t pk[4][4];
  // Rounded-weight sums: per key block over fp8 pools (each block divides by its value scale),
  // one sum over bf16 pools.
  float trb[FP8 ? 4 : 1] = {};
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    const bf16x8 a = op[i % PF];
    if (i + PF < NM) op[i % PF] = operand(i + PF);
    if (i < NPV) {
      const int ks = i / DT, d = i % DT;
      R.oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, R.pb[ks], R.oacc[d], 0, 0, 0);
    } else {
      const int j = i - NPV, s = j / 2, mt = j % 2;
      R.sacc[NXT][mt] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, R.qb[s], s == 0 ? zero : R.sacc[NXT][mt], 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (FIRST || (q * SPAN) / 16 != i) continue;
      const int ks = q >> 2, u = q & 3, mt = ks >> 1, e0 = 8 * (ks & 1) + 2 * u;
      const float p0 = fast_exp2(fmaf(R.sacc[CUR][mt][e0], slk[ks], -mref));
      const float p1 = fast_exp2(fmaf(R.sacc[CUR][mt][e0 + 1], slk[ks], -mref));
      pk[ks][u] = FP8 ? pack_bf16x2(p0 * svb[ks], p1 * svb[ks]) : pack_bf16x2(p0, p1);
      trb[FP8 ? ks : 0] = dot2(pk[ks][u], kBf16OnePair, trb[FP8 ? ks : 0]);
      // P^T(t-1) of this 16-key step had its last use in slot DT*ks + DT - 1 < i.
      if (u == 3) R.pb[ks] = __builtin_bit_cast(bf16x8, u32x4{pk[ks][0], pk[ks][1], pk[ks][2], pk[ks][3]});
    }
    stage(i);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (FIRST) {
    pipe_softmax_with_max<D, CUR, FP8>(R, h, slk, svb, rsv, tr);
    return;
  }
  if constexpr (FP8) {
    tr = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) tr = fmaf(trb[b], rsv[b], tr);
  } else {
    tr = trb[0];
  }
  // A row whose tile outgrew the running max (or whose max was -inf): redo the tile with its max.
  if (__builtin_expect(__ballot(!(tr <= kPipeOverflow)) != 0, 0))
    pipe_softmax_with_max<D, CUR, FP8>(R, h, slk, svb, rsv, tr);
}

template <int D, int G, bool CAUSAL, bool FP8>
__device__ void pipe_tile(const uint16_t* __restrict__ q, int Hq, const void* __restrict__ k_cache,
                          const void* __restrict__ v_cache, const float* __restrict__ k_scale,
                          const float* __restrict__ v_scale, int Hkv, int g,
                          const int32_t* __restrict__ bt, int L, int tok0, int ntok, int pos0,
                          int kv_begin, int kv_end, float sl, void* out, int out_f32, float* lse_out,
                          char* smem_raw) {
  using S = TileSmem<D>;
  using PS = PipeSmem<D>;
  constexpr int NB = PS::NB;
  constexpr int KSTEPS = D / 16;
  constexpr int DT = D / 32;
  constexpr int CH = D / 8;             // 16-byte chunks per key row
  constexpr int LPT = CH;               // lanes per key row when staging
  constexpr int KPI = 64 / LPT;         // key rows per wave load
  constexpr int NI = kBlockSize / KPI;  // loads per lane per block (K rows; V^T chunks alike)
  static_assert(NI == D / 32, "staging layout");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31;
  const int h = lane >> 5;
  uint16_t* smem = reinterpret_cast<uint16_t*>(smem_raw);
  uint16_t* kbuf0 = smem;
  uint16_t* vbuf0 = smem + PS::V_OFF;

  PipeRegs<D> R;
  const int pr = 32 * wave + n;
  const int tq = pr / G;
  const int hh = pr % G;
  const bool row_valid = tq < ntok;
  R.qpos = row_valid ? pos0 + tq : 0x7fffffff;
  {
    const u32x4* qrow =
        reinterpret_cast<const u32x4*>(q + ((int64_t)(tok0 + (row_valid ? tq : 0)) * Hq + g * G + hh) * D);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const u32x4 v = row_valid ? qrow[2 * s + h] : u32x4{0u, 0u, 0u, 0u};
      R.qb[s] = __builtin_bit_cast(bf16x8, v);
    }
  }
#pragma unroll
  for (int d = 0; d < DT; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) R.oacc[d][e] = 0.f;
  R.m = -INFINITY;
  R.lr = 0.f;

  const int ntiles = (kv_end - kv_begin + kKvTile - 1) / kKvTile;
  if (ntiles > 0) {
    // Staging: waves 0-3 copy the K rows (key KPI*i + lane/LPT, chunk lane % LPT) and waves 4-7
    // the V^T chunks (chunk lane + 64i of the dim-major block tile is dim (lane >> 1) + 32i,
    // tokens 8*(lane & 1)..+7) of cache block (wave & 3) of a tile.  Within each block's 16 keys
    // the V^T row holds the 4-key groups in the order 0, 2, 1, 3 (the key order of a lane's P^T
    // operand), so a chunk is stored as two 8-byte halves.  Loads are unconditional (past the
    // end they re-read the last block); values of keys past the end are zeroed at store time.
    // The staging code is written per job (J = 1 job per wave).
    constexpr int J = 1;
    const int sblk = wave & 3;
    const int sc = lane % LPT;
    const int sr = lane / LPT;
    const int64_t tile_stride = (int64_t)kBlockSize * CH;
    const int64_t blk_stride = (int64_t)Hkv * tile_stride;
    const int last_blk = (kv_end - 1) / kBlockSize;
    const int blk0 = kv_begin / kBlockSize + sblk;
    // Physical ids of the wave's blocks of 64 consecutive tiles, one per lane (read back with
    // readlane, so the per-tile address needs no memory wait); refreshed every 64 tiles.
    // fp8 pools: the waves that copy K also hold the key and value scales of those blocks,
    // alike, and put each tile's scales into scale slot tile % 8 (read by every wave in the
    // tile's softmax step; the slot is rewritten five steps later, past two barriers).
    using C8 = ChunkV<FP8>;
    float* scl = reinterpret_cast<float*>(smem_raw + PS::SC_OFF);
    int bid_base = 0;
    int bid = tile_of(bt, min(blk0 + 4 * lane, last_blk), L);
    float bks = 1.f, bvs = 1.f;
    auto load_scales = [&]() __attribute__((always_inline)) {
      if constexpr (FP8) {
        if (wave < 4) {
          bks = k_scale[(int64_t)(bid >> L) * Hkv + g];
          bvs = v_scale[(int64_t)(bid >> L) * Hkv + g];
        }
      }
    };
    load_scales();
    auto block_id = [&](int tile, float& ks, float& vs) __attribute__((always_inline)) -> int {
      if (tile - bid_base >= 64) {
        bid_base = tile;
        bid = tile_of(bt, min(blk0 + 4 * (tile + lane), last_blk), L);
        load_scales();
      }
      ks = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bks), tile - bid_base));
      vs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bvs), tile - bid_base));
      return __builtin_amdgcn_readlane(bid, tile - bid_base);
    };
    bool jv[J];                // the job copies V
    const C8* jbase[J];        // pool base of the job's kv head
    int soff[J], sstep[J];     // LDS offset (bf16 units) of chunk i: soff + i * sstep
#pragma unroll
    for (int j = 0; j < J; ++j) {
      jv[j] = wave >= 4;
      jbase[j] = reinterpret_cast<const C8*>(jv[j] ? v_cache : k_cache) + (int64_t)g * tile_stride;
      // Chunk lane + 64i of the block tile: ((KPI*i + sr)*CH + sc) is that same index for K rows.
      soff[j] = jv[j] ? PS::V_OFF + (lane >> 1) * S::VP + kBlockSize * sblk + 4 * (lane & 1)
                      : (kBlockSize * sblk + sr) * S::KP + sc * 8;
      sstep[j] = jv[j] ? 32 * S::VP : KPI * S::KP;
    }
    // Tile x goes to K buffer x % NB or V buffer x % NB.
    auto load = [&](int j, int tile, C8 (&r)[NI], float& ks, float& vs) __attribute__((always_inline)) -> int {
      const int lb = blk0 + 4 * tile;
      const C8* p = jbase[j] + (int64_t)block_id(tile, ks, vs) * blk_stride;
#pragma unroll
      for (int i = 0; i < NI; ++i) r[i] = p[lane + 64 * i];
      return jv[j] ? kv_end - lb * kBlockSize : kBlockSize;
    };
    // Stores chunk i of a loaded tile into LDS buffer `buf` (chunk 0 of a K job also stores the
    // block's scales into scale slot `slot`).  Values of keys past the end are zeroed.
    auto store_chunk = [&](int j, int i, int buf, const C8 (&rc)[NI], int nvalid, float ks, float vs, int slot)
        __attribute__((always_inline)) {
      uint16_t* dst = smem + buf * (jv[j] ? S::V_ELEMS : S::K_ELEMS);
      if constexpr (FP8) {
        if (i == 0 && !jv[j] && lane == 0) {
          scl[8 * slot + sblk] = ks;
          scl[8 * slot + 4 + sblk] = vs;
        }
      }
      u32x4 r = widen8(rc[i]);
      if (nvalid < kBlockSize) {
        // Only the last tile takes this branch; the empty asm keeps the compiler from computing
        // the mask (8 compares) ahead of the branch on every step.
        int nv = nvalid;
        asm volatile("" : "+s"(nv));
        const int t0 = 8 * (lane & 1);
        u32x4 msk;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          msk[u] = (t0 + 2 * u < nv ? 0x0000ffffu : 0u) | (t0 + 2 * u + 1 < nv ? 0xffff0000u : 0u);
        r &= msk;
      }
      if (jv[j]) {
        // Tokens 8 th .. 8 th + 3 go to group slot th, tokens 8 th + 4 .. + 7 to slot 2 + th.
        *reinterpret_cast<u32x2*>(dst + soff[j] + i * sstep[j]) = u32x2{r[0], r[1]};
        *reinterpret_cast<u32x2*>(dst + soff[j] + i * sstep[j] + 8) = u32x2{r[2], r[3]};
      } else {
        *reinterpret_cast<u32x4*>(dst + soff[j] + i * sstep[j]) = r;
      }
    };
    auto store = [&](int j, int buf, const C8 (&rc)[NI], int nvalid, float ks, float vs, int slot)
        __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < NI; ++i) store_chunk(j, i, buf, rc, nvalid, ks, vs, slot);
    };

    // Prologue: K(0), K(1), K(2) and V(0) in LDS and the loads of K(3) and V(1) in flight,
    // V(-1) = 0 (no tile before the first), S^T(0) computed.
    C8 st[J][NI];
    int nv[J];
    float ksv[J], vsv[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (!jv[j]) {
#pragma unroll
        for (int x = 0; x < 3; ++x) {
          nv[j] = load(j, x, st[j], ksv[j], vsv[j]);
          store(j, x, st[j], nv[j], ksv[j], vsv[j], x);
        }
        nv[j] = load(j, 3, st[j], ksv[j], vsv[j]);
      } else {
        nv[j] = load(j, 0, st[j], ksv[j], vsv[j]);
        store(j, 0, st[j], nv[j], ksv[j], vsv[j], 0);
        nv[j] = load(j, 1, st[j], ksv[j], vsv[j]);
      }
    }
    {
      u32x4* z = reinterpret_cast<u32x4*>(vbuf0 + (NB - 1) * S::V_ELEMS);
      for (int i = threadIdx.x; i < S::V_ELEMS / 8; i += 512) z[i] = u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    {
      const floatx16 zero = {};
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kbuf0 + (32 * mt + n) * S::KP + 16 * s + 8 * h);
          R.sacc[0][mt] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, R.qb[s], s == 0 ? zero : R.sacc[0][mt], 0, 0, 0);
        }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) R.pb[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});

    // Step t: compute S^T(t+1), P.V(t-1) and softmax(t); spread over its MFMA slots, store the
    // tile loaded in step t-1 (K(t+3) / V(t+1)) into LDS and then load the next one (K(t+4) /
    // V(t+2)), so each load has a whole step to arrive.  K(x) is stored in step x-3 and first
    // read in step x-1; V(x) is stored in step x-1 and first read in step x+1; each buffer's
    // previous tile was last read four steps before the store.  So one barrier before every even
    // step orders every store against its reads (the steps alternate the S^T sets, so even steps
    // are the CUR == 0 ones).  Step 0 takes tile 0's softmax with its maximum.
    constexpr int ST0 = 2;  // first slot with a staging store
    auto step = [&](auto cur, auto first, int t) __attribute__((always_inline)) {
      constexpr int CUR = decltype(cur)::value;
      constexpr bool FIRST = decltype(first)::value;
      if constexpr (CUR == 0) __syncthreads();
      TileScales tsc;
      if constexpr (FP8) tsc = read_scales(scl + 8 * (t % PS::SC_SLOTS));
      const int k0 = kv_begin + t * kKvTile;
      if ((k0 + kKvTile > kv_end) || (CAUSAL && k0 + kKvTile - 1 > pos0))
        pipe_mask<D, CUR, CAUSAL>(R, h, k0, kv_end);
      const int sbuf = (jv[0] ? t + 1 : t + 3) & (NB - 1);
      auto stage = [&](int i) __attribute__((always_inline)) {
        if (i >= ST0 && i < ST0 + NI)
          store_chunk(0, i - ST0, sbuf, st[0], nv[0], ksv[0], vsv[0], (t + 3) % PS::SC_SLOTS);
        if (i == ST0 + NI) nv[0] = load(0, jv[0] ? t + 2 : t + 4, st[0], ksv[0], vsv[0]);
      };
      float tr;
      // A wave in its matrix/softmax block issues ahead of the other wave on its SIMD while that
      // one waits at the barrier (equal priority measured 1-3 % slower).
      __builtin_amdgcn_s_setprio(1);
      pipe_step<D, CUR, FP8, FIRST>(R, kbuf0 + ((t + 1) & (NB - 1)) * S::K_ELEMS,
                                    vbuf0 + ((t - 1) & (NB - 1)) * S::V_ELEMS, n, h, sl, tsc, tr, stage);
      __builtin_amdgcn_s_setprio(0);
      R.lr += tr;
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using First = std::true_type;
    using Next = std::false_type;
    step(C0(), First(), 0);
    int t = 1;
    for (; t + 1 < ntiles; t += 2) {
      step(C1(), Next(), t);
      step(C0(), Next(), t + 1);
    }
    if (t < ntiles) step(C1(), Next(), t);
    // The last P.V (tile ntiles - 1, stored by the last step).
    __syncthreads();
    const uint16_t* vlast = vbuf0 + ((ntiles - 1) & (NB - 1)) * S::V_ELEMS;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) pipe_pv_step<D>(R, vlast, n, h, ks);
  }

  const float lr = R.lr + other_half(R.lr, h);
  if (!row_valid) return;
  const float inv = (lr > 0.f) ? 1.f / lr : 0.f;
  const int64_t orow = (int64_t)(tok0 + tq) * Hq + g * G + hh;
#pragma unroll
  for (int d = 0; d < DT; ++d) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int dim = 32 * d + 8 * jj + 4 * h;
      const float v0 = R.oacc[d][4 * jj] * inv, v1 = R.oacc[d][4 * jj + 1] * inv;
      const float v2 = R.oacc[d][4 * jj + 2] * inv, v3 = R.oacc[d][4 * jj + 3] * inv;
      if (out_f32) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + orow * D + dim) = make_float4(v0, v1, v2, v3);
      } else {
        uint2 w;
        w.x = pack_bf16x2(v0, v1);
        w.y = pack_bf16x2(v2, v3);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + orow * D + dim) = w;
      }
    }
  }
  if (lse_out && h == 0) lse_out[orow] = (lr > 0.f) ? (R.m + __log2f(lr)) * kLn2 : -INFINITY;
}

// DECODE_ONLY instantiations carry no MFMA path, so they need far fewer registers and run
// more waves per SIMD; a plan with any prefill tile uses the full kernel, with 4 or 8 waves
// per workgroup (8 when the batch carries enough prefill rows to fill 256-row tiles).
template <int D, int G, bool DECODE_ONLY, int NW, bool FP8>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW),
                          amdgpu_waves_per_eu(DECODE_ONLY ? (G >= 8 ? PKV_DECODE_WAVES_G8 : PKV_DECODE_WAVES) : 2)))
void varlen_kernel(VarlenArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int x = blockIdx.x;
  const int g = x % a.num_kv_heads;
  const WorkItem it = a.items[x / a.num_kv_heads];
  if (DECODE_ONLY || it.kind == kDecode) {
    decode_item<D, G, NW, FP8, FP8 ? 2 : 1>(a, it, g, smem);
  } else {
    const int r = it.seq;
    const int ctx = a.context_lens[r];
    const int tok0 = a.query_start_loc[r] + it.q_begin;
    const int32_t* bt = a.block_tables + (int64_t)r * a.bt_stride;
    // A key split of a short row writes fp32 partial states (rows partial_base + token) that
    // the reduce merges; otherwise the tile writes the output rows of its tokens.
    const bool part = it.partial_base >= 0;
    mfma_tile<D, G, true, NW, FP8>(a.q, a.num_q_heads, a.k_cache, a.v_cache, a.k_scale, a.v_scale,
                                   a.num_kv_heads, g, bt, a.bt_shift, tok0, it.q_count, ctx + it.q_begin,
                                   it.kv_begin, it.kv_end, a.scale_log2, part ? (void*)a.part_o : a.out,
                                   part ? 1 : a.out_f32, part ? a.part_lse : a.lse,
                                   part ? it.partial_base : tok0, smem);
  }
}

// Short items (rows of a few query tokens over long contexts) in a kernel of their own: their
// two-column-group MFMA path needs a register budget of two waves per SIMD, which the decode
// kernels must not inherit.
template <int D, int G, bool FP8>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kShortWaves, 64 * kShortWaves), amdgpu_waves_per_eu(2, 2)))
void short_kernel(VarlenArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int x = blockIdx.x;
  const int g = x % a.num_kv_heads;
  short_item<D, G, kShortWaves, FP8>(a, a.items[x / a.num_kv_heads], g, smem);
}

// Decode batch with a device-side work split, for graph capture: the grid depends only on
// (num_seqs, splits), each workgroup takes row x / (splits * Hkv), split (x / Hkv) % splits and
// kv head x % Hkv, and reads the row's length from seq_lens on the device.  A split past the
// row's end is an empty state (lse -inf) that the reduce weights by zero; a row of length 0
// gets output 0 and lse -inf.  Partial rows are laid out split-major (split * T + token).
template <int D, int G, bool FP8>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256),
                          amdgpu_waves_per_eu(G >= 8 ? PKV_DECODE_WAVES_G8 : PKV_DECODE_WAVES)))
void decode_graph_kernel(VarlenArgs a, int32_t splits, int32_t split_keys, int32_t num_tokens) {
  extern __shared__ __align__(16) char smem[];
  const int x = blockIdx.x;
  const int g = x % a.num_kv_heads;
  const int s = (x / a.num_kv_heads) % splits;
  const int r = x / (a.num_kv_heads * splits);
  WorkItem it;
  it.seq = r;
  it.kind = kDecode;
  it.q_begin = 0;
  it.q_count = splits;
  it.kv_begin = s * split_keys;
  it.kv_end = min(a.seq_lens[r], (s + 1) * split_keys);  // may be <= kv_begin: an empty state
  it.split = s;
  it.partial_base = splits > 1 ? s * num_tokens + a.query_start_loc[r] - s : -1;
  decode_item<D, G, 4, FP8, FP8 ? 2 : 1>(a, it, g, smem);
}

// Wide-tile kernels: 256-row pipelined tiles on 8 waves (two per SIMD).
template <int D, int G, bool FP8>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void prefill_wide_kernel(VarlenArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int x = blockIdx.x;
  const int g = x % a.num_kv_heads;
  const WorkItem it = a.items[x / a.num_kv_heads];
  const int r = it.seq;
  const int ctx = a.context_lens[r];
  const int tok0 = a.query_start_loc[r] + it.q_begin;
  const int32_t* bt = a.block_tables + (int64_t)r * a.bt_stride;
  pipe_tile<D, G, true, FP8>(a.q, a.num_q_heads, a.k_cache, a.v_cache, a.k_scale, a.v_scale, a.num_kv_heads,
                             g, bt, a.bt_shift, tok0, it.q_count, ctx + it.q_begin, it.kv_begin, it.kv_end, a.scale_log2,
                             a.out, a.out_f32, a.lse, smem);
}

template <int D, int G, bool FP8>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void cascade_kernel(CascadeArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int x = blockIdx.x;
  const int g = x % a.num_kv_heads;
  const int rest = x / a.num_kv_heads;
  const int tile = rest % a.num_tiles;
  const int seg = rest / a.num_tiles;
  constexpr int TOK = kWideTileRows / G;
  const int tok0 = tile * TOK;
  const int ntok = min(TOK, a.num_tokens - tok0);
  const int kv_begin = seg * a.seg_len;
  const int kv_end = min(a.prefix_len, kv_begin + a.seg_len);
  float* out = a.out;
  float* lse = a.lse;
  if (a.num_segments > 1) {
    out = a.part_o + (int64_t)seg * a.num_tokens * a.num_q_heads * D;
    lse = a.part_lse + (int64_t)seg * a.num_tokens * a.num_q_heads;
  }
  pipe_tile<D, G, false, FP8>(a.q, a.num_q_heads, a.k_cache, a.v_cache, a.k_scale, a.v_scale, a.num_kv_heads,
                              g, a.prefix_bt, a.bt_shift, tok0, ntok, 0, kv_begin, kv_end, a.scale_log2, out, 1,
                              lse, smem);
}

// One wave per (token, head) row; lane holds D/64 consecutive dims.
constexpr int kReduceBatch = 8;  // splits a row's states are loaded for at once
template <int D>
__global__ __launch_bounds__(256) void reduce_kernel(ReduceArgs a) {
  constexpr int V = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int Hq = a.num_q_heads;
  const int64_t token = row / Hq;
  if (token >= a.num_tokens) return;
  const int head = (int)(row - token * Hq);
  int64_t base, stride;
  int count;
  if (a.token_split) {
    base = a.token_split[3 * token];
    count = a.token_split[3 * token + 1];
    stride = a.token_split[3 * token + 2];
    if (count <= 1) return;  // written directly by the attention kernel
  } else {
    base = token;
    count = a.uniform_count;
    stride = a.num_tokens;
  }
  // One wave per row: the split layout is the same for every lane.
  count = __builtin_amdgcn_readfirstlane(count);
  float mx = -INFINITY;
  float acc[V];
#pragma unroll
  for (int e = 0; e < V; ++e) acc[e] = 0.f;
  float z = 0.f;
  if (count <= kReduceBatch) {
    // Every split's (lse, o) loads are issued before the first is used, so the partial states,
    // which the attention launch just wrote, arrive in one memory round trip; the arithmetic
    // and its order are those of the loops for more splits.
    float ls[kReduceBatch], po[kReduceBatch][V];
#pragma unroll
    for (int s = 0; s < kReduceBatch; ++s) {
      ls[s] = -INFINITY;
#pragma unroll
      for (int e = 0; e < V; ++e) po[s][e] = 0.f;
      if (s < count) {
        const int64_t prow = (base + s * stride) * Hq + head;
        ls[s] = a.part_lse[prow];
        const float* src = a.part_o + prow * D + lane * V;
#pragma unroll
        for (int e = 0; e < V; ++e) po[s][e] = src[e];
      }
    }
#pragma unroll
    for (int s = 0; s < kReduceBatch; ++s) mx = fmaxf(mx, ls[s]);
    if (mx != -INFINITY) {
#pragma unroll
      for (int s = 0; s < kReduceBatch; ++s) {
        if (s < count) {
          const float w = (ls[s] == -INFINITY) ? 0.f : __expf(ls[s] - mx);
          z += w;
#pragma unroll
          for (int e = 0; e < V; ++e) acc[e] = fmaf(w, po[s][e], acc[e]);
        }
      }
    }
  } else {
    for (int s = 0; s < count; ++s) mx = fmaxf(mx, a.part_lse[(base + s * stride) * Hq + head]);
    if (mx != -INFINITY) {
      for (int s = 0; s < count; ++s) {
        const int64_t prow = (base + s * stride) * Hq + head;
        const float ls = a.part_lse[prow];
        const float w = (ls == -INFINITY) ? 0.f : __expf(ls - mx);
        z += w;
        const float* src = a.part_o + prow * D + lane * V;
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] = fmaf(w, src[e], acc[e]);
      }
    }
  }
  const float inv = (z > 0.f) ? 1.f / z : 0.f;
  const int64_t orow = token * Hq + head;
  if (a.out_f32) {
    float* dst = reinterpret_cast<float*>(a.out) + orow * D + lane * V;
#pragma unroll
    for (int e = 0; e < V; ++e) dst[e] = acc[e] * inv;
  } else {
    uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + orow * D + lane * V;
    if constexpr (V == 1) {
      const __bf16 b = (__bf16)(acc[0] * inv);
      dst[0] = __builtin_bit_cast(uint16_t, b);
    } else {
#pragma unroll
      for (int e = 0; e < V; e += 2)
        *reinterpret_cast<uint32_t*>(dst + e) = pack_bf16x2(acc[e] * inv, acc[e + 1] * inv);
    }
  }
  if (a.lse && lane == 0) a.lse[orow] = (z > 0.f) ? mx + __logf(z) : -INFINITY;
}

template <int D, int G, int NW>
size_t varlen_smem(bool has_prefill) {
  const size_t dec = (size_t)DecodeSmem<D, G, NW>::BYTES;
  const size_t pre = has_prefill ? (size_t)TileSmem<D>::BYTES : 0;
  return dec > pre ? dec : pre;
}

constexpr bool kFp8 = PKV_KV_FP8 != 0;


// Decode items in a launch of their own: 4-wave workgroups, or one-wave ones (decode_waves == 1,
// which the plan picks only when every decode item fits one wave).
template <int D, int G>
void launch_decode_only(const VarlenArgs& a, int n_decode, int decode_waves, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)n_decode * a.num_kv_heads));
  if constexpr (G >= 8) {
    if (decode_waves == 1) {
      const size_t smem = varlen_smem<D, G, 1>(false);
      hipLaunchKernelGGL((varlen_kernel<D, G, true, 1, kFp8>), grid, dim3(64), smem, stream, a);
      return;
    }
  }
  const size_t smem = varlen_smem<D, G, 4>(false);
  hipLaunchKernelGGL((varlen_kernel<D, G, true, 4, kFp8>), grid, dim3(256), smem, stream, a);
}

template <int D, int G>
hipError_t launch_varlen_t(const VarlenArgs& a, int n_prefill, int n_decode, int n_short, int tile_rows,
                           int decode_waves, hipStream_t stream) {
  const int Hkv = a.num_kv_heads;
  if (n_prefill + n_decode > 0) {
    if (n_prefill == 0) {
      launch_decode_only<D, G>(a, n_decode, decode_waves, stream);
    } else if (tile_rows == kWideTileRows) {
      // Wide prefill tiles, then the decode items in a kernel of their own (the wide tile's
      // register budget allows two waves per SIMD, too few for the decode path).
      auto kern = prefill_wide_kernel<D, G, kFp8>;
      hipLaunchKernelGGL(kern, dim3((unsigned)((int64_t)n_prefill * Hkv)), dim3(512),
                         (size_t)PipeSmem<D>::BYTES, stream, a);
      if (n_decode > 0) {
        VarlenArgs b = a;
        b.items = a.items + n_prefill;
        b.num_items = n_decode;
        launch_decode_only<D, G>(b, n_decode, decode_waves, stream);
      }
    } else {
      auto kern = varlen_kernel<D, G, false, 4, kFp8>;
      const size_t smem = varlen_smem<D, G, 4>(true);
      hipLaunchKernelGGL(kern, dim3((unsigned)((int64_t)(n_prefill + n_decode) * Hkv)), dim3(256), smem,
                         stream, a);
    }
  }
  if (n_short > 0) {
    VarlenArgs b = a;
    b.items = a.items + n_prefill + n_decode;
    b.num_items = n_short;
    const size_t smem = (size_t)ShortSmem<D, kShortWaves>::BYTES;
    hipLaunchKernelGGL((short_kernel<D, G, kFp8>), dim3((unsigned)((int64_t)n_short * Hkv)), dim3(64 * kShortWaves), smem,
                       stream, b);
  }
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_decode_graph_t(const VarlenArgs& a, int num_seqs, int splits, int split_keys, int num_tokens,
                                 hipStream_t stream) {
  const int64_t grid = (int64_t)num_seqs * splits * a.num_kv_heads;
  if (grid == 0) return hipSuccess;
  const size_t smem = varlen_smem<D, G, 4>(false);
  hipLaunchKernelGGL((decode_graph_kernel<D, G, kFp8>), dim3((unsigned)grid), dim3(256), smem, stream, a, splits,
                     split_keys, num_tokens);
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_cascade_t(const CascadeArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)a.num_tiles * a.num_segments * a.num_kv_heads;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((cascade_kernel<D, G, kFp8>), dim3((unsigned)grid), dim3(512), (size_t)PipeSmem<D>::BYTES,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

#define PKV_DISPATCH_DG(D_, G_, CALL)                 \
  switch (D_) {                                       \
    case 64:                                          \
      switch (G_) {                                   \
        case 1: return CALL(64, 1);                   \
        case 2: return CALL(64, 2);                   \
        case 4: return CALL(64, 4);                   \
        case 8: return CALL(64, 8);                   \
      }                                               \
      break;                                          \
    case 128:                                         \
      switch (G_) {                                   \
        case 1: return CALL(128, 1);                  \
        case 2: return CALL(128, 2);                  \
        case 4: return CALL(128, 4);                  \
        case 8: return CALL(128, 8);                  \
      }                                               \
      break;                                          \
  }                                                   \
  return hipErrorInvalidValue;

#if PKV_KV_FP8
#define PKV_KV_NAME(name) name##_fp8
#else
#define PKV_KV_NAME(name) name
#endif

hipError_t PKV_KV_NAME(launch_varlen)(const VarlenArgs& a, int head_dim, int group, int n_prefill,
                                      int n_decode, int n_short, int tile_rows, int decode_waves,
                                      hipStream_t stream) {
#define CALL_V(D, G) launch_varlen_t<D, G>(a, n_prefill, n_decode, n_short, tile_rows, decode_waves, stream)
  PKV_DISPATCH_DG(head_dim, group, CALL_V)
#undef CALL_V
}

hipError_t PKV_KV_NAME(launch_cascade)(const CascadeArgs& a, int head_dim, int group,
                                       hipStream_t stream) {
#define CALL_C(D, G) launch_cascade_t<D, G>(a, stream)
  PKV_DISPATCH_DG(head_dim, group, CALL_C)
#undef CALL_C
}

hipError_t PKV_KV_NAME(launch_decode_graph)(const VarlenArgs& a, int head_dim, int group, int num_seqs,
                                           int splits, int split_keys, int num_tokens,
                                           hipStream_t stream) {
#define CALL_G(D, G) launch_decode_graph_t<D, G>(a, num_seqs, splits, split_keys, num_tokens, stream)
  PKV_DISPATCH_DG(head_dim, group, CALL_G)
#undef CALL_G
}

#if !PKV_KV_FP8
hipError_t launch_reduce(const ReduceArgs& a, int head_dim, hipStream_t stream) {
  const int64_t rows = (int64_t)a.num_tokens * a.num_q_heads;
  if (rows == 0) return hipSuccess;
  const unsigned grid = (unsigned)((rows + 3) / 4);
  if (head_dim == 64)
    hipLaunchKernelGGL(reduce_kernel<64>, dim3(grid), dim3(256), 0, stream, a);
  else if (head_dim == 128)
    hipLaunchKernelGGL(reduce_kernel<128>, dim3(grid), dim3(256), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}
#endif

}  // namespace pkv
