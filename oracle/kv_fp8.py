"""CPU oracle for an FP8 (e4m3) KV cache -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may
import this module; the HIP library never does.

Quantising the KV cache to a low-precision float such as FP8 shrinks its storage and speeds
up attention, which matters most for long contexts [2048ai.net vLLM V1 article, quantisation
section].  Readings taken where the pages are silent:

* the format is OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7) and 3 mantissa bits,
  subnormals, no infinities, the all-ones magnitude 0x7f is NaN, largest finite value 448;
* each (physical block, kv head) tile of each pool has one fp32 scale, supplied by the caller
  (k_scale and v_scale, [num_blocks, Hkv]): a code stored in that tile means
  code_value * scale (one scale per kv head, or per pool, is the case of equal entries);
* quantising x (a bf16 value) computes y = fp32(x * fp32(1 / scale)) in fp32, clamps y to
  [-448, 448] (NaN stays NaN) and rounds to the nearest e4m3 value, ties to the even code;
* attention over fp8 pools is the same softmax attention over the dequantised keys and
  values (code value * scale, exact in fp64).

Pool layouts and slots are those of the bf16 cache (keys [NB, Hkv, 16, D], values
[NB, Hkv, D, 16] for 16-token blocks; [NB, R, Hkv, 16, D] and [NB, R, Hkv, D, 16] for blocks of
16 R tokens), one byte per element; the scales are per physical block of any size.
"""

from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .paged_attention import (
    attention_state,
    bf16_to_f64,
    causal_visible,
    default_scale,
    key_tile_len,
    tiles,
    value_tile_len,
)

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Value of each e4m3 code (uint8) as fp64: (-1)^s * 2^(e-7) * (1 + m/8), or 2^-6 * m/8
    for e == 0; magnitude 0x7f is NaN."""
    c = np.asarray(codes, dtype=np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0**-6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = np.where(s == 1, -mag, mag)
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


_POS = e4m3_decode(np.arange(0x7F))  # the 127 non-negative finite values, ascending


def e4m3_encode(x) -> np.ndarray:
    """Nearest e4m3 code of each fp32 value, ties to the even code, |x| > 448 saturating to
    the largest finite code, NaN to 0x7f."""
    xs = np.asarray(x, dtype=np.float32)
    a = np.minimum(np.abs(xs).astype(np.float64), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS, a), 1, 126)  # first value >= a (clipped)
    lo = hi - 1
    d_lo, d_hi = a - _POS[lo], _POS[hi] - a
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a == 0.0, 0, pick)
    code = pick | np.where(np.signbit(xs), 0x80, 0)
    return np.where(np.isnan(xs), 0x7F, code).astype(np.uint8)


def quantize(x_bf16, scale: float) -> np.ndarray:
    """e4m3 codes of bf16 values (bit patterns) under one fp32 scale (module reading)."""
    x = (np.asarray(x_bf16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    inv = np.float32(1.0) / np.float32(scale)
    with np.errstate(invalid="ignore", over="ignore"):
        y = (x * inv).astype(np.float32)
    return e4m3_encode(y)


def reshape_and_cache_fp8(k, v, k_cache, v_cache, slots, k_scale, v_scale, block_size: int):
    """Return copies of the fp8 pools with token t's K/V, quantised under the scales of the
    block its slot falls in, at that slot; slots < 0 or past the pool are skipped.  k, v are
    bf16 bits [T, Hkv, D]; k_scale, v_scale fp32 [num_blocks, Hkv]."""
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    kt, vt = tiles(kc), tiles(vc)
    T = key_tile_len(kc)
    assert kt.shape[1] * T == block_size and value_tile_len(vc) == T
    for t, s in enumerate(np.asarray(slots, dtype=np.int64)):
        b, o = divmod(int(s), block_size)
        if s < 0 or b >= kc.shape[0]:
            continue
        for g in range(k.shape[1]):
            kt[b, o // T, g, o % T, :] = quantize(k[t, g, :], k_scale[b][g])
            vt[b, o // T, g, :, o % T] = quantize(v[t, g, :], v_scale[b][g])
    return kc, vc


def dequantize_keys(k_cache, k_scale, block_table_row, num_keys: int, kv_head: int, block_size: int):
    """Keys 0..num_keys-1 of one request and kv head as fp64 [num_keys, D]."""
    T = key_tile_len(k_cache)
    assert tiles(k_cache).shape[1] * T == block_size
    j = np.arange(num_keys)
    phys = np.asarray(block_table_row, dtype=np.int64)[j // block_size]
    o = j % block_size
    ks = np.asarray(k_scale, dtype=np.float32)[phys, kv_head].astype(np.float64)
    return e4m3_decode(tiles(k_cache)[phys, o // T, kv_head, o % T, :]) * ks[:, None]


def dequantize_values(v_cache, v_scale, block_table_row, num_keys: int, kv_head: int, block_size: int):
    """Values 0..num_keys-1 of one request and kv head as fp64 [num_keys, D] (the pool is
    dim-major)."""
    T = value_tile_len(v_cache)
    assert tiles(v_cache).shape[1] * T == block_size
    j = np.arange(num_keys)
    phys = np.asarray(block_table_row, dtype=np.int64)[j // block_size]
    o = j % block_size
    vs = np.asarray(v_scale, dtype=np.float32)[phys, kv_head].astype(np.float64)
    return e4m3_decode(tiles(v_cache)[phys, o // T, kv_head, :, o % T]) * vs[:, None]


def paged_attention_fp8(
    q,
    k_cache,
    v_cache,
    k_scale,
    v_scale,
    block_tables,
    query_start_loc,
    context_lens,
    seq_lens,
    block_size: int,
    scale: Optional[float] = None,
    rows: Optional[np.ndarray] = None,
) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of every new token over its request's dequantised paged keys/values (fp64);
    the same definition as the bf16 oracle, with key j of kv head g equal to
    e4m3_decode(code) * k_scale[block of j, g] (values alike)."""
    q = np.asarray(q)
    T, Hq, D = q.shape
    Hkv = tiles(k_cache).shape[2]
    G = Hq // Hkv
    sc = default_scale(D) if scale is None or scale <= 0 else float(scale)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    ctx = np.asarray(context_lens, dtype=np.int64)
    sl = np.asarray(seq_lens, dtype=np.int64)
    o = np.full((T, Hq, D), np.nan)
    lse = np.full((T, Hq), np.nan)
    want = None if rows is None else set(int(x) for x in np.asarray(rows))
    for r in range(len(ctx)):
        t0, t1 = int(qsl[r]), int(qsl[r + 1])
        if t1 == t0:
            continue
        toks = [t for t in range(t0, t1) if want is None or t in want]
        if not toks:
            continue
        n = int(sl[r])
        vis = causal_visible(int(ctx[r]), t1 - t0, n)
        for g in range(Hkv):
            K = dequantize_keys(k_cache, k_scale, block_tables[r], n, g, block_size)
            V = dequantize_values(v_cache, v_scale, block_tables[r], n, g, block_size)
            for hh in range(G):
                h = g * G + hh
                tt = np.array(toks)
                s = sc * (bf16_to_f64(q[tt, h, :]) @ K.T)
                s = np.where(vis[tt - t0], s, -np.inf)
                oo, ll = attention_state(s, V)
                o[tt, h, :] = oo
                lse[tt, h] = ll
    return o, lse


def cascade_prefix_attention_fp8(
    q, k_cache, v_cache, k_scale, v_scale, prefix_block_table, prefix_len: int, block_size: int,
    scale: Optional[float] = None,
) -> Tuple[np.ndarray, np.ndarray]:
    """State of every query token over the dequantised shared prefix keys 0..prefix_len-1
    (no mask: every query comes after the prefix) [2048ai.net vLLM V1 article, "Cascade
    Inference"].  Returns (o [T, Hq, D], lse [T, Hq]) in fp64."""
    q = np.asarray(q)
    T, Hq, D = q.shape
    Hkv = tiles(k_cache).shape[2]
    G = Hq // Hkv
    sc = default_scale(D) if scale is None or scale <= 0 else float(scale)
    o = np.zeros((T, Hq, D), dtype=np.float64)
    lse = np.full((T, Hq), -np.inf, dtype=np.float64)
    for g in range(Hkv):
        K = dequantize_keys(k_cache, k_scale, prefix_block_table, prefix_len, g, block_size)
        V = dequantize_values(v_cache, v_scale, prefix_block_table, prefix_len, g, block_size)
        for hh in range(G):
            h = g * G + hh
            s = sc * (bf16_to_f64(q[:, h, :]) @ K.T)
            o[:, h, :], lse[:, h] = attention_state(s, V)
    return o, lse
