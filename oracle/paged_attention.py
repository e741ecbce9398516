"""CPU fp64 oracle for attention over a paged KV cache.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the HIP library: it never loads the shared
library, includes none of its headers and takes no constant from it.

Everything here is the plain definition written out in numpy float64, slow
on purpose so that it can be checked against the pages by eye:

* Paging [vLLM principles, ch. 11 section 11.2 "PagedAttention", "分页思想"
  and the Block Table example]: the cache is cut into fixed-size blocks of
  ``block_size`` tokens; a request's block table maps its logical block
  ``p // block_size`` to a physical block, anywhere in the pool, and token
  ``p`` sits at offset ``p % block_size`` inside it.  Two requests may name
  the same physical blocks (a shared, read-only prefix).
* Batched, chunked and prefix-cached prefill [Tencent Cloud article on vLLM
  inference acceleration, sections on batched prefill, chunked prefill and
  prefix caching]: prompts of several requests are concatenated into one
  token list (``query_start_loc`` delimits them); a chunk after the first
  attends to the cached keys of earlier chunks plus, causally, to its own
  tokens; a prefix-cache hit means the first ``context_len`` tokens are
  already cached and the new tokens start at position ``context_len``.
* KV caching [2048ai.net vLLM V1 article, "KV Caching"]: the keys and values
  of every processed token are stored and reused by later steps.
* Cascade inference [2048ai.net vLLM V1 article, "Cascade Inference"]: the
  attention state of the queries over the shared prefix and over each
  unique suffix are computed separately and combined by an associative,
  commutative merge of (output, log-sum-exp) states.

Readings taken where the pages are silent:
softmax scale 1/sqrt(head_dim); q head h reads kv head h // (Hq/Hkv); the key
pool is laid out [num_blocks, Hkv, block_size, head_dim] (token-major) and the
value pool [num_blocks, Hkv, head_dim, block_size] (dim-major); a new token at position
p = context_len + i sees keys 0..p (its own key included, written to the
cache before attention); LSE is the natural log of the scaled scores; an
empty key set has state (o = 0, lse = -inf); slot = -1 means "do not write".
"""

from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np


# ---------------------------------------------------------------------------
# bf16 decoding (exact): a bf16 value is the upper 16 bits of an fp32 value.
# ---------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Pool layout.  Blocks hold a fixed number of tokens, such as 16 or 256 ("11. vLLM principles",
# section 11.2).  A physical block of bs = R * T tokens is R consecutive tiles of T tokens:
# keys [NB, R, Hkv, T, D] (a key is one row of its tile), values [NB, R, Hkv, D, T] (the T
# tokens of one dimension are contiguous).  With R = 1 the tile axis is dropped: keys
# [NB, Hkv, bs, D], values [NB, Hkv, D, bs].  The library uses T = 16: one tile for 16-token
# blocks, bs / 16 tiles for larger blocks.  (Layout reading: the pages fix no layout.)
# ---------------------------------------------------------------------------
def tiles(pool: np.ndarray) -> np.ndarray:
    """The pool as [NB, R, Hkv, T, D] (keys) or [NB, R, Hkv, D, T] (values); a view."""
    return pool[:, None] if pool.ndim == 4 else pool


def key_tile_len(k_cache: np.ndarray) -> int:
    return tiles(k_cache).shape[3]


def value_tile_len(v_cache: np.ndarray) -> int:
    return tiles(v_cache).shape[4]


def default_scale(head_dim: int) -> float:
    """Scaled dot-product attention scale (reading: 1/sqrt(D); the pages give none)."""
    return 1.0 / math.sqrt(head_dim)


# ---------------------------------------------------------------------------
# Slot mapping and the cache write.
# ---------------------------------------------------------------------------
def token_positions(context_len: int, query_len: int) -> np.ndarray:
    """Absolute positions of a request's new tokens: they follow its cached ones."""
    return np.arange(context_len, context_len + query_len, dtype=np.int64)


def slot_mapping(block_tables, query_start_loc, context_lens, block_size: int) -> np.ndarray:
    """Flat pool slot of every new token (int64 [T]).

    Token i of request r sits at position p = context_lens[r] + i; its
    logical block p // block_size is the physical block block_tables[r, that],
    and the slot is physical_block * block_size + p % block_size.
    """
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    ctx = np.asarray(context_lens, dtype=np.int64)
    bt = np.asarray(block_tables, dtype=np.int64)
    out = np.empty(int(qsl[-1]), dtype=np.int64)
    for r in range(len(ctx)):
        p = token_positions(int(ctx[r]), int(qsl[r + 1] - qsl[r]))
        phys = bt[r, p // block_size]
        out[qsl[r] : qsl[r + 1]] = phys * block_size + p % block_size
    return out


def reshape_and_cache(k, v, k_cache, v_cache, slots, block_size: int) -> Tuple[np.ndarray, np.ndarray]:
    """Return copies of the pools with token t's K/V stored at its slot (bitwise; slot < 0 skipped).

    A slot names (block, offset); offset o lies in tile o // 16 of the block, at position o % 16.
    Token t's key is one row of that key tile, its value one column of that value tile (pool
    layout above).
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    kt, vt = tiles(kc), tiles(vc)
    T = key_tile_len(kc)
    assert kt.shape[1] * T == block_size and value_tile_len(vc) == T
    for t, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if s < 0:
            continue
        b, o = divmod(int(s), block_size)
        kt[b, o // T, :, o % T, :] = k[t]
        vt[b, o // T, :, :, o % T] = v[t]
    return kc, vc


def copy_blocks(k_cache, v_cache, block_pairs) -> Tuple[np.ndarray, np.ndarray]:
    """Return copies of the pools where every physical block dst of a pair (src, dst) holds the
    bits of block src, in both pools and every kv head (the copy-on-write of a shared block
    ["11. vLLM principles", section 11.2]).  Pairs outside the pool, or with src == dst, are
    skipped; all copies read the pools as they were before the call."""
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    nb = k_cache.shape[0]
    for src, dst in np.asarray(block_pairs, dtype=np.int64).reshape(-1, 2):
        if 0 <= src < nb and 0 <= dst < nb and src != dst:
            kc[dst] = k_cache[src]
            vc[dst] = v_cache[src]
    return kc, vc


# ---------------------------------------------------------------------------
# Gathering keys/values through a block table.
# ---------------------------------------------------------------------------
def gather_keys(k_cache, block_table_row, num_keys: int, kv_head: int, block_size: int) -> np.ndarray:
    """Keys 0..num_keys-1 of one kv head, in logical order, as fp64 [num_keys, D]."""
    T = key_tile_len(k_cache)
    assert tiles(k_cache).shape[1] * T == block_size
    j = np.arange(num_keys)
    phys = np.asarray(block_table_row, dtype=np.int64)[j // block_size]
    o = j % block_size
    return bf16_to_f64(tiles(k_cache)[phys, o // T, kv_head, o % T, :]).reshape(num_keys, k_cache.shape[-1])


def gather_values(v_cache, block_table_row, num_keys: int, kv_head: int, block_size: int) -> np.ndarray:
    """Values 0..num_keys-1 of one kv head, in logical order, as fp64 [num_keys, D]."""
    T = value_tile_len(v_cache)
    vt = tiles(v_cache)
    assert vt.shape[1] * T == block_size
    j = np.arange(num_keys)
    phys = np.asarray(block_table_row, dtype=np.int64)[j // block_size]
    o = j % block_size
    return bf16_to_f64(vt[phys, o // T, kv_head, :, o % T]).reshape(num_keys, vt.shape[3])


# ---------------------------------------------------------------------------
# Softmax attention state over a key set.
# ---------------------------------------------------------------------------
def attention_state(scores: np.ndarray, values: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax-weighted values and log-sum-exp for each row of ``scores``.

    ``scores`` is [M, N] (already scaled; -inf marks keys a row does not see),
    ``values`` is [N, D].  Row state: m = max_j s_j, Z = sum_j exp(s_j - m),
    o = sum_j exp(s_j - m) / Z * v_j, lse = m + ln Z.  A row that sees no key
    gets (o = 0, lse = -inf).
    """
    M = scores.shape[0]
    D = values.shape[1]
    o = np.zeros((M, D), dtype=np.float64)
    lse = np.full(M, -np.inf, dtype=np.float64)
    if scores.shape[1] == 0:
        return o, lse
    m = scores.max(axis=1)
    live = np.isfinite(m)
    if not live.any():
        return o, lse
    w = np.exp(scores[live] - m[live, None])
    z = w.sum(axis=1)
    o[live] = (w @ values) / z[:, None]
    lse[live] = m[live] + np.log(z)
    return o, lse


def causal_visible(context_len: int, query_len: int, num_keys: int) -> np.ndarray:
    """Boolean [query_len, num_keys]: token i (position context_len + i) sees key j iff j <= context_len + i."""
    p = token_positions(context_len, query_len)
    return np.arange(num_keys)[None, :] <= p[:, None]


def paged_attention(
    q,
    k_cache,
    v_cache,
    block_tables,
    query_start_loc,
    context_lens,
    seq_lens,
    block_size: int,
    scale: Optional[float] = None,
    rows: Optional[np.ndarray] = None,
    row_tile: int = 256,
) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of every new token over its request's paged keys (fp64).

    ``q`` is bf16 bits [T, Hq, D]; pools are the caches *after* the step's
    new keys/values were written.  For token t = query_start_loc[r] + i at
    position p = context_lens[r] + i and q head h, kv head g = h // G:
    keys/values 0..p come from the pools through block_tables[r]; the result
    is the softmax state of scale * q . k over them.

    ``rows`` (optional) restricts the work to those token indices; other rows
    of the outputs are left as NaN.  Returns (o [T, Hq, D], lse [T, Hq]).
    """
    q = np.asarray(q)
    T, Hq, D = q.shape
    Hkv = tiles(k_cache).shape[2]
    if Hq % Hkv:
        raise ValueError("q heads must be a multiple of kv heads")
    G = Hq // Hkv
    sc = default_scale(D) if scale is None or scale <= 0 else float(scale)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    ctx = np.asarray(context_lens, dtype=np.int64)
    sl = np.asarray(seq_lens, dtype=np.int64)
    o = np.full((T, Hq, D), np.nan, dtype=np.float64)
    lse = np.full((T, Hq), np.nan, dtype=np.float64)
    want = None if rows is None else np.zeros(T, dtype=bool)
    if want is not None:
        want[np.asarray(rows, dtype=np.int64)] = True
    for r in range(len(ctx)):
        t0, t1 = int(qsl[r]), int(qsl[r + 1])
        ql = t1 - t0
        if ql == 0:
            continue
        if sl[r] != ctx[r] + ql:
            raise ValueError(f"request {r}: seq_len != context_len + query_len")
        toks = np.arange(t0, t1)
        if want is not None:
            toks = toks[want[t0:t1]]
            if toks.size == 0:
                continue
        n = int(sl[r])
        vis_all = causal_visible(int(ctx[r]), ql, n)
        for g in range(Hkv):
            K = gather_keys(k_cache, block_tables[r], n, g, block_size)
            V = gather_values(v_cache, block_tables[r], n, g, block_size)
            for a in range(0, toks.size, row_tile):
                tt = toks[a : a + row_tile]
                vis = vis_all[tt - t0]
                for hh in range(G):
                    h = g * G + hh
                    Q = bf16_to_f64(q[tt, h, :])
                    s = sc * (Q @ K.T)
                    s = np.where(vis, s, -np.inf)
                    oo, ll = attention_state(s, V)
                    o[tt, h, :] = oo
                    lse[tt, h] = ll
    return o, lse


def cascade_prefix_attention(
    q, k_cache, v_cache, prefix_block_table, prefix_len: int, block_size: int, scale: Optional[float] = None
) -> Tuple[np.ndarray, np.ndarray]:
    """State of every query token over the shared prefix keys 0..prefix_len-1 (no mask).

    All queries come after the prefix, so every one of them sees every prefix key.
    Returns (o [T, Hq, D], lse [T, Hq]) in fp64.
    """
    q = np.asarray(q)
    T, Hq, D = q.shape
    Hkv = tiles(k_cache).shape[2]
    G = Hq // Hkv
    sc = default_scale(D) if scale is None or scale <= 0 else float(scale)
    o = np.zeros((T, Hq, D), dtype=np.float64)
    lse = np.full((T, Hq), -np.inf, dtype=np.float64)
    for g in range(Hkv):
        K = gather_keys(k_cache, prefix_block_table, prefix_len, g, block_size)
        V = gather_values(v_cache, prefix_block_table, prefix_len, g, block_size)
        for hh in range(G):
            h = g * G + hh
            s = sc * (bf16_to_f64(q[:, h, :]) @ K.T)
            o[:, h, :], lse[:, h] = attention_state(s, V)
    return o, lse


def merge_attn_states(o_a, lse_a, o_b, lse_b) -> Tuple[np.ndarray, np.ndarray]:
    """Combine the states of two disjoint key sets into the state of their union.

    With Z = exp(lse): o = (Z_a o_a + Z_b o_b) / (Z_a + Z_b) and
    lse = ln(Z_a + Z_b), evaluated shifted by max(lse_a, lse_b).  The empty
    state (0, -inf) is the identity, and two empty states give (0, -inf).
    """
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    m = np.maximum(lse_a, lse_b)
    empty = ~np.isfinite(m)
    ms = np.where(empty, 0.0, m)
    wa = np.where(np.isfinite(lse_a), np.exp(lse_a - ms), 0.0)
    wb = np.where(np.isfinite(lse_b), np.exp(lse_b - ms), 0.0)
    z = wa + wb
    zs = np.where(empty, 1.0, z)
    o = (wa[..., None] * np.asarray(o_a, np.float64) + wb[..., None] * np.asarray(o_b, np.float64)) / zs[..., None]
    lse = np.where(empty, -np.inf, ms + np.log(zs))
    return o, lse
