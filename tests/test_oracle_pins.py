"""Pins for the CPU fp64 oracle: page values, closed forms, independent routines, brute force.

None of these re-types the oracle's own formula: each pin comes from a
different direction (a value the pages print, a closed form, torch's fp64
scaled-dot-product attention, a dense attention written here over
contiguous keys, 50-digit decimal arithmetic, or an algebraic invariant).
"""

import decimal
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_examples.json")


@pytest.fixture(scope="module")
def page():
    with open(GOLDEN) as f:
        return json.load(f)


def rand_bf16(rng, *shape):
    return W.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def empty_pool(nb, hkv, bs, d):
    return np.full((nb, hkv, bs, d), W.BF16_NAN, dtype=np.uint16)


def empty_vpool(nb, hkv, bs, d):
    return np.full((nb, hkv, d, bs), W.BF16_NAN, dtype=np.uint16)


def token_view(pool):
    """Key pool [NB, H, bs, D] (or [NB, R, H, 16, D]) -> [NB*bs, H, D]: flat token slots (an
    independent way to address a slot)."""
    if pool.ndim == 5:
        nb, r, h, t, d = pool.shape
        return pool.transpose(0, 1, 3, 2, 4).reshape(nb * r * t, h, d)
    nb, h, bs, d = pool.shape
    return pool.transpose(0, 2, 1, 3).reshape(nb * bs, h, d)


def vtoken_view(pool):
    """Value pool [NB, H, D, bs] (or [NB, R, H, D, 16]) -> [NB*bs, H, D]."""
    if pool.ndim == 5:
        nb, r, h, d, t = pool.shape
        return pool.transpose(0, 1, 4, 2, 3).reshape(nb * r * t, h, d)
    nb, h, d, bs = pool.shape
    return pool.transpose(0, 3, 1, 2).reshape(nb * bs, h, d)


# ---------------------------------------------------------------------------
# Page values
# ---------------------------------------------------------------------------
def test_batched_prefill_concatenation(page):
    ex = page["batched_prefill"]
    wl = W.tiny_prefill(seed=0)
    st = wl.steps[0]
    assert list(st.query_lens) == ex["prompt_lens"]
    assert st.num_tokens == ex["total_tokens"]
    assert list(st.query_start_loc) == [0, 31, 60, 90]
    assert list(st.context_lens) == [0, 0, 0]


def test_slot_mapping_paging_figure(page):
    ex = page["paging_figure"]
    bs = ex["block_size"]
    bt = np.array([ex["logical_to_physical"]], dtype=np.int32)
    slots = O.slot_mapping(bt, [0, 48], [0], bs)
    for (lo, hi), phys in zip(ex["token_ranges"], ex["logical_to_physical"]):
        assert list(slots[lo : hi + 1]) == list(range(phys * bs, phys * bs + bs))


def test_slot_mapping_chunk_over_cache(page):
    ex = page["chunk_over_cache"]
    bt = np.array([[7, 2, 11]], dtype=np.int32)
    c, n = ex["cached_tokens"], ex["chunk_tokens"]
    slots = O.slot_mapping(bt, [0, n], [c], 16)
    # positions 16..30 are the first 15 slots of logical block 1 (physical 2)
    assert list(slots) == list(range(2 * 16, 2 * 16 + 15))
    assert c + n == 31


def test_slot_mapping_prefix_hit(page):
    ex = page["prefix_cache_hit"]
    c, total = ex["cached_tokens"], ex["total_tokens"]
    bt = np.array([[40, 41, 42, 43, 44, 45, 46]], dtype=np.int32)  # 7 blocks cover 107 tokens
    slots = O.slot_mapping(bt, [0, total - c], [c], 16)
    assert O.token_positions(c, total - c)[0] == ex["first_position"]
    assert slots[0] == 43 * 16 + 0  # position 48 = logical block 3, offset 0
    assert slots[-1] == 46 * 16 + 10  # position 106 = logical block 6, offset 10
    assert len(slots) == 59


def test_slot_mapping_multi_request_and_padding():
    bt = np.array([[5, 9, 0], [1, 2, 3]], dtype=np.int32)
    slots = O.slot_mapping(bt, [0, 3, 5], [15, 31], 16)
    # request 0: positions 15, 16, 17 -> (5, 15), (9, 0), (9, 1)
    # request 1: positions 31, 32 -> (2, 15), (3, 0)
    assert list(slots) == [5 * 16 + 15, 9 * 16, 9 * 16 + 1, 2 * 16 + 15, 3 * 16]


def test_tile_counts_of_chunked_prefill(page):
    ex = page["chunked_prefill"]
    n, c = ex["prompt_tokens"], ex["chunk_tokens"]
    full = O.causal_visible(0, n, n)
    # the page's 48^2 counts every 16x16 tile of the dense score matrix
    assert full.size // (c * c) == ex["full_cost_in_16x16_tiles"]
    chunk_tiles = 0
    chunk_pairs = 0
    for k in range(n // c):
        vis = O.causal_visible(k * c, c, (k + 1) * c)
        chunk_tiles += vis.size // (c * c)
        chunk_pairs += int(vis.sum())
        # the last row of chunk k sees all keys so far, the first sees k*c+1
        assert vis[0].sum() == k * c + 1 and vis[-1].sum() == (k + 1) * c
    assert chunk_tiles == ex["chunked_cost_in_16x16_tiles"]
    # exact causal work is the same either way: 48*49/2 pairs
    assert chunk_pairs == int(full.sum()) == n * (n + 1) // 2 == 1176
    # a full prefill that skips fully masked tiles also visits 6 tiles
    tiles = full.reshape(n // c, c, n // c, c).any(axis=(1, 3))
    assert int(tiles.sum()) == ex["chunked_cost_in_16x16_tiles"]


def test_prefix_hit_visible_keys_closed_form(page):
    """q = 0 gives uniform weights: o = mean of visible values and lse = ln(#visible)."""
    ex = page["prefix_cache_hit"]
    c, total = ex["cached_tokens"], ex["total_tokens"]
    bs, hkv, d = 16, 1, 4
    rng = np.random.default_rng(5)
    nblk = -(-total // bs)
    bt = rng.permutation(20)[:nblk].astype(np.int32)[None, :]
    kp = empty_pool(20, hkv, bs, d)
    vp = empty_vpool(20, hkv, bs, d)
    # V_j = (j, 1, 0, 0), exact in bf16 for j < 256; keys arbitrary
    vals = np.zeros((total, hkv, d), np.float32)
    vals[:, 0, 0] = np.arange(total)
    vals[:, 0, 1] = 1.0
    kv = rand_bf16(rng, total, hkv, d)
    slots = O.slot_mapping(bt, [0, total], [0], bs)
    kp, vp = O.reshape_and_cache(kv, W.f32_to_bf16_bits(vals), kp, vp, slots, bs)
    q = np.zeros((total - c, 1, d), np.uint16)
    o, lse = O.paged_attention(q, kp, vp, bt, [0, total - c], [c], [total], bs)
    nvis = 2 * o[:, 0, 0] + 1
    assert nvis[0] == pytest.approx(c + 1, abs=1e-9)  # first new row sees 49 keys
    assert nvis[-1] == pytest.approx(total, abs=1e-9)  # last sees all 107
    assert np.allclose(lse[:, 0], np.log(np.arange(c + 1, total + 1)), atol=1e-12)
    assert np.allclose(o[:, 0, 1], 1.0, atol=1e-15)


def test_shared_block_tables_give_identical_prefix_states(page):
    ex = page["block_table_sharing"]
    bs, hkv, hq, d = 16, 2, 4, 8
    rng = np.random.default_rng(11)
    kp = rand_bf16(rng, 16, hkv, bs, d)
    vp = rand_bf16(rng, 16, hkv, d, bs)
    ta = np.array(ex["table_a"], np.int32)
    tb = np.array(ex["table_b"], np.int32)
    q = rand_bf16(rng, 3, hq, d)
    n_shared = len(ex["shared_logical_blocks"]) * bs
    oa, la = O.cascade_prefix_attention(q, kp, vp, ta, n_shared, bs)
    ob, lb = O.cascade_prefix_attention(q, kp, vp, tb, n_shared, bs)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)
    # beyond the shared blocks the two tables diverge
    oa3, _ = O.cascade_prefix_attention(q, kp, vp, ta, 3 * bs, bs)
    ob3, _ = O.cascade_prefix_attention(q, kp, vp, tb, 3 * bs, bs)
    assert not np.allclose(oa3, ob3)


# ---------------------------------------------------------------------------
# Cache write
# ---------------------------------------------------------------------------
def test_reshape_and_cache_bitwise():
    rng = np.random.default_rng(3)
    nb, h, bs, d, t = 12, 3, 16, 8, 40
    kp = rng.integers(0, 1 << 16, size=(nb, h, bs, d), dtype=np.uint16)
    vp = rng.integers(0, 1 << 16, size=(nb, h, d, bs), dtype=np.uint16)
    k = rng.integers(0, 1 << 16, size=(t, h, d), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, size=(t, h, d), dtype=np.uint16)
    slots = rng.choice(nb * bs, size=t, replace=False).astype(np.int64)
    slots[::7] = -1
    k2, v2 = O.reshape_and_cache(k, v, kp, vp, slots, bs)
    fk, fv = token_view(k2), vtoken_view(v2)
    fk0, fv0 = token_view(kp), vtoken_view(vp)
    written = np.zeros(nb * bs, bool)
    for i, s in enumerate(slots):
        if s >= 0:
            assert np.array_equal(fk[s], k[i]) and np.array_equal(fv[s], v[i])
            written[s] = True
    assert np.array_equal(fk[~written], fk0[~written])
    assert np.array_equal(fv[~written], fv0[~written])


# ---------------------------------------------------------------------------
# Independent attention routines
# ---------------------------------------------------------------------------
def _sdpa_fp64(q, k, v, mask, scale):
    """torch fp64 SDPA over one request: q [L, H, D], k/v [S, H, D], mask [L, S] bool."""
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2)[None]
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.from_numpy(mask), scale=scale
    )
    return out[0].permute(1, 0, 2).numpy()


def test_copy_blocks_bits_and_skips():
    """Copied blocks hold the source bits in both pools; untouched blocks keep theirs; pairs
    outside the pool and src == dst change nothing."""
    rng = np.random.default_rng(21)
    nb, hkv, bs, d = 12, 2, 16, 8
    kp = rand_bf16(rng, nb, hkv, bs, d)
    vp = rand_bf16(rng, nb, hkv, d, bs)
    pairs = np.array([[3, 9], [4, 4], [0, 11], [-1, 2], [5, 12]], dtype=np.int32)
    kc, vc = O.copy_blocks(kp, vp, pairs)
    for b in range(nb):
        src = {9: 3, 11: 0}.get(b, b)
        assert np.array_equal(kc[b], kp[src]) and np.array_equal(vc[b], vp[src]), b
    assert np.array_equal(kp, rand_bf16(np.random.default_rng(21), nb, hkv, bs, d))  # inputs untouched


def test_copy_on_write_keeps_the_sharer_unchanged(page):
    """["11. vLLM principles", 11.2 block-table example] A = [3, 7, 11] and B = [3, 7, 5] share
    physical blocks 3 and 7.  B takes a private copy of block 7 (to block 12) before writing a
    token into it; afterwards A's attention is the same as before, and B's equals attention over
    its own keys laid out in a fresh pool."""
    ex = page["block_table_sharing"]
    a_bt, b_bt = np.array(ex["table_a"]), np.array(ex["table_b"])
    rng = np.random.default_rng(22)
    nb, hkv, bs, d, hq = 16, 1, 16, 8, 2
    kp = rand_bf16(rng, nb, hkv, bs, d)
    vp = rand_bf16(rng, nb, hkv, d, bs)
    q = rand_bf16(rng, 2, hq, d)
    ctx_len = 40  # both requests see 41 keys: blocks 0..2
    qsl = np.array([0, 1, 2])
    ctx = np.array([ctx_len, ctx_len])
    seq = ctx + 1
    bts = np.stack([a_bt, b_bt]).astype(np.int32)
    before_o, before_l = O.paged_attention(q, kp, vp, bts, qsl, ctx, seq, bs)
    # B copies shared block 7 and overwrites one of its tokens (slot 12*16 + 5) in its copy.
    kc, vc = O.copy_blocks(kp, vp, np.array([[b_bt[1], 12]]))
    b_new = b_bt.copy()
    b_new[1] = 12
    kn = rand_bf16(rng, 1, hkv, d)
    vn = rand_bf16(rng, 1, hkv, d)
    kc, vc = O.reshape_and_cache(kn, vn, kc, vc, np.array([12 * bs + 5]), bs)
    bts2 = np.stack([a_bt, b_new]).astype(np.int32)
    after_o, after_l = O.paged_attention(q, kc, vc, bts2, qsl, ctx, seq, bs)
    assert np.array_equal(after_o[0], before_o[0]) and np.array_equal(after_l[0], before_l[0])
    # B against its keys copied block by block into a fresh pool (blocks 0, 1, 2).
    fk = np.stack([kc[b] for b in b_new])
    fv = np.stack([vc[b] for b in b_new])
    ref_o, ref_l = O.paged_attention(q[1:], fk, fv, np.array([[0, 1, 2]], np.int32), [0, 1], [ctx_len],
                                     [ctx_len + 1], bs)
    assert np.array_equal(after_o[1], ref_o[0]) and np.array_equal(after_l[1], ref_l[0])
    assert not np.allclose(after_o[1], before_o[1])  # the write did reach B


def test_tiny_prefill_matches_torch_sdpa():
    wl = W.tiny_prefill(seed=1)
    st = wl.steps[0]
    bs = wl.block_size
    slots = O.slot_mapping(st.block_tables, st.query_start_loc, st.context_lens, bs)
    kp, vp = O.reshape_and_cache(st.k, st.v, wl.k_cache, wl.v_cache, slots, bs)
    o, _ = O.paged_attention(st.q, kp, vp, st.block_tables, st.query_start_loc, st.context_lens, st.seq_lens, bs)
    G = wl.group
    for r in range(st.num_seqs):
        a, b = st.query_start_loc[r], st.query_start_loc[r + 1]
        q = O.bf16_to_f64(st.q[a:b])
        k = np.repeat(O.bf16_to_f64(st.k[a:b]), G, axis=1)
        v = np.repeat(O.bf16_to_f64(st.v[a:b]), G, axis=1)
        L = b - a
        mask = np.tril(np.ones((L, L), bool))
        ref = _sdpa_fp64(q, k, v, mask, 1.0 / math.sqrt(wl.head_dim))
        assert np.max(np.abs(o[a:b] - ref)) < 1e-12


def _dense_attention(q, keys, vals, positions, scale):
    """Dense causal attention over contiguous keys: row i sees keys 0..positions[i]."""
    s = scale * np.einsum("lhd,shd->lhs", q, keys)
    n = keys.shape[0]
    s = np.where(np.arange(n)[None, None, :] <= positions[:, None, None], s, -np.inf)
    s = s - s.max(axis=2, keepdims=True)
    w = np.exp(s)
    w /= w.sum(axis=2, keepdims=True)
    return np.einsum("lhs,shd->lhd", w, vals)


@pytest.mark.parametrize("block_size", [16, 32, 256])
def test_mixed_batch_matches_dense_contiguous_attention(block_size):
    """Paging invariance: the paged oracle equals dense attention on keys laid out in logical order."""
    wl = W.mixed_llama8b(seed=2, num_decode=6, ctx_range=(20, 90 if block_size == 16 else 600), block_size=block_size)
    bs, G = wl.block_size, wl.group
    kp, vp = wl.k_cache, wl.v_cache
    # logical key history per request, tracked here without the oracle's gather
    hist_k, hist_v = {}, {}
    for st in wl.steps:
        slots = O.slot_mapping(st.block_tables, st.query_start_loc, st.context_lens, bs)
        kp, vp = O.reshape_and_cache(st.k, st.v, kp, vp, slots, bs)
        o, _ = O.paged_attention(st.q, kp, vp, st.block_tables, st.query_start_loc, st.context_lens, st.seq_lens, bs)
        for r in range(st.num_seqs):
            rid = int(st.request_ids[r])
            a, b = st.query_start_loc[r], st.query_start_loc[r + 1]
            c = int(st.context_lens[r])
            if rid not in hist_k:
                # cached history before the first step: read it through the flat token view
                tv_k, tv_v = token_view(wl.k_cache), vtoken_view(wl.v_cache)
                phys = [int(st.block_tables[r][j // bs]) * bs + j % bs for j in range(c)]
                hist_k[rid] = [O.bf16_to_f64(tv_k[s]) for s in phys]
                hist_v[rid] = [O.bf16_to_f64(tv_v[s]) for s in phys]
            hist_k[rid] += [O.bf16_to_f64(x) for x in st.k[a:b]]
            hist_v[rid] += [O.bf16_to_f64(x) for x in st.v[a:b]]
            keys = np.repeat(np.stack(hist_k[rid]), G, axis=1)
            vals = np.repeat(np.stack(hist_v[rid]), G, axis=1)
            pos = np.arange(c, c + (b - a))
            ref = _dense_attention(O.bf16_to_f64(st.q[a:b]), keys, vals, pos, 1 / math.sqrt(wl.head_dim))
            assert np.max(np.abs(o[a:b] - ref)) < 1e-12


def test_physical_permutation_invariance():
    wl = W.decode_only(seed=3, num_seqs=5, ctx_range=(17, 70))
    st = wl.steps[0]
    bs = wl.block_size
    rng = np.random.default_rng(9)
    perm = rng.permutation(wl.num_blocks)
    kp2 = np.empty_like(wl.k_cache)
    vp2 = np.empty_like(wl.v_cache)
    kp2[perm] = wl.k_cache
    vp2[perm] = wl.v_cache
    bt2 = perm[st.block_tables].astype(np.int32)
    res = []
    for kp, vp, bt in ((wl.k_cache, wl.v_cache, st.block_tables), (kp2, vp2, bt2)):
        slots = O.slot_mapping(bt, st.query_start_loc, st.context_lens, bs)
        kq, vq = O.reshape_and_cache(st.k, st.v, kp, vp, slots, bs)
        res.append(O.paged_attention(st.q, kq, vq, bt, st.query_start_loc, st.context_lens, st.seq_lens, bs))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])


# ---------------------------------------------------------------------------
# Chunked prefill, prefix caching, cascade: equal to the single-pass result
# ---------------------------------------------------------------------------
def _run_steps(q, k, v, chunks, context0, bt, pools, bs):
    """Feed one request's tokens in chunks; returns per-token outputs stacked and final pools."""
    kp, vp = pools
    outs, lses = [], []
    done = context0
    pos = 0
    for n in chunks:
        qsl = [0, n]
        slots = O.slot_mapping(bt, qsl, [done], bs)
        kp, vp = O.reshape_and_cache(k[pos : pos + n], v[pos : pos + n], kp, vp, slots, bs)
        o, l = O.paged_attention(q[pos : pos + n], kp, vp, bt, qsl, [done], [done + n], bs)
        outs.append(o)
        lses.append(l)
        done += n
        pos += n
    return np.concatenate(outs), np.concatenate(lses), (kp, vp)


@pytest.mark.parametrize("total,chunks", [(48, [16, 16, 16]), (31, [16, 15]), (70, [1, 33, 5, 31])])
def test_chunked_equals_unchunked(total, chunks):
    rng = np.random.default_rng(total)
    bs, hkv, hq, d = 16, 2, 6, 16
    q = rand_bf16(rng, total, hq, d)
    k = rand_bf16(rng, total, hkv, d)
    v = rand_bf16(rng, total, hkv, d)
    nb = 12
    bt = rng.permutation(nb)[None, :].astype(np.int32)
    pools = (empty_pool(nb, hkv, bs, d), empty_vpool(nb, hkv, bs, d))
    o1, l1, p1 = _run_steps(q, k, v, [total], 0, bt, pools, bs)
    o2, l2, p2 = _run_steps(q, k, v, chunks, 0, bt, pools, bs)
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12
    assert np.array_equal(p1[0], p2[0]) and np.array_equal(p1[1], p2[1])


def test_prefix_cached_equals_suffix_of_full(page):
    ex = page["prefix_cache_hit"]
    total, c = ex["total_tokens"], ex["cached_tokens"]
    rng = np.random.default_rng(107)
    bs, hkv, hq, d = 16, 2, 4, 32
    q = rand_bf16(rng, total, hq, d)
    k = rand_bf16(rng, total, hkv, d)
    v = rand_bf16(rng, total, hkv, d)
    nb = 10
    bt = rng.permutation(nb)[None, :7].astype(np.int32)
    pools = (empty_pool(nb, hkv, bs, d), empty_vpool(nb, hkv, bs, d))
    full_o, full_l, _ = _run_steps(q, k, v, [total], 0, bt, pools, bs)
    # the cache already holds tokens 0..47 (written by an earlier request)
    slots = O.slot_mapping(bt, [0, c], [0], bs)
    cached = O.reshape_and_cache(k[:c], v[:c], *pools, slots, bs)
    hit_o, hit_l, _ = _run_steps(q[c:], k[c:], v[c:], [total - c], c, bt, cached, bs)
    assert np.max(np.abs(hit_o - full_o[c:])) < 1e-12
    assert np.max(np.abs(hit_l - full_l[c:])) < 1e-12


def test_cascade_plus_merge_equals_single_pass():
    wl = W.cascade_shared_prefix(seed=4, num_queries=12, prefix=64, suffix_range=(1, 40), num_q_heads=16)
    st = wl.steps[0]
    cv = wl.cascade
    bs = wl.block_size
    slots = O.slot_mapping(st.block_tables, st.query_start_loc, st.context_lens, bs)
    kp, vp = O.reshape_and_cache(st.k, st.v, wl.k_cache, wl.v_cache, slots, bs)
    full_o, full_l = O.paged_attention(st.q, kp, vp, st.block_tables, st.query_start_loc, st.context_lens, st.seq_lens, bs)
    po, pl = O.cascade_prefix_attention(st.q, kp, vp, cv.prefix_block_table, cv.prefix_len, bs)
    sbt = st.block_tables[:, cv.prefix_blocks(bs) :]
    so, sl = O.paged_attention(st.q, kp, vp, sbt, st.query_start_loc, cv.suffix_context_lens, cv.suffix_seq_lens, bs)
    mo, ml = O.merge_attn_states(po, pl, so, sl)
    assert np.max(np.abs(mo - full_o)) < 1e-12
    assert np.max(np.abs(ml - full_l)) < 1e-12


def test_split_at_any_key_and_merge():
    rng = np.random.default_rng(21)
    n, d = 37, 8
    s = rng.standard_normal((5, n)) * 3
    vals = rng.standard_normal((n, d))
    whole = O.attention_state(s, vals)
    for cut in range(0, n + 1):
        a = O.attention_state(s[:, :cut], vals[:cut])
        b = O.attention_state(s[:, cut:], vals[cut:])
        m = O.merge_attn_states(a[0], a[1], b[0], b[1])
        assert np.max(np.abs(m[0] - whole[0])) < 1e-13
        assert np.max(np.abs(m[1] - whole[1])) < 1e-13


# ---------------------------------------------------------------------------
# Merge algebra
# ---------------------------------------------------------------------------
def test_merge_commutative_associative_identity():
    rng = np.random.default_rng(8)
    shape = (6, 3)
    st = [(rng.standard_normal(shape + (5,)), rng.standard_normal(shape) * 4) for _ in range(3)]
    ab = O.merge_attn_states(*st[0], *st[1])
    ba = O.merge_attn_states(*st[1], *st[0])
    assert np.array_equal(ab[0], ba[0]) and np.array_equal(ab[1], ba[1])
    left = O.merge_attn_states(*ab, *st[2])
    bc = O.merge_attn_states(*st[1], *st[2])
    right = O.merge_attn_states(*st[0], *bc)
    assert np.max(np.abs(left[0] - right[0])) < 1e-13 and np.max(np.abs(left[1] - right[1])) < 1e-13
    empty = (np.zeros(shape + (5,)), np.full(shape, -np.inf))
    ident = O.merge_attn_states(*st[0], *empty)
    assert np.max(np.abs(ident[0] - st[0][0])) < 1e-15 and np.array_equal(ident[1], st[0][1])
    both = O.merge_attn_states(*empty, *empty)
    assert np.array_equal(both[0], empty[0]) and np.all(np.isneginf(both[1]))
    assert not np.isnan(both[0]).any()


# ---------------------------------------------------------------------------
# Closed forms and brute force
# ---------------------------------------------------------------------------
def _single_request(q, k, v, bs=4, ctx=0):
    """Run one request of len(k) keys whose last len(q) tokens are new, through a shuffled pool."""
    n, hkv, d = k.shape
    nb = -(-n // bs) + 3
    bt = np.random.default_rng(n).permutation(nb)[None, :].astype(np.int32)
    kp, vp = empty_pool(nb, hkv, bs, d), empty_vpool(nb, hkv, bs, d)
    slots = O.slot_mapping(bt, [0, n], [0], bs)
    kp, vp = O.reshape_and_cache(k, v, kp, vp, slots, bs)
    L = q.shape[0]
    return O.paged_attention(q, kp, vp, bt, [0, L], [n - L], [n], bs)


def test_one_key_returns_its_value_exactly():
    rng = np.random.default_rng(1)
    q = rand_bf16(rng, 1, 4, 16)
    k = rand_bf16(rng, 1, 2, 16)
    v = rand_bf16(rng, 1, 2, 16)
    o, lse = _single_request(q, k, v)
    assert np.array_equal(o[0], np.repeat(O.bf16_to_f64(v[0]), 2, axis=0))
    s = O.bf16_to_f64(q[0]) @ np.repeat(O.bf16_to_f64(k[0]), 2, axis=0).T / 4.0
    assert np.allclose(lse[0], np.diag(s), atol=1e-15)


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(2)
    n = 23
    k = rand_bf16(rng, n, 1, 8)
    v = rand_bf16(rng, n, 1, 8)
    q = np.zeros((1, 2, 8), np.uint16)
    o, lse = _single_request(q, k, v)
    mean = O.bf16_to_f64(v).mean(axis=0)[0]
    assert np.max(np.abs(o[0] - mean)) < 1e-15
    assert np.allclose(lse[0], math.log(n), atol=1e-15)


def test_two_keys_sigmoid():
    rng = np.random.default_rng(4)
    d = 8
    q = rand_bf16(rng, 1, 1, d)
    k = rand_bf16(rng, 2, 1, d)
    v = rand_bf16(rng, 2, 1, d)
    o, lse = _single_request(q, k, v)
    qq, kk, vv = O.bf16_to_f64(q)[0, 0], O.bf16_to_f64(k)[:, 0], O.bf16_to_f64(v)[:, 0]
    s0, s1 = (kk @ qq) / math.sqrt(d)
    p0 = 1.0 / (1.0 + math.exp(s1 - s0))
    assert np.max(np.abs(o[0, 0] - (p0 * vv[0] + (1 - p0) * vv[1]))) < 1e-15
    assert abs(lse[0, 0] - (s0 + math.log1p(math.exp(s1 - s0)))) < 1e-14


def test_gqa_equals_mha_on_repeated_kv():
    rng = np.random.default_rng(6)
    n, hkv, G, d = 29, 2, 3, 16
    q = rand_bf16(rng, 5, hkv * G, d)
    k = rand_bf16(rng, n, hkv, d)
    v = rand_bf16(rng, n, hkv, d)
    o1, l1 = _single_request(q, k, v)
    o2, l2 = _single_request(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_brute_force_decimal_50_digits():
    decimal.getcontext().prec = 50
    D = decimal.Decimal
    rng = np.random.default_rng(12)
    for n in range(1, 7):
        d = 3
        q = rand_bf16(rng, 2, 2, d)
        k = rand_bf16(rng, n, 1, d)
        v = rand_bf16(rng, n, 1, d)
        o, lse = _single_request(q, k, v, bs=2)
        qf, kf, vf = O.bf16_to_f64(q), O.bf16_to_f64(k), O.bf16_to_f64(v)
        scale = D(1) / D(d).sqrt()
        for i in range(2):
            p = n - 2 + i  # query i is at position p, sees keys 0..p
            for h in range(2):
                if p < 0:
                    continue
                s = [scale * sum(D(float(qf[i, h, x])) * D(float(kf[j, 0, x])) for x in range(d)) for j in range(p + 1)]
                m = max(s)
                e = [(sj - m).exp() for sj in s]
                z = sum(e)
                for x in range(d):
                    ref = sum(e[j] * D(float(vf[j, 0, x])) for j in range(p + 1)) / z
                    assert abs(float(ref) - o[i, h, x]) < 1e-14
                assert abs(float(m + z.ln()) - lse[i, h]) < 1e-14


def test_row_subset_matches_full():
    wl = W.decode_only(seed=5, num_seqs=6, ctx_range=(10, 50))
    st = wl.steps[0]
    bs = wl.block_size
    slots = O.slot_mapping(st.block_tables, st.query_start_loc, st.context_lens, bs)
    kp, vp = O.reshape_and_cache(st.k, st.v, wl.k_cache, wl.v_cache, slots, bs)
    args = (st.q, kp, vp, st.block_tables, st.query_start_loc, st.context_lens, st.seq_lens, bs)
    full = O.paged_attention(*args)
    part = O.paged_attention(*args, rows=np.array([1, 4]))
    assert np.array_equal(full[0][[1, 4]], part[0][[1, 4]])
    assert np.isnan(part[0][0]).all()


def test_workload_poison_covers_unwritten_slots():
    """The generator leaves NaN wherever no token is cached, and finite values where one is."""
    wl = W.mixed_llama8b(seed=0, num_decode=3, ctx_range=(20, 40))
    st = wl.steps[0]
    bs = wl.block_size
    for tv in (token_view(wl.k_cache), vtoken_view(wl.v_cache)):
        for r in range(st.num_seqs):
            c = int(st.context_lens[r])
            cached = [int(st.block_tables[r][j // bs]) * bs + j % bs for j in range(c)]
            assert np.isfinite(W.bf16_bits_to_f32(tv[cached])).all()
            fut = [int(st.block_tables[r][j // bs]) * bs + j % bs for j in range(c, int(st.seq_lens[r]))]
            assert np.isnan(W.bf16_bits_to_f32(tv[fut])).all()


# ---------------------------------------------------------------------------
# Blocks of 16 R tokens: a block of R tiles behaves as R blocks of 16 tokens
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("bs", [32, 64, 256])
def test_large_block_is_r_16_token_blocks(bs):
    """A block of bs = 16 R tokens is R consecutive 16-token tiles: the pool read as a bs=16 pool
    of R x the blocks, with table entry R b + i for tile i of block b, must give the same slots'
    bytes and the same attention, bit for bit."""
    wl = W.mixed_llama8b(seed=5, num_decode=7, ctx_range=(200, 900), block_size=bs)
    R = bs // 16
    kp, vp = wl.k_cache, wl.v_cache
    k16 = kp.reshape(wl.num_blocks * R, wl.num_kv_heads, 16, wl.head_dim)
    v16 = vp.reshape(wl.num_blocks * R, wl.num_kv_heads, wl.head_dim, 16)
    for st in wl.steps:
        bt16 = (st.block_tables[:, :, None] * R + np.arange(R)[None, None, :]).reshape(st.num_seqs, -1).astype(np.int32)
        sbig = O.slot_mapping(st.block_tables, st.query_start_loc, st.context_lens, bs)
        s16 = O.slot_mapping(bt16, st.query_start_loc, st.context_lens, 16)
        assert np.array_equal(sbig, s16)
        kp, vp = O.reshape_and_cache(st.k, st.v, kp, vp, sbig, bs)
        k16, v16 = O.reshape_and_cache(st.k, st.v, k16, v16, s16, 16)
        assert np.array_equal(kp.reshape(k16.shape), k16) and np.array_equal(vp.reshape(v16.shape), v16)
        args = (st.query_start_loc, st.context_lens, st.seq_lens)
        obig, lbig = O.paged_attention(st.q, kp, vp, st.block_tables, *args, bs)
        o16, l16 = O.paged_attention(st.q, k16, v16, bt16, *args, 16)
        assert np.array_equal(obig, o16) and np.array_equal(lbig, l16)
