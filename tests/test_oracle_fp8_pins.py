"""Pins for the FP8 (e4m3) half of the CPU oracle.

The format is pinned from outside the oracle's own code: code values from the bit-field
definition evaluated in exact rational arithmetic, the nearest-value rule by exhaustive search
over every finite code in rational arithmetic, the printed corner values of the format (1.0,
448, the smallest subnormal), hand-worked ties, and the cache and attention functions against
the bf16 oracle on inputs where the two must agree exactly.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import workloads as W


def _code_value(c):
    """Exact value of code c from the bit fields (sign, 4-bit exponent with bias 7, 3-bit
    mantissa; exponent 0 is subnormal); None for the NaN codes."""
    s, e, m = c >> 7, (c >> 3) & 15, c & 7
    if e == 15 and m == 7:
        return None
    mag = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -mag if s else mag


FINITE = [c for c in range(256) if _code_value(c) is not None]


def _nearest_even(x):
    """Exhaustive nearest finite code to the rational x (clamped to +-448), ties to the code
    with an even mantissa; -0 for negative values that round to zero."""
    x = max(min(x, Fraction(448)), Fraction(-448))
    best = None
    for c in FINITE:
        v = _code_value(c)
        if (c >> 7) != (1 if x < 0 else 0):
            continue  # codes of the other sign are never nearer (zero has both signs)
        d = abs(v - x)
        if best is None or d < best[0] or (d == best[0] and (c & 1) == 0 and (best[1] & 1) == 1):
            best = (d, c)
    return best[1]


def test_code_table_from_bit_fields():
    vals = O.e4m3_decode(np.arange(256, dtype=np.uint8))
    for c in range(256):
        v = _code_value(c)
        if v is None:
            assert np.isnan(vals[c]), c
        else:
            assert vals[c] == float(v), c
    assert len(FINITE) == 254


def test_corner_values():
    d = lambda c: float(O.e4m3_decode(np.uint8(c)))  # noqa: E731
    assert d(0x38) == 1.0
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x01) == 2.0**-9  # smallest subnormal
    assert d(0x08) == 2.0**-6  # smallest normal
    assert d(0x07) == 7 * 2.0**-9  # largest subnormal
    assert d(0x80) == 0.0 and np.signbit(O.e4m3_decode(np.uint8(0x80)))
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))


def test_values_strictly_increase_with_the_code():
    pos = O.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(O.e4m3_decode(np.arange(0x80, 0xFF, dtype=np.uint8)), -pos)


def test_encode_round_trips_every_finite_code():
    codes = np.array(FINITE, dtype=np.uint8)
    assert np.array_equal(O.e4m3_encode(O.e4m3_decode(codes).astype(np.float32)), codes)


@pytest.mark.parametrize(
    "x,code",
    [
        (1.0625, 0x38),  # halfway 1.0 / 1.125: even mantissa 0
        (1.1875, 0x3A),  # halfway 1.125 / 1.25: even mantissa 2
        (2.0**-10, 0x00),  # halfway 0 / 2^-9
        (3 * 2.0**-10, 0x02),  # halfway 2^-9 / 2^-8
        (5 * 2.0**-10, 0x02),  # halfway 2*2^-9 / 3*2^-9
        (432.0, 0x7E),  # halfway 416 / 448
        (-1.0625, 0xB8),
        (-(2.0**-12), 0x80),  # rounds to -0
        (449.0, 0x7E),
        (480.0, 0x7E),
        (1e30, 0x7E),
        (float("inf"), 0x7E),
        (-1e30, 0xFE),
        (float("-inf"), 0xFE),
        (0.0, 0x00),
        (-0.0, 0x80),
    ],
)
def test_encode_ties_and_saturation(x, code):
    assert int(O.e4m3_encode(np.float32(x))) == code


def test_encode_nan():
    assert int(O.e4m3_encode(np.float32("nan"))) == 0x7F


def test_encode_matches_exhaustive_rational_search():
    rng = np.random.default_rng(11)
    # values around every binade of the format, plus exact midpoints and the saturation range
    xs = list((rng.standard_normal(400) * np.exp2(rng.integers(-12, 10, 400))).astype(np.float32))
    pos = [_code_value(c) for c in FINITE if 0 < c < 0x7F]
    xs += [np.float32(float((a + b) / 2)) for a, b in zip(pos[::3], pos[1::3])]
    xs += [np.float32(v) for v in (447.9, 448.1, 463.9, 464.0, 500.0)]
    got = O.e4m3_encode(np.array(xs, dtype=np.float32))
    for x, c in zip(xs, got):
        assert int(c) == _nearest_even(Fraction(float(x))), x


def test_quantize_divides_by_the_scale_in_fp32():
    rng = np.random.default_rng(5)
    x = W.f32_to_bf16_bits(rng.standard_normal(2000).astype(np.float32) * 4)
    xf = W.bf16_bits_to_f32(x)
    # a power-of-two scale: x / s is exact, so the codes are those of x / s
    assert np.array_equal(O.quantize(x, 0.25), O.e4m3_encode(xf * np.float32(4.0)))
    # a general scale: y = fp32(x * fp32(1 / s)) rounded to the nearest code
    s = np.float32(0.0173)
    inv = np.float32(1.0) / s
    for xi, c in zip(xf[:300], O.quantize(x[:300], s)):
        y = np.float32(xi * inv)
        assert int(c) == _nearest_even(Fraction(float(y)))


def test_reshape_and_cache_fp8_places_like_the_bf16_cache():
    """Byte placement equals the bf16 cache's on the same slots; each token is quantised with
    the scale of the block its slot falls in."""
    rng = np.random.default_rng(7)
    nb, h, bs, d, t = 9, 2, 16, 8, 50
    k = W.f32_to_bf16_bits(rng.standard_normal((t, h, d)).astype(np.float32))
    v = W.f32_to_bf16_bits(rng.standard_normal((t, h, d)).astype(np.float32))
    ks = rng.uniform(0.01, 0.1, (nb, h)).astype(np.float32)
    vs = rng.uniform(0.01, 0.1, (nb, h)).astype(np.float32)
    slots = rng.choice(nb * bs, size=t, replace=False).astype(np.int64)
    slots[::9] = -1
    slots[4] = nb * bs + 3  # past the pool: skipped
    kp = np.full((nb, h, bs, d), 0x7F, np.uint8)
    vp = np.full((nb, h, d, bs), 0x7F, np.uint8)
    k8, v8 = O.reshape_and_cache_fp8(k, v, kp, vp, slots, ks, vs, bs)
    # expected codes per token, then placed by the bf16 cache into uint16 pools
    kq = np.zeros((t, h, d), np.uint16)
    vq = np.zeros((t, h, d), np.uint16)
    for i, s in enumerate(slots):
        b = s // bs
        if 0 <= s < nb * bs:
            for g in range(h):
                kq[i, g] = O.e4m3_encode(W.bf16_bits_to_f32(k[i, g]) * (np.float32(1) / ks[b, g]))
                vq[i, g] = O.e4m3_encode(W.bf16_bits_to_f32(v[i, g]) * (np.float32(1) / vs[b, g]))
    ok = (slots >= 0) & (slots < nb * bs)
    k16, v16 = O.reshape_and_cache(kq[ok], vq[ok], kp.astype(np.uint16), vp.astype(np.uint16), slots[ok], bs)
    assert np.array_equal(k8, k16.astype(np.uint8)) and np.array_equal(v8, v16.astype(np.uint8))


def test_attention_fp8_equals_bf16_attention_on_exact_values():
    """With power-of-two scales every dequantised value is a bf16 number, so attention over the
    fp8 pools must equal the bf16 oracle's attention over pools holding those numbers."""
    wl = W.mixed_llama8b(seed=4, num_decode=4, ctx_range=(20, 70))
    st = wl.steps[0]
    bs = wl.block_size
    c = W.fp8_cache(wl, seed=4)
    rng = np.random.default_rng(2)
    ks = np.exp2(rng.integers(-5, -1, (wl.num_blocks, wl.num_kv_heads))).astype(np.float32)
    vs = np.exp2(rng.integers(-5, -1, (wl.num_blocks, wl.num_kv_heads))).astype(np.float32)
    slots = O.slot_mapping(st.block_tables, st.query_start_loc, st.context_lens, bs)
    k8, v8 = O.reshape_and_cache_fp8(st.k, st.v, c.k_cache, c.v_cache, slots, ks, vs, bs)
    # the same numbers as bf16 pools (exact: e4m3 values times powers of two fit bf16)
    kb = W.f32_to_bf16_bits((O.e4m3_decode(k8) * ks[:, :, None, None]).astype(np.float32))
    vb = W.f32_to_bf16_bits((O.e4m3_decode(v8) * vs[:, :, None, None]).astype(np.float32))
    args = (st.block_tables, st.query_start_loc, st.context_lens, st.seq_lens, bs)
    o8, l8 = O.paged_attention_fp8(st.q, k8, v8, ks, vs, *args)
    ob, lb = O.paged_attention(st.q, kb, vb, *args)
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb)


def test_attention_fp8_scales_follow_the_block():
    """Doubling the value scales of one physical block changes exactly the rows whose keys
    use that block; doubling every key scale of a request is attention at twice the scale."""
    wl = W.decode_only(seed=6, num_seqs=3, ctx_range=(40, 60), num_q_heads=8)
    st = wl.steps[0]
    bs = wl.block_size
    c = W.fp8_cache(wl, seed=6)
    slots = O.slot_mapping(st.block_tables, st.query_start_loc, st.context_lens, bs)
    k8, v8 = O.reshape_and_cache_fp8(st.k, st.v, c.k_cache, c.v_cache, slots, c.k_scale, c.v_scale, bs)
    args = (st.block_tables, st.query_start_loc, st.context_lens, st.seq_lens, bs)
    o0, l0 = O.paged_attention_fp8(st.q, k8, v8, c.k_scale, c.v_scale, *args)
    blk = int(st.block_tables[1][0])
    vs2 = c.v_scale.copy()
    vs2[blk] *= 2
    o1, l1 = O.paged_attention_fp8(st.q, k8, v8, c.k_scale, vs2, *args)
    assert np.array_equal(l1, l0)
    assert np.array_equal(o1[[0, 2]], o0[[0, 2]]) and not np.allclose(o1[1], o0[1])
    ks2 = c.k_scale * np.float32(2)
    o2, l2 = O.paged_attention_fp8(st.q, k8, v8, ks2, c.v_scale, *args)
    o3, l3 = O.paged_attention_fp8(st.q, k8, v8, c.k_scale, c.v_scale, *args, scale=2 / np.sqrt(wl.head_dim))
    np.testing.assert_allclose(o2, o3, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l2, l3, rtol=1e-12, atol=1e-12)


def test_cascade_prefix_fp8_equals_bf16_cascade_on_exact_values():
    wl = W.cascade_shared_prefix(seed=2, num_queries=6, prefix=64, suffix_range=(1, 40), num_q_heads=8,
                                 num_kv_heads=2, head_dim=64)
    st, cv, bs = wl.steps[0], wl.cascade, wl.block_size
    c = W.fp8_cache(wl, seed=2)
    rng = np.random.default_rng(8)
    ks = np.exp2(rng.integers(-5, -1, (wl.num_blocks, wl.num_kv_heads))).astype(np.float32)
    vs = np.exp2(rng.integers(-5, -1, (wl.num_blocks, wl.num_kv_heads))).astype(np.float32)
    kb = W.f32_to_bf16_bits((O.e4m3_decode(c.k_cache) * ks[:, :, None, None]).astype(np.float32))
    vb = W.f32_to_bf16_bits((O.e4m3_decode(c.v_cache) * vs[:, :, None, None]).astype(np.float32))
    o8, l8 = O.cascade_prefix_attention_fp8(st.q, c.k_cache, c.v_cache, ks, vs, cv.prefix_block_table, cv.prefix_len, bs)
    ob, lb = O.cascade_prefix_attention(st.q, kb, vb, cv.prefix_block_table, cv.prefix_len, bs)
    assert np.all(np.isfinite(l8))
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb)


def test_fp8_block_size_256_is_sixteen_16_token_blocks():
    """fp8 pools of 256-token blocks: cache bytes and attention equal those of the bs=16 view of
    the same memory, with each 256-token block's scales repeated over its 16 tiles."""
    wl = W.decode_only(seed=9, num_seqs=4, ctx_range=(300, 700), block_size=256)
    st, R = wl.steps[0], 16
    c = W.fp8_cache(wl, seed=9)
    bt16 = (st.block_tables[:, :, None] * R + np.arange(R)[None, None, :]).reshape(st.num_seqs, -1).astype(np.int32)
    ks16, vs16 = np.repeat(c.k_scale, R, axis=0), np.repeat(c.v_scale, R, axis=0)
    k16 = c.k_cache.reshape(wl.num_blocks * R, wl.num_kv_heads, 16, wl.head_dim)
    v16 = c.v_cache.reshape(wl.num_blocks * R, wl.num_kv_heads, wl.head_dim, 16)
    s256 = O.slot_mapping(st.block_tables, st.query_start_loc, st.context_lens, 256)
    k8, v8 = O.reshape_and_cache_fp8(st.k, st.v, c.k_cache, c.v_cache, s256, c.k_scale, c.v_scale, 256)
    k8b, v8b = O.reshape_and_cache_fp8(st.k, st.v, k16, v16, s256, ks16, vs16, 16)
    assert np.array_equal(k8.reshape(k8b.shape), k8b) and np.array_equal(v8.reshape(v8b.shape), v8b)
    args = (st.query_start_loc, st.context_lens, st.seq_lens)
    o1, l1 = O.paged_attention_fp8(st.q, k8, v8, c.k_scale, c.v_scale, st.block_tables, *args, 256)
    o2, l2 = O.paged_attention_fp8(st.q, k8b, v8b, ks16, vs16, bt16, *args, 16)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
