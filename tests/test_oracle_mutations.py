"""The oracle pins catch plausible mistakes.

Each case below plants one mistake in a step of the CPU oracle: an off-by-one causal mask, a
wrong scale, the wrong kv head, shifted positions, a transposed value operand, a missing
softmax normalisation, an LSE in the wrong base, a merge with its weights swapped, and a cache
write at the wrong offset, a block copy that forgets the values, a 256-token block read with
its kv heads outside its tiles; and in the FP8 half, a wrong
exponent bias, ties rounded away from zero, no saturation, a multiplied instead of divided
scale, one kv head's scale for all, the wrong block's scale, an ignored key scale.  For each,
the pins of test_oracle_pins.py and test_oracle_fp8_pins.py run against the mutated oracle,
and at least one must fail.  The mutations live here, on the CPU, and are undone after each
case.
"""

import inspect
import json
import math
import sys

import numpy as np
import pytest

import oracle  # noqa: F401  (the package; its functions are what the pins call)
import test_oracle_fp8_pins as fp8_pins
import test_oracle_pins as pins

OM = sys.modules["oracle.paged_attention"]  # the modules whose globals the oracle's calls resolve
F8 = sys.modules["oracle.kv_fp8"]


def _pin_calls():
    """Every pin as a zero-argument callable (fixtures and parameters filled in)."""
    with open(pins.GOLDEN) as f:
        page = json.load(f)
    calls = []
    items = [(n, f) for mod in (pins, fp8_pins) for n, f in sorted(vars(mod).items(), key=lambda x: x[0])]
    for name, fn in items:
        if not name.startswith("test_") or not callable(fn):
            continue
        params = list(inspect.signature(fn).parameters)
        marks = getattr(fn, "pytestmark", [])
        grids = [m for m in marks if m.name == "parametrize"]
        if grids:
            names = [s.strip() for s in grids[0].args[0].split(",")]
            for values in grids[0].args[1]:
                kw = dict(zip(names, values if len(names) > 1 else [values]))
                calls.append((f"{name}{values}", lambda fn=fn, kw=kw: fn(**kw)))
        elif params == ["page"]:
            calls.append((name, lambda fn=fn: fn(page)))
        elif not params:
            calls.append((name, fn))
    return calls


def _patch(attr, fn):
    """Replace `attr` in the oracle module that defines it and in the package namespace."""
    mod = F8 if hasattr(F8, attr) and getattr(F8, attr).__module__ == F8.__name__ else OM
    saved = [(mod, attr, getattr(mod, attr))]
    if hasattr(oracle, attr) and callable(getattr(oracle, attr)):
        saved.append((oracle, attr, getattr(oracle, attr)))
        setattr(oracle, attr, fn)
    setattr(mod, attr, fn)
    return saved


def _restore(saved):
    for mod, attr, fn in saved:
        setattr(mod, attr, fn)


ORIG = {name: getattr(OM, name) for name in (
    "causal_visible", "default_scale", "gather_keys", "gather_values", "token_positions",
    "attention_state", "merge_attn_states", "reshape_and_cache", "copy_blocks", "tiles")}
ORIG8 = {name: getattr(F8, name) for name in (
    "e4m3_decode", "e4m3_encode", "quantize", "reshape_and_cache_fp8", "dequantize_keys",
    "dequantize_values")}


def causal_strict(context_len, query_len, num_keys):
    p = ORIG["token_positions"](context_len, query_len)
    return np.arange(num_keys)[None, :] < p[:, None]  # a row no longer sees its own key


def scale_one_over_d(head_dim):
    return 1.0 / head_dim


def keys_of_next_head(k_cache, row, num_keys, kv_head, block_size):
    return ORIG["gather_keys"](k_cache, row, num_keys, (kv_head + 1) % k_cache.shape[1], block_size)


def values_token_major(v_cache, row, num_keys, kv_head, block_size):
    j = np.arange(num_keys)
    phys = np.asarray(row, dtype=np.int64)[j // block_size]
    x = OM.bf16_to_f64(v_cache[phys, kv_head, j % block_size, :])  # reads a dim-major pool as token-major
    return x.reshape(num_keys, -1)[:, : v_cache.shape[2]]


def positions_shifted(context_len, query_len):
    return np.arange(context_len + 1, context_len + query_len + 1, dtype=np.int64)


def state_unnormalised(scores, values):
    o, lse = ORIG["attention_state"](scores, values)
    z = np.exp(np.where(np.isfinite(lse), lse - np.max(np.where(np.isfinite(scores), scores, -np.inf), axis=1,
                                                        initial=-np.inf), 0.0))
    return o * z[:, None], lse


def state_lse_base2(scores, values):
    o, lse = ORIG["attention_state"](scores, values)
    m = np.max(scores, axis=1, initial=-np.inf) if scores.shape[1] else lse
    return o, np.where(np.isfinite(lse), m + (lse - m) / math.log(2.0), lse)


def merge_swapped(o_a, lse_a, o_b, lse_b):
    o, lse = ORIG["merge_attn_states"](o_a, lse_a, o_b, lse_b)
    o2, _ = ORIG["merge_attn_states"](o_a, lse_b, o_b, lse_a)  # weights of a and b exchanged
    return o2, lse


def cache_write_next_offset(k, v, k_cache, v_cache, slots, block_size):
    s = np.asarray(slots, dtype=np.int64)
    shifted = np.where(s < 0, s, (s // block_size) * block_size + (s % block_size + 1) % block_size)
    return ORIG["reshape_and_cache"](k, v, k_cache, v_cache, shifted, block_size)


def copy_keys_only(k_cache, v_cache, block_pairs):
    kc, _ = ORIG["copy_blocks"](k_cache, v_cache, block_pairs)
    return kc, np.array(v_cache, copy=True)


def tiles_heads_outer(pool):
    """Reads a block of several tiles as [Hkv, tiles] instead of [tiles, Hkv]."""
    if pool.ndim == 4:
        return ORIG["tiles"](pool)
    nb, r, h = pool.shape[:3]
    return pool.reshape(nb, h, r, *pool.shape[3:]).transpose(0, 2, 1, 3, 4)


def decode_bias_8(codes):
    return ORIG8["e4m3_decode"](codes) * 0.5


def encode_ties_away(x):
    xs = np.asarray(x, dtype=np.float32)
    up = np.nextafter(np.abs(xs), np.float32(np.inf)) * np.sign(xs)  # nudges a tie outwards
    return ORIG8["e4m3_encode"](np.where(np.isfinite(xs), up, xs).astype(np.float32))


def encode_no_saturation(x):
    xs = np.asarray(x, dtype=np.float32)
    c = ORIG8["e4m3_encode"](xs)
    return np.where(np.abs(xs) > 448, np.uint8(0x7F), c).astype(np.uint8)


def quantize_times_scale(x_bf16, scale):
    return ORIG8["quantize"](x_bf16, 1.0 / float(scale))


def cache_fp8_head0_scale(k, v, k_cache, v_cache, slots, k_scale, v_scale, block_size):
    ks = np.repeat(np.asarray(k_scale)[:, :1], np.asarray(k_scale).shape[1], axis=1)
    return ORIG8["reshape_and_cache_fp8"](k, v, k_cache, v_cache, slots, ks, v_scale, block_size)


def values_scale_of_block0(v_cache, v_scale, row, num_keys, kv_head, block_size):
    vs = np.broadcast_to(np.asarray(v_scale)[:1], np.asarray(v_scale).shape)
    return ORIG8["dequantize_values"](v_cache, vs, row, num_keys, kv_head, block_size)


def keys_unscaled(k_cache, k_scale, row, num_keys, kv_head, block_size):
    return ORIG8["dequantize_keys"](k_cache, np.ones_like(np.asarray(k_scale)), row, num_keys, kv_head, block_size)


MUTATIONS = [
    ("causal_visible", causal_strict),
    ("default_scale", scale_one_over_d),
    ("gather_keys", keys_of_next_head),
    ("gather_values", values_token_major),
    ("token_positions", positions_shifted),
    ("attention_state", state_unnormalised),
    ("attention_state", state_lse_base2),
    ("merge_attn_states", merge_swapped),
    ("reshape_and_cache", cache_write_next_offset),
    ("copy_blocks", copy_keys_only),
    ("tiles", tiles_heads_outer),
    ("e4m3_decode", decode_bias_8),
    ("e4m3_encode", encode_ties_away),
    ("e4m3_encode", encode_no_saturation),
    ("quantize", quantize_times_scale),
    ("reshape_and_cache_fp8", cache_fp8_head0_scale),
    ("dequantize_values", values_scale_of_block0),
    ("dequantize_keys", keys_unscaled),
]


@pytest.mark.parametrize("attr,mutant", MUTATIONS, ids=[m[1].__name__ for m in MUTATIONS])
def test_pins_catch_planted_mistake(attr, mutant):
    saved = _patch(attr, mutant)
    failed = []
    try:
        with np.errstate(all="ignore"):
            for name, call in _pin_calls():
                try:
                    call()
                except Exception:  # an assertion or any error the mistake provokes
                    failed.append(name)
    finally:
        _restore(saved)
    assert failed, f"no pin fails when {attr} is replaced by {mutant.__name__}"


def test_pins_pass_on_the_unmutated_oracle():
    for name, call in _pin_calls():
        call()
