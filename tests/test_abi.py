"""CPU checks of the C ABI: the library loads, exports every declared symbol, and its host-side
logic (validation, workspace sizing, the varlen work plan) behaves — no compute call is made."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")


@pytest.fixture(scope="module")
def P():
    import paged_kv_cache_285_amd as pkg
    from paged_kv_cache_285_amd import _lib

    if not os.path.exists(_lib.LIB_PATH):
        from paged_kv_cache_285_amd import build

        build.build()
    return pkg


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    from paged_kv_cache_285_amd._lib import EXPORTS

    assert declared_functions() == sorted(EXPORTS)


def test_library_exports_every_declared_symbol(P):
    h = ctypes.CDLL(P._lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(h, name), f"{name} not exported"
    assert P.version().startswith("pkv")


def shape(P, **kw):
    d = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, num_blocks=1000, bt_stride=64)
    d.update(kw)
    return P.make_shape(**d)


def test_shape_validation_errors(P):
    lib = P.lib()
    for bad in (dict(head_dim=96), dict(num_q_heads=12), dict(num_q_heads=48, num_kv_heads=4), dict(block_size=48)):
        s = shape(P, **bad)
        rc = lib.pkv_reshape_and_cache(None, None, None, None, None, 0, ctypes.byref(s), None)
        assert rc == -1, bad
        assert lib.pkv_last_error()
    s = shape(P)
    assert lib.pkv_reshape_and_cache(None, None, None, None, None, 0, ctypes.byref(s), None) == 0
    assert lib.pkv_reshape_and_cache(None, None, None, None, None, 5, ctypes.byref(s), None) == -1
    assert lib.pkv_cascade_prefix_attention(None, None, None, None, None, None, 100, 4, ctypes.byref(s), None, 0, None) == -3
    assert lib.pkv_merge_attn_states(None, 0, None, None, None, None, None, 4, 8, 6, None) == -1
    assert lib.pkv_reshape_and_cache(None, None, None, None, None, 0, None, None) == -1
    assert lib.pkv_copy_blocks(None, None, None, 0, ctypes.byref(s), None) == 0
    assert lib.pkv_copy_blocks(None, None, None, -2, ctypes.byref(s), None) == -1
    assert lib.pkv_copy_blocks(None, None, None, 3, ctypes.byref(s), None) == -1


@pytest.mark.parametrize("bs", [32, 64, 128, 256])
def test_block_sizes_accepted_and_checked(P, bs):
    lib = P.lib()
    s = shape(P, block_size=bs, num_blocks=100, bt_stride=4)
    assert lib.pkv_reshape_and_cache(None, None, None, None, None, 0, ctypes.byref(s), None) == 0
    # 4 entries of bs tokens cover 4 * bs tokens; one more does not
    ok_plan, _ = P.plan_varlen_host([0, 1], [4 * bs - 1], [4 * bs], s)
    assert ok_plan.num_items >= 1
    with pytest.raises(P.PkvError):
        P.plan_varlen_host([0, 1], [4 * bs], [4 * bs + 1], s)
    assert lib.pkv_cascade_prefix_attention(None, None, None, None, None, None, 2 * bs + 16, 4, ctypes.byref(s), None, 0, None) == -3
    huge = shape(P, block_size=bs, num_blocks=(1 << 31) // (bs // 16))
    assert lib.pkv_reshape_and_cache(None, None, None, None, None, 0, ctypes.byref(huge), None) == -1
    fits = shape(P, block_size=bs, num_blocks=((1 << 31) - 1) // (bs // 16))
    assert lib.pkv_reshape_and_cache(None, None, None, None, None, 0, ctypes.byref(fits), None) == 0


@pytest.mark.parametrize("bs", [0, 8, 24, 48, 96, 512, -16])
def test_other_block_sizes_rejected(P, bs):
    s = shape(P, block_size=bs)
    assert P.lib().pkv_reshape_and_cache(None, None, None, None, None, 0, ctypes.byref(s), None) == -1
    assert b"block_size" in P.lib().pkv_last_error()


def test_decode_entry_points_validate_before_launching(P):
    lib = P.lib()
    s = shape(P)  # bt_stride 64 x 16 keys = 1024 keys per row at most
    z = ctypes.c_void_p(0)
    assert lib.pkv_paged_attention_decode(z, 0, z, z, z, z, z, z, z, 0, 100, ctypes.byref(s), z, 0, z) == 0
    assert lib.pkv_paged_attention_decode(z, 0, z, z, z, z, z, z, z, 4, 100, ctypes.byref(s), z, 0, z) == -1
    assert lib.pkv_paged_attention_decode(z, 0, z, z, z, z, z, z, z, 4, 5000, ctypes.byref(s), z, 0, z) == -1
    assert b"bt_stride" in lib.pkv_last_error()
    assert lib.pkv_paged_attention_decode(z, 3, z, z, z, z, z, z, z, 4, 100, ctypes.byref(s), z, 0, z) == -1
    assert lib.pkv_paged_attention_decode_fp8(z, 0, z, z, z, z, z, z, z, z, z, 4, 100, ctypes.byref(s), z, 0, z) == -1
    # long rows need partial states: too small a workspace is refused before any launch
    fake = ctypes.c_void_p(256)  # never dereferenced: the size check comes first
    s600 = shape(P, bt_stride=600)
    assert lib.pkv_paged_attention_decode(fake, 0, z, fake, fake, fake, fake, fake, fake, 256, 8192,
                                          ctypes.byref(s600), fake, 16, z) == -2
    # one split needs no workspace; long rows need partial states
    assert P.decode_workspace_size(8, 256, s) == 0
    assert P.decode_workspace_size(256, 8192, shape(P, bt_stride=600)) > 0


def test_fp8_entry_points_validate_before_launching(P):
    lib = P.lib()
    s = shape(P)
    z = ctypes.c_void_p(0)
    assert lib.pkv_reshape_and_cache_fp8(z, z, z, z, z, z, z, 0, ctypes.byref(s), z) == 0
    assert lib.pkv_reshape_and_cache_fp8(z, z, z, z, z, z, z, 5, ctypes.byref(s), z) == -1
    assert lib.pkv_append_kv_fp8(z, z, z, z, z, z, z, z, z, z, 2, 3, ctypes.byref(s), z) == -1
    assert lib.pkv_copy_blocks_fp8(z, z, z, z, z, 0, ctypes.byref(s), z) == 0
    assert lib.pkv_copy_blocks_fp8(z, z, z, z, z, 2, ctypes.byref(s), z) == -1
    assert lib.pkv_cascade_prefix_attention_fp8(z, z, z, z, z, z, z, z, 100, 4, ctypes.byref(s), z, 0, z) == -3
    assert lib.pkv_paged_attention_varlen_fp8(z, 0, z, z, z, z, z, z, z, z, z, z, 1, 1, ctypes.byref(s), None, z, 0, z) == -1
    bad = shape(P, head_dim=96)
    assert lib.pkv_append_kv_fp8(z, z, z, z, z, z, z, z, z, z, 2, 3, ctypes.byref(bad), z) == -1
    assert b"head_dim" in lib.pkv_last_error()


def test_plan_rejects_inconsistent_metadata(P):
    s = shape(P)
    with pytest.raises(P.PkvError, match="seq_lens"):
        P.plan_varlen_host([0, 3], [5], [7], s)
    with pytest.raises(P.PkvError, match="query_start_loc"):
        P.plan_varlen_host([1, 3], [5], [7], s)
    with pytest.raises(P.PkvError, match="bt_stride"):
        P.plan_varlen_host([0, 1], [64 * 16], [64 * 16 + 1], s)


@pytest.mark.parametrize("lengths", [(1, 1, 1, 2, 5, 17, 100, 300), (1, 1, 2, 5, 8, 12, 16, 17)])
def test_plan_covers_every_row_exactly_once(P, lengths):
    s = shape(P, bt_stride=600)
    rng = np.random.default_rng(0)
    B = 40
    ql = rng.choice(lengths, size=B)
    ctx = rng.integers(0, 5000, size=B)
    qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    seq = (ctx + ql).astype(np.int32)
    plan, items = P.plan_varlen_host(qsl, ctx, seq, s)
    assert plan.num_items == len(items) == plan.num_prefill_items + plan.num_decode_items + plan.num_short_items
    G = 4
    tok_per_tile = plan.tile_rows // G
    cover_tok = np.zeros(int(qsl[-1]), int)
    dec_keys = {}
    cut_keys = {}
    short_keys = {}
    partial_rows = []
    for seqi, kind, qb, qc, kb, ke, pbase, split in items:
        if kind == 2:
            # a short row (2 .. 32 / G tokens) split by keys like a decode row
            assert 1 < ql[seqi] and ql[seqi] * G <= 32 and qb == 0 and qc == ql[seqi]
            cover_tok[qsl[seqi] : qsl[seqi] + qc] += split == 0
            short_keys.setdefault(seqi, []).append((kb, ke, pbase, split))
        elif kind == 1 and pbase >= 0:
            # a key split of a short row: the whole row, keys [kb, ke), partial rows pbase + t
            assert 32 < ql[seqi] * G <= 64 and qb == 0 and qc == ql[seqi] and seq[seqi] > 1024
            cover_tok[qsl[seqi] : qsl[seqi] + qc] += split == 0
            cut_keys.setdefault(seqi, []).append((kb, ke, pbase, split))
        elif kind == 1:
            assert ql[seqi] > 1 and 0 < qc <= tok_per_tile
            cover_tok[qsl[seqi] + qb : qsl[seqi] + qb + qc] += 1
            assert kb == 0 and ke == min(seq[seqi], ctx[seqi] + qb + qc)
        else:
            assert ql[seqi] == 1
            cover_tok[qsl[seqi]] += split == 0
            dec_keys.setdefault(seqi, []).append((kb, ke, pbase, split, qc))
    assert (cover_tok == 1).all()
    for r, ranges in cut_keys.items():
        ranges.sort()
        assert ranges[0][0] == 0 and ranges[-1][1] == seq[r] and len(ranges) == -(-seq[r] // 1024)
        for i, (a, b) in enumerate(zip(ranges, ranges[1:])):
            assert a[1] == b[0] == 1024 * (i + 1)
        base = ranges[0][2]
        for i, x in enumerate(ranges):
            assert x[3] == i and x[2] == base + i * ql[r]
        partial_rows += list(range(base, base + len(ranges) * ql[r]))
    for r, ranges in short_keys.items():
        ranges.sort()
        assert ranges[0][0] == 0 and ranges[-1][1] == seq[r]
        for a, b in zip(ranges, ranges[1:]):
            assert a[1] == b[0] and a[1] % 16 == 0
        if len(ranges) == 1:
            assert ranges[0][2] == -1
        else:
            base = ranges[0][2]
            for i, x in enumerate(ranges):
                assert x[3] == i and x[2] == base + i * ql[r]
            partial_rows += list(range(base, base + len(ranges) * ql[r]))
    for r, ranges in dec_keys.items():
        ranges.sort()
        assert ranges[0][0] == 0 and ranges[-1][1] == seq[r]
        for a, b in zip(ranges, ranges[1:]):
            assert a[1] == b[0] and a[1] % 16 == 0
        assert all(x[3] == i and x[4] == len(ranges) for i, x in enumerate(ranges))
        if len(ranges) == 1:
            assert ranges[0][2] == -1
        else:
            partial_rows += list(range(ranges[0][2], ranges[0][2] + len(ranges)))
    # every partial row belongs to exactly one (token, split)
    assert sorted(partial_rows) == list(range(plan.num_partials))
    # heaviest first within each kind
    pre = items[items[:, 1] == 1]
    cost = pre[:, 3].astype(np.int64) * (pre[:, 5] - pre[:, 4])
    assert (np.diff(cost) <= 0).all()
    assert (items[: plan.num_prefill_items, 1] == 1).all()
    dec = items[items[:, 1] == 0]
    assert (np.diff(dec[:, 5] - dec[:, 4]) <= 0).all()


def test_decode_waves_one_only_for_many_short_g8_items(P):
    """A decode-only plan asks for one-wave workgroups only when every item has at most 64
    blocks, q heads share a kv head eight at a time and there are at least 4096 (item, kv head)
    workgroups; otherwise four waves."""
    rng = np.random.default_rng(3)

    def plan(B, lo, hi, Hq, Hkv=8, extra_ql=()):
        ql = np.array([1] * B + list(extra_ql))
        ctx = rng.integers(lo, hi + 1, size=len(ql))
        qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
        s = shape(P, num_q_heads=Hq, num_kv_heads=Hkv, bt_stride=600, num_blocks=60000)
        p, items = P.plan_varlen_host(qsl, ctx, (ctx + ql).astype(np.int32), s)
        return p, items

    p, items = plan(512, 63, 1023, 64)  # the cascade suffix pass's shape
    assert p.decode_waves == 1
    assert ((items[:, 5] + 15) // 16 - items[:, 4] // 16).max() <= 64
    assert plan(512, 63, 1023, 32)[0].decode_waves == 4  # G = 4
    assert plan(400, 63, 1023, 64)[0].decode_waves == 4  # 3200 workgroups
    assert plan(512, 63, 2000, 64)[0].decode_waves == 4  # items over 64 blocks
    assert plan(512, 63, 1023, 64, extra_ql=(40,))[0].decode_waves == 4  # 128-row tiles beside


def test_one_wave_decode_items_always_fit_one_wave(P):
    """Over random G = 8 decode-only batches (300..1200 rows, contexts up to 100..3000 keys),
    a plan that asks for one-wave workgroups never holds a decode item over 64 blocks (one
    block id per lane), and some of them ask for it."""
    rng = np.random.default_rng(7)
    s = shape(P, num_q_heads=64, num_kv_heads=8, bt_stride=200, num_blocks=200000)
    ones = 0
    for _ in range(100):
        B = int(rng.integers(300, 1200))
        ctx = rng.integers(0, int(rng.integers(100, 3000)), size=B)
        qsl = np.arange(B + 1, dtype=np.int32)
        plan, items = P.plan_varlen_host(qsl, ctx, (ctx + 1).astype(np.int32), s)
        if plan.decode_waves == 1:
            ones += 1
            assert ((items[:, 5] + 15) // 16 - items[:, 4] // 16).max() <= 64
    assert ones > 0


def test_workspace_bound_holds_for_every_plan(P):
    rng = np.random.default_rng(1)
    for trial in range(40):
        bs = int(rng.choice([16, 32, 64, 128, 256]))
        s = shape(P, bt_stride=-(-10500 // bs), block_size=bs, num_q_heads=int(rng.choice([8, 16, 32, 64])))
        B = int(rng.integers(1, 300))
        # decode rows, short rows (ql * G <= 32), cut rows (<= 64), tiles, and empty rows
        ql = rng.choice([0, 1, 1, 1, 2, 3, 4, 8, 12, 16, 32, 64, 500], size=B)
        ctx = rng.integers(0, 10000, size=B)
        qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
        seq = (ctx + ql).astype(np.int32)
        plan, items = P.plan_varlen_host(qsl, ctx, seq, s)
        bound = P.varlen_workspace_size(B, int(qsl[-1]), int(seq.max()), s)
        assert plan.workspace_used <= bound
        # one-wave decode workgroups hold one block id per lane: every decode item <= 64 blocks
        assert plan.decode_waves in (1, 4)
        if plan.decode_waves == 1:
            dec = items[items[:, 1] == 0]
            assert ((dec[:, 5] + 15) // 16 - dec[:, 4] // 16).max() <= 64


def test_binding_rejects_buffers_smaller_than_the_shape(P):
    """The Python binding compares every buffer's size with the shape it passes and raises
    before the library is called (on CPU tensors the size check comes first, so a correctly
    sized CPU tensor fails only the device check)."""
    import torch

    s = P.make_shape(8, 2, 64, 10, 4)
    pool = 10 * 2 * 16 * 64
    T, B = 5, 2
    good = dict(
        q=torch.zeros(T * 8 * 64, dtype=torch.int16),
        k_cache=torch.zeros(pool, dtype=torch.int16),
        v_cache=torch.zeros(pool, dtype=torch.int16),
        block_tables=torch.zeros(B * 4, dtype=torch.int32),
        query_start_loc=torch.zeros(B + 1, dtype=torch.int32),
        context_lens=torch.zeros(B, dtype=torch.int32),
        seq_lens=torch.zeros(B, dtype=torch.int32),
    )
    plan = P.PkvVarlenPlan()
    ws = torch.zeros(256, dtype=torch.uint8)

    def call(**kw):
        a = dict(good)
        a.update(kw)
        return P.paged_attention_varlen(a["q"].view(T, 8, 64) if a["q"].numel() == T * 512 else a["q"],
                                        a["k_cache"], a["v_cache"], a["block_tables"], a["query_start_loc"],
                                        a["context_lens"], a["seq_lens"], s, plan, ws,
                                        out=torch.zeros(T * 8 * 64, dtype=torch.int16))

    with pytest.raises(ValueError, match="device tensor"):
        call()
    for name, n in (("k_cache", pool - 1), ("v_cache", pool // 2), ("block_tables", B * 4 - 1),
                    ("query_start_loc", B), ("seq_lens", B - 1)):
        with pytest.raises(ValueError, match=f"{name} holds"):
            call(**{name: torch.zeros(n, dtype=good[name].dtype)})
    with pytest.raises(ValueError, match="lse holds"):
        P.paged_attention_varlen(good["q"].view(T, 8, 64), good["k_cache"], good["v_cache"], good["block_tables"],
                                 good["query_start_loc"], good["context_lens"], good["seq_lens"], s, plan, ws,
                                 out=torch.zeros(T * 8 * 64, dtype=torch.int16), lse=torch.zeros(T * 8 - 1))
    with pytest.raises(ValueError, match="v holds"):
        P.reshape_and_cache(torch.zeros((T, 2, 64), dtype=torch.int16), torch.zeros((T, 2, 32), dtype=torch.int16),
                            good["k_cache"], good["v_cache"], torch.zeros(T, dtype=torch.int64), s)
    with pytest.raises(ValueError, match="k_scale holds"):
        P.reshape_and_cache_fp8(torch.zeros((T, 2, 64), dtype=torch.int16), torch.zeros((T, 2, 64), dtype=torch.int16),
                                torch.zeros(pool, dtype=torch.uint8), torch.zeros(pool, dtype=torch.uint8),
                                torch.zeros(10 * 2 - 1), torch.zeros(10 * 2), torch.zeros(T, dtype=torch.int64), s)
    with pytest.raises(ValueError, match="prefix_block_table holds"):
        P.cascade_prefix_attention(good["q"].view(T, 8, 64), good["k_cache"], good["v_cache"],
                                   torch.zeros(1, dtype=torch.int32), 32, s)
    with pytest.raises(ValueError, match="out_b holds"):
        P.merge_attn_states(torch.zeros((T, 8, 64)), torch.zeros((T, 8)), torch.zeros((T, 8, 63)),
                            torch.zeros((T, 8)))


def test_decode_noalloc_refuses_a_batch_beyond_its_scratch(P):
    """The allocation-free decode checks the batch's partial-state bytes against its device
    scratch before touching the device."""
    lib = P.lib()
    s = shape(P, num_blocks=1 << 20, bt_stride=4096)
    assert P.decode_workspace_size(4096, 65536, s) > P.PKV_DECODE_SCRATCH_BYTES
    rc = lib.pkv_paged_attention_decode_noalloc(ctypes.c_void_p(16), 0, None, ctypes.c_void_p(16), ctypes.c_void_p(16),
                                                ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16),
                                                ctypes.c_void_p(16), 4096, 65536, ctypes.byref(s), None)
    assert rc == -2
    assert "scratch" in lib.pkv_last_error().decode()
