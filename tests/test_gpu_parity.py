"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle, on seeded workloads.

Cache writes and slot mappings must match bit for bit; attention outputs must hold max abs
error <= 1e-2 (bf16 output rounding excepted, and reported) and relative L2 <= 5e-3.
"""

import sys

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU, skipped
    pytest.skip("no GPU", allow_module_level=True)

import paged_kv_cache_285_amd as P  # noqa: E402
from _gpu import (  # noqa: E402
    DeviceWorkload,
    many_requests,
    bf16_out_to_f64,
    check_attention,
    check_lse,
    lse_rows_from_rounded_weights,
    dev16,
    dev32,
    host16,
)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_and_check(wl, rows_per_step=None, check_pools=True, want_lse=True, out_dtype=torch.bfloat16, seed=0,
                  expect_tile_rows=None, scale=None, check_steps=None):
    """Run every step of ``wl`` on the GPU and compare with the oracle (optionally on sampled rows);
    ``check_steps``: compare only those steps (every step by default); ``scale``: a softmax scale
    other than 1/sqrt(head_dim), for both."""
    bs = wl.block_size
    dw = DeviceWorkload(wl, scale=scale or 0.0)
    kp, vp = wl.k_cache, wl.v_cache
    rng = np.random.default_rng(seed)
    stats = []
    for si, st in enumerate(wl.steps):
        say(f"  step {si}: B={st.num_seqs} T={st.num_tokens}")
        slots_g, out_g, lse_g, plan = dw.run_step(st, out_dtype=out_dtype, want_lse=want_lse)
        torch.cuda.synchronize()
        if expect_tile_rows is not None:
            assert plan.tile_rows == expect_tile_rows, plan.tile_rows
        slots_o = O.slot_mapping(st.block_tables, st.query_start_loc, st.context_lens, bs)
        assert np.array_equal(slots_g.cpu().numpy(), slots_o), "slot mapping differs"
        kp, vp = O.reshape_and_cache(st.k, st.v, kp, vp, slots_o, bs)
        if check_pools:
            assert np.array_equal(host16(dw.k_cache), kp), "k_cache bits differ"
            assert np.array_equal(host16(dw.v_cache), vp), "v_cache bits differ"
        else:
            touched = np.unique(slots_o // bs)
            assert np.array_equal(host16(dw.k_cache[touched]), kp[touched]), "k_cache bits differ"
            assert np.array_equal(host16(dw.v_cache[touched]), vp[touched]), "v_cache bits differ"
        rows = None
        if check_steps is not None and si not in check_steps:
            continue
        if rows_per_step is not None and st.num_tokens > rows_per_step:
            rows = np.sort(rng.choice(st.num_tokens, size=rows_per_step, replace=False))
            # always include the first and last token of every prefill row and the longest decode row
            extra = list(st.query_start_loc[:-1]) + list(st.query_start_loc[1:] - 1)
            extra.append(int(st.query_start_loc[int(np.argmax(st.seq_lens))]))
            rows = np.unique(np.concatenate([rows, np.array(extra)]))
        o_ref, l_ref = O.paged_attention(
            st.q, kp, vp, st.block_tables, st.query_start_loc, st.context_lens, st.seq_lens, bs, rows=rows,
            scale=scale,
        )
        o_gpu = bf16_out_to_f64(out_g)
        sel = slice(None) if rows is None else rows
        r = check_attention(o_gpu[sel], o_ref[sel], f"{wl.name} step {si}", bf16_out=out_dtype != torch.float32)
        if want_lse:
            loose = lse_rows_from_rounded_weights(st, wl.num_q_heads // wl.num_kv_heads, plan.tile_rows)
            r["lse_max_abs"] = check_lse(lse_g.cpu().numpy()[sel], l_ref[sel], f"{wl.name} step {si} lse",
                                         rounded=loose[sel])
        stats.append(r)
        say(f"    plan items={plan.num_items} tile_rows={plan.tile_rows} partials={plan.num_partials} bps={plan.blocks_per_split} {r}")
    return stats


def test_tiny_prefill_parity():
    say("tiny_prefill seed 0..2")
    for seed in range(3):
        run_and_check(W.tiny_prefill(seed=seed))


def test_mixed_batch_small_parity():
    say("mixed_llama8b small")
    run_and_check(W.mixed_llama8b(seed=1, num_decode=12, ctx_range=(17, 700)))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_mixed_batch_full_parity(seed):
    say(f"mixed_llama8b full (64 decode rows, ctx 128..4096), seed {seed}")
    run_and_check(W.mixed_llama8b(seed=seed))


def test_decode_small_parity_fp32_out():
    say("decode_only small, fp32 out")
    run_and_check(W.decode_only(seed=2, num_seqs=24, ctx_range=(1, 3000)), out_dtype=torch.float32)


def test_decode_group8_parity():
    say("decode_only G=8 small")
    run_and_check(W.decode_only(seed=3, num_seqs=20, ctx_range=(1, 2500), num_q_heads=64))


def test_long_chunked_prefill_small_parity():
    say("long_chunked_prefill small: 1024-token prompt in 4 chunks of 256, 6 decode rows")
    run_and_check(W.long_chunked_prefill(seed=1, prompt=1024, chunk=256, num_decode=6, decode_ctx=333))


def test_long_chunked_prefill_8wave_tiles_parity():
    """512-token chunks x 4 q heads per kv head = 2048 packed rows: the plan picks 256-row tiles."""
    say("long_chunked_prefill small with 8-wave tiles: 1536-token prompt in 3 chunks of 512")
    stats = run_and_check(W.long_chunked_prefill(seed=2, prompt=1536, chunk=512, num_decode=5, decode_ctx=700))
    assert stats


def test_spec_verify_small_parity():
    """Query length 1 + 4 drafted tokens over cached contexts: small causal-offset MFMA tiles."""
    say("spec_verify small: 12 rows of 5 tokens, ctx U[1, 700]")
    run_and_check(W.spec_verify(seed=1, num_seqs=12, ctx_range=(1, 700)))
    say("spec_verify: 6 rows of 5 tokens and 4 of 8, ctx U[1100, 3000]")
    run_and_check(W.spec_verify(seed=2, num_seqs=6, ctx_range=(1100, 3000)))
    run_and_check(W.spec_verify(seed=3, num_seqs=4, draft=7, ctx_range=(1100, 3000)))


def test_short_rows_split_at_key_boundaries():
    """Rows split by keys with a split starting before, at and after the first query token's
    position, so that some tokens see no key of a split (an empty state the reduce must weigh by
    zero): rows of 12 tokens (48 packed rows at G 4) over contexts around 1024 and 2048 are cut
    tiles with 1024-key splits; rows of 2, 5 and 16 tokens over long contexts are split too
    (short items: equal pieces)."""
    say("rows split by keys around the query tokens' positions")
    ctxs = [1019, 1020, 1023, 1024, 1025, 2043, 2047, 2048]
    reqs = [W.RequestSpec(c, [12]) for c in ctxs] + [W.RequestSpec(c, [5]) for c in (3071, 1100, 2500)]
    reqs += [W.RequestSpec(1500, [16]), W.RequestSpec(1030, [2])]
    wl = W.build("split_edges", reqs, num_q_heads=32, num_kv_heads=8, head_dim=128, seed=13)
    st = wl.steps[0]
    shape = P.make_shape(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_blocks, wl.bt_stride)
    _, items = P.plan_varlen_host(st.query_start_loc, st.context_lens, st.seq_lens, shape)
    cut = items[(items[:, 1] == 1) & (items[:, 6] >= 0)]
    # every row around 1024 / 2048 has a split starting inside its query tokens' positions
    for r, c in enumerate(ctxs):
        starts = cut[cut[:, 0] == r, 4]
        assert any(c - 5 <= b <= c + 11 for b in starts if b > 0), (c, starts)
    assert (items[:, 1] == 2).sum() > 3  # short rows split as well
    run_and_check(wl)


@pytest.mark.parametrize("head_dim,group", [(64, 1), (128, 2), (128, 8), (64, 4)])
def test_short_rows_every_shape(head_dim, group):
    """Rows of 2 .. 32 / G query tokens (short items: MFMA columns = packed (token, q head) rows)
    with contexts from empty to a few thousand keys, split or not, for several shapes."""
    say(f"short rows, D={head_dim} G={group}")
    rng = np.random.default_rng(head_dim + group)
    qmax = 32 // group
    reqs = [W.RequestSpec(int(c), [int(q)]) for c, q in zip(rng.integers(0, 3000, 10), rng.integers(2, qmax + 1, 10))]
    reqs += [W.RequestSpec(0, [qmax]), W.RequestSpec(17, [2]), W.RequestSpec(1, [1])]
    wl = W.build("short_rows", reqs, num_q_heads=8 * group, num_kv_heads=8, head_dim=head_dim, seed=head_dim * group)
    run_and_check(wl)


@pytest.mark.parametrize("case", ["mixed", "wide"])
def test_fp32_output_from_every_item_kind(case):
    """fp32 output (and LSE) from decode rows, short rows, 128-row tiles and, for "wide",
    256-row pipelined tiles: every kernel's fp32 store path against the oracle."""
    say(f"fp32 output: {case}")
    if case == "mixed":
        reqs = [W.RequestSpec(c, [1]) for c in (2500, 900, 30)]
        reqs += [W.RequestSpec(1500, [4]), W.RequestSpec(200, [150]), W.RequestSpec(0, [40])]
        wl = W.build("fp32_mixed", reqs, num_q_heads=16, num_kv_heads=4, head_dim=128, seed=41)
        run_and_check(wl, out_dtype=torch.float32)
    else:
        reqs = [W.RequestSpec(100, [1024 + 19]), W.RequestSpec(700, [1])]
        wl = W.build("fp32_wide", reqs, num_q_heads=4, num_kv_heads=2, head_dim=64, seed=42)
        run_and_check(wl, out_dtype=torch.float32, expect_tile_rows=256)


def test_lengths_at_block_tile_and_split_edges():
    """Contexts and chunk ends on either side of a 16-key block, a 64-key MFMA tile and a
    1024-key split: decode rows, short rows and tile rows in one batch."""
    say("lengths at block, tile and split edges")
    dec = [(0, 1), (15, 1), (16, 1), (63, 1), (64, 1), (1023, 1), (1024, 1), (1025, 1)]
    short = [(15, 2), (16, 3), (63, 5), (64, 8), (1023, 2), (1024, 7)]
    tiles = [(0, 16), (15, 17), (48, 16), (63, 65), (64, 64), (1023, 33), (1024, 64), (0, 129)]
    reqs = [W.RequestSpec(c, [q]) for c, q in dec + short + tiles]
    wl = W.build("edges", reqs, num_q_heads=8, num_kv_heads=2, head_dim=128, seed=43)
    run_and_check(wl)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_one_wave_decode_items(out_dtype):
    """Many short G = 8 decode rows (520 rows of 1..1000 keys, 64 q / 8 kv heads): the plan runs
    them as one-wave workgroups; every row against the oracle."""
    say(f"one-wave decode items ({out_dtype})")
    wl = W.decode_only(seed=45, num_seqs=520, ctx_range=(1, 1000), num_q_heads=64)
    st = wl.steps[0]
    shape = P.make_shape(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_blocks, wl.bt_stride,
                         block_size=wl.block_size)
    plan, _ = P.plan_varlen_host(st.query_start_loc, st.context_lens, st.seq_lens, shape)
    assert plan.decode_waves == 1
    run_and_check(wl, out_dtype=out_dtype)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_split_counts_around_the_reduce_batch(out_dtype):
    """Decode rows cut into 7, 8, 9, 10 and 17 key splits beside unsplit rows: the split-KV
    reduce loads up to 8 splits' states in one round and takes more in a loop; both against
    the oracle."""
    say(f"split counts 7..17 around the reduce's batch of 8 ({out_dtype})")
    reqs = [W.RequestSpec(c, [1]) for c in (1791, 2047, 2048, 2303, 2559, 4351, 100, 0)]
    wl = W.build("reduce_batch_edges", reqs, num_q_heads=32, num_kv_heads=8, head_dim=128, seed=44)
    st = wl.steps[0]
    shape = P.make_shape(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_blocks, wl.bt_stride,
                         block_size=wl.block_size)
    _, items = P.plan_varlen_host(st.query_start_loc, st.context_lens, st.seq_lens, shape)
    splits = np.bincount(items[:, 0], minlength=len(reqs))
    assert {7, 8, 9, 10, 17} <= set(splits.tolist()) and 1 in splits, splits
    run_and_check(wl, out_dtype=out_dtype)


def test_spec_verify_full_size_every_row():
    say("spec_verify full: 64 rows of 5 tokens, ctx U[1024, 4096], every row")
    run_and_check(W.spec_verify(seed=0), check_pools=False)


def test_graph_capture_replays_match_eager():
    """The step's cache write and attention (decode splits with their reduce, and prefill tiles)
    captured in a HIP graph: every replay, with eager work and synchronisation in between,
    gives the eager result bit for bit.  The plan is uploaded before capture."""
    say("graph capture: mixed batch step 0")
    wl = W.mixed_llama8b(seed=6, num_decode=24, ctx_range=(100, 3000))
    st = wl.steps[0]
    dw = DeviceWorkload(wl)
    t = dw.step_tensors(st)
    plan = P.plan_varlen(dw.ws, st.query_start_loc, st.context_lens, st.seq_lens, dw.shape)
    assert plan.num_partials > 0 and plan.num_prefill_items > 0
    out = torch.empty(st.q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(st.q.shape[:2], dtype=torch.float32, device="cuda")

    def step():
        P.append_kv(t["k"], t["v"], dw.k_cache, dw.v_cache, t["bt"], t["qsl"], t["ctx"], dw.shape)
        P.paged_attention_varlen(t["q"], dw.k_cache, dw.v_cache, t["bt"], t["qsl"], t["ctx"], t["seq"], dw.shape,
                                 plan, dw.ws, out=out, lse=lse)

    step()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        step()  # warm the side stream before capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.synchronize()
    scratch = torch.zeros(1 << 20, device="cuda")
    for rep in range(3):
        out.zero_()
        lse.zero_()
        scratch.add_(1.0)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), f"replay {rep}: output differs"
        assert torch.equal(lse, ref_l), f"replay {rep}: lse differs"


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_decode_device_split_matches_oracle(out_dtype):
    """Decode with the work split on the device (no host plan): against the oracle, and a row of
    length 0 gives output 0 and lse -inf."""
    say(f"decode with device-side split, out {out_dtype}")
    wl = W.decode_only(seed=41, num_seqs=20, ctx_range=(1, 5000))
    st = wl.steps[0]
    dw = DeviceWorkload(wl)
    t = dw.step_tensors(st)
    P.append_kv(t["k"], t["v"], dw.k_cache, dw.v_cache, t["bt"], t["qsl"], t["ctx"], dw.shape)
    max_seq = wl.bt_stride * wl.block_size  # the longest row the block tables can hold
    ws = P.alloc_workspace(P.decode_workspace_size(st.num_seqs, max_seq, dw.shape))
    lse = torch.empty(st.q.shape[:2], dtype=torch.float32, device="cuda")
    out = P.paged_attention_decode(t["q"], dw.k_cache, dw.v_cache, t["bt"], t["qsl"], t["seq"], dw.shape, max_seq,
                                   workspace=ws, out_dtype=out_dtype, lse=lse)
    torch.cuda.synchronize()
    slots = O.slot_mapping(st.block_tables, st.query_start_loc, st.context_lens, wl.block_size)
    kp, vp = O.reshape_and_cache(st.k, st.v, wl.k_cache, wl.v_cache, slots, wl.block_size)
    ref, lref = O.paged_attention(st.q, kp, vp, st.block_tables, st.query_start_loc, st.context_lens, st.seq_lens,
                                  wl.block_size)
    r = check_attention(bf16_out_to_f64(out), ref, "device-split decode", bf16_out=out_dtype != torch.float32)
    check_lse(lse.cpu().numpy(), lref, "device-split decode lse")
    say(f"    {r}")
    seq0 = t["seq"].clone()
    seq0[3] = 0
    out0 = P.paged_attention_decode(t["q"], dw.k_cache, dw.v_cache, t["bt"], t["qsl"], seq0, dw.shape, max_seq,
                                    workspace=ws, out_dtype=out_dtype, lse=lse)
    torch.cuda.synchronize()
    assert not bf16_out_to_f64(out0)[3].any() and bool(torch.isneginf(lse[3]).all())


@pytest.mark.parametrize("head_dim,group", [(64, 1), (64, 2), (128, 8)])
def test_decode_device_split_every_shape(head_dim, group):
    """The device-split decode at the head sizes and groupings the varlen tests cover apart from
    D 128 / G 4: 12 rows of 1..3000 keys against the oracle."""
    say(f"device-split decode D={head_dim} G={group}")
    reqs = [W.RequestSpec(int(c), [1]) for c in np.random.default_rng(47).integers(0, 3000, size=12)]
    wl = W.build("dsplit_shapes", reqs, num_q_heads=2 * group, num_kv_heads=2, head_dim=head_dim, seed=47)
    st = wl.steps[0]
    dw = DeviceWorkload(wl)
    t = dw.step_tensors(st)
    P.append_kv(t["k"], t["v"], dw.k_cache, dw.v_cache, t["bt"], t["qsl"], t["ctx"], dw.shape)
    max_seq = wl.bt_stride * wl.block_size
    ws = P.alloc_workspace(P.decode_workspace_size(st.num_seqs, max_seq, dw.shape))
    lse = torch.empty(st.q.shape[:2], dtype=torch.float32, device="cuda")
    out = P.paged_attention_decode(t["q"], dw.k_cache, dw.v_cache, t["bt"], t["qsl"], t["seq"], dw.shape, max_seq,
                                   workspace=ws, lse=lse)
    torch.cuda.synchronize()
    slots = O.slot_mapping(st.block_tables, st.query_start_loc, st.context_lens, wl.block_size)
    kp, vp = O.reshape_and_cache(st.k, st.v, wl.k_cache, wl.v_cache, slots, wl.block_size)
    ref, lref = O.paged_attention(st.q, kp, vp, st.block_tables, st.query_start_loc, st.context_lens, st.seq_lens,
                                  wl.block_size)
    r = check_attention(bf16_out_to_f64(out), ref, f"device-split decode D={head_dim} G={group}")
    check_lse(lse.cpu().numpy(), lref, "device-split decode lse")
    say(f"    {r}")


def test_decode_step_graph_replays_with_new_metadata():
    """A decode step (fused cache write + device-split decode) for a padded bucket of 8 rows is
    captured once in a HIP graph, then replayed for three different batches written into the
    same buffers (5 real rows, 3 padding rows of length 0 whose cache writes go to a spare
    block), with eager work between replays: every replay matches the eager call bit for bit
    and the oracle to tolerance."""
    say("graph capture of a bucketed decode step, replayed with new metadata")
    B, real, NB, WST, max_seq = 8, 5, 1200, 200, 3200
    wls = []
    for i in range(3):
        rng = np.random.default_rng(100 + i)
        ctxs = rng.integers(10, 3000, size=real)
        reqs = [W.RequestSpec(int(c), [1]) for c in ctxs]
        wls.append(W.build("bucket", reqs, num_q_heads=32, num_kv_heads=8, head_dim=128, seed=100 + i,
                           num_blocks=NB, bt_stride=WST))
    shape = P.make_shape(32, 8, 128, NB, WST)

    def padded(wl):
        st = wl.steps[0]
        used = {int(b) for r in range(real) for b in st.block_tables[r, : (int(st.seq_lens[r]) + 15) // 16]}
        spare = max(set(range(NB)) - used)  # padding rows write here; no real row reads it
        bt = np.full((B, WST), spare, np.int32)
        bt[:real] = st.block_tables
        qsl = np.arange(B + 1, dtype=np.int32)
        ctx = np.zeros(B, np.int32)
        ctx[:real] = st.context_lens
        seq = np.zeros(B, np.int32)
        seq[:real] = st.seq_lens
        pad = lambda x: np.concatenate([x, np.zeros((B - real,) + x.shape[1:], x.dtype)])  # noqa: E731
        return dict(q=pad(st.q), k=pad(st.k), v=pad(st.v), bt=bt, qsl=qsl, ctx=ctx, seq=seq)

    m0 = padded(wls[0])
    buf = {k: (dev16(v) if v.dtype == np.uint16 else dev32(v)) for k, v in m0.items()}
    kc, vc = dev16(wls[0].k_cache), dev16(wls[0].v_cache)
    ws = P.alloc_workspace(P.decode_workspace_size(B, max_seq, shape))
    out = torch.empty((B, 32, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, 32), dtype=torch.float32, device="cuda")

    def step():
        P.append_kv(buf["k"], buf["v"], kc, vc, buf["bt"], buf["qsl"], buf["ctx"], shape)
        P.paged_attention_decode(buf["q"], kc, vc, buf["bt"], buf["qsl"], buf["seq"], shape, max_seq, workspace=ws,
                                 out=out, lse=lse)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.synchronize()
    scratch = torch.zeros(1 << 20, device="cuda")
    for i, wl in enumerate(wls):
        m = padded(wl)
        for k, v in m.items():
            buf[k].copy_(torch.from_numpy(v.view(np.int16) if v.dtype == np.uint16 else v))
        kc.copy_(torch.from_numpy(wl.k_cache.view(np.int16)))
        vc.copy_(torch.from_numpy(wl.v_cache.view(np.int16)))
        out.zero_()
        lse.zero_()
        scratch.add_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_g, l_g = out.clone(), lse.clone()
        # eager on the same inputs (the cache write is idempotent)
        step()
        torch.cuda.synchronize()
        assert torch.equal(o_g.view(torch.int16), out.view(torch.int16)), f"replay {i}: differs from eager"
        assert torch.equal(l_g, lse), f"replay {i}: lse differs from eager"
        st = wl.steps[0]
        slots = O.slot_mapping(st.block_tables, st.query_start_loc, st.context_lens, wl.block_size)
        kp, vp = O.reshape_and_cache(st.k, st.v, wl.k_cache, wl.v_cache, slots, wl.block_size)
        ref, lref = O.paged_attention(st.q, kp, vp, st.block_tables, st.query_start_loc, st.context_lens,
                                      st.seq_lens, wl.block_size)
        check_attention(bf16_out_to_f64(o_g)[:real], ref, f"graph replay {i}")
        check_lse(l_g.cpu().numpy()[:real], lref, f"graph replay {i} lse")
        assert not bf16_out_to_f64(o_g)[real:].any() and bool(torch.isneginf(l_g[real:]).all())


WIDE_SHAPES = [(64, 1), (64, 2), (64, 4), (64, 8), (128, 1), (128, 2), (128, 4), (128, 8)]


@pytest.mark.parametrize("head_dim,group", WIDE_SHAPES)
def test_wide_tiles_every_shape(head_dim, group):
    """A batch with >= 2048 packed prefill rows (256-row tiles, launched apart from its decode
    rows) at every supported (head_dim, q heads per kv head): a ragged chunk over a cached
    context, a short prompt and three decode rows."""
    say(f"wide tiles D={head_dim} G={group}")
    reqs = [W.RequestSpec(300, [2048 // group + 37]), W.RequestSpec(0, [100])]
    reqs += [W.RequestSpec(c, [1]) for c in (1, 700, 1500)]
    wl = W.build("wide", reqs, num_q_heads=2 * group, num_kv_heads=2, head_dim=head_dim, seed=11)
    run_and_check(wl, expect_tile_rows=256)


@pytest.mark.parametrize("head_dim,group", [(64, 1), (64, 8), (128, 1), (128, 2)])
def test_cascade_every_shape(head_dim, group):
    say(f"cascade D={head_dim} G={group}")
    wl = W.cascade_shared_prefix(seed=5, num_queries=70, prefix=1040, suffix_range=(1, 200),
                                 num_q_heads=2 * group, num_kv_heads=2, head_dim=head_dim)
    _cascade_check(wl)


def test_single_key_rows_are_exact():
    """One visible key: p = 1 exactly, so the output is that key's value, bit for bit."""
    say("single-key rows")
    wl = W.decode_only(seed=4, num_seqs=9, ctx_range=(0, 0))
    dw = DeviceWorkload(wl)
    st = wl.steps[0]
    _, out, lse, _ = dw.run_step(st, want_lse=True)
    torch.cuda.synchronize()
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), np.repeat(st.v, wl.group, axis=1))


def test_append_kv_matches_oracle_bitwise():
    """Slot mapping and cache write fused in one launch: slots and pool bits equal the oracle's."""
    say("append_kv (fused slot mapping + cache write)")
    wl = W.mixed_llama8b(seed=4, num_decode=9, ctx_range=(5, 300))
    dw = DeviceWorkload(wl)
    kp, vp = wl.k_cache, wl.v_cache
    for st in wl.steps:
        t = dw.step_tensors(st)
        slots = torch.empty(st.num_tokens, dtype=torch.int64, device="cuda")
        P.append_kv(t["k"], t["v"], dw.k_cache, dw.v_cache, t["bt"], t["qsl"], t["ctx"], dw.shape, slot_mapping=slots)
        torch.cuda.synchronize()
        ref = O.slot_mapping(st.block_tables, st.query_start_loc, st.context_lens, wl.block_size)
        assert np.array_equal(slots.cpu().numpy(), ref)
        kp, vp = O.reshape_and_cache(st.k, st.v, kp, vp, ref, wl.block_size)
        assert np.array_equal(host16(dw.k_cache), kp) and np.array_equal(host16(dw.v_cache), vp)


def test_copy_blocks_matches_oracle_bitwise():
    say("copy_blocks: 40 pairs over the mixed batch pools, plus skipped pairs")
    wl = W.mixed_llama8b(seed=7, num_decode=8)
    dw = DeviceWorkload(wl)
    rng = np.random.default_rng(7)
    perm = rng.permutation(wl.num_blocks)
    pairs = np.stack([perm[:40], perm[40:80]], axis=1).astype(np.int32)  # no block in two pairs
    pairs = np.concatenate([pairs, [[-1, 3], [5, wl.num_blocks], [9, 9]]]).astype(np.int32)
    P.copy_blocks(dw.k_cache, dw.v_cache, dev32(pairs), dw.shape)
    torch.cuda.synchronize()
    kc, vc = O.copy_blocks(wl.k_cache, wl.v_cache, pairs)
    assert np.array_equal(host16(dw.k_cache), kc), "k_cache bits differ"
    assert np.array_equal(host16(dw.v_cache), vc), "v_cache bits differ"


def test_plan_reuse_is_bit_identical():
    """The same plan run three times over split-KV rows gives identical bits and matches the oracle."""
    say("plan reuse with split-KV rows")
    wl = W.decode_only(seed=8, num_seqs=12, ctx_range=(3000, 9000))
    st = wl.steps[0]
    dw = DeviceWorkload(wl)
    t = dw.step_tensors(st)
    P.append_kv(t["k"], t["v"], dw.k_cache, dw.v_cache, t["bt"], t["qsl"], t["ctx"], dw.shape)
    plan = P.plan_varlen(dw.ws, st.query_start_loc, st.context_lens, st.seq_lens, dw.shape)
    assert plan.num_partials > 0
    outs = []
    for _ in range(3):
        outs.append(
            P.paged_attention_varlen(
                t["q"], dw.k_cache, dw.v_cache, t["bt"], t["qsl"], t["ctx"], t["seq"], dw.shape, plan, dw.ws
            )
        )
    torch.cuda.synchronize()
    a = [o.view(torch.int16).cpu().numpy() for o in outs]
    assert np.array_equal(a[0], a[1]) and np.array_equal(a[0], a[2])
    slots = O.slot_mapping(st.block_tables, st.query_start_loc, st.context_lens, wl.block_size)
    kp, vp = O.reshape_and_cache(st.k, st.v, wl.k_cache, wl.v_cache, slots, wl.block_size)
    ref, _ = O.paged_attention(st.q, kp, vp, st.block_tables, st.query_start_loc, st.context_lens, st.seq_lens, wl.block_size)
    check_attention(bf16_out_to_f64(outs[2]), ref, "plan reuse")


def test_permutation_invariance_and_rerun_bit_identical():
    say("physical permutation invariance")
    wl = W.decode_only(seed=5, num_seqs=10, ctx_range=(30, 900))
    st = wl.steps[0]
    dw = DeviceWorkload(wl)
    _, o1, _, _ = dw.run_step(st)
    _, o1b, _, _ = dw.run_step(st)  # re-run (cache write is idempotent)
    rng = np.random.default_rng(1)
    perm = rng.permutation(wl.num_blocks)
    wl2 = W.decode_only(seed=5, num_seqs=10, ctx_range=(30, 900))
    k2 = np.empty_like(wl2.k_cache)
    v2 = np.empty_like(wl2.v_cache)
    k2[perm] = wl2.k_cache
    v2[perm] = wl2.v_cache
    wl2.k_cache, wl2.v_cache = k2, v2
    wl2.steps[0].block_tables = perm[wl2.steps[0].block_tables].astype(np.int32)
    dw2 = DeviceWorkload(wl2)
    _, o2, _, _ = dw2.run_step(wl2.steps[0])
    torch.cuda.synchronize()
    a = o1.view(torch.int16).cpu().numpy()
    assert np.array_equal(a, o1b.view(torch.int16).cpu().numpy())
    assert np.array_equal(a, o2.view(torch.int16).cpu().numpy())


def _scale_bf16(bits: np.ndarray, factor: float) -> np.ndarray:
    """bf16 bit patterns times a power of two (exact while nothing overflows)."""
    x = (bits.astype(np.uint32) << 16).view(np.float32) * np.float32(factor)
    assert np.isfinite(x).all()
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _large_scores(wl, factor=16.0):
    """Every query times `factor`: scaled scores then spread over ~+-70 in log2 units, so the
    running maximum of a row moves by far more than its 2^8 window after the first tile or block
    and the kernels take their rescale branches (output and row sum times exp2(m_old - m_new)),
    which N(0, 1) queries never reach.  Most rows' softmax then sits on one or two keys."""
    for st in wl.steps:
        st.q[...] = _scale_bf16(st.q, factor)
    return wl


@pytest.mark.parametrize("case", ["mixed", "wide"])
def test_large_scores_take_the_rescale_paths(case):
    """Decode rows (split and unsplit), a speculative-verify row (short item), a chunk over a
    cached context (128-row tiles) and, for "wide", a long chunk on 256-row pipelined tiles, all
    with queries 16x N(0, 1), so that one key dominates many rows."""
    say(f"large scores: {case}")
    if case == "mixed":
        reqs = [W.RequestSpec(c, [1]) for c in (3000, 1500, 700, 40)]
        reqs += [W.RequestSpec(2000, [5]), W.RequestSpec(300, [200])]
        wl = W.build("large_mixed", reqs, num_q_heads=8, num_kv_heads=2, head_dim=128, seed=21)
        run_and_check(_large_scores(wl))
    else:
        reqs = [W.RequestSpec(300, [2048 // 4 + 37]), W.RequestSpec(2500, [1])]
        wl = W.build("large_wide", reqs, num_q_heads=8, num_kv_heads=2, head_dim=128, seed=22)
        run_and_check(_large_scores(wl), expect_tile_rows=256)


def test_large_scores_cascade():
    say("large scores: cascade")
    wl = W.cascade_shared_prefix(seed=23, num_queries=70, prefix=1040, suffix_range=(1, 200),
                                 num_q_heads=16, num_kv_heads=2, head_dim=128)
    _cascade_check(_large_scores(wl))


def test_cascade_prefix_cut_into_segments():
    """Too few query tiles to fill the chip: the prefix pass cuts a 4112-key prefix (not a
    multiple of the 64-key tile) into key segments, the last one ragged, and merges them."""
    say("cascade with key segments")
    wl = W.cascade_shared_prefix(seed=25, num_queries=20, prefix=4112, suffix_range=(1, 100),
                                 num_q_heads=16, num_kv_heads=2, head_dim=128)
    _cascade_check(wl)


def test_cascade_small_parity():
    say("cascade small")
    wl = W.cascade_shared_prefix(seed=1, num_queries=40, prefix=1024, suffix_range=(1, 300))
    _cascade_check(wl)


def _cascade_check(wl, rows=None, scale=None, every_row=False):
    """GPU prefix pass, suffix pass and merge against the oracle.  With rows, the prefix pass and
    the merged output are compared on those rows only (the merged output against single-pass
    attention).  With every_row, the prefix and suffix passes and the merged output are compared
    on every row against the oracle's own prefix pass, suffix pass and merge (which the CPU pins
    tie to single-pass attention), and rows still picks the rows checked against single-pass
    attention."""
    bs = wl.block_size
    st = wl.steps[0]
    cv = wl.cascade
    dw = DeviceWorkload(wl, scale=scale or 0.0)
    t = dw.step_tensors(st)
    slots = P.compute_slot_mapping(t["bt"], t["qsl"], t["ctx"], dw.shape, st.num_tokens)
    P.reshape_and_cache(t["k"], t["v"], dw.k_cache, dw.v_cache, slots, dw.shape)
    # prefix pass
    pbt = dev32(cv.prefix_block_table)
    cws = P.alloc_workspace(P.cascade_workspace_size(st.num_tokens, cv.prefix_len, dw.shape))
    o_p, l_p = P.cascade_prefix_attention(t["q"], dw.k_cache, dw.v_cache, pbt, cv.prefix_len, dw.shape, cws)
    # suffix pass: the same varlen kernel over the suffix view of the block tables
    pb = cv.prefix_blocks(bs)
    sbt_np = np.ascontiguousarray(st.block_tables[:, pb:])
    sshape = P.make_shape(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_blocks, sbt_np.shape[1],
                          block_size=wl.block_size, scale=scale or 0.0)
    sctx, sseq = dev32(cv.suffix_context_lens), dev32(cv.suffix_seq_lens)
    plan = P.plan_varlen(dw.ws, st.query_start_loc, cv.suffix_context_lens, cv.suffix_seq_lens, sshape)
    l_s = torch.empty((st.num_tokens, wl.num_q_heads), dtype=torch.float32, device="cuda")
    o_s = P.paged_attention_varlen(
        t["q"], dw.k_cache, dw.v_cache, dev32(sbt_np), t["qsl"], sctx, sseq, sshape, plan, dw.ws,
        out_dtype=torch.float32, lse=l_s,
    )
    lse_m = torch.empty_like(l_s)
    out = P.merge_attn_states(o_p, l_p, o_s, l_s, lse_out=lse_m)
    torch.cuda.synchronize()
    slots_o = O.slot_mapping(st.block_tables, st.query_start_loc, st.context_lens, bs)
    kp, vp = O.reshape_and_cache(st.k, st.v, wl.k_cache, wl.v_cache, slots_o, bs)
    if every_row:
        po, pl = O.cascade_prefix_attention(st.q, kp, vp, cv.prefix_block_table, cv.prefix_len, bs, scale=scale)
        check_attention(o_p.cpu().numpy().astype(np.float64), po, "cascade prefix, every row", bf16_out=False)
        check_lse(l_p.cpu().numpy(), pl, "cascade prefix lse, every row", rounded=True)
        so, sl = O.paged_attention(st.q, kp, vp, sbt_np, st.query_start_loc, cv.suffix_context_lens,
                                   cv.suffix_seq_lens, bs, scale=scale)
        check_attention(o_s.cpu().numpy().astype(np.float64), so, "cascade suffix, every row", bf16_out=False)
        check_lse(l_s.cpu().numpy(), sl, "cascade suffix lse, every row")
        mo, ml = O.merge_attn_states(po, pl, so, sl)
        r = check_attention(bf16_out_to_f64(out), mo, "cascade merged vs oracle merge, every row")
        check_lse(lse_m.cpu().numpy(), ml, "cascade merged lse, every row", rounded=True)
        say(f"    cascade merged, every row {r}")
        if rows is None:
            return
    sel = slice(None) if rows is None else rows
    qs = st.q if rows is None else st.q[rows]
    po, pl = O.cascade_prefix_attention(qs, kp, vp, cv.prefix_block_table, cv.prefix_len, bs, scale=scale)
    check_attention(o_p.cpu().numpy().astype(np.float64)[sel], po, "cascade prefix", bf16_out=False)
    check_lse(l_p.cpu().numpy()[sel], pl, "cascade prefix lse", rounded=True)
    fo, fl = O.paged_attention(st.q, kp, vp, st.block_tables, st.query_start_loc, st.context_lens, st.seq_lens, bs, rows=rows,
                               scale=scale)
    r = check_attention(bf16_out_to_f64(out)[sel], fo[sel], "cascade merged vs single pass")
    check_lse(lse_m.cpu().numpy()[sel], fl[sel], "cascade merged lse", rounded=True)
    say(f"    cascade merged {r}")


def test_merge_kernel_matches_oracle():
    say("merge kernel")
    rng = np.random.default_rng(7)
    T, H, D = 37, 8, 128
    oa, ob = rng.standard_normal((T, H, D)), rng.standard_normal((T, H, D))
    la, lb = rng.standard_normal((T, H)) * 5, rng.standard_normal((T, H)) * 5
    la[0, :3] = -np.inf
    lb[1, :2] = -np.inf
    la[2, 0] = lb[2, 0] = -np.inf
    oa[la == -np.inf] = 0
    ob[lb == -np.inf] = 0
    f = lambda x: torch.from_numpy(x.astype(np.float32)).cuda()  # noqa: E731
    lo = torch.empty((T, H), dtype=torch.float32, device="cuda")
    out = P.merge_attn_states(f(oa), f(la), f(ob), f(lb), out_dtype=torch.float32, lse_out=lo)
    torch.cuda.synchronize()
    ref_o, ref_l = O.merge_attn_states(oa.astype(np.float32), la.astype(np.float32), ob.astype(np.float32), lb.astype(np.float32))
    assert np.max(np.abs(out.cpu().numpy() - ref_o)) < 1e-5
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(lo.cpu().numpy()), fin)
    assert np.max(np.abs(lo.cpu().numpy()[fin] - ref_l[fin])) < 1e-5
    assert not np.isnan(out.cpu().numpy()).any()


def test_empty_and_zero_length_rows():
    say("empty batch and zero-length rows")
    wl = W.decode_only(seed=6, num_seqs=4, ctx_range=(20, 60))
    dw = DeviceWorkload(wl)
    st = wl.steps[0]
    dw.run_step(st)  # writes every row's new token into the pools
    slots_o = O.slot_mapping(st.block_tables, st.query_start_loc, st.context_lens, wl.block_size)
    kp, vp = O.reshape_and_cache(st.k, st.v, wl.k_cache, wl.v_cache, slots_o, wl.block_size)
    # the same rows again, but row 1 brings no new token (all of its keys are cached)
    qsl = np.array([0, 1, 1, 2, 3], np.int32)
    ctx = st.context_lens.copy()
    ctx[1] = st.seq_lens[1]
    seq = (ctx + np.diff(qsl)).astype(np.int32)
    q = st.q[[0, 2, 3]]
    plan = P.plan_varlen(dw.ws, qsl, ctx, seq, dw.shape)
    out = P.paged_attention_varlen(
        dev16(q), dw.k_cache, dw.v_cache, dev32(st.block_tables), dev32(qsl), dev32(ctx), dev32(seq), dw.shape, plan, dw.ws
    )
    torch.cuda.synchronize()
    o_ref, _ = O.paged_attention(q, kp, vp, st.block_tables, qsl, ctx, seq, wl.block_size)
    check_attention(bf16_out_to_f64(out), o_ref, "zero-length row")
    plan0 = P.plan_varlen(dw.ws, [0], [], [], dw.shape)
    assert plan0.num_items == 0


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_full_size_every_row(seed):
    """Full decode-only size (256 rows, ctx 1024..8192) in the launch configuration bench times,
    every row against the oracle."""
    say(f"decode_only full size, every row, seed {seed}")
    run_and_check(W.decode_only(seed=seed), check_pools=False)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_cascade_full_size_every_row(seed):
    """Full cascade size (512 queries x 64 heads, 16384-token prefix, suffixes 64..1024) in the
    launch configuration bench times: every row of the three passes against the oracle's, and
    24 sampled rows of the merged output against single-pass attention."""
    say(f"cascade full size (512 queries, 16384-token prefix), every row, seed {seed}")
    wl = W.cascade_shared_prefix(seed=seed)
    rows = np.sort(np.random.default_rng(3).choice(wl.steps[0].num_tokens, 24, replace=False))
    _cascade_check(wl, rows=rows, every_row=True)


@pytest.mark.parametrize("seed", [1, 2])
def test_long_chunked_prefill_full_size_last_chunk_other_seeds(seed):
    """The full long prefill with the other correctness seeds: every step runs, every row of the
    last (2048 prompt rows over 32768 keys and the 128 decode rows) is compared."""
    say(f"long_chunked_prefill full size, last chunk every row, seed {seed}")
    wl = W.long_chunked_prefill(seed=seed)
    run_and_check(wl, check_pools=False, want_lse=False, check_steps=(len(wl.steps) - 1,))


@pytest.mark.parametrize("chunks", [(0, 8), (8, 11), (11, 13), (13, 15), (15, 16)])
def test_long_chunked_prefill_full_size_every_row(chunks):
    """Full long-prefill size (a 32768-token prompt in 16 chunks of 2048 beside 128 decode rows)
    in the launch configuration bench times, every row: each case runs all 16 steps and compares
    every row of the steps in [chunks) (2048 prompt rows over up to 32768 keys and the 128 decode
    rows each); the cases split the oracle's work, which grows with the chunk index."""
    say(f"long_chunked_prefill full size (32768-token prompt in 16 chunks + 128 decode rows), steps {chunks}")
    wl = W.long_chunked_prefill(seed=0)
    run_and_check(wl, check_pools=False, want_lse=False, check_steps=range(*chunks))


# ---------------------------------------------------------------------------
# 256-token blocks: the same kernels, block tables naming blocks of 16 tiles
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("case", ["mixed", "decode", "wide"])
def test_block_size_256_parity(case):
    say(f"256-token blocks: {case}")
    if case == "mixed":
        run_and_check(W.mixed_llama8b(seed=21, num_decode=12, ctx_range=(20, 900), block_size=256),
                      expect_tile_rows=128)
    elif case == "decode":
        run_and_check(W.decode_only(seed=22, num_seqs=24, ctx_range=(30, 6000), block_size=256))
    else:
        wl = W.long_chunked_prefill(seed=23, prompt=4096, chunk=2048, num_decode=8, decode_ctx=300, block_size=256)
        run_and_check(wl, rows_per_step=200, expect_tile_rows=256)


def test_block_size_256_cascade():
    say("256-token blocks: cascade prefix + suffix + merge")
    _cascade_check(W.cascade_shared_prefix(seed=24, num_queries=40, prefix=1024, suffix_range=(1, 300),
                                           block_size=256))


def test_block_size_256_copy_blocks_bitwise():
    say("256-token blocks: copy_blocks")
    wl = W.mixed_llama8b(seed=25, num_decode=8, ctx_range=(100, 3000), block_size=256)
    dw = DeviceWorkload(wl)
    perm = np.random.default_rng(25).permutation(wl.num_blocks)
    n = wl.num_blocks // 2
    pairs = np.stack([perm[:n], perm[n:2 * n]], axis=1).astype(np.int32)
    P.copy_blocks(dw.k_cache, dw.v_cache, dev32(pairs), dw.shape)
    torch.cuda.synchronize()
    kc, vc = O.copy_blocks(wl.k_cache, wl.v_cache, pairs)
    assert np.array_equal(host16(dw.k_cache), kc) and np.array_equal(host16(dw.v_cache), vc)


def test_block_size_256_full_size_decode_every_row():
    say("256-token blocks: decode_only full size, every row")
    run_and_check(W.decode_only(seed=0, block_size=256), check_pools=False)


# ---------------------------------------------------------------------------
# Blocks of 32, 64 and 128 tokens (2, 4 and 8 tiles of 16 tokens)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("bs", [32, 64, 128])
@pytest.mark.parametrize("case", ["mixed", "decode"])
def test_block_sizes_32_to_128_parity(case, bs):
    say(f"{bs}-token blocks: {case}")
    if case == "mixed":
        run_and_check(W.mixed_llama8b(seed=60 + bs, num_decode=12, ctx_range=(20, 1500), block_size=bs))
    else:
        run_and_check(W.decode_only(seed=61 + bs, num_seqs=24, ctx_range=(1, 6000), block_size=bs))


@pytest.mark.parametrize("bs", [32, 128])
def test_block_sizes_wide_tiles_and_cascade(bs):
    say(f"{bs}-token blocks: 256-row tiles, then cascade prefix + suffix + merge")
    wl = W.long_chunked_prefill(seed=62 + bs, prompt=4096, chunk=2048, num_decode=8, decode_ctx=300, block_size=bs)
    run_and_check(wl, rows_per_step=200, expect_tile_rows=256)
    _cascade_check(W.cascade_shared_prefix(seed=63 + bs, num_queries=40, prefix=1024, suffix_range=(1, 300),
                                           block_size=bs))


def test_block_size_64_copy_on_write_then_device_split_decode():
    """64-token blocks, copy-on-write: a third of the requests' blocks are copied into spare
    blocks (bit for bit, as the oracle's copy) and those block-table entries are pointed at the
    copies; the fused append and the device-split decode over the remapped tables then match
    the oracle over the same tables."""
    say("64-token blocks: copy_blocks into spare blocks, remapped tables, device-split decode")
    wl = W.decode_only(seed=64, num_seqs=20, ctx_range=(1, 5000), block_size=64)
    st = wl.steps[0]
    dw = DeviceWorkload(wl)
    used = np.concatenate([st.block_tables[r, : -(-int(st.seq_lens[r]) // wl.block_size)] for r in range(st.num_seqs)])
    spare = np.setdiff1d(np.arange(wl.num_blocks), st.block_tables)
    rng = np.random.default_rng(64)
    n = min(len(spare), len(used) // 3)
    src = rng.choice(used, size=n, replace=False)
    dst = rng.choice(spare, size=n, replace=False)
    pairs = np.stack([src, dst], axis=1).astype(np.int32)
    P.copy_blocks(dw.k_cache, dw.v_cache, dev32(pairs), dw.shape)
    torch.cuda.synchronize()
    kc, vc = O.copy_blocks(wl.k_cache, wl.v_cache, pairs)
    assert np.array_equal(host16(dw.k_cache), kc) and np.array_equal(host16(dw.v_cache), vc)
    remap = np.arange(wl.num_blocks, dtype=np.int32)
    remap[src] = dst
    bt = remap[st.block_tables]
    t = dw.step_tensors(st)
    t["bt"] = dev32(bt)
    P.append_kv(t["k"], t["v"], dw.k_cache, dw.v_cache, t["bt"], t["qsl"], t["ctx"], dw.shape)
    max_seq = wl.bt_stride * wl.block_size
    ws = P.alloc_workspace(P.decode_workspace_size(st.num_seqs, max_seq, dw.shape))
    lse = torch.empty(st.q.shape[:2], dtype=torch.float32, device="cuda")
    out = P.paged_attention_decode(t["q"], dw.k_cache, dw.v_cache, t["bt"], t["qsl"], t["seq"], dw.shape, max_seq,
                                   workspace=ws, lse=lse)
    torch.cuda.synchronize()
    slots = O.slot_mapping(bt, st.query_start_loc, st.context_lens, wl.block_size)
    kp, vp = O.reshape_and_cache(st.k, st.v, kc, vc, slots, wl.block_size)
    assert np.array_equal(host16(dw.k_cache), kp) and np.array_equal(host16(dw.v_cache), vp)
    ref, lref = O.paged_attention(st.q, kp, vp, bt, st.query_start_loc, st.context_lens, st.seq_lens, wl.block_size)
    say(f"    {n} blocks copied; {check_attention(bf16_out_to_f64(out), ref, 'device-split decode, 64-token blocks')}")
    check_lse(lse.cpu().numpy(), lref, "device-split decode lse, 64-token blocks")


@pytest.mark.parametrize("num_req,num_kv_heads,head_dim", [(900, 2, 64), (200, 1, 64), (3000, 8, 128)])
def test_slot_search_over_many_requests(num_req, num_kv_heads, head_dim):
    """Slot mapping and the fused append over batches with more requests than a workgroup has
    threads and long runs of requests with no new token: slots and pool bits equal the
    oracle's (the same slots as without the empty requests)."""
    wl, st, qsl, ctx, bt = many_requests(11 + num_req, num_req, num_kv_heads, head_dim)
    say(f"slot search: {len(ctx)} requests ({num_req} with tokens), T={st.num_tokens}, Hkv={num_kv_heads}, D={head_dim}")
    ref = O.slot_mapping(bt, qsl, ctx, wl.block_size)
    assert np.array_equal(ref, O.slot_mapping(st.block_tables, st.query_start_loc, st.context_lens, wl.block_size))
    shape = P.make_shape(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_blocks, wl.bt_stride,
                         block_size=wl.block_size)
    btd, qsld, ctxd = dev32(bt), dev32(qsl), dev32(ctx)
    slots = P.compute_slot_mapping(btd, qsld, ctxd, shape, st.num_tokens)
    torch.cuda.synchronize()
    assert np.array_equal(slots.cpu().numpy(), ref), "slot mapping differs"
    kc, vc = dev16(wl.k_cache), dev16(wl.v_cache)
    slots2 = torch.empty(st.num_tokens, dtype=torch.int64, device="cuda")
    P.append_kv(dev16(st.k), dev16(st.v), kc, vc, btd, qsld, ctxd, shape, slot_mapping=slots2)
    torch.cuda.synchronize()
    assert np.array_equal(slots2.cpu().numpy(), ref), "append_kv slots differ"
    kp, vp = O.reshape_and_cache(st.k, st.v, wl.k_cache, wl.v_cache, ref, wl.block_size)
    assert np.array_equal(host16(kc), kp) and np.array_equal(host16(vc), vp), "pool bits differ"


def test_slots_past_the_table_or_before_zero_are_skipped():
    """Requests whose positions run past the block table, or are negative, get slot -1 for
    those tokens and write nothing; the other requests' slots and pool bits equal the oracle's."""
    wl = W.decode_only(seed=31, num_seqs=40, ctx_range=(5, 600))
    st = wl.steps[0]
    B = st.num_seqs
    ql = np.diff(st.query_start_loc).astype(np.int64)
    bad_past, bad_neg = [3, 17, 29], [8, 30]
    ql2 = ql.copy()
    ql2[bad_past + bad_neg] = 3
    ctx2 = st.context_lens.astype(np.int64).copy()
    ctx2[bad_past] = wl.bt_stride * wl.block_size + np.array([0, 5, 40])  # every position past the table
    ctx2[bad_neg] = -4  # positions -4, -3, -2
    qsl2 = np.concatenate([[0], np.cumsum(ql2)]).astype(np.int32)
    T = int(qsl2[-1])
    rng = np.random.default_rng(31)
    k = W.f32_to_bf16_bits(rng.standard_normal((T, wl.num_kv_heads, wl.head_dim)).astype(np.float32))
    v = W.f32_to_bf16_bits(rng.standard_normal((T, wl.num_kv_heads, wl.head_dim)).astype(np.float32))
    good = np.array([r for r in range(B) if r not in bad_past + bad_neg])
    good_tok = np.concatenate([np.arange(qsl2[r], qsl2[r + 1]) for r in good])
    qsl_good = np.concatenate([[0], np.cumsum(ql2[good])]).astype(np.int32)
    ref = np.full(T, -1, dtype=np.int64)
    ref[good_tok] = O.slot_mapping(st.block_tables[good], qsl_good, ctx2[good], wl.block_size)
    dw = DeviceWorkload(wl)
    btd, qsld, ctxd = dev32(st.block_tables), dev32(qsl2), dev32(ctx2)
    slots = P.compute_slot_mapping(btd, qsld, ctxd, dw.shape, T)
    slots2 = torch.empty(T, dtype=torch.int64, device="cuda")
    P.append_kv(dev16(k), dev16(v), dw.k_cache, dw.v_cache, btd, qsld, ctxd, dw.shape, slot_mapping=slots2)
    torch.cuda.synchronize()
    assert np.array_equal(slots.cpu().numpy(), ref) and np.array_equal(slots2.cpu().numpy(), ref)
    kp, vp = O.reshape_and_cache(k, v, wl.k_cache, wl.v_cache, ref, wl.block_size)
    assert np.array_equal(host16(dw.k_cache), kp) and np.array_equal(host16(dw.v_cache), vp)


@pytest.mark.parametrize("bs", [16, 256])
def test_slot_mapping_past_2_pow_31(bs):
    """Block ids near the top of the int32 range: slots (block id x block size + offset) pass
    2^31 and must come out as exact int64 values (no pool is touched)."""
    say(f"slot mapping above 2^31, block size {bs}")
    rng = np.random.default_rng(bs)
    B, W_ = 30, 6
    num_blocks = (1 << 31) // (bs // 16) - 1
    bt = rng.integers(num_blocks // 2, num_blocks, size=(B, W_)).astype(np.int32)
    ql = rng.integers(0, 5, size=B)
    ctx = rng.integers(0, W_ * bs - 4, size=B)
    qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    ref = O.slot_mapping(bt, qsl, ctx.astype(np.int32), bs)
    assert ref.max() >= 1 << 31
    shape = P.make_shape(8, 2, 128, num_blocks, W_, block_size=bs)
    slots = P.compute_slot_mapping(dev32(bt), dev32(qsl), dev32(ctx), shape, int(qsl[-1]))
    torch.cuda.synchronize()
    assert np.array_equal(slots.cpu().numpy(), ref)


@pytest.mark.parametrize("group,head_dim", [(8, 128), (4, 64)])
def test_one_kv_head(group, head_dim):
    """A single kv head (multi-query attention): decode rows with and without splits, a short
    row, 128-row tiles, and then 256-row tiles and the cascade, all on one kv head."""
    say(f"one kv head, G={group}, D={head_dim}")
    reqs = [W.RequestSpec(c, [1]) for c in (2000, 300, 7)]
    reqs += [W.RequestSpec(600, [2]), W.RequestSpec(100, [90])]
    wl = W.build("mqa_mixed", reqs, num_q_heads=group, num_kv_heads=1, head_dim=head_dim, seed=44 + group)
    run_and_check(wl)
    reqs = [W.RequestSpec(50, [2048 // group + 11]), W.RequestSpec(900, [1])]
    wl = W.build("mqa_wide", reqs, num_q_heads=group, num_kv_heads=1, head_dim=head_dim, seed=45 + group)
    run_and_check(wl, expect_tile_rows=256)
    _cascade_check(W.cascade_shared_prefix(seed=46 + group, num_queries=30, prefix=1024, suffix_range=(1, 200),
                                           num_q_heads=group, num_kv_heads=1, head_dim=head_dim))


def test_explicit_softmax_scale():
    """pkv_shape.scale > 0 replaces 1/sqrt(head_dim) in every path (decode, short, 128-row and
    256-row tiles, cascade prefix and suffix), against the oracle at the same scale.  0.05
    against the default 0.088 at D 128: scores 0.57x as large, a difference far beyond the
    tolerance in rows of many keys, and no row that one key dominates."""
    say("explicit softmax scale 0.05")
    reqs = [W.RequestSpec(c, [1]) for c in (1800, 60)]
    reqs += [W.RequestSpec(700, [3]), W.RequestSpec(40, [70])]
    run_and_check(W.build("scaled_mixed", reqs, num_q_heads=8, num_kv_heads=2, head_dim=128, seed=47), scale=0.05)
    reqs = [W.RequestSpec(0, [2048 // 4 + 5])]
    run_and_check(W.build("scaled_wide", reqs, num_q_heads=8, num_kv_heads=2, head_dim=128, seed=48),
                  expect_tile_rows=256, scale=0.05)
    _cascade_check(W.cascade_shared_prefix(seed=49, num_queries=24, prefix=1024, suffix_range=(1, 100),
                                           num_q_heads=8, num_kv_heads=2, head_dim=128), scale=0.05)
