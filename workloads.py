"""Seeded synthetic workloads for attention over a paged KV cache.

This module builds inputs only.  It draws request lengths, a random
permutation of the physical block pool, block tables and bf16 values, and
it carries no attention arithmetic: no slot computation, no scores, no
softmax.  Both the CPU oracle (``oracle/``) and the HIP library are fed from
here; neither one's results ever flow back into it.

Value recipe (used by every workload):
  * every float is an N(0,1) fp32 draw rounded to bf16 with
    round-to-nearest-even; values travel as raw bf16 bit patterns (uint16);
  * integer uniform draws are inclusive on both ends;
  * draw order: lengths, pool permutation, prior-cache K/V (written straight
    into the pools at the slots of tokens already cached before the first
    step), then per step new K, new V and Q;
  * large arrays are drawn in fixed 4 Mi-element chunks, each from its own
    PCG64 stream keyed by (seed, array tag, chunk index), so the values do not
    depend on how many threads draw them;
  * pools: keys [num_blocks, Hkv, 16, D] (token-major), values
    [num_blocks, Hkv, D, 16] (dim-major); a pool of 16 R-token blocks (R > 1, e.g. 256-token
    blocks) holds R such 16-token tiles per block: keys [num_blocks, R, Hkv, 16, D], values
    [num_blocks, R, Hkv, D, 16];
  * every pool slot that holds no cached token (unreferenced blocks, block
    table padding and the not-yet-written tail of each request) is set to
    bf16 NaN so that a kernel reading outside the visible keys shows up.

The five workloads mirror the shapes the pages use: the 31+29+30 batched
prefill of the Tencent Cloud article ("how vLLM implements inference
acceleration", batched-prefill paragraph); the 48-token prompt in three
16-token chunks, the 16-cached + 15-token chunk and the 107-token prompt with
48 prefix-cached tokens (same article, chunked-prefill and prefix-caching
sections); a decode-only batch; a long chunked prefill beside decode rows;
and the shared-prefix batch of cascade inference (2048ai.net vLLM V1 article,
"Cascade Inference").
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
_CHUNK = 1 << 22

WORKLOAD_NAMES = (
    "tiny_prefill",
    "mixed_llama8b",
    "decode_only",
    "long_chunked_prefill",
    "cascade_shared_prefix",
)

_TAGS = {"pool_k": 1, "pool_v": 2, "new_k": 3, "new_v": 4, "q": 5, "fp8_k": 6, "fp8_v": 7, "fp8_scale": 8}
FP8_NAN = np.uint8(0x7F)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even; NaN stays a quiet NaN."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    out = ((u + (np.uint32(0x7FFF) + lsb)) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_bf16(n: int, seed: int, tag: int, sub: int = 0) -> np.ndarray:
    """n N(0,1) values as bf16 bits, drawn chunk by chunk from keyed PCG64 streams."""
    out = np.empty(n, dtype=np.uint16)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def fill(ci: int) -> None:
        lo = ci * _CHUNK
        hi = min(n, lo + _CHUNK)
        ss = np.random.SeedSequence(entropy=seed, spawn_key=(tag, sub, ci))
        g = np.random.Generator(np.random.PCG64(ss))
        out[lo:hi] = f32_to_bf16_bits(g.standard_normal(hi - lo, dtype=np.float32))

    if nchunks <= 1:
        if n:
            fill(0)
    else:
        with ThreadPoolExecutor(max_workers=_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


@dataclass
class Step:
    """Metadata and new tensors of one attention call over a mixed batch."""

    query_start_loc: np.ndarray  # int32 [B+1]
    context_lens: np.ndarray  # int32 [B]  tokens cached before this step
    seq_lens: np.ndarray  # int32 [B]  keys visible after this step
    block_tables: np.ndarray  # int32 [B, W]
    request_ids: np.ndarray  # int32 [B]  which logical request each row is
    k: np.ndarray  # bf16 bits [T, Hkv, D]
    v: np.ndarray  # bf16 bits [T, Hkv, D]
    q: np.ndarray  # bf16 bits [T, Hq, D]

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def query_lens(self) -> np.ndarray:
        return np.diff(self.query_start_loc).astype(np.int32)


@dataclass
class CascadeView:
    """The shared-prefix split of a cascade step.

    ``prefix_block_table`` lists the physical blocks of the shared prefix;
    the suffix pass reads ``block_tables[:, prefix_blocks:]`` with the
    suffix-relative lengths below.
    """

    prefix_len: int
    prefix_block_table: np.ndarray  # int32 [prefix_len / bs]
    suffix_context_lens: np.ndarray  # int32 [B]
    suffix_seq_lens: np.ndarray  # int32 [B]

    def prefix_blocks(self, block_size: int) -> int:
        return self.prefix_len // block_size


@dataclass
class Workload:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    bt_stride: int
    k_cache: np.ndarray  # bf16 bits [NB, Hkv, bs, D] (initial contents; token-major)
    v_cache: np.ndarray  # bf16 bits [NB, Hkv, D, bs] (dim-major)
    steps: List[Step]
    cascade: Optional[CascadeView] = None
    notes: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


@dataclass
class RequestSpec:
    """One logical request: ``context`` tokens already cached, then one chunk per step (0 = idle)."""

    context: int
    chunks: Sequence[int]


def build(
    name: str,
    requests: Sequence[RequestSpec],
    *,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    block_size: int = 16,
    seed: int = 0,
    rng: Optional[np.random.Generator] = None,
    pool_factor: float = 1.2,
    num_blocks: Optional[int] = None,
    bt_stride: Optional[int] = None,
    shared_prefix: int = 0,
    distinct_padding: bool = False,
    poison: bool = True,
) -> Workload:
    """Lay the requests out in a randomly permuted block pool and draw all values.

    ``shared_prefix`` tokens (a multiple of ``block_size``) at the start of every
    request live in one set of physical blocks that every block table names.
    ``distinct_padding`` fills block-table entries past a request's last block
    with further distinct physical ids instead of one spare poisoned block.
    """
    bs = block_size
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    if shared_prefix % bs:
        raise ValueError("shared prefix must be block aligned")
    nreq = len(requests)
    nsteps = max(len(r.chunks) for r in requests)
    final = [r.context + sum(r.chunks) for r in requests]
    nblk = [-(-f // bs) for f in final]
    pblk = shared_prefix // bs
    own = [b - pblk for b in nblk]
    if min(own) < 0:
        raise ValueError("request shorter than the shared prefix")
    W = bt_stride if bt_stride is not None else max(nblk)
    if W < max(nblk):
        raise ValueError("block table stride too small")
    used = pblk + sum(own)
    pad_needed = nreq * W - sum(nblk) if distinct_padding else 1
    if num_blocks is None:
        num_blocks = max(int(math.ceil(pool_factor * used)), used + pad_needed)
    if num_blocks < used + pad_needed:
        raise ValueError("pool too small")

    perm = rng.permutation(num_blocks).astype(np.int32)
    cur = 0
    prefix_ids = perm[cur : cur + pblk]
    cur += pblk
    tables = np.empty((nreq, W), dtype=np.int32)
    for r in range(nreq):
        tables[r, :pblk] = prefix_ids
        tables[r, pblk : nblk[r]] = perm[cur : cur + own[r]]
        cur += own[r]
    if distinct_padding:
        for r in range(nreq):
            k = W - nblk[r]
            tables[r, nblk[r] :] = perm[cur : cur + k]
            cur += k
    else:
        spare = perm[cur]
        cur += 1
        for r in range(nreq):
            tables[r, nblk[r] :] = spare

    H, D = num_kv_heads, head_dim
    nelem = num_blocks * H * bs * D
    if bs > 16:
        if bs % 16:
            raise ValueError("blocks above 16 tokens must be whole 16-token tiles")
        R = bs // 16
        k_cache = normal_bf16(nelem, seed, _TAGS["pool_k"]).reshape(num_blocks, R, H, 16, D)
        v_cache = normal_bf16(nelem, seed, _TAGS["pool_v"]).reshape(num_blocks, R, H, D, 16)
    else:
        R = 1
        k_cache = normal_bf16(nelem, seed, _TAGS["pool_k"]).reshape(num_blocks, H, bs, D)
        v_cache = normal_bf16(nelem, seed, _TAGS["pool_v"]).reshape(num_blocks, H, D, bs)
    k5 = k_cache if R > 1 else k_cache[:, None]  # [NB, R, H, T, D] view
    v5 = v_cache if R > 1 else v_cache[:, None]
    T = bs // R
    if poison:
        referenced = np.zeros(num_blocks, dtype=bool)
        for r in range(nreq):
            referenced[tables[r, : nblk[r]]] = True
        k_cache[~referenced] = BF16_NAN
        v_cache[~referenced] = BF16_NAN
        # Slots at or past each request's cached length hold no token yet.
        for r in range(nreq):
            start = max(requests[r].context, shared_prefix)
            for pos_blk in range(start // bs, nblk[r]):
                lo = max(start - pos_blk * bs, 0)
                phys = tables[r, pos_blk]
                for t in range(R):
                    lt = min(max(lo - t * T, 0), T)
                    k5[phys, t, :, lt:, :] = BF16_NAN
                    v5[phys, t, :, :, lt:] = BF16_NAN

    steps: List[Step] = []
    done = [r.context for r in requests]
    for s in range(nsteps):
        rows = [r for r in range(nreq) if s < len(requests[r].chunks) and requests[r].chunks[s] > 0]
        qlen = np.array([requests[r].chunks[s] for r in rows], dtype=np.int32)
        ctx = np.array([done[r] for r in rows], dtype=np.int32)
        qsl = np.zeros(len(rows) + 1, dtype=np.int32)
        np.cumsum(qlen, out=qsl[1:])
        T = int(qsl[-1])
        k = normal_bf16(T * H * D, seed, _TAGS["new_k"], s).reshape(T, H, D)
        v = normal_bf16(T * H * D, seed, _TAGS["new_v"], s).reshape(T, H, D)
        q = normal_bf16(T * num_q_heads * D, seed, _TAGS["q"], s).reshape(T, num_q_heads, D)
        steps.append(
            Step(
                query_start_loc=qsl,
                context_lens=ctx,
                seq_lens=(ctx + qlen).astype(np.int32),
                block_tables=np.ascontiguousarray(tables[rows]),
                request_ids=np.array(rows, dtype=np.int32),
                k=k,
                v=v,
                q=q,
            )
        )
        for i, r in enumerate(rows):
            done[r] += int(qlen[i])

    cascade = None
    if shared_prefix:
        last = steps[-1]
        cascade = CascadeView(
            prefix_len=shared_prefix,
            prefix_block_table=prefix_ids.copy(),
            suffix_context_lens=(last.context_lens - shared_prefix).astype(np.int32),
            suffix_seq_lens=(last.seq_lens - shared_prefix).astype(np.int32),
        )
    return Workload(
        name=name,
        num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads,
        head_dim=head_dim,
        block_size=bs,
        num_blocks=num_blocks,
        bt_stride=W,
        k_cache=k_cache,
        v_cache=v_cache,
        steps=steps,
        cascade=cascade,
    )


@dataclass
class Fp8Cache:
    """An FP8 (e4m3 byte code) KV cache in the layouts of the bf16 pools, with one fp32 scale per
    (physical block, kv head) tile of each pool."""

    k_cache: np.ndarray  # uint8 [NB, Hkv, bs, D]
    v_cache: np.ndarray  # uint8 [NB, Hkv, D, bs]
    k_scale: np.ndarray  # float32 [NB, Hkv]
    v_scale: np.ndarray  # float32 [NB, Hkv]


def random_codes(n: int, seed: int, tag: int, max_magnitude: int = 0x57) -> np.ndarray:
    """n random e4m3 byte codes: magnitude byte uniform on [0, max_magnitude] (0x57 is 15.0,
    below the NaN code 0x7f), sign bit uniform; drawn chunk by chunk like normal_bf16."""
    out = np.empty(n, dtype=np.uint8)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def fill(ci: int) -> None:
        lo = ci * _CHUNK
        hi = min(n, lo + _CHUNK)
        ss = np.random.SeedSequence(entropy=seed, spawn_key=(tag, 0, ci))
        g = np.random.Generator(np.random.PCG64(ss))
        mag = g.integers(0, max_magnitude, size=hi - lo, endpoint=True, dtype=np.uint8)
        sign = g.integers(0, 1, size=hi - lo, endpoint=True, dtype=np.uint8) << np.uint8(7)
        out[lo:hi] = mag | sign

    if nchunks <= 1:
        if n:
            fill(0)
    else:
        with ThreadPoolExecutor(max_workers=_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def fp8_cache(wl: "Workload", seed: int = 0, scale_range=(0.04, 0.12)) -> Fp8Cache:
    """FP8 pools for a workload: every element the bf16 pools hold as a cached value gets a
    random code (random_codes), every poisoned element the NaN code 0x7f; the scales are
    uniform fp32 draws on scale_range, one per (block, kv head) of each pool."""
    kc = random_codes(wl.k_cache.size, seed, _TAGS["fp8_k"]).reshape(wl.k_cache.shape)
    vc = random_codes(wl.v_cache.size, seed, _TAGS["fp8_v"]).reshape(wl.v_cache.shape)
    kc[wl.k_cache == BF16_NAN] = FP8_NAN
    vc[wl.v_cache == BF16_NAN] = FP8_NAN
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=(_TAGS["fp8_scale"],))))
    lo, hi = scale_range
    shape = (wl.num_blocks, wl.num_kv_heads)
    ks = g.uniform(lo, hi, size=shape).astype(np.float32)
    vs = g.uniform(lo, hi, size=shape).astype(np.float32)
    return Fp8Cache(k_cache=kc, v_cache=vc, k_scale=ks, v_scale=vs)


def _rng(seed: int, which: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, which])))


def tiny_prefill(seed: int = 0) -> Workload:
    """3 prompts of 31, 29, 30 tokens batched into 90 query tokens; 4 q / 2 kv heads, D=64.

    Block tables have 8 logical entries per request, all 24 distinct physical
    ids drawn from one permutation of a 64-block pool (only the first two per
    request hold tokens).
    """
    reqs = [RequestSpec(0, [31]), RequestSpec(0, [29]), RequestSpec(0, [30])]
    return build(
        "tiny_prefill",
        reqs,
        num_q_heads=4,
        num_kv_heads=2,
        head_dim=64,
        seed=seed,
        rng=_rng(seed, 0),
        num_blocks=64,
        bt_stride=8,
        distinct_padding=True,
    )


def mixed_llama8b(seed: int = 0, num_decode: int = 64, ctx_range=(128, 4096), block_size: int = 16) -> Workload:
    """Mixed continuous batch on a Llama-3-8B-shaped layer (32 q / 8 kv heads, D=128).

    Three steps over one pool:
      A: a 48-token prompt in chunks of 16/16/16;
      C: a 31-token prompt as 16 then 15 (the 16-cached + 15-token chunk);
      B: a 107-token prompt whose first 48 tokens are prefix-cached (one step, 59 tokens from position 48);
      plus ``num_decode`` decode rows, context uniform in ``ctx_range``, one token per step.
    """
    rng = _rng(seed, 1)
    dctx = rng.integers(ctx_range[0], ctx_range[1] + 1, size=num_decode)
    reqs = [RequestSpec(0, [16, 16, 16]), RequestSpec(0, [16, 15]), RequestSpec(48, [59])]
    reqs += [RequestSpec(int(c), [1, 1, 1]) for c in dctx]
    return build("mixed_llama8b", reqs, num_q_heads=32, num_kv_heads=8, head_dim=128, seed=seed, rng=rng,
                 block_size=block_size)


def decode_only(seed: int = 0, num_seqs: int = 256, ctx_range=(1024, 8192), num_q_heads: int = 32,
                block_size: int = 16) -> Workload:
    """Memory-bound decode: one query token per sequence, context uniform in ``ctx_range``."""
    rng = _rng(seed, 2)
    ctx = rng.integers(ctx_range[0], ctx_range[1] + 1, size=num_seqs)
    reqs = [RequestSpec(int(c), [1]) for c in ctx]
    return build("decode_only", reqs, num_q_heads=num_q_heads, num_kv_heads=8, head_dim=128, seed=seed, rng=rng,
                 block_size=block_size)


def long_chunked_prefill(
    seed: int = 0, prompt: int = 32768, chunk: int = 2048, num_decode: int = 128, decode_ctx: int = 2048,
    block_size: int = 16,
) -> Workload:
    """One long prompt prefilled in fixed chunks against its growing paged context, beside decode rows."""
    rng = _rng(seed, 3)
    n = prompt // chunk
    reqs = [RequestSpec(0, [chunk] * n)]
    reqs += [RequestSpec(decode_ctx, [1] * n) for _ in range(num_decode)]
    return build("long_chunked_prefill", reqs, num_q_heads=32, num_kv_heads=8, head_dim=128, seed=seed, rng=rng,
                 block_size=block_size)


def spec_verify(seed: int = 0, num_seqs: int = 64, draft: int = 4, ctx_range=(1024, 4096)) -> Workload:
    """Speculative-decoding verification rows: each request scores its next token plus ``draft``
    drafted tokens (query length 1 + draft) against its cached context in one pass, as the
    Tencent Cloud article's speculative decoding / MTP section describes with four drafts;
    Llama-3-8B-shaped."""
    rng = _rng(seed, 5)
    ctx = rng.integers(ctx_range[0], ctx_range[1] + 1, size=num_seqs)
    reqs = [RequestSpec(int(c), [1 + draft]) for c in ctx]
    return build("spec_verify", reqs, num_q_heads=32, num_kv_heads=8, head_dim=128, seed=seed, rng=rng)


def cascade_shared_prefix(
    seed: int = 0,
    num_queries: int = 512,
    prefix: int = 16384,
    suffix_range=(64, 1024),
    num_q_heads: int = 64,
    num_kv_heads: int = 8,
    head_dim: int = 128,
    block_size: int = 16,
) -> Workload:
    """Decode queries that all share one physical prefix, plus unique suffixes (which include the new token).

    Default: the 70B-shaped head slice, 64 q / 8 kv heads, D=128.
    """
    rng = _rng(seed, 4)
    suf = rng.integers(suffix_range[0], suffix_range[1] + 1, size=num_queries)
    reqs = [RequestSpec(prefix + int(s) - 1, [1]) for s in suf]
    return build(
        "cascade_shared_prefix",
        reqs,
        num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads,
        head_dim=head_dim,
        seed=seed,
        rng=rng,
        shared_prefix=prefix,
        block_size=block_size,
    )


_BUILDERS = {
    "tiny_prefill": tiny_prefill,
    "mixed_llama8b": mixed_llama8b,
    "decode_only": decode_only,
    "long_chunked_prefill": long_chunked_prefill,
    "cascade_shared_prefix": cascade_shared_prefix,
    "spec_verify": spec_verify,
}


def make_workload(name, seed: int = 0, **kw) -> Workload:
    """Build a workload by name or by its 0-based index in ``WORKLOAD_NAMES``."""
    if isinstance(name, int):
        name = WORKLOAD_NAMES[name]
    return _BUILDERS[name](seed=seed, **kw)
