"""Python face of libpkv: one function per C entry point, same names, torch tensors in and out.

Only argument marshalling happens here (dtype/device/contiguity checks, pointer extraction,
the current HIP stream).  Every step of the attention path runs in the HIP kernels of
libpkv.so.  bf16 tensors may be passed as torch.bfloat16 or as raw 16-bit views.
"""

from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import numpy as np
import torch

from ._lib import PKV_DTYPE_BF16, PKV_DTYPE_F32, PkvShape, PkvVarlenPlan, check, lib

_16BIT = (torch.bfloat16, torch.int16, torch.uint16)
# FP8 (e4m3) pools: raw byte codes, or torch's float8_e4m3fn view of the same bytes.
_FP8 = (torch.uint8,) + ((torch.float8_e4m3fn,) if hasattr(torch, "float8_e4m3fn") else ())
_F32 = (torch.float32,)


def make_shape(
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    num_blocks: int,
    bt_stride: int,
    block_size: int = 16,
    scale: float = 0.0,
) -> PkvShape:
    return PkvShape(num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, bt_stride, scale)


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, name: str, dtypes=None) -> ctypes.c_void_p:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return ctypes.c_void_p(t.data_ptr())


def _opt(t: Optional[torch.Tensor], name: str, dtypes=None) -> ctypes.c_void_p:
    return ctypes.c_void_p(0) if t is None else _dev(t, name, dtypes)


def _need(t: Optional[torch.Tensor], n: int, name: str) -> None:
    """Raise unless tensor ``t`` (if given) holds at least ``n`` elements: a buffer smaller than
    the sizes passed to the library would be read or written out of bounds on the device."""
    if t is not None and isinstance(t, torch.Tensor) and t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} elements, the call needs {n}")


def _pool_elems(shape: PkvShape) -> int:
    """Elements of one pool (keys or values) of this shape."""
    return int(shape.num_blocks) * int(shape.num_kv_heads) * int(shape.block_size) * int(shape.head_dim)


def _need_meta(block_tables, query_start_loc, context_lens, seq_lens, num_seqs: int, shape: PkvShape) -> None:
    _need(block_tables, num_seqs * int(shape.bt_stride), "block_tables")
    _need(query_start_loc, num_seqs + 1, "query_start_loc")
    _need(context_lens, num_seqs, "context_lens")
    _need(seq_lens, num_seqs, "seq_lens")


def _need_pools(k_cache, v_cache, shape: PkvShape, k_scale=None, v_scale=None) -> None:
    _need(k_cache, _pool_elems(shape), "k_cache")
    _need(v_cache, _pool_elems(shape), "v_cache")
    _need(k_scale, int(shape.num_blocks) * int(shape.num_kv_heads), "k_scale")
    _need(v_scale, int(shape.num_blocks) * int(shape.num_kv_heads), "v_scale")


def _need_new_kv(k, v, num_tokens: int, shape: PkvShape) -> None:
    n = num_tokens * int(shape.num_kv_heads) * int(shape.head_dim)
    _need(k, n, "k")
    _need(v, n, "v")


def _need_q_out(q, out, lse, num_tokens: int, shape: PkvShape) -> None:
    n = num_tokens * int(shape.num_q_heads)
    _need(q, n * int(shape.head_dim), "q")
    _need(out, n * int(shape.head_dim), "out")
    _need(lse, n, "lse")


def _host_i32(x, name: str) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    a = np.ascontiguousarray(np.asarray(x), dtype=np.int32)
    if a.ndim != 1:
        raise ValueError(f"{name} must be one-dimensional")
    return a


def version() -> str:
    return lib().pkv_version().decode()


def compute_slot_mapping(
    block_tables: torch.Tensor,
    query_start_loc: torch.Tensor,
    context_lens: torch.Tensor,
    shape: PkvShape,
    num_tokens: int,
    out: Optional[torch.Tensor] = None,
) -> torch.Tensor:
    """Slot of every new token (int64 [num_tokens]) from the block tables."""
    num_seqs = int(context_lens.numel())
    if out is None:
        out = torch.empty(num_tokens, dtype=torch.int64, device=block_tables.device)
    _need(out, num_tokens, "slot_mapping")
    _need_meta(block_tables, query_start_loc, context_lens, None, num_seqs, shape)
    check(
        lib().pkv_compute_slot_mapping(
            _dev(out, "slot_mapping", (torch.int64,)),
            _dev(block_tables, "block_tables", (torch.int32,)),
            _dev(query_start_loc, "query_start_loc", (torch.int32,)),
            _dev(context_lens, "context_lens", (torch.int32,)),
            num_seqs,
            num_tokens,
            ctypes.byref(shape),
            _stream(),
        )
    )
    return out


def reshape_and_cache(
    k: torch.Tensor,
    v: torch.Tensor,
    k_cache: torch.Tensor,
    v_cache: torch.Tensor,
    slot_mapping: torch.Tensor,
    shape: PkvShape,
) -> None:
    """Write the new tokens' K/V bits into the paged pools at their slots (in place)."""
    num_tokens = int(k.shape[0])
    _need_new_kv(k, v, num_tokens, shape)
    _need_pools(k_cache, v_cache, shape)
    _need(slot_mapping, num_tokens, "slot_mapping")
    check(
        lib().pkv_reshape_and_cache(
            _dev(k, "k", _16BIT),
            _dev(v, "v", _16BIT),
            _dev(k_cache, "k_cache", _16BIT),
            _dev(v_cache, "v_cache", _16BIT),
            _dev(slot_mapping, "slot_mapping", (torch.int64,)),
            num_tokens,
            ctypes.byref(shape),
            _stream(),
        )
    )


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, block_pairs: torch.Tensor, shape: PkvShape) -> None:
    """Copy physical blocks src -> dst in both pools (rows {src, dst} of int32 ``block_pairs``)."""
    _need_pools(k_cache, v_cache, shape)
    _need(block_pairs, 2 * int(block_pairs.shape[0]), "block_pairs")
    check(
        lib().pkv_copy_blocks(
            _dev(k_cache, "k_cache", _16BIT),
            _dev(v_cache, "v_cache", _16BIT),
            _dev(block_pairs, "block_pairs", (torch.int32,)),
            int(block_pairs.shape[0]),
            ctypes.byref(shape),
            _stream(),
        )
    )


def append_kv(
    k: torch.Tensor,
    v: torch.Tensor,
    k_cache: torch.Tensor,
    v_cache: torch.Tensor,
    block_tables: torch.Tensor,
    query_start_loc: torch.Tensor,
    context_lens: torch.Tensor,
    shape: PkvShape,
    slot_mapping: Optional[torch.Tensor] = None,
) -> Optional[torch.Tensor]:
    """Slot mapping and cache write in one launch; also fills ``slot_mapping`` when given."""
    _need_new_kv(k, v, int(k.shape[0]), shape)
    _need_pools(k_cache, v_cache, shape)
    _need_meta(block_tables, query_start_loc, context_lens, None, int(context_lens.numel()), shape)
    _need(slot_mapping, int(k.shape[0]), "slot_mapping")
    check(
        lib().pkv_append_kv(
            _opt(slot_mapping, "slot_mapping", (torch.int64,)),
            _dev(k, "k", _16BIT),
            _dev(v, "v", _16BIT),
            _dev(k_cache, "k_cache", _16BIT),
            _dev(v_cache, "v_cache", _16BIT),
            _dev(block_tables, "block_tables", (torch.int32,)),
            _dev(query_start_loc, "query_start_loc", (torch.int32,)),
            _dev(context_lens, "context_lens", (torch.int32,)),
            int(context_lens.numel()),
            int(k.shape[0]),
            ctypes.byref(shape),
            _stream(),
        )
    )
    return slot_mapping


def reshape_and_cache_fp8(
    k: torch.Tensor,
    v: torch.Tensor,
    k_cache: torch.Tensor,
    v_cache: torch.Tensor,
    k_scale: torch.Tensor,
    v_scale: torch.Tensor,
    slot_mapping: torch.Tensor,
    shape: PkvShape,
) -> None:
    """Quantise the new tokens' bf16 K/V to e4m3 under their blocks' scales (fp32
    [num_blocks, Hkv]) and write them into the fp8 pools at their slots (in place)."""
    _need_new_kv(k, v, int(k.shape[0]), shape)
    _need_pools(k_cache, v_cache, shape, k_scale, v_scale)
    _need(slot_mapping, int(k.shape[0]), "slot_mapping")
    check(
        lib().pkv_reshape_and_cache_fp8(
            _dev(k, "k", _16BIT),
            _dev(v, "v", _16BIT),
            _dev(k_cache, "k_cache", _FP8),
            _dev(v_cache, "v_cache", _FP8),
            _dev(k_scale, "k_scale", _F32),
            _dev(v_scale, "v_scale", _F32),
            _dev(slot_mapping, "slot_mapping", (torch.int64,)),
            int(k.shape[0]),
            ctypes.byref(shape),
            _stream(),
        )
    )


def append_kv_fp8(
    k: torch.Tensor,
    v: torch.Tensor,
    k_cache: torch.Tensor,
    v_cache: torch.Tensor,
    k_scale: torch.Tensor,
    v_scale: torch.Tensor,
    block_tables: torch.Tensor,
    query_start_loc: torch.Tensor,
    context_lens: torch.Tensor,
    shape: PkvShape,
    slot_mapping: Optional[torch.Tensor] = None,
) -> Optional[torch.Tensor]:
    """append_kv into fp8 pools: slot mapping and quantising cache write in one launch."""
    _need_new_kv(k, v, int(k.shape[0]), shape)
    _need_pools(k_cache, v_cache, shape, k_scale, v_scale)
    _need_meta(block_tables, query_start_loc, context_lens, None, int(context_lens.numel()), shape)
    _need(slot_mapping, int(k.shape[0]), "slot_mapping")
    check(
        lib().pkv_append_kv_fp8(
            _opt(slot_mapping, "slot_mapping", (torch.int64,)),
            _dev(k, "k", _16BIT),
            _dev(v, "v", _16BIT),
            _dev(k_cache, "k_cache", _FP8),
            _dev(v_cache, "v_cache", _FP8),
            _dev(k_scale, "k_scale", _F32),
            _dev(v_scale, "v_scale", _F32),
            _dev(block_tables, "block_tables", (torch.int32,)),
            _dev(query_start_loc, "query_start_loc", (torch.int32,)),
            _dev(context_lens, "context_lens", (torch.int32,)),
            int(context_lens.numel()),
            int(k.shape[0]),
            ctypes.byref(shape),
            _stream(),
        )
    )
    return slot_mapping


def copy_blocks_fp8(
    k_cache: torch.Tensor,
    v_cache: torch.Tensor,
    k_scale: torch.Tensor,
    v_scale: torch.Tensor,
    block_pairs: torch.Tensor,
    shape: PkvShape,
) -> None:
    """copy_blocks for fp8 pools: the blocks' bytes and their per-kv-head scales."""
    _need_pools(k_cache, v_cache, shape, k_scale, v_scale)
    _need(block_pairs, 2 * int(block_pairs.shape[0]), "block_pairs")
    check(
        lib().pkv_copy_blocks_fp8(
            _dev(k_cache, "k_cache", _FP8),
            _dev(v_cache, "v_cache", _FP8),
            _dev(k_scale, "k_scale", _F32),
            _dev(v_scale, "v_scale", _F32),
            _dev(block_pairs, "block_pairs", (torch.int32,)),
            int(block_pairs.shape[0]),
            ctypes.byref(shape),
            _stream(),
        )
    )


def varlen_workspace_size(num_seqs: int, num_tokens: int, max_seq_len: int, shape: PkvShape) -> int:
    return int(lib().pkv_varlen_workspace_size(num_seqs, num_tokens, max_seq_len, ctypes.byref(shape)))


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def plan_varlen(
    workspace: torch.Tensor,
    query_start_loc,
    context_lens,
    seq_lens,
    shape: PkvShape,
) -> PkvVarlenPlan:
    """Build the work list from host copies of the metadata and upload it into ``workspace``."""
    qsl = _host_i32(query_start_loc, "query_start_loc")
    ctx = _host_i32(context_lens, "context_lens")
    sl = _host_i32(seq_lens, "seq_lens")
    plan = PkvVarlenPlan()
    check(
        lib().pkv_plan_varlen(
            ctypes.byref(plan),
            _dev(workspace, "workspace", (torch.uint8,)),
            workspace.numel(),
            qsl.ctypes.data_as(ctypes.c_void_p),
            ctx.ctypes.data_as(ctypes.c_void_p),
            sl.ctypes.data_as(ctypes.c_void_p),
            int(ctx.shape[0]),
            int(qsl[-1]) if qsl.size else 0,
            ctypes.byref(shape),
            _stream(),
        )
    )
    return plan


def plan_varlen_host(query_start_loc, context_lens, seq_lens, shape: PkvShape) -> Tuple[PkvVarlenPlan, np.ndarray]:
    """Host-only planning (no device work): the plan summary and the work items [n, 8] int32."""
    qsl = _host_i32(query_start_loc, "query_start_loc")
    ctx = _host_i32(context_lens, "context_lens")
    sl = _host_i32(seq_lens, "seq_lens")
    plan = PkvVarlenPlan()
    args = (
        qsl.ctypes.data_as(ctypes.c_void_p),
        ctx.ctypes.data_as(ctypes.c_void_p),
        sl.ctypes.data_as(ctypes.c_void_p),
        int(ctx.shape[0]),
        int(qsl[-1]) if qsl.size else 0,
        ctypes.byref(shape),
    )
    check(lib().pkv_plan_varlen_host(ctypes.byref(plan), None, 0, *args))
    items = np.zeros((max(plan.num_items, 1), 8), dtype=np.int32)
    check(lib().pkv_plan_varlen_host(ctypes.byref(plan), items.ctypes.data_as(ctypes.c_void_p), items.shape[0], *args))
    return plan, items[: plan.num_items]


def paged_attention_varlen(
    q: torch.Tensor,
    k_cache: torch.Tensor,
    v_cache: torch.Tensor,
    block_tables: torch.Tensor,
    query_start_loc: torch.Tensor,
    context_lens: torch.Tensor,
    seq_lens: torch.Tensor,
    shape: PkvShape,
    plan: PkvVarlenPlan,
    workspace: torch.Tensor,
    out: Optional[torch.Tensor] = None,
    out_dtype: torch.dtype = torch.bfloat16,
    lse: Optional[torch.Tensor] = None,
) -> torch.Tensor:
    """Attention of every new token over its paged keys for a mixed decode/prefill batch."""
    num_tokens = int(q.shape[0])
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    _need_q_out(q, out, lse, num_tokens, shape)
    _need_pools(k_cache, v_cache, shape)
    _need_meta(block_tables, query_start_loc, context_lens, seq_lens, int(context_lens.numel()), shape)
    code = PKV_DTYPE_F32 if out.dtype == torch.float32 else PKV_DTYPE_BF16
    check(
        lib().pkv_paged_attention_varlen(
            _dev(out, "out", _16BIT + (torch.float32,)),
            code,
            _opt(lse, "lse", (torch.float32,)),
            _dev(q, "q", _16BIT),
            _dev(k_cache, "k_cache", _16BIT),
            _dev(v_cache, "v_cache", _16BIT),
            _dev(block_tables, "block_tables", (torch.int32,)),
            _dev(query_start_loc, "query_start_loc", (torch.int32,)),
            _dev(context_lens, "context_lens", (torch.int32,)),
            _dev(seq_lens, "seq_lens", (torch.int32,)),
            int(context_lens.numel()),
            num_tokens,
            ctypes.byref(shape),
            ctypes.byref(plan),
            _dev(workspace, "workspace", (torch.uint8,)),
            workspace.numel(),
            _stream(),
        )
    )
    return out


def paged_attention_varlen_fp8(
    q: torch.Tensor,
    k_cache: torch.Tensor,
    v_cache: torch.Tensor,
    k_scale: torch.Tensor,
    v_scale: torch.Tensor,
    block_tables: torch.Tensor,
    query_start_loc: torch.Tensor,
    context_lens: torch.Tensor,
    seq_lens: torch.Tensor,
    shape: PkvShape,
    plan: PkvVarlenPlan,
    workspace: torch.Tensor,
    out: Optional[torch.Tensor] = None,
    out_dtype: torch.dtype = torch.bfloat16,
    lse: Optional[torch.Tensor] = None,
) -> torch.Tensor:
    """paged_attention_varlen over fp8 (e4m3) pools with per-(block, kv head) scales."""
    num_tokens = int(q.shape[0])
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    _need_q_out(q, out, lse, num_tokens, shape)
    _need_pools(k_cache, v_cache, shape, k_scale, v_scale)
    _need_meta(block_tables, query_start_loc, context_lens, seq_lens, int(context_lens.numel()), shape)
    code = PKV_DTYPE_F32 if out.dtype == torch.float32 else PKV_DTYPE_BF16
    check(
        lib().pkv_paged_attention_varlen_fp8(
            _dev(out, "out", _16BIT + (torch.float32,)),
            code,
            _opt(lse, "lse", (torch.float32,)),
            _dev(q, "q", _16BIT),
            _dev(k_cache, "k_cache", _FP8),
            _dev(v_cache, "v_cache", _FP8),
            _dev(k_scale, "k_scale", _F32),
            _dev(v_scale, "v_scale", _F32),
            _dev(block_tables, "block_tables", (torch.int32,)),
            _dev(query_start_loc, "query_start_loc", (torch.int32,)),
            _dev(context_lens, "context_lens", (torch.int32,)),
            _dev(seq_lens, "seq_lens", (torch.int32,)),
            int(context_lens.numel()),
            num_tokens,
            ctypes.byref(shape),
            ctypes.byref(plan),
            _dev(workspace, "workspace", (torch.uint8,)),
            workspace.numel(),
            _stream(),
        )
    )
    return out


def decode_workspace_size(num_seqs: int, max_seq_len: int, shape: PkvShape) -> int:
    return int(lib().pkv_decode_workspace_size(num_seqs, max_seq_len, ctypes.byref(shape)))


def paged_attention_decode(
    q: torch.Tensor,
    k_cache: torch.Tensor,
    v_cache: torch.Tensor,
    block_tables: torch.Tensor,
    query_start_loc: torch.Tensor,
    seq_lens: torch.Tensor,
    shape: PkvShape,
    max_seq_len: int,
    workspace: Optional[torch.Tensor] = None,
    out: Optional[torch.Tensor] = None,
    out_dtype: torch.dtype = torch.bfloat16,
    lse: Optional[torch.Tensor] = None,
    k_scale: Optional[torch.Tensor] = None,
    v_scale: Optional[torch.Tensor] = None,
) -> torch.Tensor:
    """Decode attention (one query token per row) with the work split on the device: the
    launches depend only on (rows, max_seq_len), so the call can be captured in a graph and
    replayed with new metadata in the same buffers.  With k_scale / v_scale the pools are fp8."""
    num_seqs = int(seq_lens.numel())
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    code = PKV_DTYPE_F32 if out.dtype == torch.float32 else PKV_DTYPE_BF16
    _need_q_out(q, out, lse, num_seqs, shape)
    _need_pools(k_cache, v_cache, shape, k_scale, v_scale)
    _need_meta(block_tables, query_start_loc, None, seq_lens, num_seqs, shape)
    ws = workspace
    common = (
        _dev(block_tables, "block_tables", (torch.int32,)),
        _dev(query_start_loc, "query_start_loc", (torch.int32,)),
        _dev(seq_lens, "seq_lens", (torch.int32,)),
        num_seqs,
        int(max_seq_len),
        ctypes.byref(shape),
        _opt(ws, "workspace", (torch.uint8,)),
        0 if ws is None else ws.numel(),
        _stream(),
    )
    head = (_dev(out, "out", _16BIT + (torch.float32,)), code, _opt(lse, "lse", (torch.float32,)), _dev(q, "q", _16BIT))
    if k_scale is None:
        check(lib().pkv_paged_attention_decode(
            *head, _dev(k_cache, "k_cache", _16BIT), _dev(v_cache, "v_cache", _16BIT), *common))
    else:
        check(lib().pkv_paged_attention_decode_fp8(
            *head, _dev(k_cache, "k_cache", _FP8), _dev(v_cache, "v_cache", _FP8),
            _dev(k_scale, "k_scale", _F32), _dev(v_scale, "v_scale", _F32), *common))
    return out


def paged_attention_decode_noalloc(
    q: torch.Tensor,
    k_cache: torch.Tensor,
    v_cache: torch.Tensor,
    block_tables: torch.Tensor,
    query_start_loc: torch.Tensor,
    seq_lens: torch.Tensor,
    shape: PkvShape,
    max_seq_len: int,
    out: torch.Tensor,
    lse: Optional[torch.Tensor] = None,
) -> torch.Tensor:
    """paged_attention_decode with its partial states in the library's device scratch: no
    workspace, and (with ``out`` given) nothing allocated, so it can be called where allocation
    is not allowed.  Calls that may overlap on one GPU race on the shared scratch."""
    num_seqs = int(seq_lens.numel())
    code = PKV_DTYPE_F32 if out.dtype == torch.float32 else PKV_DTYPE_BF16
    _need_q_out(q, out, lse, num_seqs, shape)
    _need_pools(k_cache, v_cache, shape)
    _need_meta(block_tables, query_start_loc, None, seq_lens, num_seqs, shape)
    check(
        lib().pkv_paged_attention_decode_noalloc(
            _dev(out, "out", _16BIT + (torch.float32,)),
            code,
            _opt(lse, "lse", (torch.float32,)),
            _dev(q, "q", _16BIT),
            _dev(k_cache, "k_cache", _16BIT),
            _dev(v_cache, "v_cache", _16BIT),
            _dev(block_tables, "block_tables", (torch.int32,)),
            _dev(query_start_loc, "query_start_loc", (torch.int32,)),
            _dev(seq_lens, "seq_lens", (torch.int32,)),
            num_seqs,
            int(max_seq_len),
            ctypes.byref(shape),
            _stream(),
        )
    )
    return out


def cascade_workspace_size(num_tokens: int, prefix_len: int, shape: PkvShape) -> int:
    return int(lib().pkv_cascade_workspace_size(num_tokens, prefix_len, ctypes.byref(shape)))


def cascade_prefix_attention(
    q: torch.Tensor,
    k_cache: torch.Tensor,
    v_cache: torch.Tensor,
    prefix_block_table: torch.Tensor,
    prefix_len: int,
    shape: PkvShape,
    workspace: Optional[torch.Tensor] = None,
    out: Optional[torch.Tensor] = None,
    lse: Optional[torch.Tensor] = None,
) -> Tuple[torch.Tensor, torch.Tensor]:
    """State (fp32 output, LSE) of every query over the shared prefix keys."""
    T, Hq = int(q.shape[0]), int(q.shape[1])
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    _need_q_out(q, out, lse, T, shape)
    _need(prefix_block_table, int(prefix_len) // max(int(shape.block_size), 1), "prefix_block_table")
    _need_pools(k_cache, v_cache, shape)
    ws = workspace
    check(
        lib().pkv_cascade_prefix_attention(
            _dev(out, "out_prefix", (torch.float32,)),
            _dev(lse, "lse_prefix", (torch.float32,)),
            _dev(q, "q", _16BIT),
            _dev(k_cache, "k_cache", _16BIT),
            _dev(v_cache, "v_cache", _16BIT),
            _dev(prefix_block_table, "prefix_block_table", (torch.int32,)),
            int(prefix_len),
            T,
            ctypes.byref(shape),
            _opt(ws, "workspace", (torch.uint8,)),
            0 if ws is None else ws.numel(),
            _stream(),
        )
    )
    return out, lse


def cascade_prefix_attention_fp8(
    q: torch.Tensor,
    k_cache: torch.Tensor,
    v_cache: torch.Tensor,
    k_scale: torch.Tensor,
    v_scale: torch.Tensor,
    prefix_block_table: torch.Tensor,
    prefix_len: int,
    shape: PkvShape,
    workspace: Optional[torch.Tensor] = None,
    out: Optional[torch.Tensor] = None,
    lse: Optional[torch.Tensor] = None,
) -> Tuple[torch.Tensor, torch.Tensor]:
    """cascade_prefix_attention over fp8 (e4m3) pools with per-(block, kv head) scales."""
    T, Hq = int(q.shape[0]), int(q.shape[1])
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    _need_q_out(q, out, lse, T, shape)
    _need(prefix_block_table, int(prefix_len) // max(int(shape.block_size), 1), "prefix_block_table")
    _need_pools(k_cache, v_cache, shape, k_scale, v_scale)
    ws = workspace
    check(
        lib().pkv_cascade_prefix_attention_fp8(
            _dev(out, "out_prefix", (torch.float32,)),
            _dev(lse, "lse_prefix", (torch.float32,)),
            _dev(q, "q", _16BIT),
            _dev(k_cache, "k_cache", _FP8),
            _dev(v_cache, "v_cache", _FP8),
            _dev(k_scale, "k_scale", _F32),
            _dev(v_scale, "v_scale", _F32),
            _dev(prefix_block_table, "prefix_block_table", (torch.int32,)),
            int(prefix_len),
            T,
            ctypes.byref(shape),
            _opt(ws, "workspace", (torch.uint8,)),
            0 if ws is None else ws.numel(),
            _stream(),
        )
    )
    return out, lse


def merge_attn_states(
    out_a: torch.Tensor,
    lse_a: torch.Tensor,
    out_b: torch.Tensor,
    lse_b: torch.Tensor,
    out: Optional[torch.Tensor] = None,
    out_dtype: torch.dtype = torch.bfloat16,
    lse_out: Optional[torch.Tensor] = None,
) -> torch.Tensor:
    """Merge two attention states over disjoint key sets into the state of their union."""
    T, H, D = (int(x) for x in out_a.shape)
    if out is None:
        out = torch.empty((T, H, D), dtype=out_dtype, device=out_a.device)
    code = PKV_DTYPE_F32 if out.dtype == torch.float32 else PKV_DTYPE_BF16
    for t, nm, n in ((out, "out", T * H * D), (out_b, "out_b", T * H * D), (lse_a, "lse_a", T * H),
                     (lse_b, "lse_b", T * H), (lse_out, "lse_out", T * H)):
        _need(t, n, nm)
    check(
        lib().pkv_merge_attn_states(
            _dev(out, "out", _16BIT + (torch.float32,)),
            code,
            _opt(lse_out, "lse_out", (torch.float32,)),
            _dev(out_a, "out_a", (torch.float32,)),
            _dev(lse_a, "lse_a", (torch.float32,)),
            _dev(out_b, "out_b", (torch.float32,)),
            _dev(lse_b, "lse_b", (torch.float32,)),
            T,
            H,
            D,
            _stream(),
        )
    )
    return out


def timing_begin() -> None:
    """Start bracketing every varlen attention kernel launch with HIP events (this thread)."""
    check(lib().pkv_timing_begin())


def timing_end() -> Tuple[float, int]:
    """Stop timing; return (summed kernel milliseconds, number of timed launches)."""
    ms = ctypes.c_double()
    n = ctypes.c_int32()
    check(lib().pkv_timing_end(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def timing_durations() -> np.ndarray:
    """Per-launch kernel milliseconds of the window the last timing_end() closed."""
    n = lib().pkv_timing_durations(None, 0)
    check(min(n, 0))
    buf = np.zeros(max(n, 1), dtype=np.float64)
    got = lib().pkv_timing_durations(buf.ctypes.data_as(ctypes.c_void_p), n)
    check(min(got, 0))
    return buf[:n]
