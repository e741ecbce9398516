"""ctypes binding of libpkv.so (argument marshalling only).

Every function here forwards device pointers, sizes and the current HIP stream to one C entry
point of ``include/pkv.h``; no attention arithmetic happens in Python.  There is no fallback:
if the shared library is missing or fails to load, every call raises.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpkv.so")

PKV_DTYPE_BF16 = 0
PKV_DTYPE_F32 = 1

# Entry points declared in include/pkv.h (kept in sync by tests/test_abi.py).
PKV_DECODE_SCRATCH_BYTES = 32 << 20  # device scratch of pkv_paged_attention_decode_noalloc

EXPORTS = (
    "pkv_varlen_workspace_size",
    "pkv_compute_slot_mapping",
    "pkv_reshape_and_cache",
    "pkv_append_kv",
    "pkv_reshape_and_cache_fp8",
    "pkv_append_kv_fp8",
    "pkv_copy_blocks",
    "pkv_copy_blocks_fp8",
    "pkv_plan_varlen",
    "pkv_plan_varlen_host",
    "pkv_paged_attention_varlen",
    "pkv_paged_attention_varlen_fp8",
    "pkv_decode_workspace_size",
    "pkv_paged_attention_decode",
    "pkv_paged_attention_decode_noalloc",
    "pkv_paged_attention_decode_fp8",
    "pkv_cascade_workspace_size",
    "pkv_cascade_prefix_attention",
    "pkv_cascade_prefix_attention_fp8",
    "pkv_merge_attn_states",
    "pkv_timing_begin",
    "pkv_timing_end",
    "pkv_timing_durations",
    "pkv_last_error",
    "pkv_version",
)


class PkvShape(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("bt_stride", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


class PkvVarlenPlan(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_tokens", ctypes.c_int32),
        ("num_items", ctypes.c_int32),
        ("num_prefill_items", ctypes.c_int32),
        ("num_decode_items", ctypes.c_int32),
        ("num_partials", ctypes.c_int32),
        ("blocks_per_split", ctypes.c_int32),
        ("has_splits", ctypes.c_int32),
        ("workspace_used", ctypes.c_int64),
        ("head_dim", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("tile_rows", ctypes.c_int32),
        ("num_short_items", ctypes.c_int32),
        ("decode_waves", ctypes.c_int32),
    ]


class PkvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libpkv error {code}: {msg}")
        self.code = code


_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_SHAPE = ctypes.POINTER(PkvShape)
_PLAN = ctypes.POINTER(PkvVarlenPlan)

_SIGS = {
    "pkv_varlen_workspace_size": (_SZ, [_I32, _I32, _I32, _SHAPE]),
    "pkv_compute_slot_mapping": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I32, _SHAPE, _P]),
    "pkv_reshape_and_cache": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _SHAPE, _P]),
    "pkv_append_kv": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _SHAPE, _P]),
    "pkv_reshape_and_cache_fp8": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _SHAPE, _P]),
    "pkv_append_kv_fp8": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _SHAPE, _P]),
    "pkv_copy_blocks": (ctypes.c_int, [_P, _P, _P, _I32, _SHAPE, _P]),
    "pkv_copy_blocks_fp8": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _SHAPE, _P]),
    "pkv_plan_varlen": (ctypes.c_int, [_PLAN, _P, _SZ, _P, _P, _P, _I32, _I32, _SHAPE, _P]),
    "pkv_plan_varlen_host": (ctypes.c_int, [_PLAN, _P, _I32, _P, _P, _P, _I32, _I32, _SHAPE]),
    "pkv_paged_attention_varlen": (
        ctypes.c_int,
        [_P, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _SHAPE, _PLAN, _P, _SZ, _P],
    ),
    "pkv_paged_attention_varlen_fp8": (
        ctypes.c_int,
        [_P, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _SHAPE, _PLAN, _P, _SZ, _P],
    ),
    "pkv_decode_workspace_size": (_SZ, [_I32, _I32, _SHAPE]),
    "pkv_paged_attention_decode": (
        ctypes.c_int,
        [_P, _I32, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _SHAPE, _P, _SZ, _P],
    ),
    "pkv_paged_attention_decode_noalloc": (
        ctypes.c_int,
        [_P, _I32, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _SHAPE, _P],
    ),
    "pkv_paged_attention_decode_fp8": (
        ctypes.c_int,
        [_P, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _SHAPE, _P, _SZ, _P],
    ),
    "pkv_cascade_workspace_size": (_SZ, [_I32, _I32, _SHAPE]),
    "pkv_cascade_prefix_attention": (
        ctypes.c_int,
        [_P, _P, _P, _P, _P, _P, _I32, _I32, _SHAPE, _P, _SZ, _P],
    ),
    "pkv_cascade_prefix_attention_fp8": (
        ctypes.c_int,
        [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _SHAPE, _P, _SZ, _P],
    ),
    "pkv_merge_attn_states": (ctypes.c_int, [_P, _I32, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P]),
    "pkv_timing_begin": (ctypes.c_int, []),
    "pkv_timing_end": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)]),
    "pkv_timing_durations": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]),
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_version": (ctypes.c_char_p, []),
}


def lib() -> ctypes.CDLL:
    """Load libpkv.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_285_amd.build` "
                "(there is no non-HIP fallback)"
            )
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def check(rc: int) -> None:
    if rc != 0:
        raise PkvError(rc, lib().pkv_last_error().decode())
