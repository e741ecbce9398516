"""Attention over a paged KV cache on AMD MI355X (gfx950): HIP kernels behind a C ABI.

The compute path lives in ``libpkv.so`` (built from ``csrc/`` by ``build.py``); this package
is its thin Python binding.  Importing it does not load the library; the first call does, and
raises if the library has not been built.
"""

from ._lib import (  # noqa: F401
    PKV_DECODE_SCRATCH_BYTES,
    PKV_DTYPE_BF16,
    PKV_DTYPE_F32,
    PkvError,
    PkvShape,
    PkvVarlenPlan,
    lib,
)
from .ops import (  # noqa: F401
    alloc_workspace,
    append_kv,
    append_kv_fp8,
    cascade_prefix_attention,
    cascade_prefix_attention_fp8,
    cascade_workspace_size,
    compute_slot_mapping,
    copy_blocks,
    copy_blocks_fp8,
    decode_workspace_size,
    make_shape,
    merge_attn_states,
    paged_attention_decode,
    paged_attention_decode_noalloc,
    paged_attention_varlen,
    paged_attention_varlen_fp8,
    plan_varlen,
    plan_varlen_host,
    reshape_and_cache,
    reshape_and_cache_fp8,
    timing_begin,
    timing_durations,
    timing_end,
    varlen_workspace_size,
    version,
)
