"""CPU fp64 oracle for paged-KV attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package.  The product path (the HIP
library and its Python binding) never imports, calls or links it.

Pins: every function here is checked in ``tests/test_oracle_pins.py`` and
``tests/test_oracle_fp8_pins.py`` against closed forms, page values, a
separately written dense attention, torch's fp64 scaled-dot-product attention,
50-digit brute force, and exact rational nearest-value search for the FP8
format.  No function is "parity unpinned".
"""

from .paged_attention import (  # noqa: F401
    attention_state,
    bf16_to_f64,
    cascade_prefix_attention,
    causal_visible,
    copy_blocks,
    default_scale,
    gather_keys,
    gather_values,
    merge_attn_states,
    paged_attention,
    reshape_and_cache,
    slot_mapping,
    token_positions,
)
from .kv_fp8 import (  # noqa: F401
    cascade_prefix_attention_fp8,
    dequantize_keys,
    dequantize_values,
    e4m3_decode,
    e4m3_encode,
    paged_attention_fp8,
    quantize,
    reshape_and_cache_fp8,
)
