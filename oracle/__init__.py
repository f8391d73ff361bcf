"""fp64 CPU oracle for attention over a paged, block-table-indexed KV cache.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link this package: only
the tests, the smoke check and the benchmark's CPU-baseline leg use it. It shares no code with the HIP
library (no kernels, headers, helpers or constant tables); the two meet only at the seeded input
generators in ``workloads``.

Everything here is the plain definition, in float64, with no tiling, no blocking and no fusion.
bf16 inputs are widened exactly (bf16 -> f32 -> f64). Every function cites the passage it follows.
"""
from .attention import (  # noqa: F401
    kv_head_of,
    key_visible,
    gather_tokens,
    attend_rows,
    paged_decode,
    paged_decode_pairs,
    decode_partials,
    merge_partials,
    ragged_prefill,
    ragged_prefill_rows,
    paged_prefill,
    paged_prefill_rows,
    reshape_and_cache,
    validate_block_tables,
    STATUS,
)
from .blocks import copy_blocks, swap_blocks  # noqa: F401,E402
from .fp8 import (  # noqa: F401,E402
    e4m3_value, e4m3_decode, e4m3_encode, quantize, dequantize, reshape_and_cache_fp8, paged_decode_fp8,
)
from .stream import paged_decode_window, streamed_decode  # noqa: F401,E402
