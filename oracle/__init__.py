"""CPU fp64 oracle for one grouped-query attention step with RoPE over a KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code, constants
or helpers with the HIP library in ``gqa_attention_rope_amd/``.

Parity status of each function is stated in the module docstring of
``gqa_oracle``: every function is pinned to something other than itself.
"""

from .gqa_oracle import (  # noqa: F401
    visible_rows,
    bf16_to_f64,
    f64_to_bf16,
    rope_frequencies,
    llama3_scaled_frequencies,
    yarn_frequencies,
    rope_attention_factor,
    rotate_pairs,
    rope_rotate,
    rope_append,
    attend,
    attend_bruteforce,
    kv_cache_bytes,
)
