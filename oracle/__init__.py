"""fp64 CPU oracle for exact attention -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library.
"""

from .attention import (  # noqa: F401
    allowed_mask,
    attention_decode,
    attention_backward,
    attention_dense,
    attention_flops,
    attention_fp8,
    attention_kvcache,
    attention_varlen,
    e4m3_decode,
    merge_states,
    online_attention,
    sdpa,
    sdpa_backward,
)
