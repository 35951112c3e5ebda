"""MI355X (gfx950) attention forward: tiled prefill with online softmax,
packed variable-length prefill and split-KV decode, behind the C ABI of
libfa.so (include/fa.h).  This package is the thin Python binding plus the
build script, the seeded input generators and the workload table."""

from .binding import (  # noqa: F401
    EXPORTED,
    FA_ERR_INVALID_ARG,
    FA_ERR_LAUNCH,
    FA_ERR_UNSUPPORTED,
    FA_DECODE_SCRATCH_BYTES,
    FA_ERR_WORKSPACE,
    FA_OK,
    LIB_PATH,
    FAError,
    attention,
    attention_backward,
    attention_fp8,
    attention_kvcache,
    attention_varlen,
    decode,
    fa_bwd,
    fa_bwd_workspace_size,
    fa_decode,
    fa_decode_noalloc,
    fa_decode_workspace_size,
    fa_fwd,
    fa_fwd_fp32,
    fa_fwd_fp8,
    fa_fwd_kvcache,
    fa_status_string,
    load_library,
)
