"""The five synthetic workloads, by name and size.

Shapes follow the pages' workload kinds: a small single-head check, a
medium prefill batch, an 8000-token prompt ("How FlashAttention accelerates
Transformer attention with IO-aware tiling" (wiblog.cn), section "Why the
intermediate matrices slow standard attention"), a packed batch of mixed
prompt lengths (its section "Is it worth enabling", short/medium/long
groups) and token-by-token decode against a KV cache (its section
"Training, prefill and decode", table 1).
"""

from __future__ import annotations

import math

SMALL_FP32 = dict(name="dense_fp32_b1_h1_n256_d64", kind="dense", dtype="f32", batch=1,
                  heads=1, seqlen=256, d=64, causal=False, window_left=-1, seed=11)
PREFILL_2K = dict(name="dense_bf16_b4_h16_n2048_d128", kind="dense", dtype="bf16", batch=4,
                  heads=16, seqlen=2048, d=128, causal=False, window_left=-1, seed=22)
LONG_8K = dict(name="dense_bf16_b1_h32_n8000_d128_causal", kind="dense", dtype="bf16",
               batch=1, heads=32, seqlen=8000, d=128, causal=True, window_left=-1, seed=33)
VARLEN = dict(name="varlen_bf16_16seq_128to4096_h16_d64_causal_w1024", kind="varlen",
              dtype="bf16", nseq=16, len_lo=128, len_hi=4096, heads=16, d=64, causal=True,
              window_left=1024, seed=44)
DECODE = dict(name="decode_bf16_b64_h32_len1024to32768_d128_chunk256", kind="decode",
              dtype="bf16", batch=64, heads=32, len_lo=1024, len_hi=32768, max_len=32768,
              d=128, chunk=256, seed=55)

ALL = [SMALL_FP32, PREFILL_2K, LONG_8K, VARLEN, DECODE]

# Chunked prefill against a KV cache (several new tokens per sequence): a
# synthetic workload of the next step after single-token decode, not one of
# the five configurations above.
KVCACHE = dict(name="kvcache_bf16_b8_h32_new512_len1024to16384_d128_causal", kind="kvcache",
               dtype="bf16", batch=8, heads=32, n_new=512, len_lo=1024, len_hi=16384,
               max_len=16384, d=128, causal=True, seed=66)


def default_scale(d: int) -> float:
    """1 / sqrt(d), the scale of the attention definition."""
    return 1.0 / math.sqrt(d)
