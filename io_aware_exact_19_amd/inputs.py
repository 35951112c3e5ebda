"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random numbers and packs them; it holds none of the
attention arithmetic.  Recipe (the pages print no data, so every workload is
synthetic):

* values are i.i.d. N(0, 1): ``torch.randn`` in float32 from a
  ``torch.Generator`` seeded with a per-tensor sub-seed, then rounded to
  bfloat16 (round-to-nearest-even) when the workload is bf16;
* "peaked" runs multiply the rounded Q by 4 (a power of two, so exact);
* sequence lengths are integers drawn uniformly from [lo, hi] inclusive with
  ``torch.randint`` from their own sub-seed;
* e4m3 workloads draw the same fp32 N(0, 1) values, pick one factor per
  (batch, head) block of a tensor, amax / 448 (448 is the largest finite e4m3
  value), and store round-to-nearest-even e4m3 codes of value / factor
  (torch's float8_e4m3fn conversion); the factor is the block's
  dequantisation factor;
* KV caches too large for host memory are generated on the device, one
  sub-seed per sequence, and rows past each sequence's length are filled with
  NaN so that a read of padding shows up in the output.
"""

from __future__ import annotations

import torch

_STREAM = {"q": 1, "k": 2, "v": 3, "lengths": 4, "dout": 5}


def subseed(seed: int, name: str, index: int = 0) -> int:
    """Independent seed per (workload seed, tensor name, sequence index)."""
    return (int(seed) * 16 + _STREAM[name]) * 1_000_003 + int(index)


def normal(shape, seed: int, dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """i.i.d. N(0,1) drawn in float32 on ``device`` and rounded to ``dtype``."""
    g = torch.Generator(device=device).manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device)
    return x.to(dtype)


def lengths(n: int, lo: int, hi: int, seed: int) -> torch.Tensor:
    """n integer lengths uniform on [lo, hi] (inclusive), int64, on the CPU."""
    g = torch.Generator().manual_seed(subseed(seed, "lengths"))
    return torch.randint(lo, hi + 1, (n,), generator=g, dtype=torch.int64)


def cu_seqlens(lens) -> torch.Tensor:
    """Packing offsets [0, l0, l0+l1, ...] as int32."""
    lens = torch.as_tensor(lens, dtype=torch.int64)
    out = torch.zeros(lens.numel() + 1, dtype=torch.int64)
    out[1:] = torch.cumsum(lens, 0)
    return out.to(torch.int32)


def dense_qkv(batch, seq_q, seq_k, heads, d, seed, dtype=torch.bfloat16, q_mult=1.0):
    """Q [B, seq_q, H, d], K/V [B, seq_k, H, d] on the CPU."""
    q = normal((batch, seq_q, heads, d), subseed(seed, "q"), dtype)
    k = normal((batch, seq_k, heads, d), subseed(seed, "k"), dtype)
    v = normal((batch, seq_k, heads, d), subseed(seed, "v"), dtype)
    if q_mult != 1.0:
        q = q * q_mult
    return q, k, v


def varlen_qkv(lens, heads, d, seed, dtype=torch.bfloat16):
    """Packed Q/K/V [sum(lens), H, d] (self-attention: same lengths for Q and K)."""
    total = int(torch.as_tensor(lens).sum())
    q = normal((total, heads, d), subseed(seed, "q"), dtype)
    k = normal((total, heads, d), subseed(seed, "k"), dtype)
    v = normal((total, heads, d), subseed(seed, "v"), dtype)
    return q, k, v


def varlen_qkv_pair(lens_q, lens_k, heads, d, seed, dtype=torch.bfloat16):
    """Packed Q [sum(lens_q), H, d] and K/V [sum(lens_k), H, d]: sequence i
    has lens_q[i] queries and lens_k[i] keys (cross-length packing)."""
    tq = int(torch.as_tensor(lens_q).sum())
    tk = int(torch.as_tensor(lens_k).sum())
    q = normal((tq, heads, d), subseed(seed, "q"), dtype)
    k = normal((tk, heads, d), subseed(seed, "k"), dtype)
    v = normal((tk, heads, d), subseed(seed, "v"), dtype)
    return q, k, v


def decode_cache(batch, max_len, heads, d, seqlens, seed, device, name, dtype=torch.bfloat16,
                 pad=float("nan")):
    """KV cache [B, max_len, H, d]: sequence b's first seqlens[b] rows drawn
    N(0,1) from sub-seed (seed, name, b); the remaining rows set to ``pad``."""
    cache = torch.empty((batch, max_len, heads, d), dtype=dtype, device=device)
    for b in range(batch):
        n = int(seqlens[b])
        cache[b, :n] = normal((n, heads, d), subseed(seed, name, b), dtype, device)
        if n < max_len:
            cache[b, n:] = pad
    return cache


def fp8_tensor(shape, seed: int, mult: float = 1.0, device="cpu"):
    """e4m3 codes (uint8 [B, n, H, d]) and per-(batch, head) dequantisation
    factors (float32 [B * H]) of i.i.d. N(0,1) values times ``mult``, drawn
    on ``device``."""
    x = normal(shape, seed, torch.float32, device) * mult
    B, _, H, _ = x.shape
    amax = x.abs().amax(dim=(1, 3))  # [B, H]
    ds = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    codes = (x / ds[:, None, :, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), ds.reshape(-1).contiguous()


def fp8_qkv(B, n_q, n_k, H, d, seed, q_mult: float = 1.0):
    """(q8, k8, v8, descale_q, descale_k, descale_v) on the CPU."""
    q8, dq = fp8_tensor((B, n_q, H, d), subseed(seed, "q"), q_mult)
    k8, dk = fp8_tensor((B, n_k, H, d), subseed(seed, "k"))
    v8, dv = fp8_tensor((B, n_k, H, d), subseed(seed, "v"))
    return q8, k8, v8, dq, dk, dv
