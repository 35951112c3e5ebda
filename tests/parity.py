"""Comparison helpers for GPU-vs-oracle parity (element by element).

Tolerances for the outputs (against the fp64 oracle on the same inputs):
bf16 output max-abs <= 2e-2 and mean-abs <= 2e-3; fp32 output max-abs <= 1e-5;
lse abs <= 1e-3 everywhere.  Rows whose oracle lse is -inf (no allowed key)
must come back as O = 0 and lse = -inf exactly.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
FP32_MAX_ABS = 1e-5
LSE_ABS = 1e-3


def to_f64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().float().cpu().double().numpy()
    return np.asarray(t, dtype=np.float64)


def bf16_floor(o_ref):
    """Error of the oracle's own output rounded to bf16: what any bf16 output
    must carry at least."""
    r = torch.from_numpy(np.asarray(o_ref)).to(torch.bfloat16).double().numpy()
    e = np.abs(r - o_ref)
    return float(e.max()), float(e.mean())


def check(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what):
    o = to_f64(o_gpu)
    assert o.shape == o_ref.shape, f"{what}: shape {o.shape} vs {o_ref.shape}"
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    err = np.abs(o - o_ref)
    max_abs, mean_abs = float(err.max()), float(err.mean())
    msg = f"[parity] {what}: O max-abs {max_abs:.3e} mean-abs {mean_abs:.3e}"
    if dtype == torch.bfloat16:
        fmax, fmean = bf16_floor(o_ref)
        msg += f" (bf16 rounding floor max {fmax:.3e} mean {fmean:.3e})"
    if lse_gpu is not None:
        lse = to_f64(lse_gpu)
        assert lse.shape == lse_ref.shape, f"{what}: lse shape {lse.shape} vs {lse_ref.shape}"
        empty = np.isneginf(lse_ref)
        assert np.array_equal(np.isneginf(lse), empty), f"{what}: -inf rows differ"
        live = ~empty
        lerr = float(np.abs(lse[live] - lse_ref[live]).max()) if live.any() else 0.0
        msg += f"; lse max-abs {lerr:.3e}"
        assert lerr <= LSE_ABS, f"{what}: lse error {lerr:.3e} > {LSE_ABS}"
    print(msg, file=sys.stderr, flush=True)
    if dtype == torch.bfloat16:
        assert max_abs <= BF16_MAX_ABS, f"{what}: max-abs {max_abs:.3e} > {BF16_MAX_ABS}"
        assert mean_abs <= BF16_MEAN_ABS, f"{what}: mean-abs {mean_abs:.3e} > {BF16_MEAN_ABS}"
    else:
        assert max_abs <= FP32_MAX_ABS, f"{what}: max-abs {max_abs:.3e} > {FP32_MAX_ABS}"
    return max_abs, mean_abs


def announce(what):
    """Name the case before a GPU step, flushed, so a crash still names it."""
    print(f"[gpu-case] {what}", file=sys.stderr, flush=True)
