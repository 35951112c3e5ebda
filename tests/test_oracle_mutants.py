"""Planted mistakes, on the CPU: each variant below is the one-head oracle
with one plausible error (a dropped term, a wrong sign or index, a swapped
operand).  The pin battery must reject every one of them, which shows the pins
can catch that class of mistake in the oracle itself."""

import numpy as np
import pytest

import oracle
from tests import oracle_pins


def _mutant(kind):
    def impl(q, k, v, scale, causal=False, window_left=-1):
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        n_q, n_k = q.shape[0], k.shape[0]
        s = (q @ k.T) if kind == "no_scale" else scale * (q @ k.T)
        if kind == "scale_sqrt":
            s = np.sqrt(scale) * (q @ k.T)
        i = np.arange(n_q)[:, None]
        j = np.arange(n_k)[None, :]
        delta = n_k - n_q
        if kind == "top_left_causal":
            delta = 0
        ok = np.ones((n_q, n_k), dtype=bool)
        if causal and kind != "mask_ignored":
            ok &= (j < i + delta) if kind == "causal_excludes_diag" else (j <= i + delta)
        if window_left >= 0 and kind != "mask_ignored":
            if kind == "window_off_by_one":
                ok &= j > i + delta - window_left
            else:
                ok &= j >= i + delta - window_left
        s = np.where(ok, s, -np.inf)
        o = np.zeros((n_q, v.shape[1]))
        lse = np.full(n_q, -np.inf)
        live = ok.any(axis=1)
        s = s[live]
        if kind == "column_softmax":
            m = s.max(axis=0, keepdims=True)
            e = np.exp(s - m)
            p = e / e.sum(axis=0, keepdims=True)
            o[live] = np.nan_to_num(p) @ v
            lse[live] = (m.max() + np.log(e.sum(axis=1)))
            return o, lse
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        l = e.sum(axis=1)
        p = e / l[:, None]
        o[live] = (p @ k) if kind == "k_for_v" else (p @ v)
        if kind == "lse_no_max":
            lse[live] = np.log(l)
        elif kind == "lse_log2":
            lse[live] = m + np.log2(l)
        else:
            lse[live] = m + np.log(l)
        if kind == "no_normalise":
            o[live] = e @ v
        return o, lse

    return impl


MUTANTS = [
    "no_scale",
    "scale_sqrt",
    "top_left_causal",
    "causal_excludes_diag",
    "mask_ignored",
    "window_off_by_one",
    "column_softmax",
    "k_for_v",
    "lse_no_max",
    "lse_log2",
    "no_normalise",
]


def _fails_some_pin(impl):
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(impl)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    return caught


def test_unmutated_copy_passes():
    """The harness itself: the copy with no mistake passes every pin."""
    assert _fails_some_pin(_mutant("none")) == []


@pytest.mark.parametrize("kind", MUTANTS)
def test_each_planted_mistake_is_caught(kind):
    caught = _fails_some_pin(_mutant(kind))
    assert caught, f"mutant {kind} passed every pin"


def test_oracle_is_not_a_mutant():
    assert _fails_some_pin(lambda q, k, v, s, c, w: oracle.sdpa(q, k, v, s, c, w)) == []
