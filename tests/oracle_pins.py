"""Pins that tie a one-head attention implementation to facts the pages and
the mathematics fix, independent of the implementation itself.

Every ``pin_*`` takes ``impl(q, k, v, scale, causal, window_left) -> (o, lse)``
(one head, q [n_q, d], k/v [n_k, d], fp64 results) and raises AssertionError
when the implementation disagrees.  The oracle must pass all of them; each
planted mistake in ``test_oracle_mutants.py`` must fail at least one.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TIGHT = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol=TIGHT, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    err = np.where(same_inf, 0.0, np.abs(a - b))
    assert np.all(np.isfinite(err)), f"{what}: non-finite mismatch"
    scale = np.maximum(1.0, np.abs(np.where(same_inf, 0.0, b)))
    worst = float(np.max(err / scale)) if err.size else 0.0
    assert worst <= tol, f"{what}: max rel/abs error {worst:.3e} > {tol:.1e}"


def _torch_mask(n_q, n_k, causal, window_left):
    """Allowed pairs built with tril/triu (a different route from the oracle)."""
    delta = n_k - n_q
    m = torch.ones(n_q, n_k, dtype=torch.bool)
    if causal:
        m = torch.tril(m, diagonal=delta)
    if window_left >= 0:
        m = torch.triu(m, diagonal=delta - window_left)
    return m


# ---------------------------------------------------------------- library


def pin_torch_sdpa(impl):
    """PyTorch's own scaled_dot_product_attention (CPU, float64) on random
    shapes, masks and scales; lse against torch.logsumexp of the masked
    scores."""
    cases = [
        (17, 17, 8, 0.3, False, -1),
        (33, 33, 16, 0.25, True, -1),
        (40, 40, 8, 0.5, True, 5),
        (9, 23, 4, 0.7, True, -1),
        (23, 23, 8, 0.4, False, 3),
        (1, 13, 8, 0.35, True, 2),
    ]
    for t, (n_q, n_k, d, scale, causal, w) in enumerate(cases):
        r = _rng(100 + t)
        q, k, v = r.normal(size=(n_q, d)), r.normal(size=(n_k, d)), r.normal(size=(n_k, d))
        o, lse = impl(q, k, v, scale, causal, w)
        mask = _torch_mask(n_q, n_k, causal, w)
        qt, kt, vt = (torch.from_numpy(x) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt[None], kt[None], vt[None], attn_mask=mask[None], scale=scale)[0]
        s = scale * (qt @ kt.T)
        s = s.masked_fill(~mask, float("-inf"))
        ref_lse = torch.logsumexp(s, dim=-1)
        _close(o, ref.numpy(), 1e-12, f"torch sdpa o case {t}")
        _close(lse, ref_lse.numpy(), 1e-12, f"torch sdpa lse case {t}")


# ---------------------------------------------------------- closed forms


def pin_golden_hand_cases(impl):
    """Hand-derived exact values (tests/golden/hand_closed_forms.json)."""
    with open(os.path.join(GOLDEN, "hand_closed_forms.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        o, lse = impl(np.array(c["q"]), np.array(c["k"]), np.array(c["v"]), c["scale"],
                      c["causal"], c["window_left"])
        _close(o, c["o"], 1e-13, c["name"] + " o")
        _close(lse, c["lse"], 1e-13, c["name"] + " lse")


def pin_zero_query(impl):
    """Q = 0: every allowed score is 0, so O_i is the plain mean of the
    allowed V rows and lse_i = ln(number of allowed keys)."""
    r = _rng(7)
    for n_q, n_k, causal, w in [(12, 12, False, -1), (12, 12, True, -1), (15, 15, True, 4),
                                (6, 10, True, -1)]:
        q = np.zeros((n_q, 8))
        k, v = r.normal(size=(n_k, 8)), r.normal(size=(n_k, 5))
        o, lse = impl(q, k, v, 0.5, causal, w)
        delta = n_k - n_q
        for i in range(n_q):
            hi = min(n_k - 1, i + delta) if causal else n_k - 1
            lo = max(0, i + delta - w) if w >= 0 else 0
            _close(o[i], v[lo:hi + 1].mean(axis=0), 1e-13, f"zero-q row {i}")
            _close(lse[i], math.log(hi - lo + 1), 1e-13, f"zero-q lse row {i}")


def pin_single_key(impl):
    """n_k = 1: the softmax over one key is 1, so O_i = V_0 and
    lse_i = scale * q_i . k_0."""
    r = _rng(8)
    q, k, v = r.normal(size=(9, 16)), r.normal(size=(1, 16)), r.normal(size=(1, 16))
    o, lse = impl(q, k, v, 0.25, False, -1)
    _close(o, np.repeat(v, 9, axis=0), 1e-13, "single key o")
    _close(lse, 0.25 * (q @ k[0]), 1e-13, "single key lse")


def pin_causal_first_row(impl):
    """Causal with n_q = n_k: row 0 sees key 0 only, so O_0 = V_0 and
    lse_0 = scale * q_0 . k_0."""
    r = _rng(9)
    q, k, v = r.normal(size=(11, 8)), r.normal(size=(11, 8)), r.normal(size=(11, 8))
    o, lse = impl(q, k, v, 0.3, True, -1)
    _close(o[0], v[0], 1e-13, "causal row 0")
    _close(lse[0], 0.3 * q[0] @ k[0], 1e-13, "causal row 0 lse")


def pin_window_zero(impl):
    """Causal with window 0: row i sees key i only, so O = V."""
    r = _rng(10)
    q, k, v = r.normal(size=(10, 8)), r.normal(size=(10, 8)), r.normal(size=(10, 8))
    o, lse = impl(q, k, v, 0.3, True, 0)
    _close(o, v, 1e-13, "window 0 o")
    _close(lse, 0.3 * np.sum(q * k, axis=1), 1e-13, "window 0 lse")


def pin_wide_window(impl):
    """A window of at least n - 1 keys removes nothing from the causal mask."""
    r = _rng(11)
    q, k, v = r.normal(size=(14, 8)), r.normal(size=(14, 8)), r.normal(size=(14, 8))
    base = impl(q, k, v, 0.3, True, -1)
    for w in (13, 14, 100):
        got = impl(q, k, v, 0.3, True, w)
        _close(got[0], base[0], 1e-13, f"wide window {w} o")
        _close(got[1], base[1], 1e-13, f"wide window {w} lse")


def pin_bottom_right(impl):
    """Causal with n_q < n_k: query i sees keys 0..i+(n_k-n_q), i.e. it equals
    unmasked attention over that key prefix."""
    r = _rng(12)
    n_q, n_k = 5, 12
    q, k, v = r.normal(size=(n_q, 8)), r.normal(size=(n_k, 8)), r.normal(size=(n_k, 8))
    o, lse = impl(q, k, v, 0.4, True, -1)
    for i in range(n_q):
        hi = i + n_k - n_q
        oi, li = impl(q[i:i + 1], k[:hi + 1], v[:hi + 1], 0.4, False, -1)
        _close(o[i], oi[0], 1e-13, f"bottom-right row {i}")
        _close(lse[i], li[0], 1e-13, f"bottom-right lse row {i}")


# ------------------------------------------------------------ invariants


def pin_row_shift(impl):
    """Adding the same amount to every score of a row leaves O unchanged and
    shifts lse by that amount: K' = K + 1 w^T shifts row i by scale*q_i.w;
    an extra q column c/scale against an extra k column of ones shifts every
    score by c."""
    r = _rng(13)
    q, k, v = r.normal(size=(16, 8)), r.normal(size=(16, 8)), r.normal(size=(16, 8))
    o, lse = impl(q, k, v, 0.35, True, 6)
    w = r.normal(size=8)
    o2, lse2 = impl(q, k + w[None, :], v, 0.35, True, 6)
    _close(o2, o, 1e-12, "row shift o")
    _close(lse2, lse + 0.35 * (q @ w), 1e-12, "row shift lse")
    c = 3.25
    q3 = np.concatenate([q, np.full((16, 1), c / 0.35)], axis=1)
    k3 = np.concatenate([k, np.ones((16, 1))], axis=1)
    o3, lse3 = impl(q3, k3, v, 0.35, True, 6)
    _close(o3, o, 1e-12, "constant shift o")
    _close(lse3, lse + c, 1e-12, "constant shift lse")


def pin_key_permutation(impl):
    """Without a mask, permuting the K and V rows together changes nothing."""
    r = _rng(14)
    q, k, v = r.normal(size=(7, 8)), r.normal(size=(19, 8)), r.normal(size=(19, 6))
    perm = r.permutation(19)
    a = impl(q, k, v, 0.3, False, -1)
    b = impl(q, k[perm], v[perm], 0.3, False, -1)
    _close(b[0], a[0], 1e-12, "permutation o")
    _close(b[1], a[1], 1e-12, "permutation lse")


def pin_linear_in_v(impl):
    """O is linear in V for fixed Q and K."""
    r = _rng(15)
    q, k = r.normal(size=(10, 8)), r.normal(size=(10, 8))
    v1, v2 = r.normal(size=(10, 8)), r.normal(size=(10, 8))
    o1 = impl(q, k, v1, 0.3, True, -1)[0]
    o2 = impl(q, k, v2, 0.3, True, -1)[0]
    o12 = impl(q, k, 2.0 * v1 - 3.0 * v2, 0.3, True, -1)[0]
    _close(o12, 2.0 * o1 - 3.0 * o2, 1e-12, "linearity")


def pin_convex_rows(impl):
    """Each output row is a convex combination of allowed V rows: it lies
    inside their per-column range, and V = all ones gives exactly ones."""
    r = _rng(16)
    q, k = 3.0 * r.normal(size=(12, 8)), r.normal(size=(12, 8))
    v = r.normal(size=(12, 4))
    o = impl(q, k, v, 0.5, True, 3)[0]
    for i in range(12):
        lo = max(0, i - 3)
        vv = v[lo:i + 1]
        assert np.all(o[i] >= vv.min(axis=0) - 1e-12) and np.all(o[i] <= vv.max(axis=0) + 1e-12)
    ones = impl(q, k, np.ones((12, 4)), 0.5, True, 3)[0]
    _close(ones, np.ones((12, 4)), 1e-13, "weights sum to one")


def pin_brute_force(impl):
    """Pure-Python loops over every tiny case: n in 1..6, d in 1..3, with and
    without the causal mask; each weight is exp(score) / sum(exp(score))."""
    r = _rng(17)
    for n in range(1, 7):
        for d in range(1, 4):
            for causal in (False, True):
                q, k, v = r.normal(size=(n, d)), r.normal(size=(n, d)), r.normal(size=(n, d))
                o, lse = impl(q, k, v, 0.6, causal, -1)
                for i in range(n):
                    keys = range(i + 1) if causal else range(n)
                    sc = [0.6 * sum(q[i][t] * k[j][t] for t in range(d)) for j in keys]
                    ex = [math.exp(x) for x in sc]
                    tot = sum(ex)
                    for c in range(d):
                        want = sum(ex[a] * v[j][c] for a, j in enumerate(keys)) / tot
                        assert abs(o[i][c] - want) <= 1e-12 * max(1.0, abs(want)), (n, d, i, c)
                    assert abs(lse[i] - math.log(tot)) <= 1e-12 * max(1.0, abs(math.log(tot)))


ALL_PINS = [
    pin_torch_sdpa,
    pin_golden_hand_cases,
    pin_zero_query,
    pin_single_key,
    pin_causal_first_row,
    pin_window_zero,
    pin_wide_window,
    pin_bottom_right,
    pin_row_shift,
    pin_key_permutation,
    pin_linear_in_v,
    pin_convex_rows,
    pin_brute_force,
]
