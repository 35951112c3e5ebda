"""CPU checks of the fp64 oracle against what the pages and the mathematics fix.

No GPU.  The one-head definition is pinned by the battery in oracle_pins;
the batched, packed, decode, recurrence, merge and FLOP-count functions are
pinned against the one-head definition and against closed forms.
"""

import math

import numpy as np
import pytest

import oracle
from tests import oracle_pins


def _oracle_one_head(q, k, v, scale, causal, window_left):
    return oracle.sdpa(q, k, v, scale, causal, window_left)


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_definition_pins(pin):
    pin(_oracle_one_head)


# ------------------------------------------------ recurrence of the pages


@pytest.mark.parametrize("block", [1, 3, 7, 16, 64])
@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (True, 5)])
def test_online_recurrence_matches_three_pass(block, causal, window):
    """The block update m', l', u' -> u / l reproduces the 3-pass result
    (global normalisation is preserved), including tails that do not fill a
    block (n = 45 is not a multiple of 7, 16 or 64)."""
    r = np.random.default_rng(block * 10 + causal)
    n, d = 45, 8
    q, k, v = 2.0 * r.normal(size=(n, d)), r.normal(size=(n, d)), r.normal(size=(n, d))
    o_ref, lse_ref = oracle.sdpa(q, k, v, 0.4, causal, window)
    o, lse = oracle.online_attention(q, k, v, 0.4, block, causal, window)
    assert np.max(np.abs(o - o_ref)) <= 1e-12
    assert np.max(np.abs(lse - lse_ref)) <= 1e-12


def test_online_recurrence_passes_pins():
    """The recurrence itself passes the definition pins at an awkward block."""
    for pin in oracle_pins.ALL_PINS:
        pin(lambda q, k, v, s, c, w: oracle.online_attention(q, k, v, s, 3, c, w))


# ------------------------------------------------------------ batching


def test_dense_heads_and_batches_independent():
    """Batched dense attention equals one-head attention on each (b, h) slice,
    and permuting heads permutes the outputs."""
    r = np.random.default_rng(3)
    B, N, H, d = 2, 19, 3, 8
    q, k, v = (r.normal(size=(B, N, H, d)) for _ in range(3))
    o, lse = oracle.attention_dense(q, k, v, 0.3, True, 4)
    for b in range(B):
        for h in range(H):
            oo, ll = oracle.sdpa(q[b, :, h], k[b, :, h], v[b, :, h], 0.3, True, 4)
            np.testing.assert_array_equal(o[b, :, h], oo)
            np.testing.assert_array_equal(lse[b, h], ll)
    perm = [2, 0, 1]
    o2, lse2 = oracle.attention_dense(q[:, :, perm], k[:, :, perm], v[:, :, perm], 0.3, True, 4)
    np.testing.assert_array_equal(o2, o[:, :, perm])
    np.testing.assert_array_equal(lse2, lse[:, perm])


def test_varlen_equals_per_sequence_dense():
    """Packed attention equals dense attention of each sequence on its own."""
    r = np.random.default_rng(4)
    lens = [5, 1, 17, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    H, d = 2, 8
    q, k, v = (r.normal(size=(cu[-1], H, d)) for _ in range(3))
    o, lse = oracle.attention_varlen(q, k, v, cu, cu, 0.3, True, 3)
    for i, n in enumerate(lens):
        a, b = cu[i], cu[i + 1]
        od, ld = oracle.attention_dense(q[None, a:b], k[None, a:b], v[None, a:b], 0.3, True, 3)
        np.testing.assert_allclose(o[a:b], od[0], rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse[:, a:b], ld[0], rtol=0, atol=1e-15)


def test_decode_equals_last_row_of_prefill():
    """One query against L cached keys equals the last row of causal prefill of
    length L (bottom-right causal lets the last row see every key), and rows
    past the length are never read (NaN padding stays out)."""
    r = np.random.default_rng(5)
    B, H, d, max_len = 3, 2, 8, 24
    lens = [24, 7, 1]
    kc, vc = r.normal(size=(B, max_len, H, d)), r.normal(size=(B, max_len, H, d))
    for b, n in enumerate(lens):
        kc[b, n:] = np.nan
        vc[b, n:] = np.nan
    q = r.normal(size=(B, 1, H, d))
    o, lse = oracle.attention_decode(q, kc, vc, lens, 0.3)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    for b, n in enumerate(lens):
        qq = r.normal(size=(1, n, H, d))
        qq[0, -1] = q[b, 0]
        op, lp = oracle.attention_dense(qq, kc[None, b, :n], vc[None, b, :n], 0.3, True)
        np.testing.assert_allclose(o[b, 0], op[0, -1], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[b], lp[0, :, -1], rtol=0, atol=1e-14)


def test_kvcache_equals_last_rows_of_prefill():
    """n_new queries against a cache of L keys (the new tokens last) equal the
    last n_new rows of causal prefill of length L; with every length equal to
    max_len the cache form is dense attention; with n_new = 1 it is decode.
    NaN padding past each length stays out."""
    r = np.random.default_rng(6)
    B, H, d, max_len, n_new = 3, 2, 8, 30, 5
    lens = [30, 12, 5]
    kc, vc = r.normal(size=(B, max_len, H, d)), r.normal(size=(B, max_len, H, d))
    for b, n in enumerate(lens):
        kc[b, n:] = np.nan
        vc[b, n:] = np.nan
    q = r.normal(size=(B, n_new, H, d))
    o, lse = oracle.attention_kvcache(q, kc, vc, lens, 0.3, True, 6)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    for b, n in enumerate(lens):
        qq = r.normal(size=(1, n, H, d))
        qq[0, n - n_new:] = q[b]
        op, lp = oracle.attention_dense(qq, kc[None, b, :n], vc[None, b, :n], 0.3, True, 6)
        np.testing.assert_allclose(o[b], op[0, n - n_new:], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[b], lp[0, :, n - n_new:], rtol=0, atol=1e-14)
    kf, vf = r.normal(size=(B, max_len, H, d)), r.normal(size=(B, max_len, H, d))
    o1, l1 = oracle.attention_kvcache(q, kf, vf, [max_len] * B, 0.3, False)
    o2, l2 = oracle.attention_dense(q, kf, vf, 0.3, False)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    o3, l3 = oracle.attention_kvcache(q[:, -1:], kc, vc, lens, 0.3, True)
    o4, l4 = oracle.attention_decode(q[:, -1:], kc, vc, lens, 0.3)
    np.testing.assert_allclose(o3, o4, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l3[:, :, 0], l4, rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (True, 2), (False, 1)])
def test_backward_matches_finite_differences(causal, window):
    """dQ, dK, dV of L = sum(O o dO) against central differences of the
    forward definition (n_q != n_k, so bottom-right masks and, with the
    window, rows and keys that see nothing are exercised)."""
    r = np.random.default_rng(11)
    n_q, n_k, d, dv_ = 5, 7, 3, 4
    q, k = r.normal(size=(n_q, d)), r.normal(size=(n_k, d))
    v, do = r.normal(size=(n_k, dv_)), r.normal(size=(n_q, dv_))
    scale = 0.7
    dq, dk, dv = oracle.sdpa_backward(q, k, v, do, scale, causal, window)

    def loss(qq, kk, vv):
        o, _ = oracle.sdpa(qq, kk, vv, scale, causal, window)
        return float((o * do).sum())

    h = 1e-6
    for x, g, idx in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(x)
        for pos in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[pos] += h
            xm[pos] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[idx], args_m[idx] = xp, xm
            num[pos] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


def test_backward_invariants():
    """Row sums of dS vanish, so the key gradients sum to zero over the keys;
    shifting every key by one vector shifts each score row by a constant,
    which changes neither P nor O: dQ and dV stay the same."""
    r = np.random.default_rng(12)
    n, d = 9, 4
    q, k, v, do = (r.normal(size=(n, d)) for _ in range(4))
    for causal in (False, True):
        dq, dk, dv = oracle.sdpa_backward(q, k, v, do, 0.5, causal)
        np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
        w = r.normal(size=d)
        dq2, _, dv2 = oracle.sdpa_backward(q, k + w[None, :], v, do, 0.5, causal)
        np.testing.assert_allclose(dq2, dq, rtol=0, atol=1e-12)
        np.testing.assert_allclose(dv2, dv, rtol=0, atol=1e-12)


def test_backward_matches_autograd():
    """Cross-check with PyTorch's autograd (fp64, CPU) through its own SDPA."""
    torch = pytest.importorskip("torch")
    r = np.random.default_rng(13)
    B, n, H, d = 2, 11, 2, 8
    q, k, v, do = (r.normal(size=(B, n, H, d)) for _ in range(4))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.3, True)
    tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3), requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=0.3)
    o.backward(torch.tensor(do.transpose(0, 2, 1, 3)))
    for got, ref in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(got, ref.grad.numpy().transpose(0, 2, 1, 3), rtol=1e-10,
                                   atol=1e-12)


@pytest.mark.parametrize("chunk", [1, 4, 7, 256])
def test_merge_of_chunks_equals_unsplit(chunk):
    """Attention over disjoint key chunks, merged by lse weights, equals
    attention over all keys, for any chunk size (split-KV equals unsplit)."""
    r = np.random.default_rng(6 + chunk)
    q, k, v = 3.0 * r.normal(size=(4, 16)), r.normal(size=(50, 16)), r.normal(size=(50, 16))
    o_ref, lse_ref = oracle.sdpa(q, k, v, 0.25)
    parts = [oracle.sdpa(q, k[a:a + chunk], v[a:a + chunk], 0.25) for a in range(0, 50, chunk)]
    o, lse = oracle.merge_states([p[0] for p in parts], [p[1] for p in parts])
    assert np.max(np.abs(o - o_ref)) <= 1e-12
    assert np.max(np.abs(lse - lse_ref)) <= 1e-12


def test_merge_ignores_empty_chunks():
    """A chunk with no allowed key (lse = -inf) carries zero weight; all-empty
    gives the empty-row convention (zeros, -inf)."""
    o_parts = np.array([[[1.0, 2.0]], [[0.0, 0.0]]])
    lse_parts = np.array([[0.5], [-np.inf]])
    o, lse = oracle.merge_states(o_parts, lse_parts)
    np.testing.assert_array_equal(o, [[1.0, 2.0]])
    np.testing.assert_array_equal(lse, [0.5])
    o, lse = oracle.merge_states(np.zeros((2, 1, 2)), np.full((2, 1), -np.inf))
    np.testing.assert_array_equal(o, np.zeros((1, 2)))
    assert np.all(np.isneginf(lse))


def test_empty_row_convention():
    """A row with no allowed key (window reaching left of the keys of a
    bottom-right causal mask with n_q > n_k) outputs zeros and lse = -inf."""
    r = np.random.default_rng(7)
    q, k, v = r.normal(size=(6, 4)), r.normal(size=(3, 4)), r.normal(size=(3, 4))
    o, lse = oracle.sdpa(q, k, v, 0.5, causal=True)
    # delta = -3: rows 0..2 have j <= i - 3 < 0 -> nothing allowed
    np.testing.assert_array_equal(o[:3], 0.0)
    assert np.all(np.isneginf(lse[:3]))
    assert np.all(np.isfinite(lse[3:]))


def test_row_subset_matches_full():
    """Evaluating a subset of query rows at their absolute positions equals
    the same rows of the full evaluation (used for sampled checks at full
    size)."""
    r = np.random.default_rng(8)
    q, k, v = r.normal(size=(40, 8)), r.normal(size=(40, 8)), r.normal(size=(40, 8))
    o, lse = oracle.sdpa(q, k, v, 0.3, True, 9)
    rows = np.array([0, 3, 17, 39])
    o2, lse2 = oracle.sdpa(q[rows], k, v, 0.3, True, 9, q_index=rows, n_q=40)
    np.testing.assert_allclose(o2, o[rows], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse2, lse[rows], rtol=0, atol=1e-15)


# ----------------------------------------------------------- FLOP count


def test_flop_count_closed_forms():
    """4 d per allowed pair: N^2 pairs unmasked, N(N+1)/2 causal, and for a
    causal window W: (W+1)(W+2)/2 + (W+1)(N-W-1) when N > W+1."""
    assert oracle.attention_flops(256, 256, 64) == 4 * 64 * 256 * 256
    assert oracle.attention_flops(2048, 2048, 128, True) == 4 * 128 * 2048 * 2049 // 2
    assert oracle.attention_flops(8000, 8000, 128, True) == 4 * 128 * 8000 * 8001 // 2
    W, N = 1024, 3000
    pairs = (W + 1) * (W + 2) // 2 + (W + 1) * (N - W - 1)
    assert oracle.attention_flops(N, N, 64, True, W) == 4 * 64 * pairs
    assert oracle.attention_flops(500, 500, 64, True, W) == 4 * 64 * 500 * 501 // 2
    # matches counting the mask directly
    m = oracle.allowed_mask(37, 50, True, 6)
    assert oracle.attention_flops(37, 50, 8, True, 6) == 4 * 8 * int(m.sum())


def test_config_sizes():
    """The headline prefill workload is 137.44 GFLOP non-causal."""
    f = 4 * 16 * oracle.attention_flops(2048, 2048, 128)
    assert f == 137438953472
    assert math.isclose(f / 1e9, 137.44, rel_tol=1e-4)
