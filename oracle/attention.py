"""Plain fp64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this module:
only the tests, the smoke check and the bench's CPU-baseline leg use it. It
shares no code with the HIP library and imports nothing from it.

What it computes, and where the pages fix it:

* The attention definition, O = softmax(Q K^T / sqrt(d)) V with the softmax
  taken over each row of the score matrix and masks restricting which
  query/key pairs interact -- "FlashAttention" (aiwiki.page),
  section "Attention and the memory bottleneck", the SDPA equation.
* The softmax is evaluated the safe three-pass way (row maximum, then the sum
  of exponentials shifted by that maximum, then the division) -- "From Online
  Softmax to FlashAttention" (cloud.tencent.cn), section 2.1/2.2, the 3-pass
  softmax.  The full score matrix is materialised, exactly the thing the
  method avoids; this module is allowed to be slow.
* The row log-sum-exp, lse_i = m_i + ln l_i, is the "compact normalisation
  information" the method keeps for the backward pass -- "FlashAttention",
  section "Training and computational complexity".  Natural log, fp64.
* ``online_attention`` is the block recurrence m' = max(m, max s_b),
  l' = e^{m-m'} l + sum_j e^{s_bj - m'}, u' = e^{m-m'} u + sum_j e^{s_bj-m'} v_bj,
  output u / l -- "FlashAttention", section "Tiling and online
  normalisation", the three update equations and the final division.  It is
  used by the tests to pin the recurrence against the 3-pass definition.
* ``sdpa_backward`` / ``attention_backward`` are the gradients of the same
  definition with respect to Q, K and V for an output gradient dO, by the
  chain rule through the materialised softmax: dV = P^T dO, dP = dO V^T,
  dS = P o (dP - rowsum(dO o O)), dQ = scale dS K, dK = scale dS^T Q.  The
  pages keep the row log-sum-exp exactly so that the backward pass can
  recompute P instead of storing it ("FlashAttention", section "Training and
  computational complexity"); the gradient formulas themselves are the
  textbook derivative of softmax(S) V, pinned in the tests by central finite
  differences.
* ``merge_states`` combines per-chunk (o_c, lse_c) pairs.  The pages do not
  name split-KV; the merge is the same rescale-and-add as the recurrence above
  applied to whole chunk states (a chunk state (m_c, l_c, u_c) has
  o_c = u_c / l_c and lse_c = m_c + ln l_c).

Readings taken where the pages are silent:

* causal alignment is bottom-right: key j is allowed for query i iff
  j <= i + (n_k - n_q);
* a left window of W keys admits keys j >= i + (n_k - n_q) - W, so with the
  causal bound a row sees at most W + 1 keys; W < 0 means no window;
* a row with no allowed key outputs zeros and lse = -inf.

* ``attention_fp8`` is the same attention on 8-bit floating-point inputs,
  the low-precision variant named in "FlashAttention", section "Versions":
  each e4m3 code is decoded to its exact value (``e4m3_decode``, written from
  the OCP float8 e4m3 definition: sign, 4 exponent bits with bias 7, 3
  mantissa bits, exponent field 0 subnormal, S.1111.111 NaN, no infinities),
  multiplied by the dequantisation factor of its (batch, head) block, and the
  fp64 definition above runs on the result.  The GPU path's own rounding of
  the probabilities is not part of the definition.

All functions take numpy arrays of any float dtype and compute in fp64.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "allowed_mask",
    "sdpa",
    "attention_dense",
    "attention_varlen",
    "attention_decode",
    "attention_kvcache",
    "sdpa_backward",
    "attention_backward",
    "online_attention",
    "merge_states",
    "attention_flops",
    "e4m3_decode",
    "attention_fp8",
]


def allowed_mask(n_q, n_k, causal=False, window_left=-1, q_index=None):
    """Boolean [len(q_index), n_k] mask of allowed (query, key) pairs.

    ``q_index`` holds the absolute query positions (defaults to 0..n_q-1) so
    that a subset of rows can be evaluated at full sequence length.
    Masks restricting query/key interaction: "FlashAttention", section
    "Attention and the memory bottleneck"; causal and sliding-window masks are
    named in section "Software integration and limitations".
    """
    if q_index is None:
        q_index = np.arange(n_q)
    i = np.asarray(q_index, dtype=np.int64)[:, None]
    j = np.arange(n_k, dtype=np.int64)[None, :]
    delta = n_k - n_q
    ok = np.ones((i.shape[0], n_k), dtype=bool)
    if causal:
        ok &= j <= i + delta
    if window_left is not None and window_left >= 0:
        ok &= j >= i + delta - window_left
    return ok


def sdpa(q, k, v, scale, causal=False, window_left=-1, q_index=None, n_q=None):
    """One head of exact attention, materialised, with the 3-pass softmax.

    q: [rows, d], k: [n_k, d], v: [n_k, d_v].  ``q_index``/``n_q`` let q be a
    subset of the rows of a longer query sequence (mask positions are
    absolute).  Returns (o [rows, d_v], lse [rows]) in fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows, n_k = q.shape[0], k.shape[0]
    if n_q is None:
        n_q = rows
    # score matrix S = scale * Q K^T, every entry materialised
    s = scale * (q @ k.T)
    ok = allowed_mask(n_q, n_k, causal, window_left, q_index)
    s = np.where(ok, s, -np.inf)
    o = np.zeros((rows, v.shape[1]), dtype=np.float64)
    lse = np.full(rows, -np.inf, dtype=np.float64)
    live = ok.any(axis=1)
    if not live.any():
        return o, lse
    s = s[live]
    # pass 1: row maximum
    m = s.max(axis=1)
    # pass 2: sum of exponentials shifted by the row maximum
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    # pass 3: normalise, then weight the value rows
    p = e / l[:, None]
    o[live] = p @ v
    lse[live] = m + np.log(l)
    return o, lse


def sdpa_backward(q, k, v, do, scale, causal=False, window_left=-1):
    """Gradients of one head of attention, materialised, fp64.

    q: [n_q, d], k: [n_k, d], v: [n_k, d_v], do: [n_q, d_v] (the gradient of
    the loss with respect to O).  P is the row softmax of the masked scores
    (3-pass, rows with no allowed key have P = 0).  Returns dq [n_q, d],
    dk [n_k, d], dv [n_k, d_v].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n_q, n_k = q.shape[0], k.shape[0]
    s = scale * (q @ k.T)
    ok = allowed_mask(n_q, n_k, causal, window_left)
    s = np.where(ok, s, -np.inf)
    p = np.zeros_like(s)
    live = ok.any(axis=1)
    if live.any():
        sl = s[live]
        m = sl.max(axis=1)
        e = np.exp(sl - m[:, None])
        p[live] = e / e.sum(axis=1)[:, None]
    o = p @ v
    dv = p.T @ do                          # O = P V
    dp = do @ v.T
    dsum = (do * o).sum(axis=1)            # = rowsum(P o dP)
    ds = p * (dp - dsum[:, None])          # softmax Jacobian applied to dP, row by row
    dq = scale * (ds @ k)                  # S = scale Q K^T
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def attention_backward(q, k, v, do, scale, causal=False, window_left=-1):
    """Dense batched gradients: q/do [B, n_q, H, d], k/v [B, n_k, H, d];
    returns dq, dk, dv in the same layouts, fp64, one ``sdpa_backward`` per
    (batch, head)."""
    q = np.asarray(q)
    B, n_q, H, d = q.shape
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            dq[b, :, h], dk[b, :, h], dv[b, :, h] = sdpa_backward(
                q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], scale, causal, window_left)
    return dq, dk, dv


def attention_dense(q, k, v, scale, causal=False, window_left=-1):
    """Dense batched attention.

    q: [B, n_q, H, d], k/v: [B, n_k, H, d] (the [batch, seq, heads, d]
    layout).  Returns o [B, n_q, H, d] and lse [B, H, n_q], fp64.  Heads and
    batch entries are independent, one ``sdpa`` each.
    """
    q = np.asarray(q)
    B, n_q, H, _ = q.shape
    n_k = k.shape[1]
    o = np.zeros((B, n_q, H, v.shape[3]), dtype=np.float64)
    lse = np.zeros((B, H, n_q), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            o[b, :, h, :], lse[b, h, :] = sdpa(
                q[b, :, h, :], k[b, :, h, :], v[b, :, h, :], scale, causal, window_left
            )
    return o, lse


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, scale, causal=False, window_left=-1):
    """Packed variable-length attention.

    q: [total_q, H, d], k/v: [total_k, H, d]; sequence i owns rows
    cu_q[i]:cu_q[i+1] of q and cu_k[i]:cu_k[i+1] of k and v.  Each sequence
    is attended independently.  Returns o [total_q, H, d], lse [H, total_q].
    """
    q = np.asarray(q)
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    total_q, H, _ = q.shape
    o = np.zeros((total_q, H, v.shape[2]), dtype=np.float64)
    lse = np.zeros((H, total_q), dtype=np.float64)
    for i in range(len(cq) - 1):
        q0, q1, k0, k1 = cq[i], cq[i + 1], ck[i], ck[i + 1]
        if q1 == q0:
            continue
        for h in range(H):
            o[q0:q1, h, :], lse[h, q0:q1] = sdpa(
                q[q0:q1, h, :], k[k0:k1, h, :], v[k0:k1, h, :], scale, causal, window_left
            )
    return o, lse


def attention_decode(q, k_cache, v_cache, seqlens_k, scale, heads=None, batches=None):
    """One new query per sequence against its cached keys and values.

    q: [B, 1, H, d]; k_cache/v_cache: [B, max_len, H, d]; sequence b attends
    to its first seqlens_k[b] cached rows (the cache already holds the current
    token, so no causal mask).  Rows past the length are never read.  Returns
    o [B, 1, H, d] and lse [B, H]; ``heads``/``batches`` restrict the work to
    a subset (the rest stays zero) for sampled checks at full size.
    """
    B, _, H, d = q.shape
    o = np.zeros((B, 1, H, v_cache.shape[3]), dtype=np.float64)
    lse = np.zeros((B, H), dtype=np.float64)
    for b in range(B) if batches is None else batches:
        n = int(seqlens_k[b])
        for h in range(H) if heads is None else heads:
            ob, lb = sdpa(q[b, :, h, :], k_cache[b, :n, h, :], v_cache[b, :n, h, :], scale)
            o[b, :, h, :] = ob
            lse[b, h] = lb[0]
    return o, lse


def attention_kvcache(q, k_cache, v_cache, seqlens_k, scale, causal=True, window_left=-1,
                      heads=None, batches=None):
    """Several new queries per sequence against its cached keys and values.

    q: [B, n_new, H, d] are the last n_new positions of each sequence;
    k_cache/v_cache: [B, max_len, H, d]; sequence b's keys are its first
    seqlens_k[b] rows (the new tokens among them, last).  Masks are relative
    to the bottom-right diagonal (delta = seqlens_k[b] - n_new), as in
    ``allowed_mask``.  Rows past the length are never read.  Returns
    o [B, n_new, H, d] and lse [B, H, n_new]; ``heads``/``batches`` restrict
    the work to a subset (the rest stays zero).
    """
    B, n_new, H, _ = q.shape
    o = np.zeros((B, n_new, H, v_cache.shape[3]), dtype=np.float64)
    lse = np.zeros((B, H, n_new), dtype=np.float64)
    for b in range(B) if batches is None else batches:
        n = int(seqlens_k[b])
        for h in range(H) if heads is None else heads:
            o[b, :, h, :], lse[b, h, :] = sdpa(
                q[b, :, h, :], k_cache[b, :n, h, :], v_cache[b, :n, h, :], scale, causal,
                window_left)
    return o, lse


def online_attention(q, k, v, scale, block, causal=False, window_left=-1):
    """Block-by-block online-softmax attention for one head, in fp64.

    Follows the update equations of "FlashAttention", section "Tiling and
    online normalisation": for each query row keep a running maximum m, an
    exponential sum l and an unnormalised output u; for every key block s_b
    set m' = max(m, max s_b), l' = e^{m-m'} l + sum_j e^{s_bj - m'},
    u' = e^{m-m'} u + sum_j e^{s_bj - m'} v_bj; the output is u / l.  Masked
    pairs carry the score -inf and so contribute e^{-inf} = 0.  This is the
    same 1-pass idea as the output surrogate of "From Online Softmax to
    FlashAttention", section 3, with the normalisation deferred to the end;
    the key blocks are the tiles of its section 4.
    Returns (o [n_q, d_v], lse [n_q]); lse = m + ln l.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_q, n_k = q.shape[0], k.shape[0]
    ok = allowed_mask(n_q, n_k, causal, window_left)
    o = np.zeros((n_q, v.shape[1]))
    lse = np.full(n_q, -np.inf)
    for i in range(n_q):
        m, l, u = -np.inf, 0.0, np.zeros(v.shape[1])
        for j0 in range(0, n_k, block):
            j1 = min(j0 + block, n_k)
            s_b = np.where(ok[i, j0:j1], scale * (k[j0:j1] @ q[i]), -np.inf)
            m_new = max(m, s_b.max())
            if m_new == -np.inf:  # nothing allowed yet: state stays empty
                continue
            rescale = np.exp(m - m_new)
            e = np.exp(s_b - m_new)
            l = rescale * l + e.sum()
            u = rescale * u + e @ v[j0:j1]
            m = m_new
        if l > 0.0:
            o[i] = u / l
            lse[i] = m + np.log(l)
    return o, lse


def merge_states(o_parts, lse_parts):
    """Combine chunk results (o_c, lse_c) of disjoint key chunks into one.

    With the chunk maximum M = max_c lse_c and weights w_c = e^{lse_c - M}:
    o = sum_c w_c o_c / sum_c w_c and lse = M + ln sum_c w_c.  This is the
    rescale of "FlashAttention", section "Tiling and online normalisation",
    applied to whole chunk states.  o_parts: [C, ..., d], lse_parts: [C, ...].
    Chunks with lse = -inf (no allowed key) carry zero weight.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    big = lse_parts.max(axis=0)
    safe = np.where(np.isfinite(big), big, 0.0)
    w = np.exp(lse_parts - safe)
    wsum = w.sum(axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = (w[..., None] * o_parts).sum(axis=0) / wsum[..., None]
        lse = safe + np.log(wsum)
    o = np.where((wsum > 0)[..., None], o, 0.0)
    lse = np.where(wsum > 0, lse, -np.inf)
    return o, lse


def attention_flops(n_q, n_k, d, causal=False, window_left=-1):
    """Algorithmic FLOPs of one head: 4 * d per allowed (query, key) pair.

    Two d-long dot products per pair (one for Q K^T, one for P V), two FLOPs
    per multiply-add.  All allowed pairs are computed -- the method keeps the
    quadratic arithmetic ("FlashAttention", section "Training and
    computational complexity").  Counted by brute force over the mask rows.
    """
    pairs = 0
    for i in range(n_q):
        hi = n_k - 1
        lo = 0
        delta = n_k - n_q
        if causal:
            hi = min(hi, i + delta)
        if window_left is not None and window_left >= 0:
            lo = max(lo, i + delta - window_left)
        if hi >= lo:
            pairs += hi - lo + 1
    return 4 * d * pairs


def e4m3_decode(codes):
    """Exact fp64 values of OCP e4m3 codes (uint8 array of any shape).

    Bit layout s eeee mmm: exponent field e > 0 gives (-1)^s (1 + m/8) 2^(e-7),
    e = 0 gives the subnormals (-1)^s (m/8) 2^-6, and the two codes with
    e = 15 and m = 7 are NaN (the format has no infinities; 0xFE = -448 is
    the most negative finite value).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = c >> 7
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def attention_fp8(q8, k8, v8, descale_q, descale_k, descale_v, scale, causal=False,
                  window_left=-1):
    """Dense attention on e4m3 codes q8 [B, n_q, H, d], k8/v8 [B, n_k, H, d]
    with one dequantisation factor per (batch, head) and tensor (arrays of
    B * H values, batch-major).  Returns o [B, n_q, H, d] and lse [B, H, n_q],
    fp64, of ``attention_dense`` on the dequantised tensors."""
    q8 = np.asarray(q8)
    B, _, H, _ = q8.shape

    def deq(codes, ds):
        f = np.asarray(ds, dtype=np.float64).reshape(B, 1, H, 1)
        return e4m3_decode(codes) * f

    return attention_dense(deq(q8, descale_q), deq(k8, descale_k), deq(v8, descale_v), scale,
                           causal, window_left)
