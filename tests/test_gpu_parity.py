"""GPU parity: the HIP path, called through the C ABI, against the fp64
oracle on the same seeded inputs, element by element.

Small shapes span several 128-row query tiles and 64-key K/V tiles with
ragged tails; the five workloads run at full size in the launch configuration
the bench times, checked on every output (2k prefill, packed batch), on every
row of four heads and sampled rows of the others (8000-token prompt) and on
every head of ten sequences (decode).
"""

import math
import sys

import numpy as np
import pytest
import torch

import io_aware_exact_19_amd as fa
import oracle
from io_aware_exact_19_amd import configs, inputs
from tests.parity import announce, check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load_library()
    yield
    torch.cuda.synchronize()


def _np(t):
    return t.float().double().numpy() if t.dtype == torch.bfloat16 else t.double().numpy()


def _dense_case(B, H, nq, nk, d, causal, W, dtype, seed, q_mult=1.0, scale=None):
    q, k, v = inputs.dense_qkv(B, nq, nk, H, d, seed, dtype, q_mult)
    s = 1.0 / math.sqrt(d) if scale is None else scale
    what = f"dense B{B} H{H} nq{nq} nk{nk} d{d} causal{int(causal)} W{W} {dtype} x{q_mult}"
    announce(what)
    o, lse = fa.attention(q.cuda(), k.cuda(), v.cuda(), scale=s, causal=causal, window_left=W)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_dense(_np(q), _np(k), _np(v), s, causal, W)
    check(o.cpu(), lse.cpu(), o_ref, lse_ref, dtype, what)
    return o.cpu(), lse.cpu(), o_ref, lse_ref


SMALL_BF16 = [
    # B, H, nq, nk, d, causal, window
    (1, 2, 300, 300, 128, False, -1),
    (2, 3, 300, 300, 128, True, -1),
    (1, 2, 517, 517, 64, True, 100),
    (1, 2, 200, 333, 128, True, -1),   # n_q < n_k: bottom-right causal
    (1, 2, 333, 200, 64, True, -1),    # n_q > n_k: the first 133 rows see no key
    (1, 1, 1, 1, 128, False, -1),
    (1, 2, 63, 63, 128, True, -1),
    (1, 2, 65, 65, 64, False, -1),
    (1, 2, 200, 200, 128, True, 0),    # window 0: O = V
    (1, 2, 200, 200, 64, True, 500),   # window wider than the sequence
    (1, 2, 130, 130, 128, False, 7),   # window without causal
    (3, 1, 129, 64, 64, False, -1),
    (1, 2, 1, 700, 128, True, -1),     # one query at the end of 700 keys
    # d = 128 runs the two-group kernel (256 query rows per workgroup)
    (1, 2, 700, 700, 128, True, 100),  # window: first needed tile > 0, several workgroups
    (1, 2, 333, 200, 128, True, -1),   # n_q > n_k: rows without keys, dead waves
    (2, 2, 600, 600, 128, False, 150), # window without causal, several tiles
    (1, 3, 1000, 1000, 128, True, 1024),  # window wider than the sequence
    (1, 1, 257, 257, 128, True, 31),   # window narrower than a tile
    (1, 1, 513, 1100, 128, False, -1), # n_q just past two workgroups, ragged keys
]


@pytest.mark.parametrize("B,H,nq,nk,d,causal,W", SMALL_BF16)
def test_dense_bf16_small(B, H, nq, nk, d, causal, W):
    _dense_case(B, H, nq, nk, d, causal, W, torch.bfloat16, seed=1000 + nq + nk + d + W)


def test_dense_bf16_peaked():
    """Q multiplied by 4: peaked softmax rows."""
    _dense_case(2, 2, 256, 256, 128, False, -1, torch.bfloat16, seed=7, q_mult=4.0)
    _dense_case(1, 2, 300, 300, 64, True, -1, torch.bfloat16, seed=8, q_mult=4.0)


def test_window_zero_returns_v_exactly():
    """Causal with window 0: each row sees only its own key, so O = V bit for
    bit (p = 1) and lse = scale * q.k."""
    o, lse, o_ref, _ = _dense_case(1, 2, 150, 150, 128, True, 0, torch.bfloat16, seed=9)
    _, _, v = inputs.dense_qkv(1, 150, 150, 2, 128, 9, torch.bfloat16)
    assert torch.equal(o, v)


def test_rows_without_keys_are_zero():
    o, lse, o_ref, lse_ref = _dense_case(1, 2, 333, 200, 64, True, -1, torch.bfloat16, seed=10)
    assert torch.all(o[:, :133] == 0)
    assert torch.all(torch.isneginf(lse[:, :, :133]))


def test_no_keys_at_all():
    q = inputs.normal((2, 5, 3, 64), 1).cuda()
    k = torch.empty((2, 0, 3, 64), dtype=torch.bfloat16, device="cuda")
    announce("dense seqlen_k=0")
    o, lse = fa.attention(q, k, k.clone(), causal=False)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("B,H,nq,nk,causal,W", [
    (2, 64, 700, 400, True, -1),    # 384 items, partial second round; whole tiles without keys
    (1, 264, 300, 300, False, -1),  # 528 items, partial third round, no mask
    (2, 72, 520, 520, True, 200),   # 432 items, causal + window (first needed tile > 0)
])
def test_persistent_grid(B, H, nq, nk, causal, W):
    """More d = 128 query tiles than compute units: each workgroup walks
    several items (mirrored order in odd rounds, the next item's tiles and Q
    queued during the current item's last step)."""
    _dense_case(B, H, nq, nk, 128, causal, W, torch.bfloat16, seed=31)


@pytest.mark.parametrize("B,H,nq,nk,d,causal,W", [
    (1, 2, 300, 300, 128, True, -1),
    (1, 1, 100, 37, 64, True, 5),
    (2, 2, 130, 130, 64, False, -1),
])
def test_dense_fp32_small(B, H, nq, nk, d, causal, W):
    _dense_case(B, H, nq, nk, d, causal, W, torch.float32, seed=2000 + nq + nk)


def test_workload_small_fp32():
    c = configs.SMALL_FP32
    _dense_case(c["batch"], c["heads"], c["seqlen"], c["seqlen"], c["d"], c["causal"],
                c["window_left"], torch.float32, c["seed"])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("q_mult", [1.0, 4.0])
def test_workload_prefill_2k(causal, q_mult):
    """B4 H16 N2048 d128 bf16, every output checked."""
    c = configs.PREFILL_2K
    _dense_case(c["batch"], c["heads"], c["seqlen"], c["seqlen"], c["d"], causal, -1,
                torch.bfloat16, c["seed"], q_mult=q_mult)


def test_workload_long_8k():
    """B1 H32 N8000 causal d128: sampled rows (every tile boundary near the
    start, the middle and the 64-row tail tile) of every head, and every row
    of four heads."""
    c = configs.LONG_8K
    N, H, d = c["seqlen"], c["heads"], c["d"]
    q, k, v = inputs.dense_qkv(1, N, N, H, d, c["seed"])
    s = configs.default_scale(d)
    announce("long 8k causal")
    o, lse = fa.attention(q.cuda(), k.cuda(), v.cuda(), scale=s, causal=True)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    rng = np.random.default_rng(3)
    rows = sorted(set([0, 1, 2, 63, 64, 127, 128, 129, 3999, 4000, 7871, 7872, 7935, 7936,
                       7937, 7990, 7998, 7999] + list(rng.integers(0, N, 24))))
    rows = np.array(rows)
    qn, kn, vn = _np(q), _np(k), _np(v)
    o_ref = np.zeros((len(rows), H, d))
    lse_ref = np.zeros((H, len(rows)))
    for h in range(H):
        o_ref[:, h], lse_ref[h] = oracle.sdpa(qn[0, rows, h], kn[0, :, h], vn[0, :, h], s, True,
                                             q_index=rows, n_q=N)
    check(o[0, rows], lse[0][:, rows], o_ref, lse_ref, torch.bfloat16, "long 8k sampled rows")
    # every row of four heads (first, last and two inside, on different XCDs)
    for h in (0, 11, 22, 31):
        o_h, lse_h = oracle.sdpa(qn[0, :, h], kn[0, :, h], vn[0, :, h], s, True)
        check(o[0, :, h], lse[0, h], o_h, lse_h, torch.bfloat16, f"long 8k head {h}, all rows")


def _varlen_case(lens, H, d, causal, W, seed, heads_checked=None):
    lens = torch.as_tensor(lens)
    cu = inputs.cu_seqlens(lens)
    q, k, v = inputs.varlen_qkv(lens, H, d, seed)
    s = configs.default_scale(d)
    what = f"varlen nseq{len(lens)} H{H} d{d} causal{int(causal)} W{W}"
    announce(what)
    cu_d = cu.cuda()
    o, lse = fa.attention_varlen(q.cuda(), k.cuda(), v.cuda(), cu_d, cu_d, int(lens.max()),
                                 int(lens.max()), scale=s, causal=causal, window_left=W)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    hs = list(range(H)) if heads_checked is None else heads_checked
    qn, kn, vn = _np(q[:, hs]), _np(k[:, hs]), _np(v[:, hs])
    o_ref, lse_ref = oracle.attention_varlen(qn, kn, vn, cu.numpy(), cu.numpy(), s, causal, W)
    check(o[:, hs], lse[hs], o_ref, lse_ref, torch.bfloat16, what)
    return q, k, v, cu, o, lse


def test_varlen_small():
    _varlen_case([5, 1, 300, 129, 64, 0, 200], 2, 64, True, 50, seed=31)
    _varlen_case([130, 70, 257], 3, 128, False, -1, seed=32)
    _varlen_case([1000, 17, 513], 2, 128, True, -1, seed=33)
    _varlen_case([0, 1, 2, 300, 700, 5, 256, 257], 2, 128, True, 64, seed=35)


def _scaled_case(q, k, v, causal, W, what):
    """Dense bf16 case on given CPU inputs, checked element by element."""
    d = q.shape[-1]
    s = 1.0 / math.sqrt(d)
    announce(what)
    o, lse = fa.attention(q.cuda(), k.cuda(), v.cuda(), scale=s, causal=causal, window_left=W)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_dense(_np(q), _np(k), _np(v), s, causal, W)
    check(o.cpu(), lse.cpu(), o_ref, lse_ref, torch.bfloat16, what)


@pytest.mark.parametrize("d", [64, 128])
def test_growing_scores_rescale_repeatedly(d):
    """Scores rise along the keys (K row j carries j times a direction that Q
    points along), so the row maximum grows from tile to tile and the lazy
    reference must move many times; the output is dominated by the last
    allowed keys."""
    B, H, N = 1, 2, 900
    q, k, v = inputs.dense_qkv(B, N, N, H, d, 61)
    ramp = torch.linspace(0.0, 400.0, N).view(1, N, 1, 1)
    k = (k.float() * 0.05 + ramp * torch.ones(d) / math.sqrt(d) * 0.5).to(torch.bfloat16)
    q = (q.float() * 0.05 + torch.ones(d) / math.sqrt(d) * 4.0).to(torch.bfloat16)
    for causal in (False, True):
        _scaled_case(q, k, v, causal, -1, f"growing scores d{d} causal{int(causal)}")


@pytest.mark.parametrize("d", [64, 128])
def test_extreme_score_magnitudes(d):
    """Scores of several hundred in natural units (exp would overflow fp32
    without the reference shift), with the maximum placed in a late tile."""
    B, H, N = 1, 2, 600
    q, k, v = inputs.dense_qkv(B, N, N, H, d, 62)
    q = (q.float() * 16.0).to(torch.bfloat16)
    k = (k.float() * 16.0).to(torch.bfloat16)
    _scaled_case(q, k, v, False, -1, f"extreme scores d{d}")
    _scaled_case(q, k, v, True, 200, f"extreme scores d{d} causal window")


def test_key_range_beyond_one_buffer_window():
    """More than 2^32 bytes of keys for one head at a head stride of 16 KiB
    (64 heads x d 128): the d = 128 kernel addresses K/V through buffer
    windows of at most 2^32 bytes and must move its window part-way through
    the keys.  4.3 GB each for K and V, generated on the device; sampled
    (row, head) outputs checked against the oracle."""
    H, d, n_q = 64, 128, 64
    win = (2 ** 32 - 1) // (H * d * 2) // 64 * 64   # keys per window
    n_k = win + 1000
    dev = "cuda"
    announce(f"dense n_q {n_q} n_k {n_k} H{H} d{d} (window {win} keys)")
    q = inputs.normal((1, n_q, H, d), 71, device=dev)
    k = inputs.normal((1, n_k, H, d), 72, device=dev)
    v = inputs.normal((1, n_k, H, d), 73, device=dev)
    s = 1.0 / math.sqrt(d)
    for causal in (False, True):
        o, lse = fa.attention(q, k, v, scale=s, causal=causal)
        torch.cuda.synchronize()
        for h in (0, 37, 63):
            kh, vh = _np(k[0, :, h].cpu()), _np(v[0, :, h].cpu())
            rows = np.array([0, 31, 63])
            o_ref, lse_ref = oracle.sdpa(_np(q[0, rows, h].cpu()), kh, vh, s, causal,
                                         q_index=rows, n_q=n_q)
            check(o[0, rows, h].cpu(), lse[0, h, rows].cpu(), o_ref, lse_ref, torch.bfloat16,
                  f"window crossing causal{int(causal)} head {h}")
    del q, k, v
    torch.cuda.empty_cache()


def test_d64_keys_beyond_4gib():
    """More than 2^32 bytes of keys (and values) at d = 64 (128 heads, a
    16 KiB row) with a ragged last tile: the four-wave kernel rebuilds each
    tile's descriptor from a 64-bit base.  Generated on the device; sampled
    (row, head) outputs checked against the oracle."""
    H, d, n_q = 128, 64, 64
    n_k = 2 ** 32 // (H * d * 2) + 1000
    dev = "cuda"
    announce(f"dense d64 n_q {n_q} n_k {n_k} H{H} (K, V {n_k * H * d * 2 / 2 ** 30:.2f} GiB each)")
    q = inputs.normal((1, n_q, H, d), 74, device=dev)
    k = inputs.normal((1, n_k, H, d), 75, device=dev)
    v = inputs.normal((1, n_k, H, d), 76, device=dev)
    s = 1.0 / math.sqrt(d)
    rows = np.array([0, 31, 63])
    for causal in (False, True):
        o, lse = fa.attention(q, k, v, scale=s, causal=causal)
        torch.cuda.synchronize()
        for h in (0, 77, 127):
            kh, vh = _np(k[0, :, h].cpu()), _np(v[0, :, h].cpu())
            o_ref, lse_ref = oracle.sdpa(_np(q[0, rows, h].cpu()), kh, vh, s, causal,
                                         q_index=rows, n_q=n_q)
            check(o[0, rows, h].cpu(), lse[0, h, rows].cpu(), o_ref, lse_ref, torch.bfloat16,
                  f"d64 beyond 4 GiB causal{int(causal)} head {h}")
    del q, k, v
    torch.cuda.empty_cache()


def test_varlen_equals_per_sequence_dense():
    """The packed call and one dense call per sequence run the same tiles in
    the same order: identical bits."""
    lens = [300, 129, 1, 450]
    q, k, v, cu, o, lse = _varlen_case(lens, 2, 64, True, 100, seed=34)
    for i, n in enumerate(lens):
        a, b = int(cu[i]), int(cu[i + 1])
        od, ld = fa.attention(q[None, a:b].cuda(), k[None, a:b].cuda(), v[None, a:b].cuda(),
                              causal=True, window_left=100)
        torch.cuda.synchronize()
        assert torch.equal(od[0].cpu(), o[a:b])
        assert torch.equal(ld[0].cpu(), lse[:, a:b])


def test_workload_varlen():
    """16 sequences, lengths U[128, 4096], H16 d64, causal + window 1024;
    every head checked on every row of every sequence."""
    c = configs.VARLEN
    lens = inputs.lengths(c["nseq"], c["len_lo"], c["len_hi"], c["seed"])
    _varlen_case(lens, c["heads"], c["d"], c["causal"], c["window_left"], c["seed"])


def _decode_case(B, H, max_len, d, lens, chunk, seed, pairs=None):
    lens = torch.as_tensor(lens, dtype=torch.int32)
    what = f"decode B{B} H{H} max_len{max_len} d{d} chunk{chunk}"
    announce(what)
    kc = inputs.decode_cache(B, max_len, H, d, lens, seed, "cuda", "k")
    vc = inputs.decode_cache(B, max_len, H, d, lens, seed, "cuda", "v")
    q = inputs.normal((B, 1, H, d), inputs.subseed(seed, "q")).cuda()
    s = configs.default_scale(d)
    o, lse = fa.decode(q, kc, vc, lens.cuda(), scale=s, chunk=chunk)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(H)]
    o_ref = np.zeros((len(pairs), d))
    lse_ref = np.zeros(len(pairs))
    got_o = torch.zeros((len(pairs), d), dtype=torch.bfloat16)
    got_l = torch.zeros(len(pairs))
    qn = _np(q.cpu())
    rows_of = {}
    for i, (b, h) in enumerate(pairs):
        n = int(lens[b])
        if b not in rows_of:  # one host copy of a sequence's valid rows, all heads
            rows_of.clear()
            rows_of[b] = (kc[b, :n].cpu(), vc[b, :n].cpu())
        kb, vb = rows_of[b]
        ob, lb = oracle.sdpa(qn[b, :, h], _np(kb[:, h]), _np(vb[:, h]), s)
        o_ref[i], lse_ref[i] = ob[0], lb[0]
        got_o[i], got_l[i] = o[b, 0, h], lse[b, h]
    check(got_o, got_l, o_ref, lse_ref, torch.bfloat16, what)
    del kc, vc
    return q, o, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("chunk", [64, 256, 512])
def test_decode_small(d, chunk):
    """Padding rows are NaN: any read past a sequence's length poisons O."""
    _decode_case(3, 2, 1000, d, [1, 257, 1000], chunk, seed=41)


@pytest.mark.parametrize("H,d,chunk", [(3, 128, 256), (20, 128, 128), (40, 64, 64), (33, 64, 512)])
def test_decode_ragged_heads(H, d, chunk):
    """Head counts that leave the last head group of a workgroup partly
    empty; lengths on, just before and just after chunk and step edges."""
    _decode_case(4, H, 1030, d, [16, 511, 1030, 513], chunk, seed=44)


def test_decode_empty_sequence():
    q, o, lse = _decode_case(2, 2, 64, 128, [0, 5], 64, seed=42, pairs=[(1, 0), (1, 1)])
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))


def test_decode_equals_prefill_last_row():
    """One query against L cached keys is the last row of causal prefill."""
    L, H, d = 777, 2, 128
    kc = inputs.decode_cache(1, 1024, H, d, [L], 43, "cuda", "k")
    vc = inputs.decode_cache(1, 1024, H, d, [L], 43, "cuda", "v")
    q = inputs.normal((1, 1, H, d), 5).cuda()
    announce("decode vs prefill")
    od, ld = fa.decode(q, kc, vc, torch.tensor([L], dtype=torch.int32, device="cuda"), chunk=128)
    op, lp = fa.attention(q, kc[:, :L].contiguous(), vc[:, :L].contiguous(), causal=True)
    torch.cuda.synchronize()
    assert (od.float() - op.float()).abs().max().item() <= 2e-2
    assert (ld - lp[:, :, 0]).abs().max().item() <= 1e-3


# Backward tolerance, relative to the largest reference gradient entry of each
# tensor: P and dS are rounded to bf16 before their products (relative error
# up to 2^-8 each), D = rowsum(dO o O) uses the bf16 forward output, and the
# gradients are rounded to bf16 once; each stays well inside 2 % of the
# tensor's largest entry at the element level and 0.2 % on average.
BWD_MAX_REL = 2e-2
BWD_MEAN_REL = 2e-3


def _bwd_case(B, H, n_q, n_k, d, causal, W, seed, q_mult=1.0):
    what = f"bwd B{B} H{H} nq{n_q} nk{n_k} d{d} causal{int(causal)} W{W} x{q_mult}"
    announce(what)
    q, k, v = inputs.dense_qkv(B, n_q, n_k, H, d, seed, torch.bfloat16, q_mult)
    do = inputs.normal((B, n_q, H, d), inputs.subseed(seed, "dout"))
    s = configs.default_scale(d)
    qc, kc, vc, dc = (x.cuda() for x in (q, k, v, do))
    o, lse = fa.attention(qc, kc, vc, scale=s, causal=causal, window_left=W)
    dq, dk, dv = fa.attention_backward(qc, kc, vc, o, lse, dc, scale=s, causal=causal,
                                       window_left=W)
    torch.cuda.synchronize()
    refs = oracle.attention_backward(_np(q), _np(k), _np(v), _np(do), s, causal, W)
    msg = []
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        g = _np(got.cpu())
        assert np.all(np.isfinite(g)), f"{what}: non-finite {name}"
        top = max(float(np.abs(ref).max()), 1e-30)
        err = np.abs(g - ref) / top
        msg.append(f"{name} max {err.max():.2e} mean {err.mean():.2e} (of {top:.2e})")
        assert err.max() <= BWD_MAX_REL, f"{what}: {name} max rel {err.max():.3e}"
        assert err.mean() <= BWD_MEAN_REL, f"{what}: {name} mean rel {err.mean():.3e}"
    print(f"[parity] {what}: " + "; ".join(msg), file=sys.stderr, flush=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_q,n_k,causal,W,qm", [(300, 300, False, -1, 1.0), (257, 700, True, -1, 1.0),
                                                 (1000, 1000, True, 100, 1.0), (129, 64, False, -1, 1.0),
                                                 (512, 512, True, -1, 4.0)])
def test_backward(d, n_q, n_k, causal, W, qm):
    """dQ, dK, dV against the fp64 oracle's chain rule on the same bf16 inputs,
    with o and lse from the forward kernel."""
    _bwd_case(2, 3, n_q, n_k, d, causal, W, seed=71, q_mult=qm)


def _kvcache_case(B, H, max_len, d, lens, n_new, causal, W, seed, pairs=None):
    lens = torch.as_tensor(lens, dtype=torch.int32)
    what = f"kvcache B{B} H{H} max_len{max_len} d{d} new{n_new} causal{int(causal)} W{W}"
    announce(what)
    kc = inputs.decode_cache(B, max_len, H, d, lens, seed, "cuda", "k")
    vc = inputs.decode_cache(B, max_len, H, d, lens, seed, "cuda", "v")
    q = inputs.normal((B, n_new, H, d), inputs.subseed(seed, "q")).cuda()
    s = configs.default_scale(d)
    o, lse = fa.attention_kvcache(q, kc, vc, lens.cuda(), scale=s, causal=causal, window_left=W)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(H)]
    o_ref = np.zeros((len(pairs), n_new, d))
    lse_ref = np.zeros((len(pairs), n_new))
    got_o = torch.zeros((len(pairs), n_new, d), dtype=torch.bfloat16)
    got_l = torch.zeros((len(pairs), n_new))
    qn = _np(q.cpu())
    for i, (b, h) in enumerate(pairs):
        n = int(lens[b])
        o_ref[i], lse_ref[i] = oracle.sdpa(qn[b, :, h], _np(kc[b, :n, h].cpu()),
                                           _np(vc[b, :n, h].cpu()), s, causal, W)
        got_o[i], got_l[i] = o[b, :, h], lse[b, h]
    check(got_o, got_l, o_ref, lse_ref, torch.bfloat16, what)
    del kc, vc


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_new,causal,W", [(1, True, -1), (5, True, -1), (300, True, -1),
                                            (300, True, 100), (77, False, -1)])
def test_kvcache_small(d, n_new, causal, W):
    """New tokens at the end of cached sequences (NaN past each length), bottom-right causal."""
    _kvcache_case(3, 4, 1100, d, [1100, 700, 300], n_new, causal, W, seed=47)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal,W", [(True, -1), (True, 100), (False, 150)])
def test_kvcache_longest_first(d, causal, W):
    """batch * heads a multiple of 8 under a mask, heads a multiple of 8: the
    KV-cache work order that starts sequences longest cache first (ranked in
    the kernel, ties by index), with equal lengths, an empty cache and caches
    shorter than the new tokens (rows without keys)."""
    _kvcache_case(5, 8, 1100, d, [700, 1100, 0, 1100, 200], 300, causal, W, seed=53)


def test_kvcache_queries_without_keys():
    """A sequence shorter than the chunk: its first queries see no key (O = 0, lse = -inf)."""
    _kvcache_case(2, 2, 64, 128, [3, 64], 5, True, -1, seed=48)


def test_kvcache_full_cache_equals_dense():
    """Every length equal to max_len: the cache form is plain dense attention."""
    B, H, d, L, n = 2, 4, 128, 640, 256
    q, k, v = (x.cuda() for x in inputs.dense_qkv(B, L, L, H, d, 49))
    announce("kvcache vs dense")
    ok, lk = fa.attention_kvcache(q[:, L - n:].contiguous(), k, v,
                                  torch.full((B,), L, dtype=torch.int32, device="cuda"))
    od, ld = fa.attention(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(ok, od[:, L - n:]) and torch.equal(lk, ld[:, :, L - n:])


def test_workload_kvcache():
    """B8 H32 d128, 512 new tokens against caches of U[1024, 16384] keys (NaN
    padded): 4 sequences x 2 heads checked against the oracle on all rows."""
    c = configs.KVCACHE
    lens = inputs.lengths(c["batch"], c["len_lo"], c["len_hi"], c["seed"]).to(torch.int32)
    bs = [int(lens.argmax()), int(lens.argmin()), 3, 6]
    pairs = [(b, h) for b in bs for h in (0, 31)]
    _kvcache_case(c["batch"], c["heads"], c["max_len"], c["d"], lens, c["n_new"], c["causal"],
                  -1, c["seed"], pairs)
    torch.cuda.empty_cache()


def test_workload_decode():
    """B64 H32, lengths U[1024, 32768], d128, 256-key chunks, full-size NaN
    padded caches; all 32 heads of 10 sequences (the longest, the shortest
    and 8 drawn at random) checked against the oracle."""
    c = configs.DECODE
    lens = inputs.lengths(c["batch"], c["len_lo"], c["len_hi"], c["seed"]).to(torch.int32)
    rng = np.random.default_rng(5)
    bs = [int(lens.argmax()), int(lens.argmin())]
    bs += [int(b) for b in rng.permutation(c["batch"]) if int(b) not in bs][:8]
    pairs = [(b, h) for b in bs for h in range(c["heads"])]
    _decode_case(c["batch"], c["heads"], c["max_len"], c["d"], lens, c["chunk"], c["seed"], pairs)
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# Kernel branches reached only by particular shapes: the longest-first work
# order (batch * heads a multiple of 8 with a mask, several tiles per head),
# packed batches whose key lengths differ from their query lengths, a single
# key for many queries, and windows far wider than any sequence.


@pytest.mark.parametrize("causal,W", [(True, -1), (True, 256), (False, 300)])
def test_backward_headline_shape(causal, W):
    """B4 H16 N2048 d128: 64 (batch, head) units, so the dK/dV and dQ kernels
    take their longest-first order under a mask; every element of dQ, dK and
    dV against the oracle."""
    c = configs.PREFILL_2K
    _bwd_case(c["batch"], c["heads"], c["seqlen"], c["seqlen"], c["d"], causal, W, seed=c["seed"])


@pytest.mark.parametrize("B,H,n_q,n_k,causal,W", [
    (2, 64, 520, 777, False, -1),   # ragged last 256-row unit (8 rows), n_q < n_k
    (4, 64, 520, 777, True, -1),    # the same under a causal mask
    (2, 64, 1100, 600, True, 100),  # n_q > n_k: rows without keys; window
    (2, 64, 1000, 1000, False, 200),  # window only
])
def test_backward_dq_eight_waves(B, H, n_q, n_k, causal, W):
    """At d = 128 the dQ kernel runs eight waves (256 query rows) per
    workgroup when batch * heads * ceil(n_q / 256) reaches the CU count (256
    here), or twice it under a mask: these shapes take that variant with
    ragged tails and masks."""
    masked = causal or W >= 0
    assert B * H * -(-n_q // 256) >= (2 if masked else 1) * 256
    _bwd_case(B, H, n_q, n_k, 128, causal, W, seed=79)


@pytest.mark.parametrize("B,H,n_q,n_k,W", [
    (2, 64, 100, 1000, 50),   # key tiles 0-5 of every head are seen by no query row
    (1, 128, 300, 1400, 400),  # the same mixed with long items
])
def test_backward_persistent_empty_items(B, H, n_q, n_k, W):
    """More (batch, head, key tile) items than CUs at d = 128: the dK/dV
    kernel walks several items per workgroup, here with many items that no
    query row can see (a left window far behind the queries), so an item
    without tiles follows and precedes items with tiles."""
    _bwd_case(B, H, n_q, n_k, 128, False, W, seed=97)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,n_q,n_k,causal,W", [
    (2, 4, 700, 700, True, -1),
    (2, 4, 700, 700, True, 150),
    (1, 8, 600, 600, False, 200),
    (1, 8, 500, 900, True, -1),    # n_q < n_k
    (1, 8, 650, 400, True, 100),   # n_q > n_k: rows without keys
])
def test_backward_longest_first(d, B, H, n_q, n_k, causal, W):
    """batch * heads = 8 with several 128-row tiles per head: the masked
    branch of the backward work order at both head dims."""
    _bwd_case(B, H, n_q, n_k, d, causal, W, seed=73)


@pytest.mark.parametrize("B,H,n_q,n_k,causal,W", [
    (2, 4, 600, 600, True, -1),    # 5 query tiles per head, longest first
    (1, 8, 700, 700, True, 150),
    (1, 8, 500, 500, False, 100),  # window only: earlier tiles are the long ones
    (2, 4, 389, 389, True, -1),    # ragged last tile
    (1, 8, 450, 800, True, 64),    # n_q < n_k
    (1, 16, 700, 300, True, -1),   # n_q > n_k: whole tiles without keys
])
def test_d64_longest_first(B, H, n_q, n_k, causal, W):
    """The d = 64 kernel's longest-first order with several tiles per head."""
    _dense_case(B, H, n_q, n_k, 64, causal, W, torch.bfloat16, seed=81 + n_q + W)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_new,W", [(400, -1), (600, 200)])
def test_kvcache_longest_first(d, n_new, W):
    """KV-cache launches with batch * heads = 8 and several query tiles per
    head (the longest-first order over caches of different lengths)."""
    _kvcache_case(2, 4, 1300, d, [1300, 900], n_new, True, W, seed=83)


def _varlen_pair_case(lens_q, lens_k, H, d, causal, W, seed):
    lq, lk = torch.as_tensor(lens_q), torch.as_tensor(lens_k)
    cu_q, cu_k = inputs.cu_seqlens(lq), inputs.cu_seqlens(lk)
    q, k, v = inputs.varlen_qkv_pair(lq, lk, H, d, seed)
    s = configs.default_scale(d)
    what = f"varlen cross nq{list(lens_q)} nk{list(lens_k)} H{H} d{d} causal{int(causal)} W{W}"
    announce(what)
    o, lse = fa.attention_varlen(q.cuda(), k.cuda(), v.cuda(), cu_q.cuda(), cu_k.cuda(),
                                 max(int(lq.max()), 1), max(int(lk.max()), 1), scale=s,
                                 causal=causal, window_left=W)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_varlen(_np(q), _np(k), _np(v), cu_q.numpy(), cu_k.numpy(),
                                             s, causal, W)
    check(o.cpu(), lse.cpu(), o_ref, lse_ref, torch.bfloat16, what)
    return o.cpu(), lse.cpu(), cu_q


# per sequence: n_k > n_q, n_k < n_q (causal leaves the first rows without
# keys), n_k = 0, n_q = 0, one key, equal lengths
VARLEN_Q = [300, 129, 64, 0, 200, 5, 517, 1]
VARLEN_K = [500, 64, 0, 100, 200, 1, 300, 700]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal,W", [(True, -1), (True, 90), (False, -1), (False, 150)])
def test_varlen_cross_lengths(d, causal, W):
    """Packed sequences whose key counts differ from their query counts:
    per-sequence bottom-right alignment delta = n_k - n_q on the varlen path."""
    o, lse, cu_q = _varlen_pair_case(VARLEN_Q, VARLEN_K, 3, d, causal, W, seed=91)
    # the sequence with no keys: zeros and -inf
    a, b = int(cu_q[2]), int(cu_q[3])
    assert torch.all(o[a:b] == 0) and torch.all(torch.isneginf(lse[:, a:b]))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_single_key_many_queries(d, causal):
    """seqlen_k = 1: every row that sees the key returns V_0 exactly (p = 1)
    with lse = scale q . k_0; with the causal mask only the last row sees it."""
    n_q = 333
    o, lse, o_ref, lse_ref = _dense_case(2, 2, n_q, 1, d, causal, -1, torch.bfloat16,
                                         seed=95 + d)
    _, _, v = inputs.dense_qkv(2, n_q, 1, 2, d, 95 + d, torch.bfloat16)
    live = slice(n_q - 1, n_q) if causal else slice(0, n_q)
    assert torch.equal(o[:, live], v.expand(2, n_q, 2, d)[:, live])
    if causal:
        assert torch.all(o[:, :n_q - 1] == 0) and torch.all(torch.isneginf(lse[:, :, :n_q - 1]))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_window_near_int_max(d, causal):
    """window_left = 2^31 - 1 with n_q > n_k: the same result as no window
    (the kernels' window bound must not wrap around)."""
    _dense_case(1, 2, 400, 150, d, causal, 2 ** 31 - 1, torch.bfloat16, seed=97)
