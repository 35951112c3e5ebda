"""CPU checks of the C ABI: the library loads, exports every symbol that
include/fa.h declares, and rejects bad arguments with the documented codes
before touching the GPU (no compute call is made here)."""

import ctypes
import os
import re

import pytest

import io_aware_exact_19_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# fake, 16-byte aligned, never dereferenced: every call below fails its
# argument check (or is a no-op) before any pointer is used
P = 0x10000
NULL_STREAM = 0


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.skip("libfa.so not built")
    return fa.load_library()


def test_header_declares_the_binding_names():
    assert _declared_functions() == sorted(fa.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_status_strings(lib):
    assert fa.fa_status_string(0) == "FA_OK"
    for code in (-1, -2, -3, -4):
        assert fa.fa_status_string(code).startswith("FA_ERR")
    assert fa.fa_status_string(7) == "unknown fa_status"


def _fwd(fn=fa.fa_fwd, **kw):
    args = dict(q=P, k=P, v=P, o=P, lse=P, batch=2, heads=4, seqlen_q=64, seqlen_k=64, d=128,
                scale=0.125, causal=0, window_left=-1, cu_seqlens_q=None, cu_seqlens_k=None,
                stream=NULL_STREAM)
    args.update(kw)
    return fn(**args)


@pytest.mark.parametrize("fn", [fa.fa_fwd, fa.fa_fwd_fp32])
@pytest.mark.parametrize("bad,code", [
    (dict(q=0), fa.FA_ERR_INVALID_ARG),
    (dict(k=0), fa.FA_ERR_INVALID_ARG),
    (dict(v=0), fa.FA_ERR_INVALID_ARG),
    (dict(o=0), fa.FA_ERR_INVALID_ARG),
    (dict(q=P + 2), fa.FA_ERR_INVALID_ARG),
    (dict(o=P + 8), fa.FA_ERR_INVALID_ARG),
    (dict(lse=P + 2), fa.FA_ERR_INVALID_ARG),
    (dict(batch=-1), fa.FA_ERR_INVALID_ARG),
    (dict(heads=-3), fa.FA_ERR_INVALID_ARG),
    (dict(seqlen_q=-1), fa.FA_ERR_INVALID_ARG),
    (dict(seqlen_k=-5), fa.FA_ERR_INVALID_ARG),
    (dict(d=0), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_INVALID_ARG),
    (dict(d=256), fa.FA_ERR_INVALID_ARG),
    (dict(d=-64), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-0.1), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(cu_seqlens_q=P), fa.FA_ERR_INVALID_ARG),
    (dict(cu_seqlens_k=P), fa.FA_ERR_INVALID_ARG),
])
def test_fwd_rejects(lib, fn, bad, code):
    assert _fwd(fn, **bad) == code


def test_fwd_fp32_varlen_unsupported(lib):
    assert _fwd(fa.fa_fwd_fp32, cu_seqlens_q=P, cu_seqlens_k=P) == fa.FA_ERR_UNSUPPORTED


def test_fwd_varlen_misaligned_offsets(lib):
    assert _fwd(cu_seqlens_q=P + 2, cu_seqlens_k=P) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("empty", [dict(batch=0), dict(heads=0), dict(seqlen_q=0)])
def test_fwd_empty_is_noop(lib, empty):
    # nothing to compute: returns before any HIP call, even with null pointers
    assert _fwd(q=0, k=0, v=0, o=0, **empty) == fa.FA_OK


def _dec(**kw):
    args = dict(q=P, k_cache=P, v_cache=P, seqlens_k=P, o=P, lse=P, batch=4, heads=8,
                max_len=1000, d=128, scale=0.1, chunk=256, workspace=P, workspace_bytes=1 << 30,
                stream=NULL_STREAM)
    args.update(kw)
    return fa.fa_decode(**args)


@pytest.mark.parametrize("bad,code", [
    (dict(q=0), fa.FA_ERR_INVALID_ARG),
    (dict(k_cache=0), fa.FA_ERR_INVALID_ARG),
    (dict(v_cache=0), fa.FA_ERR_INVALID_ARG),
    (dict(seqlens_k=0), fa.FA_ERR_INVALID_ARG),
    (dict(o=0), fa.FA_ERR_INVALID_ARG),
    (dict(seqlens_k=P + 2), fa.FA_ERR_INVALID_ARG),
    (dict(k_cache=P + 4), fa.FA_ERR_INVALID_ARG),
    (dict(batch=-1), fa.FA_ERR_INVALID_ARG),
    (dict(max_len=0), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_INVALID_ARG),
    (dict(d=32), fa.FA_ERR_INVALID_ARG),
    (dict(chunk=100), fa.FA_ERR_UNSUPPORTED),
    (dict(chunk=0), fa.FA_ERR_INVALID_ARG),
    # one 512-key chunk of 16384 heads x 128 dims spans 2 GiB of cache rows
    (dict(batch=1, heads=16384, max_len=512, chunk=512), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(workspace_bytes=16), fa.FA_ERR_WORKSPACE),
])
def test_decode_rejects(lib, bad, code):
    assert _dec(**bad) == code


def _kvc(**kw):
    args = dict(q=P, k_cache=P, v_cache=P, seqlens_k=P, o=P, lse=P, batch=4, heads=8,
                seqlen_q=32, max_len=1000, d=128, scale=0.1, causal=1, window_left=-1,
                stream=NULL_STREAM)
    args.update(kw)
    return fa.fa_fwd_kvcache(**args)


@pytest.mark.parametrize("bad,code", [
    (dict(seqlens_k=0), fa.FA_ERR_INVALID_ARG),
    (dict(seqlens_k=P + 2), fa.FA_ERR_INVALID_ARG),
    (dict(q=0), fa.FA_ERR_INVALID_ARG),
    (dict(k_cache=0), fa.FA_ERR_INVALID_ARG),
    (dict(v_cache=P + 8), fa.FA_ERR_INVALID_ARG),
    (dict(max_len=0), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_INVALID_ARG),
    (dict(batch=0), fa.FA_OK),
    (dict(seqlen_q=0), fa.FA_OK),
])
def test_kvcache_rejects(lib, bad, code):
    assert _kvc(**bad) == code


def _bwd(**kw):
    args = dict(q=P, k=P, v=P, o=P, dout=P, lse=P, dq=P, dk=P, dv=P, batch=2, heads=4, seqlen_q=64,
                seqlen_k=64, d=128, scale=0.1, causal=0, window_left=-1, workspace=P,
                workspace_bytes=1 << 20, stream=NULL_STREAM)
    args.update(kw)
    return fa.fa_bwd(**args)


@pytest.mark.parametrize("bad,code", [
    (dict(q=0), fa.FA_ERR_INVALID_ARG),
    (dict(dout=0), fa.FA_ERR_INVALID_ARG),
    (dict(lse=0), fa.FA_ERR_INVALID_ARG),
    (dict(dk=0), fa.FA_ERR_INVALID_ARG),
    (dict(dv=P + 4), fa.FA_ERR_INVALID_ARG),
    (dict(lse=P + 2), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(causal=3), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_INVALID_ARG),
    (dict(d=0), fa.FA_ERR_INVALID_ARG),
    (dict(workspace_bytes=2 * 2 * 4 * 64 * 4 - 1), fa.FA_ERR_WORKSPACE),
    (dict(batch=0), fa.FA_OK),
])
def test_bwd_rejects(lib, bad, code):
    assert _bwd(**bad) == code


def test_bwd_workspace_size(lib):
    assert fa.fa_bwd_workspace_size(2, 4, 64) == 2 * 2 * 4 * 64 * 4
    assert fa.fa_bwd_workspace_size(0, 4, 64) == 0


def test_decode_workspace_size(lib):
    # fp32 chunk outputs [B, H, C, d], 256-byte aligned, then fp32 chunk lse [B, H, C]
    B, H, L, d, c = 64, 32, 32768, 128, 256
    C = L // c
    o_bytes = B * H * C * d * 4
    assert fa.fa_decode_workspace_size(B, H, L, d, c) == o_bytes + B * H * C * 4
    assert fa.fa_decode_workspace_size(3, 2, 1000, 64, 256) == ((3 * 2 * 4 * 64 * 4 + 255) // 256) * 256 + 3 * 2 * 4 * 4
    assert fa.fa_decode_workspace_size(0, 2, 10, 64, 64) == 0
    assert fa.fa_decode_workspace_size(1, 1, 1, 64, 0) == 0


def test_decode_workspace_exact_size_accepted_by_checks(lib):
    need = fa.fa_decode_workspace_size(4, 8, 1000, 128, 256)
    assert _dec(workspace_bytes=need - 1) == fa.FA_ERR_WORKSPACE
    assert _dec(batch=0, workspace_bytes=need) == fa.FA_OK  # no-op


def test_binding_fails_loudly_without_library(tmp_path):
    import io_aware_exact_19_amd.binding as b
    saved = b._lib
    try:
        b._lib = None
        with pytest.raises(RuntimeError, match="missing"):
            b.load_library(str(tmp_path / "nope.so"))
    finally:
        b._lib = saved


def _fp8(**kw):
    args = dict(q=P, k=P, v=P, o=P, lse=P, descale_q=P, descale_k=P, descale_v=P, batch=2,
                heads=4, seqlen_q=64, seqlen_k=100, d=128, scale=0.125, causal=0, window_left=-1,
                stream=NULL_STREAM)
    args.update(kw)
    return fa.fa_fwd_fp8(**args)


@pytest.mark.parametrize("bad,code", [
    (dict(q=0), fa.FA_ERR_INVALID_ARG),
    (dict(k=0), fa.FA_ERR_INVALID_ARG),
    (dict(v=0), fa.FA_ERR_INVALID_ARG),
    (dict(o=0), fa.FA_ERR_INVALID_ARG),
    (dict(descale_q=0), fa.FA_ERR_INVALID_ARG),
    (dict(descale_k=0), fa.FA_ERR_INVALID_ARG),
    (dict(descale_v=0), fa.FA_ERR_INVALID_ARG),
    (dict(descale_v=P + 2), fa.FA_ERR_INVALID_ARG),
    (dict(q=P + 8), fa.FA_ERR_INVALID_ARG),
    (dict(lse=P + 1), fa.FA_ERR_INVALID_ARG),
    (dict(batch=-1), fa.FA_ERR_INVALID_ARG),
    (dict(seqlen_k=-1), fa.FA_ERR_INVALID_ARG),
    (dict(d=64), fa.FA_ERR_UNSUPPORTED),   # valid head dim, no fp8 kernel for it
    (dict(d=96), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(causal=3), fa.FA_ERR_INVALID_ARG),
    (dict(heads=1 << 19), fa.FA_ERR_UNSUPPORTED),  # 64 rows of heads * 128 bytes reach 4 GiB
])
def test_fwd_fp8_rejects(lib, bad, code):
    assert _fp8(**bad) == code


@pytest.mark.parametrize("empty", [dict(batch=0), dict(heads=0), dict(seqlen_q=0)])
def test_fwd_fp8_empty_is_noop(lib, empty):
    assert _fp8(q=0, k=0, v=0, o=0, descale_q=0, descale_k=0, descale_v=0, **empty) == fa.FA_OK


def _dec_na(**kw):
    args = dict(q=P, k_cache=P, v_cache=P, seqlens_k=P, o=P, lse=P, batch=4, heads=8,
                max_len=1000, d=128, scale=0.1, chunk=256, stream=NULL_STREAM)
    args.update(kw)
    return fa.fa_decode_noalloc(**args)


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define FA_DECODE_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == fa.FA_DECODE_SCRATCH_BYTES


@pytest.mark.parametrize("bad,code", [
    (dict(q=0), fa.FA_ERR_INVALID_ARG),
    (dict(seqlens_k=P + 2), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_INVALID_ARG),
    (dict(chunk=100), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(max_len=0), fa.FA_ERR_INVALID_ARG),
    # 64 x 32 heads x 32768 keys in 256-key chunks needs 135 MB of chunk states
    (dict(batch=64, heads=32, max_len=32768, chunk=256), fa.FA_ERR_WORKSPACE),
    (dict(batch=0), fa.FA_OK),
])
def test_decode_noalloc_rejects(lib, bad, code):
    assert _dec_na(**bad) == code


def test_decode_noalloc_limit_is_the_workspace_size(lib):
    """The largest accepted call needs at most the array's bytes; one more
    chunk row of sequences does not fit."""
    need = fa.fa_decode_workspace_size(64, 32, 32768, 128, 512)
    assert need <= fa.FA_DECODE_SCRATCH_BYTES
    assert fa.fa_decode_workspace_size(64, 32, 32768, 128, 256) > fa.FA_DECODE_SCRATCH_BYTES
    # rejected before any HIP call (only the size differs from an accepted shape)
    assert _dec_na(batch=64, heads=32, max_len=32768, chunk=256) == fa.FA_ERR_WORKSPACE
