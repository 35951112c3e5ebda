"""Pins of the fp8 part of the oracle (CPU): the e4m3 decoder against the
format's definition and PyTorch's float8_e4m3fn, and the dequantised
attention against invariants that any correct dequantisation keeps."""

import math

import numpy as np
import pytest
import torch

import oracle
from io_aware_exact_19_amd import inputs


def test_e4m3_decode_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = oracle.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], mine[ok])


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x38, 1.0), (0x3C, 1.5), (0x40, 2.0), (0x7E, 448.0), (0xFE, -448.0),
    (0x08, 2.0 ** -6), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0xC0, -2.0), (0x30, 0.5),
])
def test_e4m3_decode_hand_values(code, value):
    # s eeee mmm: (1 + m/8) 2^(e-7); e = 0: (m/8) 2^-6
    assert oracle.e4m3_decode(np.array([code], dtype=np.uint8))[0] == value


def test_e4m3_decode_nan_and_negative_zero():
    out = oracle.e4m3_decode(np.array([0x7F, 0xFF, 0x80], dtype=np.uint8))
    assert np.isnan(out[0]) and np.isnan(out[1])
    assert out[2] == 0.0 and math.copysign(1.0, out[2]) == -1.0


def _case(seed=3, n_q=40, n_k=50, causal=False, W=-1):
    q8, k8, v8, dq, dk, dv = inputs.fp8_qkv(2, n_q, n_k, 3, 16, seed)
    return [t.numpy() for t in (q8, k8, v8, dq, dk, dv)]


def test_fp8_descale_v_is_linear():
    q8, k8, v8, dq, dk, dv = _case()
    o1, l1 = oracle.attention_fp8(q8, k8, v8, dq, dk, dv, 0.25, causal=True)
    o2, l2 = oracle.attention_fp8(q8, k8, v8, dq, dk, 2.0 * dv, 0.25, causal=True)  # exact in fp32
    np.testing.assert_allclose(o2, 2.0 * o1, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(l1, l2)


def test_fp8_only_the_product_of_q_and_k_factors_matters():
    q8, k8, v8, dq, dk, dv = _case()
    o1, l1 = oracle.attention_fp8(q8, k8, v8, dq, dk, dv, 0.25)
    o2, l2 = oracle.attention_fp8(q8, k8, v8, 4.0 * dq, dk / 4.0, dv, 0.25)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l2, l1, rtol=1e-12, atol=1e-12)


def test_fp8_factors_belong_to_their_own_head():
    # changing head (1, 2)'s factor moves only that head's output
    q8, k8, v8, dq, dk, dv = _case()
    o1, _ = oracle.attention_fp8(q8, k8, v8, dq, dk, dv, 0.25)
    dv2 = dv.copy()
    dv2[1 * 3 + 2] *= 2.0
    o2, _ = oracle.attention_fp8(q8, k8, v8, dq, dk, dv2, 0.25)
    np.testing.assert_allclose(o2[1, :, 2], 2.0 * o1[1, :, 2], rtol=1e-12, atol=1e-14)
    mask = np.ones(o1.shape, dtype=bool)
    mask[1, :, 2] = False
    np.testing.assert_array_equal(o2[mask], o1[mask])


def test_fp8_generator_round_trip():
    # the codes times their factor reproduce the drawn values to e4m3 precision
    x = inputs.normal((2, 30, 3, 16), inputs.subseed(9, "q"), torch.float32).double().numpy()
    q8, dq = inputs.fp8_tensor((2, 30, 3, 16), inputs.subseed(9, "q"))
    y = oracle.e4m3_decode(q8.numpy()) * dq.double().numpy().reshape(2, 1, 3, 1)
    f = dq.double().numpy().reshape(2, 1, 3, 1)
    # relative 2^-4 for normal codes, absolute 2^-10 * factor for subnormal ones
    assert np.all(np.abs(y - x) <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * f) + 1e-12)
    assert np.abs(oracle.e4m3_decode(q8.numpy())).max() <= 448.0
