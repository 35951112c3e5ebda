"""CPU checks of tests/fp8_bound.py against the model it states: values the
model fixes by hand, and the bound covering the model's own error."""

import numpy as np
import torch

import oracle
from tests import fp8_bound as fb


def _codes(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_exponents():
    e = fb.exponents(_codes([448.0, 1.0, 1.5, 2.0 ** -6, 2.0 ** -9, -3.0, 0.0]))
    assert list(e[:6]) == [8, 0, 0, -6, -9, 1] and e[6] < -1000


def test_group_of_eight_loses_small_products_of_the_big_ones_group():
    # one 448 x 448 product and 63 products of 2^-6 x 1: the big product's
    # group keeps 13 bits below 2^16 (its exponent sum), i.e. multiples of
    # 2^3, so its 7 small companions vanish; the other 7 groups are exact
    a = _codes([448.0] + [2.0 ** -6] * 63)
    b = _codes([448.0] + [1.0] * 63)
    assert fb.emulate_dot(a, b) == 448.0 ** 2 + 56 * 2.0 ** -6
    # the same with cancelling big products: +448^2 - 448^2 + 62 x 2^-6
    a = _codes([448.0, -448.0] + [1.0] * 62)
    b = _codes([448.0, 448.0] + [2.0 ** -6] * 62)
    assert fb.emulate_dot(a, b) == 56 * 2.0 ** -6


def test_products_within_seven_binades_are_exact():
    # exponent sums 0 and -7: the small product's lowest bit (2^-13) is the
    # quantum, so nothing is lost
    a = _codes([1.875] + [2.0 ** -7 * 1.875] + [0.0] * 62)
    b = _codes([1.0] + [1.0] + [0.0] * 62)
    exact = float(oracle.e4m3_decode(a) @ oracle.e4m3_decode(b))
    assert fb.emulate_dot(a, b) == exact


def test_bound_covers_the_model():
    rng = np.random.default_rng(0)
    for t in range(300):
        x = rng.standard_normal(128) * rng.choice([1.0, 4.0]) * (rng.random(128) < rng.choice([1.0, 0.5]))
        y = rng.standard_normal(128)
        a = _codes(x / max(np.abs(x).max(), 1e-30) * 448)
        b = _codes(y / np.abs(y).max() * 448)
        exact = float(oracle.e4m3_decode(a) @ oracle.e4m3_decode(b))
        bound = float(fb.score_error_bound(a[None], b[None])[0, 0])
        assert abs(fb.emulate_dot(a, b) - exact) <= bound


def test_lse_bound_first_order_form():
    # one key: lse error = the score error, bounded by the score bound
    rng = np.random.default_rng(1)
    q = _codes(rng.standard_normal((1, 128)) * 50)
    k = _codes(rng.standard_normal((1, 128)) * 50)
    b = fb.lse_error_bound(q, k, 0.5, 0.25, 0.1, np.ones((1, 1), bool))
    sb = fb.score_error_bound(q, k)[0, 0] * 0.5 * 0.25 * 0.1
    assert abs(b[0] - (sb + sb ** 2 / 2 + 4e-6)) < 1e-15
    # no allowed key: 0
    assert fb.lse_error_bound(q, k, 1.0, 1.0, 1.0, np.zeros((1, 1), bool))[0] == 0.0
