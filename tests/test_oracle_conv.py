"""Pins of the causal conv1d + SiLU oracle (CPU): torch's grouped conv1d (an independent library
routine), the impulse response, causality, the width-1 special case."""
import numpy as np
import pytest
import torch

import oracle


def _case(seed, batch, dim, L, W):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((batch, dim, L)), rng.standard_normal((dim, W)),
            rng.standard_normal(dim))


@pytest.mark.parametrize("W", [1, 2, 3, 4])
@pytest.mark.parametrize("shape", [(2, 3, 17), (1, 5, 2), (3, 2, 40)])
def test_conv_matches_torch_conv1d(W, shape):
    x, w, b = _case(W * 100 + shape[2], *shape, W)
    for bias in (b, None):
        got = oracle.conv_silu_ref(x, w, bias)
        tx = torch.from_numpy(x)
        pre = torch.nn.functional.conv1d(tx, torch.from_numpy(w)[:, None, :],
                                         None if bias is None else torch.from_numpy(bias),
                                         padding=W - 1, groups=shape[1])[..., :shape[2]]
        ref = torch.nn.functional.silu(pre).numpy()
        np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-14)


def test_conv_impulse_response():
    """x = e_j: the pre-activation at t is bias + w[j - t + W - 1] for j <= t <= j + W - 1 (the
    taps in reverse order: the newest token meets the last tap), bias elsewhere."""
    W, L, j = 4, 12, 5
    rng = np.random.default_rng(3)
    w = rng.standard_normal((1, W))
    b = np.array([0.3])
    x = np.zeros((1, 1, L))
    x[0, 0, j] = 1.0
    u = oracle.conv_silu_ref(x, w, b)[0, 0]
    for t in range(L):
        pre = b[0] + (w[0, j - t + W - 1] if j <= t <= j + W - 1 else 0.0)
        assert abs(u[t] - pre / (1.0 + np.exp(-pre))) < 1e-15


def test_conv_is_causal():
    x, w, b = _case(7, 1, 3, 30, 4)
    base = oracle.conv_silu_ref(x, w, b)
    for t in (0, 9, 29):
        x2 = x.copy()
        x2[:, :, t] += 5.0
        moved = oracle.conv_silu_ref(x2, w, b)
        np.testing.assert_array_equal(moved[:, :, :t], base[:, :, :t])
        assert np.all(moved[:, :, t] != base[:, :, t])


def test_conv_width_one_is_pointwise():
    x, w, b = _case(9, 2, 4, 10, 1)
    pre = w[None, :, 0:1] * x + b[None, :, None]
    np.testing.assert_allclose(oracle.conv_silu_ref(x, w, b), pre / (1 + np.exp(-pre)),
                               rtol=1e-15, atol=1e-15)


def test_scan_conv_ref_composes():
    rng = np.random.default_rng(11)
    x, w, b = _case(12, 1, 2, 20, 4)
    delta = rng.standard_normal((1, 2, 20))
    A = -np.arange(1, 17, dtype=np.float64)[None].repeat(2, 0)
    B, C = rng.standard_normal((1, 16, 20)), rng.standard_normal((1, 16, 20))
    out, last, u = oracle.scan_conv_ref(x, w, b, delta, A, B, C, None, None, None, True)
    o2, l2 = oracle.scan_ref(oracle.conv_silu_ref(x, w, b), delta, A, B, C, None, None, None, True)
    np.testing.assert_array_equal(out, o2)
    np.testing.assert_array_equal(last, l2)
