"""Pins of the oracle's depthwise causal short convolution (the DeltaNet
rebuttal, answer W2) against facts outside its own formulas:

- one channel equals numpy's full convolution with the reversed taps, cut to
  the sequence length (the library routine fixes the direction of the taps);
- a unit impulse at a sequence start returns the taps in reverse order, and
  nothing before the impulse;
- the backward pass is the adjoint: <conv(x), dy> = <x, dx> = <w, dw> (the
  map is linear in x and in w), which fails for a shifted or flipped index
  in either gradient;
- packed sequences equal the sequences filtered one by one (nothing leaks
  across a boundary), including empty and one-token sequences.
"""
import numpy as np
import pytest


@pytest.mark.parametrize("W", [1, 2, 4, 7])
def test_conv_matches_numpy_convolve(oracle_lib, W):
    rng = np.random.default_rng(81 + W)
    T, H, D = 11, 2, 3
    x = rng.standard_normal((2, T, H, D))
    w = rng.standard_normal((H, D, W))
    y = oracle_lib.short_conv(x, w)
    for b in range(2):
        for h in range(H):
            for c in range(D):
                ref = np.convolve(x[b, :, h, c], w[h, c, ::-1])[:T]
                assert np.abs(y[b, :, h, c] - ref).max() < 1e-13


def test_conv_impulse_response(oracle_lib):
    W, T = 4, 9
    w = np.arange(1.0, W + 1).reshape(1, 1, W)
    x = np.zeros((1, T, 1, 1))
    x[0, 3, 0, 0] = 1.0
    y = oracle_lib.short_conv(x, w)[0, :, 0, 0]
    assert np.all(y[:3] == 0.0)
    assert np.array_equal(y[3:3 + W], w[0, 0, ::-1])
    assert np.all(y[3 + W:] == 0.0)


@pytest.mark.parametrize("W", [1, 3, 4])
def test_conv_backward_is_adjoint(oracle_lib, W):
    rng = np.random.default_rng(90 + W)
    cu = np.array([0, 5, 5, 6, 14], dtype=np.int32)
    H, D = 2, 4
    x = rng.standard_normal((1, 14, H, D))
    w = rng.standard_normal((H, D, W))
    dy = rng.standard_normal((1, 14, H, D))
    y = oracle_lib.short_conv(x, w, cu)
    dx, dw = oracle_lib.short_conv_bwd(x, w, dy, cu)
    lhs = np.sum(y * dy)
    assert abs(lhs - np.sum(x * dx)) < 1e-12 * max(1.0, abs(lhs))
    assert abs(lhs - np.sum(w * dw)) < 1e-12 * max(1.0, abs(lhs))
    # a gradient of a linear map does not depend on the point: one entry by a difference
    e = np.zeros_like(x)
    e[0, 7, 1, 2] = 1.0
    assert abs(np.sum((oracle_lib.short_conv(x + e, w, cu) - y) * dy) - dx[0, 7, 1, 2]) < 1e-12


def test_conv_packed_equals_separate(oracle_lib):
    rng = np.random.default_rng(95)
    lengths = [6, 0, 1, 9, 3]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    H, D, W = 2, 3, 4
    x = rng.standard_normal((1, int(cu[-1]), H, D))
    w = rng.standard_normal((H, D, W))
    dy = rng.standard_normal(x.shape)
    y = oracle_lib.short_conv(x, w, cu)
    dx, dw = oracle_lib.short_conv_bwd(x, w, dy, cu)
    dw_sum = np.zeros_like(w)
    for n, L in enumerate(lengths):
        t0 = int(cu[n])
        xs, dys = x[:, t0:t0 + L], dy[:, t0:t0 + L]
        assert np.array_equal(y[:, t0:t0 + L], oracle_lib.short_conv(xs, w))
        dxs, dws = oracle_lib.short_conv_bwd(xs, w, dys)
        assert np.array_equal(dx[:, t0:t0 + L], dxs)
        dw_sum += dws
    assert np.abs(dw - dw_sum).max() < 1e-12
