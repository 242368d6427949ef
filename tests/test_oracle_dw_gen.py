"""Pins for the oracle's generalised depthwise layer (R x S filters, dilation, depth
multiplier; PyTorch forum "Using optimised depthwise convolutions": a grouped
convolution with one group per input channel and k outputs per group, any filter size,
dilated in the thread's separable module) and of the DW->PW module built on it.

Each pin relies on something other than the generalised code itself: the library's
grouped, dilated convolution; pure-Python loops on tiny inputs; the oracle's plain
R x S depthwise layer (pinned in test_oracle_pins.py) with zeros inserted between the
taps or with the filters of each multiplier slot taken apart; exact shifts of one-hot
taps; and the plain 3x3 module when the generalisation is switched off.
"""
import itertools

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _rng(seed=0):
    return np.random.default_rng(seed)


def _torch_dw_gen(x, w, stride, pad, dil):
    """groups = C, out_channels = C*M: the forum page's depthwise layer."""
    xt = torch.from_numpy(x).permute(0, 3, 1, 2)
    wt = torch.from_numpy(w)[:, None]
    return F.conv2d(xt, wt, stride=stride, padding=pad, dilation=dil,
                    groups=x.shape[3]).permute(0, 2, 3, 1).numpy()


@pytest.mark.parametrize("R,dil,M,stride,pad", [
    (3, 1, 2, 1, 1), (3, 2, 1, 1, 2), (3, 2, 2, 2, 2), (5, 1, 1, 1, 2), (5, 1, 1, 2, 2),
    (5, 2, 3, 1, 3), (7, 1, 1, 1, 3), (1, 1, 4, 1, 0), (3, 3, 1, 2, 1), (5, 1, 2, 1, 0)])
def test_dw_gen_matches_torch_grouped_dilated_conv(R, dil, M, stride, pad):
    rng = _rng(R * 100 + dil * 10 + M)
    x = rng.standard_normal((2, 13, 11, 6))
    w = rng.standard_normal((6 * M, R, R))
    got = oracle.dw_gen(x, w, (stride, stride), (pad, pad), (dil, dil))
    ref = _torch_dw_gen(x, w, stride, pad, dil)
    assert got.shape == ref.shape
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_dw_gen_rectangular_filter_and_mixed_strides():
    rng = _rng(7)
    x = rng.standard_normal((1, 9, 12, 4))
    w = rng.standard_normal((8, 3, 5))
    got = oracle.dw_gen(x, w, (2, 1), (1, 2), (1, 2))
    xt = torch.from_numpy(x).permute(0, 3, 1, 2)
    ref = F.conv2d(xt, torch.from_numpy(w)[:, None], stride=(2, 1), padding=(1, 2),
                   dilation=(1, 2), groups=4).permute(0, 2, 3, 1).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_dw_gen_brute_force_tiny():
    rng = _rng(3)
    N, H, W, C, M, R, d, s, p = 1, 5, 6, 2, 2, 3, 2, 1, 2
    x = rng.integers(-3, 4, (N, H, W, C)).astype(np.float64)
    w = rng.integers(-2, 3, (C * M, R, R)).astype(np.float64)
    Ho = (H + 2 * p - ((R - 1) * d + 1)) // s + 1
    Wo = (W + 2 * p - ((R - 1) * d + 1)) // s + 1
    ref = np.zeros((N, Ho, Wo, C * M))
    for n, oh, ow, j in itertools.product(range(N), range(Ho), range(Wo), range(C * M)):
        for r, q in itertools.product(range(R), range(R)):
            ih, iw = oh * s - p + r * d, ow * s - p + q * d
            if 0 <= ih < H and 0 <= iw < W:
                ref[n, oh, ow, j] += x[n, ih, iw, j // M] * w[j, r, q]
    got = oracle.dw_gen(x, w, (s, s), (p, p), (d, d))
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("R,dil", [(3, 2), (3, 3), (5, 2)])
def test_dilated_filter_is_a_zero_inserted_dense_filter(R, dil):
    """Dilation d spaces the taps d apart: the same as a ((R-1)d+1)-wide filter with
    d-1 zeros between taps, run by the plain depthwise layer."""
    rng = _rng(R + dil)
    x = rng.standard_normal((2, 12, 10, 5))
    w = rng.standard_normal((5, R, R))
    E = (R - 1) * dil + 1
    wz = np.zeros((5, E, E))
    wz[:, ::dil, ::dil] = w
    pad = E // 2
    got = oracle.dw_gen(x, w, (1, 1), (pad, pad), (dil, dil))
    ref = oracle.dw(x, wz, (1, 1), (pad, pad))
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("M", [2, 3])
def test_depth_multiplier_interleaves_per_slot_depthwise_layers(M):
    """Output channel c*M + i is filter slot i of input channel c: the result is M
    plain depthwise layers (one per slot) interleaved along the channels."""
    rng = _rng(M)
    x = rng.standard_normal((1, 9, 8, 4))
    w = rng.standard_normal((4 * M, 3, 3))
    got = oracle.dw_gen(x, w, (1, 1), (1, 1), (1, 1))
    for i in range(M):
        ref = oracle.dw(x, w[i::M], (1, 1), (1, 1))
        assert np.array_equal(got[..., i::M], ref)


@pytest.mark.parametrize("r,q,dil", [(0, 0, 2), (2, 1, 2), (1, 2, 3), (4, 0, 1)])
def test_one_hot_dilated_tap_is_an_exact_shift(r, q, dil):
    R = 5 if r == 4 else 3
    pad = (R - 1) * dil // 2
    rng = _rng(11)
    x = rng.standard_normal((1, 10, 9, 3))
    w = np.zeros((3, R, R))
    w[:, r, q] = 1.0
    t = oracle.dw_gen(x, w, (1, 1), (pad, pad), (dil, dil))
    dh, dw = r * dil - pad, q * dil - pad
    for oh, ow in itertools.product(range(10), range(9)):
        ih, iw = oh + dh, ow + dw
        want = x[0, ih, iw] if (0 <= ih < 10 and 0 <= iw < 9) else np.zeros(3)
        assert np.array_equal(t[0, oh, ow], want)


def test_one_by_one_depthwise_filter_scales_each_channel():
    rng = _rng(5)
    x = rng.standard_normal((2, 4, 5, 3))
    w = rng.standard_normal((6, 1, 1))
    t = oracle.dw_gen(x, w, (1, 1), (0, 0), (1, 1))
    ref = np.repeat(x, 2, axis=3) * w[:, 0, 0]
    assert np.array_equal(t, ref)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_dwpw_gen_without_generalisation_is_the_plain_module(dtype):
    rng = _rng(21)
    x = oracle.round_to(rng.standard_normal((2, 9, 10, 8)), dtype)
    w1 = oracle.round_to(rng.normal(0, .3, (8, 3, 3)), dtype)
    w2 = oracle.round_to(rng.normal(0, .3, (16, 8)), dtype)
    s1, b1 = rng.uniform(.5, 1.5, 8), rng.normal(0, .1, 8)
    s2, b2 = rng.uniform(.5, 1.5, 16), rng.normal(0, .1, 16)
    kw = dict(scale1=s1, bias1=b1, act1="relu6", scale2=s2, bias2=b2, act2="relu",
              dtype=dtype)
    a = oracle.dwpw_gen(x, w1, w2, (1, 1), (1, 1), (1, 1), **kw)
    b = oracle.dwpw(x, w1, w2, (1, 1), (1, 1), **kw)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_dwpw_gen_is_the_layer_by_layer_pipeline(dtype):
    """torch's dilated grouped conv, the folded batch-norm epilogue, a storage cast, a
    1x1 conv, the second epilogue and cast: the unfused network, step by step."""
    rng = _rng(31)
    M, R, d, s, p = 2, 5, 2, 2, 4
    x = oracle.round_to(rng.standard_normal((2, 17, 15, 8)), dtype)
    w1 = oracle.round_to(rng.normal(0, .2, (16, R, R)), dtype)
    w2 = oracle.round_to(rng.normal(0, .2, (24, 16)), dtype)
    s1, b1 = rng.uniform(.5, 1.5, 16), rng.normal(0, .1, 16)
    s2, b2 = rng.uniform(.5, 1.5, 24), rng.normal(0, .1, 24)
    y, t = oracle.dwpw_gen(x, w1, w2, (s, s), (p, p), (d, d), scale1=s1, bias1=b1,
                           act1="relu6", scale2=s2, bias2=b2, act2="relu", dtype=dtype,
                           return_t=True)
    cast = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    tt = _torch_dw_gen(x, w1, s, p, d)
    tt = np.clip(tt * s1 + b1, 0, 6)
    tt = torch.from_numpy(tt).to(cast).double().numpy()
    assert np.array_equal(t, tt)
    yy = tt @ w2.T
    yy = np.maximum(yy * s2 + b2, 0)
    yy = torch.from_numpy(yy).to(cast).double().numpy()
    # the 1x1 sums differ from numpy's matmul only in summation order (fp64), so the
    # rounded outputs agree except where a sum sits within fp64 noise of a midpoint
    assert np.mean(y == yy) > 0.999
    np.testing.assert_allclose(y, yy, rtol=1e-2, atol=1e-3)
