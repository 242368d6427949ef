"""CPU pins of the oracle's three-layer PW -> DW -> PW module (the inverted-residual block
of "Fusing Depthwise and Pointwise Convolutions for Efficient Inference on GPUs",
Sec. II-B and Fig. 4: pointwise expansion, depthwise 3x3, pointwise projection, with the
block's identity shortcut when the extent and channel count are unchanged).

Each pin checks the oracle against something other than itself: torch's conv2d pipeline
with its own casts, the definition written out with Python loops, identity layers,
exact integer arithmetic for the shortcut and linearity, and the sampled checker against
the full one.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _nchw(x):
    return torch.from_numpy(x).permute(0, 3, 1, 2)


def _nhwc(t):
    return t.permute(0, 2, 3, 1).numpy()


def _cast(a, dtype):
    if dtype == "f16":
        return a.astype(np.float16).astype(np.float64)
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def _act(a, act):
    if act == "relu":
        return np.maximum(a, 0.0)
    if act == "relu6":
        return np.clip(a, 0.0, 6.0)
    return a


def _torch_block(x, w1, w2, w3, stride, s, b, acts, residual, dtype):
    """The block from library routines: 1x1 conv2d, grouped 3x3 conv2d over the rounded
    intermediate (its zero padding around that intermediate), 1x1 conv2d, numpy/torch
    casts for the roundings."""
    (s1, s2, s3), (b1, b2, b3) = s, b
    K1 = w1.shape[0]
    t1 = _nhwc(F.conv2d(_nchw(x), torch.from_numpy(w1[:, :, None, None])))
    t1 = _cast(_act(t1 * s1 + b1, acts[0]), dtype)
    t2 = _nhwc(F.conv2d(_nchw(t1), torch.from_numpy(w2[:, None]), stride=stride, padding=1,
                        groups=K1))
    t2 = _cast(_act(t2 * s2 + b2, acts[1]), dtype)
    y = _nhwc(F.conv2d(_nchw(t2), torch.from_numpy(w3[:, :, None, None])))
    y = _act(y * s3 + b3, acts[2])
    if residual:
        y = y + x
    return _cast(y, dtype), t1, t2


def _draw(rng, N, H, W, C, K1, K, dtype):
    x = oracle.round_to(rng.standard_normal((N, H, W, C)), dtype)
    w1 = oracle.round_to(rng.standard_normal((K1, C)) * 0.3, dtype)
    w2 = oracle.round_to(rng.standard_normal((K1, 3, 3)) * 0.3, dtype)
    w3 = oracle.round_to(rng.standard_normal((K, K1)) * 0.2, dtype)
    s = tuple(rng.uniform(0.5, 1.5, n) for n in (K1, K1, K))
    b = tuple(rng.standard_normal(n) * 0.1 for n in (K1, K1, K))
    return x, w1, w2, w3, s, b


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("stride,residual", [(1, True), (1, False), (2, False)])
def test_pwdwpw_is_the_conv2d_pipeline(dtype, stride, residual):
    rng = _rng(41 + stride + 2 * residual)
    N, H, W, C, K1 = 2, 7, 6, 8, 24
    K = C if residual else 16
    x, w1, w2, w3, s, b = _draw(rng, N, H, W, C, K1, K, dtype)
    acts = ("relu6", "relu6", "none")
    y, t1, t2 = oracle.pwdwpw(x, w1, w2, w3, (stride, stride), (1, 1), s[0], b[0], acts[0],
                              s[1], b[1], acts[1], s[2], b[2], acts[2], residual, dtype,
                              return_t=True)
    yr, t1r, t2r = _torch_block(x, w1, w2, w3, stride, s, b, acts, residual, dtype)
    ulp = {"f32": 2.0 ** -23, "f16": 2.0 ** -10, "bf16": 2.0 ** -7}[dtype]
    assert y.shape == yr.shape == (N, (H - 1) // stride + 1, (W - 1) // stride + 1, K)
    # the torch side rounds bf16 through binary32 (a double rounding) and sums in another
    # order: allow one unit of the storage type where they differ, and demand agreement
    # almost everywhere
    for got, ref in ((t1, t1r), (t2, t2r), (y, yr)):
        assert np.all(np.abs(got - ref) <= 2 * ulp * np.maximum(np.abs(ref), 1e-3) + 1e-30)
        assert np.mean(got == ref) > 0.97


def test_pwdwpw_brute_force_tiny():
    # the definition written out with Python loops on a 4x5 image, binary16 storage
    rng = _rng(42)
    N, H, W, C, K1, K = 1, 4, 5, 3, 4, 3
    x = oracle.round_to(rng.standard_normal((N, H, W, C)), "f16")
    w1 = oracle.round_to(rng.standard_normal((K1, C)), "f16")
    w2 = oracle.round_to(rng.standard_normal((K1, 3, 3)), "f16")
    w3 = oracle.round_to(rng.standard_normal((K, K1)), "f16")
    b1, b2, s3, b3 = (rng.standard_normal(K1), rng.standard_normal(K1),
                      rng.uniform(0.5, 1.5, K), rng.standard_normal(K))
    y = oracle.pwdwpw(x, w1, w2, w3, bias1=b1, act1="relu", bias2=b2, act2="relu6",
                      scale3=s3, bias3=b3, residual=True, dtype="f16")
    h16 = lambda v: float(np.float16(v))  # noqa: E731  (round to nearest even binary16)
    t1 = [[[h16(max(sum(x[0, i, j, c] * w1[k, c] for c in range(C)) + b1[k], 0.0))
            for k in range(K1)] for j in range(W)] for i in range(H)]
    for oh in range(H):
        for ow in range(W):
            t2 = []
            for k in range(K1):
                acc = 0.0
                for r in range(3):
                    for q in range(3):
                        ih, iw = oh - 1 + r, ow - 1 + q
                        if 0 <= ih < H and 0 <= iw < W:
                            acc += t1[ih][iw][k] * w2[k, r, q]
                t2.append(h16(min(max(acc + b2[k], 0.0), 6.0)))
            for k in range(K):
                v = s3[k] * sum(t2[c] * w3[k, c] for c in range(K1)) + b3[k] + x[0, oh, ow, k]
                assert y[0, oh, ow, k] == h16(v), (oh, ow, k)


def test_pwdwpw_identity_layers_return_the_input():
    # identity expansion, a centre-tap depthwise filter and an identity projection pass
    # the input through; the shortcut then doubles it (exact in binary32)
    rng = _rng(43)
    N, H, W, C = 2, 5, 6, 8
    x = rng.integers(-50, 50, (N, H, W, C)).astype(np.float64)
    eye = np.eye(C)
    w2 = np.zeros((C, 3, 3))
    w2[:, 1, 1] = 1.0
    y = oracle.pwdwpw(x, eye, w2, eye, dtype="f32")
    assert np.array_equal(y, x)
    y = oracle.pwdwpw(x, eye, w2, eye, residual=True, dtype="f32")
    assert np.array_equal(y, 2 * x)
    # stride 2 subsamples the identity
    y = oracle.pwdwpw(x, eye, w2, eye, stride=(2, 2), dtype="f32")
    assert np.array_equal(y, x[:, ::2, ::2])


def test_pwdwpw_shortcut_adds_the_input_pixel_exactly():
    # integer data: every sum is exact in binary32, so the shortcut's effect is exactly x
    rng = _rng(44)
    N, H, W, C, K1 = 2, 6, 5, 8, 16
    x = rng.integers(-4, 5, (N, H, W, C)).astype(np.float64)
    w1 = rng.integers(-2, 3, (K1, C)).astype(np.float64)
    w2 = rng.integers(-2, 3, (K1, 3, 3)).astype(np.float64)
    w3 = rng.integers(-2, 3, (C, K1)).astype(np.float64)
    kw = dict(act1="relu", act2="relu", dtype="f32")
    y0 = oracle.pwdwpw(x, w1, w2, w3, **kw)
    y1 = oracle.pwdwpw(x, w1, w2, w3, residual=True, **kw)
    assert np.array_equal(y1 - y0, x)
    # the shortcut needs an unchanged extent and K == C
    with pytest.raises(ValueError):
        oracle.pwdwpw(x, w1, w2, w3, stride=(2, 2), residual=True, **kw)
    with pytest.raises(ValueError):
        oracle.pwdwpw(x, w1, w2, w3[:4], residual=True, **kw)


def test_pwdwpw_is_linear_in_the_projection():
    # with no activation after it, the third layer is linear in its filters: doubling w3
    # doubles the output (integer data, exact), and a zero projection leaves the bias
    rng = _rng(45)
    N, H, W, C, K1, K = 1, 5, 5, 4, 8, 6
    x = rng.integers(-3, 4, (N, H, W, C)).astype(np.float64)
    w1 = rng.integers(-2, 3, (K1, C)).astype(np.float64)
    w2 = rng.integers(-2, 3, (K1, 3, 3)).astype(np.float64)
    w3 = rng.integers(-2, 3, (K, K1)).astype(np.float64)
    b3 = rng.integers(-5, 6, K).astype(np.float64)
    kw = dict(act1="relu6", act2="relu", dtype="f32")
    y = oracle.pwdwpw(x, w1, w2, w3, **kw)
    assert np.array_equal(oracle.pwdwpw(x, w1, w2, 2 * w3, **kw), 2 * y)
    z = oracle.pwdwpw(x, w1, w2, np.zeros_like(w3), bias3=b3, **kw)
    assert np.array_equal(z, np.broadcast_to(b3, z.shape))


@pytest.mark.parametrize("stride,residual", [(1, True), (2, False)])
def test_pwdwpw_sampled_rows_equal_full_outputs(stride, residual):
    rng = _rng(46 + stride)
    N, H, W, C, K1 = 3, 9, 7, 8, 24
    K = C if residual else 12
    x, w1, w2, w3, s, b = _draw(rng, N, H, W, C, K1, K, "f16")
    kw = dict(stride=(stride, stride), scale1=s[0], bias1=b[0], act1="relu6", scale2=s[1],
              bias2=b[1], act2="relu6", scale3=s[2], bias3=b[2], residual=residual,
              dtype="f16")
    y = oracle.pwdwpw(x, w1, w2, w3, **kw)
    Ho, Wo = y.shape[1:3]
    pix = [(n, oh, ow) for n in range(N) for oh in range(Ho) for ow in range(Wo)
           if (n + oh + 2 * ow) % 3 == 0]
    ya = oracle.pwdwpw_at(x, w1, w2, w3, pix, **kw)
    assert np.array_equal(ya, np.array([y[p] for p in pix]))
