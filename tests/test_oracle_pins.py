"""Pins for the CPU oracle: checks against things other than the oracle itself.

* library routines it must reduce to: torch.nn.functional.conv2d (groups=C for the
  depthwise layer), batch_norm + relu/relu6 for the epilogue, numpy/torch casts for
  IEEE round-to-nearest-even;
* exact invariants of convolution (identity filters, one-hot taps, linearity,
  stride-2 as a subsample of stride-1, channel permutation, batch independence, a
  diagonal standard conv equal to a depthwise conv);
* facts the pages print about shapes and memory accounting (tests/golden).

A plausible mistake anywhere in the oracle (a dropped tap, a flipped filter, a wrong
padding or stride, a transposed weight, an epilogue applied in the wrong order, a
rounding in the wrong place or mode) fails at least one test here.
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import accounting
import fcm_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")


def _rng(seed=0):
    return np.random.default_rng(seed)


def _torch_dw(x, w, stride, pad):
    xt = torch.from_numpy(x).permute(0, 3, 1, 2)
    wt = torch.from_numpy(w)[:, None]
    return F.conv2d(xt, wt, stride=stride, padding=pad, groups=x.shape[3]).permute(
        0, 2, 3, 1).numpy()


def _torch_conv(x, w, stride, pad):
    xt = torch.from_numpy(x).permute(0, 3, 1, 2)
    return F.conv2d(xt, torch.from_numpy(w), stride=stride, padding=pad).permute(
        0, 2, 3, 1).numpy()


# ---------------------------------------------------------------------------------
# rounding
# ---------------------------------------------------------------------------------
def test_f16_all_patterns_and_midpoints():
    bits = np.arange(65536, dtype=np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    fin = np.isfinite(vals)
    r = oracle.round_to(vals[fin], "f16")
    assert np.array_equal(r, vals[fin])
    for b in bits[fin][::97]:
        v = float(np.uint16(b).view(np.float16))
        assert oracle.f16_bits(v) == int(b), hex(b)
    # midpoints between consecutive positive finite values: ties go to even
    pos = np.sort(np.unique(vals[fin & (vals >= 0)]))
    mids = (pos[:-1] + pos[1:]) / 2.0
    expect = mids.astype(np.float16).astype(np.float64)
    assert np.array_equal(oracle.round_to(mids, "f16"), expect)
    assert np.array_equal(oracle.round_to(-mids, "f16"), -expect)
    # just above / below the largest finite value and the overflow threshold
    edge = np.array([65504.0, 65519.0, 65519.999, 65520.0, 1e6, 2.0 ** -25,
                     2.0 ** -25 * 1.0000001, 2.0 ** -24 * 1.5, 6.0e-8, -0.0])
    with np.errstate(over="ignore"):
        expect_edge = edge.astype(np.float16).astype(np.float64)
    assert np.array_equal(oracle.round_to(edge, "f16"), expect_edge)


def test_f16_random_against_numpy():
    rng = _rng(1)
    v = rng.standard_normal(200000) * np.exp(rng.uniform(-20, 12, 200000))
    with np.errstate(over="ignore"):
        expect = v.astype(np.float16).astype(np.float64)
    assert np.array_equal(oracle.round_to(v, "f16"), expect)


def test_bf16_all_patterns_and_midpoints():
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    vals = bits.view(torch.bfloat16).to(torch.float64).numpy()
    fin = np.isfinite(vals)
    assert np.array_equal(oracle.round_to(vals[fin], "bf16"), vals[fin])
    raw = np.arange(65536)[fin]
    for b in raw[::101]:
        v = float(torch.tensor([b], dtype=torch.int32).to(torch.int16).view(
            torch.bfloat16).to(torch.float64))
        assert oracle.bf16_bits(v) == int(b), hex(int(b))
    pos = np.sort(np.unique(vals[fin & (vals >= 0)]))
    mids = (pos[:-1] + pos[1:]) / 2.0            # exactly representable in binary32
    expect = torch.from_numpy(mids.astype(np.float32)).to(torch.bfloat16).to(
        torch.float64).numpy()
    assert np.array_equal(oracle.round_to(mids, "bf16"), expect)


def test_bf16_random_against_torch():
    rng = _rng(2)
    v32 = (rng.standard_normal(200000) * np.exp(rng.uniform(-60, 60, 200000))).astype(
        np.float32)
    v = v32.astype(np.float64)
    expect = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_to(v, "bf16"), expect)


def test_f32_random_against_numpy():
    rng = _rng(3)
    v = rng.standard_normal(200000) * np.exp(rng.uniform(-80, 80, 200000))
    assert np.array_equal(oracle.round_to(v, "f32"), v.astype(np.float32).astype(np.float64))


# ---------------------------------------------------------------------------------
# layers against torch.nn.functional.conv2d in float64
# ---------------------------------------------------------------------------------
@pytest.mark.parametrize("N,H,W,C,stride,pad,R", [
    (1, 1, 1, 1, 1, 1, 3), (2, 5, 7, 8, 1, 1, 3), (2, 9, 6, 16, 2, 1, 3),
    (1, 8, 8, 24, 2, 0, 3), (3, 4, 9, 8, 1, 0, 3), (1, 6, 5, 4, 1, 0, 2),
    (1, 7, 7, 16, 1, 2, 5)])
def test_dw_matches_torch_grouped_conv(N, H, W, C, stride, pad, R):
    rng = _rng(N * 100 + H)
    x = rng.standard_normal((N, H, W, C))
    w = rng.standard_normal((C, R, R))
    t = oracle.dw(x, w, (stride, stride), (pad, pad))
    ref = _torch_dw(x, w, stride, pad)
    assert t.shape == ref.shape
    assert np.max(np.abs(t - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("C,K", [(1, 1), (8, 32), (32, 8), (24, 40)])
def test_pw_matches_torch_1x1(C, K):
    rng = _rng(C + 7 * K)
    t = rng.standard_normal((2, 5, 3, C))
    w = rng.standard_normal((K, C))
    y = oracle.pw(t, w)
    ref = _torch_conv(t, w[:, :, None, None], 1, 0)
    assert np.max(np.abs(y - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("N,H,W,C,K,stride,pad", [
    (1, 5, 5, 8, 16, 1, 1), (2, 7, 4, 16, 8, 2, 1), (1, 6, 6, 3, 5, 1, 0)])
def test_conv_matches_torch(N, H, W, C, K, stride, pad):
    rng = _rng(K)
    x = rng.standard_normal((N, H, W, C))
    w = rng.standard_normal((K, C, 3, 3))
    y = oracle.conv(x, w, (stride, stride), (pad, pad))
    ref = _torch_conv(x, w, stride, pad)
    assert np.max(np.abs(y - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("act", ["none", "relu", "relu6"])
def test_epilogue_is_folded_batchnorm_then_activation(act):
    rng = _rng(5)
    C = 12
    a = rng.standard_normal((3, 4, 5, C)) * 4
    gamma, beta = rng.uniform(0.5, 1.5, C), rng.standard_normal(C)
    mean, var, eps = rng.standard_normal(C), rng.uniform(0.5, 2.0, C), 1e-5
    scale = gamma / np.sqrt(var + eps)
    bias = beta - mean * scale
    out = oracle.epilogue(a, scale, bias, act)
    at = torch.from_numpy(a).permute(0, 3, 1, 2)
    bn = F.batch_norm(at, torch.from_numpy(mean), torch.from_numpy(var),
                      torch.from_numpy(gamma), torch.from_numpy(beta), False, 0.0, eps)
    bn = {"none": lambda v: v, "relu": F.relu, "relu6": F.relu6}[act](bn)
    ref = bn.permute(0, 2, 3, 1).numpy()
    assert np.max(np.abs(out - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))
    # null arrays are the identity
    assert np.array_equal(oracle.epilogue(a, None, None, "none"), a)


def _torch_round(a, dtype):
    if dtype == "f16":
        return a.astype(np.float16).astype(np.float64)
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_dwpw_module_is_layer_by_layer_pipeline(dtype):
    rng = _rng(11)
    N, H, W, C, K = 2, 6, 5, 8, 12
    x = oracle.round_to(rng.standard_normal((N, H, W, C)), dtype)
    wd = oracle.round_to(rng.standard_normal((C, 3, 3)) * 0.3, dtype)
    wp = oracle.round_to(rng.standard_normal((K, C)) * 0.3, dtype)
    s1, b1 = rng.uniform(0.5, 1.5, C), rng.standard_normal(C) * 0.1
    s2, b2 = rng.uniform(0.5, 1.5, K), rng.standard_normal(K) * 0.1
    y, t = oracle.dwpw(x, wd, wp, (1, 1), (1, 1), s1, b1, "relu6", s2, b2, "relu", dtype,
                       return_t=True)
    # reference pipeline from library routines; rounding by numpy/torch casts
    tt = _torch_dw(x, wd, 1, 1) * s1 + b1
    tt = np.clip(tt, 0, 6)
    tr = _torch_round(tt, dtype)
    yy = np.maximum(_torch_conv(tr, wp[:, :, None, None], 1, 0) * s2 + b2, 0)
    yr = _torch_round(yy, dtype)
    ulp = {"f32": 2.0 ** -23, "f16": 2.0 ** -10, "bf16": 2.0 ** -7}[dtype]
    # torch's bfloat16 cast rounds via binary32, so allow a rare one-ulp difference
    assert np.all(np.abs(t - tr) <= ulp * np.abs(tr) + 1e-30)
    assert np.all(np.abs(y - yr) <= 2 * ulp * np.maximum(np.abs(yr), 1e-3) + 1e-30)
    frac_exact = np.mean(y == yr)
    assert frac_exact > 0.97


def test_b2b_module_is_layer_by_layer_pipeline():
    rng = _rng(12)
    N, H, W, C, K1, K = 2, 5, 6, 8, 16, 8
    x = oracle.round_to(rng.standard_normal((N, H, W, C)), "f16")
    w1 = oracle.round_to(rng.standard_normal((K1, C, 3, 3)) * 0.1, "f16")
    w2 = oracle.round_to(rng.standard_normal((K, K1)) * 0.2, "f16")
    s1, b1 = rng.uniform(0.5, 1.5, K1), rng.standard_normal(K1) * 0.1
    s2, b2 = rng.uniform(0.5, 1.5, K), rng.standard_normal(K) * 0.1
    y, t = oracle.b2b(x, w1, w2, (1, 1), (1, 1), s1, b1, "relu", s2, b2, "relu", "f16",
                      return_t=True)
    tr = _torch_round(np.maximum(_torch_conv(x, w1, 1, 1) * s1 + b1, 0), "f16")
    yr = _torch_round(np.maximum(_torch_conv(tr, w2[:, :, None, None], 1, 0) * s2 + b2, 0),
                      "f16")
    assert np.array_equal(t, tr)
    assert np.array_equal(y, yr)


# ---------------------------------------------------------------------------------
# exact invariants
# ---------------------------------------------------------------------------------
def test_identity_depthwise_and_pointwise_are_noops():
    rng = _rng(20)
    for dtype in ("f32", "f16", "bf16"):
        x = oracle.round_to(rng.standard_normal((2, 7, 5, 16)), dtype)
        wd = np.zeros((16, 3, 3))
        wd[:, 1, 1] = 1.0
        wp = np.eye(16)
        y, t = oracle.dwpw(x, wd, wp, dtype=dtype, return_t=True)
        assert np.array_equal(t, x)
        assert np.array_equal(y, x)


@pytest.mark.parametrize("r,s", [(0, 0), (0, 2), (2, 1), (1, 0), (2, 2)])
def test_one_hot_tap_is_a_shift_with_zero_border(r, s):
    rng = _rng(21)
    x = rng.standard_normal((1, 6, 7, 4))
    w = np.zeros((4, 3, 3))
    w[:, r, s] = 1.0
    t = oracle.dw(x, w)
    xp = np.pad(x, ((0, 0), (1, 1), (1, 1), (0, 0)))
    expect = xp[:, r:r + 6, s:s + 7, :]
    assert np.array_equal(t, expect)


def test_linearity():
    rng = _rng(22)
    x1, x2 = rng.standard_normal((2, 2, 5, 6, 8))
    wd, wp = rng.standard_normal((8, 3, 3)), rng.standard_normal((5, 8))
    a, b = 0.75, -1.25
    y = oracle.pw(oracle.dw(a * x1 + b * x2, wd), wp)
    y12 = a * oracle.pw(oracle.dw(x1, wd), wp) + b * oracle.pw(oracle.dw(x2, wd), wp)
    assert np.max(np.abs(y - y12)) <= 1e-12 * np.max(np.abs(y))


def test_stride2_is_stride1_subsampled():
    rng = _rng(23)
    x = rng.standard_normal((2, 9, 8, 8))
    w = rng.standard_normal((8, 3, 3))
    t1 = oracle.dw(x, w, (1, 1), (1, 1))
    t2 = oracle.dw(x, w, (2, 2), (1, 1))
    assert np.array_equal(t2, t1[:, ::2, ::2, :])


def test_channel_permutation_and_batch_independence():
    rng = _rng(24)
    x = rng.standard_normal((3, 5, 5, 8))
    w = rng.standard_normal((8, 3, 3))
    perm = rng.permutation(8)
    t = oracle.dw(x, w)
    assert np.array_equal(oracle.dw(x[..., perm], w[perm]), t[..., perm])
    assert np.array_equal(oracle.dw(x[1:2], w), t[1:2])


def test_diagonal_standard_conv_equals_depthwise():
    rng = _rng(25)
    C = 8
    x = oracle.round_to(rng.standard_normal((2, 6, 5, C)), "f16")
    wd = oracle.round_to(rng.standard_normal((C, 3, 3)) * 0.4, "f16")
    wp = oracle.round_to(rng.standard_normal((6, C)) * 0.4, "f16")
    w1 = np.zeros((C, C, 3, 3))
    for c in range(C):
        w1[c, c] = wd[c]
    kw = dict(scale1=rng.uniform(0.5, 1.5, C), bias1=rng.standard_normal(C) * 0.1,
              act1="relu6", bias2=rng.standard_normal(6) * 0.1, act2="relu", dtype="f16")
    assert np.array_equal(oracle.b2b(x, w1, wp, **kw), oracle.dwpw(x, wd, wp, **kw))


def test_sampled_rows_equal_full_outputs():
    wl = fcm_inputs.WORKLOADS["mbv1_f16_8x112x112_c64_k128"].replace(N=2, H=9, W=20)
    inp = fcm_inputs.make_inputs(wl)
    kw = dict(stride=(1, 1), pad=(1, 1), scale1=inp["scale1"], bias1=inp["bias1"],
              act1=wl.act1, scale2=inp["scale2"], bias2=inp["bias2"], act2=wl.act2,
              dtype=wl.dtype)
    full = oracle.dwpw(inp["x"], inp["w1"], inp["w2"], **kw)
    pix = fcm_inputs.sample_pixels(wl, 40)
    rows = oracle.dwpw_at(inp["x"], inp["w1"], inp["w2"], pix, **kw)
    assert np.array_equal(rows, full[pix[:, 0], pix[:, 1], pix[:, 2]])


# ---------------------------------------------------------------------------------
# INT8: exact integer sums, binary32 requantization
# ---------------------------------------------------------------------------------
def _requant_ref(acc, scale, bias, act):
    """Integer sums (exact in float64) -> v = scale*acc + bias computed exactly in
    float64 (dyadic scale and bias keep it exact), rounded once to binary32 (what one
    fused multiply-add gives) -> clamp -> nearest integer with ties to even (numpy's
    rint) -> saturate."""
    v = (acc * scale + bias).astype(np.float32)
    if act in ("relu", "relu6"):
        v = np.maximum(v, np.float32(0))
    if act == "relu6":
        v = np.minimum(v, np.float32(6))
    return np.clip(np.rint(v.astype(np.float64)), -128, 127)


@pytest.mark.parametrize("stride,act1,act2", [(1, "relu", "relu"), (2, "none", "relu6"),
                                              (1, "relu6", "none")])
def test_i8_dwpw_is_the_integer_pipeline(stride, act1, act2):
    rng = _rng(40 + stride)
    N, H, W, C, K = 2, 9, 11, 16, 24
    x = rng.integers(-128, 128, (N, H, W, C)).astype(np.float64)
    wd = rng.integers(-127, 128, (C, 3, 3)).astype(np.float64)
    wp = rng.integers(-127, 128, (K, C)).astype(np.float64)
    # dyadic scales and biases: scale*acc + bias is exact in float64, so rounding it to
    # binary32 once is exactly what a fused multiply-add in binary32 returns
    s1 = rng.integers(1, 4096, C) / 2.0 ** 17
    b1 = rng.integers(-64, 64, C) / 8.0
    s2 = rng.integers(1, 4096, K) / 2.0 ** 19
    b2 = rng.integers(-64, 64, K) / 8.0
    y, t = oracle.dwpw(x, wd, wp, (stride, stride), (1, 1), s1, b1, act1, s2, b2, act2, "i8",
                       return_t=True)
    acc1 = _torch_dw(x, wd, stride, 1)
    assert np.all(acc1 == np.rint(acc1)) and np.abs(acc1).max() < 2 ** 24
    tr = _requant_ref(acc1, s1, b1, act1)
    acc2 = _torch_conv(tr, wp[:, :, None, None], 1, 0)
    yr = _requant_ref(acc2, s2, b2, act2)
    assert np.array_equal(t, tr)
    assert np.array_equal(y, yr)
    # the codes really reach the int8 range's ends where the activation allows it
    if act1 != "relu6":
        assert t.max() == 127 or t.min() == -128


def test_i8_rounding_ties_to_even_and_saturates():
    # identity filters and scale 1/2: every intermediate is x/2 exactly, so odd inputs
    # sit on a tie; scale 2 on the output saturates the large codes
    x = np.arange(-127, 128, dtype=np.float64).reshape(1, 1, 255, 1)
    wd = np.zeros((1, 3, 3))
    wd[0, 1, 1] = 1
    y1, t = oracle.dwpw(x, wd, np.eye(1), scale1=np.array([0.5]), dtype="i8", return_t=True)
    half = x / 2
    expect = np.where(np.abs(half - np.trunc(half)) == 0.5,
                      2 * np.round(half / 2), np.round(half))   # ties to the even neighbour
    assert np.array_equal(t, expect)
    assert np.array_equal(t.ravel()[[0, 1, 2, 125, 126, 127, 128, 129]],
                          [-64, -63, -62, -1, 0, 0, 0, 1])
    y2 = oracle.dwpw(x, wd, np.eye(1), scale1=np.array([4.0]), dtype="i8")
    assert y2.min() == -128 and y2.max() == 127
    assert np.array_equal(y2.ravel(), np.clip(4 * x.ravel(), -128, 127))


def test_i8_inputs_are_integer_codes():
    wl = fcm_inputs.WORKLOADS["mbv1i8_i8_8x112x112_c32_k64"].replace(N=1, H=8, W=8)
    inp = fcm_inputs.make_inputs(wl)
    for k in ("x", "w1", "w2"):
        a = inp[k]
        assert np.all(a == np.rint(a)) and a.min() >= -128 and a.max() <= 127
    assert accounting.alg_bytes(fcm_inputs.WORKLOADS["mbv1i8_i8_8x112x112_c32_k64"]) == (
        8 * 112 * 112 * (32 + 64) + 9 * 32 + 64 * 32 + 4 * 2 * (32 + 64))


# ---------------------------------------------------------------------------------
# the pointwise -> pointwise module
# ---------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_pwpw_module_is_layer_by_layer_pipeline(dtype):
    rng = _rng(50)
    x = oracle.round_to(rng.standard_normal((2, 5, 7, 24)), dtype)
    w1 = oracle.round_to(rng.standard_normal((40, 24)) * 0.3, dtype)
    w2 = oracle.round_to(rng.standard_normal((16, 40)) * 0.3, dtype)
    s1, b1 = rng.uniform(0.5, 1.5, 40), rng.standard_normal(40) * 0.1
    s2, b2 = rng.uniform(0.5, 1.5, 16), rng.standard_normal(16) * 0.1
    y, t = oracle.pwpw(x, w1, w2, s1, b1, "relu6", s2, b2, "relu", dtype, return_t=True)
    tr = _torch_round(np.clip(_torch_conv(x, w1[:, :, None, None], 1, 0) * s1 + b1, 0, 6), dtype)
    yr = _torch_round(np.maximum(_torch_conv(tr, w2[:, :, None, None], 1, 0) * s2 + b2, 0), dtype)
    ulp = {"f32": 2.0 ** -23, "f16": 2.0 ** -10, "bf16": 2.0 ** -7}[dtype]
    assert np.all(np.abs(t - tr) <= ulp * np.abs(tr) + 1e-30)
    assert np.all(np.abs(y - yr) <= 2 * ulp * np.maximum(np.abs(yr), 1e-3) + 1e-30)
    assert np.mean(y == yr) > 0.97


def test_pwpw_identity_first_layer_is_one_pointwise_layer():
    rng = _rng(51)
    x = oracle.round_to(rng.standard_normal((1, 4, 6, 16)), "f16")
    w2 = oracle.round_to(rng.standard_normal((8, 16)) * 0.3, "f16")
    b2 = rng.standard_normal(8) * 0.1
    y, t = oracle.pwpw(x, np.eye(16), w2, bias2=b2, act2="relu", dtype="f16", return_t=True)
    assert np.array_equal(t, x)
    assert np.array_equal(y, oracle.round_to(np.maximum(oracle.pw(x, w2) + b2, 0), "f16"))
    # and the module is a per-pixel map: any subset of pixels gives the same rows
    pix = np.array([[0, 3, 5], [0, 0, 0], [0, 2, 1]])
    assert np.array_equal(oracle.pwpw_at(x, np.eye(16), w2, pix, bias2=b2, act2="relu",
                                         dtype="f16"), y[pix[:, 0], pix[:, 1], pix[:, 2]])


def test_pwpw_accounting_closed_forms():
    wl = fcm_inputs.WORKLOADS["pwpw_f16_32x56x56_c64_k32_k64"]
    s = accounting.sizes(wl)
    P = 32 * 56 * 56
    assert (wl.Ho, wl.Wo) == (56, 56)
    assert s["t"] == P * 32 * 2
    assert accounting.alg_bytes(wl) == P * (64 + 64) * 2 + (32 * 64 + 64 * 32) * 2 + 4 * 2 * (32 + 64)
    assert accounting.flops(wl) == 2 * P * (64 * 32 + 32 * 64)


# ---------------------------------------------------------------------------------
# the pointwise -> depthwise module
# ---------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,stride,pad", [("f32", 1, 1), ("f16", 1, 1), ("bf16", 1, 1),
                                              ("f16", 2, 1), ("f16", 1, 0)])
def test_pwdw_module_is_layer_by_layer_pipeline(dtype, stride, pad):
    rng = _rng(31 + stride + 3 * pad)
    N, H, W, C, K1 = 2, 7, 6, 8, 24
    x = oracle.round_to(rng.standard_normal((N, H, W, C)), dtype)
    wp = oracle.round_to(rng.standard_normal((K1, C)) * 0.3, dtype)
    wd = oracle.round_to(rng.standard_normal((K1, 3, 3)) * 0.3, dtype)
    s1, b1 = rng.uniform(0.5, 1.5, K1), rng.standard_normal(K1) * 0.1
    s2, b2 = rng.uniform(0.5, 1.5, K1), rng.standard_normal(K1) * 0.1
    y, t = oracle.pwdw(x, wp, wd, (stride, stride), (pad, pad), s1, b1, "relu6", s2, b2,
                       "relu", dtype, return_t=True)
    # reference pipeline from library routines: 1x1 conv2d, then a grouped conv2d whose
    # zero padding surrounds the rounded intermediate; rounding by numpy/torch casts
    tr = _torch_round(np.clip(_torch_conv(x, wp[:, :, None, None], 1, 0) * s1 + b1, 0, 6),
                      dtype)
    yr = _torch_round(np.maximum(_torch_dw(tr, wd, stride, pad) * s2 + b2, 0), dtype)
    ulp = {"f32": 2.0 ** -23, "f16": 2.0 ** -10, "bf16": 2.0 ** -7}[dtype]
    assert t.shape == (N, H, W, K1) and y.shape == yr.shape
    assert np.all(np.abs(t - tr) <= ulp * np.abs(tr) + 1e-30)
    assert np.all(np.abs(y - yr) <= 2 * ulp * np.maximum(np.abs(yr), 1e-3) + 1e-30)
    assert np.mean(y == yr) > 0.97


def test_pwdw_brute_force_tiny():
    # the definition written out with Python loops on a 3x4 image
    rng = _rng(32)
    N, H, W, C, K1 = 1, 3, 4, 3, 2
    x = rng.standard_normal((N, H, W, C))
    wp = rng.standard_normal((K1, C))
    wd = rng.standard_normal((K1, 3, 3))
    b1 = rng.standard_normal(K1)
    y = oracle.pwdw(x, wp, wd, bias1=b1, act1="relu", dtype="f32")
    t = np.zeros((H, W, K1))
    for h in range(H):
        for w in range(W):
            for k in range(K1):
                v = sum(x[0, h, w, c] * wp[k, c] for c in range(C)) + b1[k]
                t[h, w, k] = float(np.float32(max(v, 0.0)))
    for oh in range(H):
        for ow in range(W):
            for k in range(K1):
                acc = 0.0
                for r in range(3):
                    for s_ in range(3):
                        ih, iw = oh - 1 + r, ow - 1 + s_
                        if 0 <= ih < H and 0 <= iw < W:
                            acc += t[ih, iw, k] * wd[k, r, s_]
                assert abs(y[0, oh, ow, k] - float(np.float32(acc))) <= 1e-6 * max(1, abs(acc))


def test_pwdw_padding_surrounds_the_intermediate():
    # x = 0: the intermediate is round(relu(bias1)) at every pixel, and with all-ones
    # depthwise filters each output counts the window positions inside the image
    # (4 in a corner, 6 on an edge, 9 inside); padding the module's input instead would
    # give 9 everywhere
    N, H, W, C, K1 = 1, 5, 6, 8, 16
    b1 = np.linspace(0.1, 1.6, K1)
    y = oracle.pwdw(np.zeros((N, H, W, C)), np.ones((K1, C)), np.ones((K1, 3, 3)),
                    bias1=b1, act1="relu", dtype="f16")
    t = oracle.round_to(b1, "f16")
    count = np.full((H, W), 9.0)
    count[0, :] -= 3
    count[-1, :] -= 3
    count[:, 0] -= 3
    count[:, -1] -= 3
    count[0, 0] = count[0, -1] = count[-1, 0] = count[-1, -1] = 4
    expect = oracle.round_to(count[:, :, None] * t[None, None, :], "f16")
    assert np.array_equal(y[0], expect)


def test_pwdw_identity_depthwise_returns_the_intermediate():
    rng = _rng(33)
    x = oracle.round_to(rng.standard_normal((2, 5, 4, 8)), "bf16")
    wp = oracle.round_to(rng.standard_normal((16, 8)) * 0.4, "bf16")
    wd = np.zeros((16, 3, 3))
    wd[:, 1, 1] = 1.0
    y, t = oracle.pwdw(x, wp, wd, scale1=rng.uniform(0.5, 1.5, 16),
                       bias1=rng.standard_normal(16) * 0.1, act1="relu6", dtype="bf16",
                       return_t=True)
    assert np.array_equal(y, t)
    # and an identity pointwise layer hands the input to the depthwise layer unchanged
    wd2 = oracle.round_to(rng.standard_normal((8, 3, 3)), "bf16")
    y2, t2 = oracle.pwdw(x, np.eye(8), wd2, dtype="bf16", return_t=True)
    assert np.array_equal(t2, x)
    assert np.array_equal(y2, oracle.round_to(_torch_dw(x, wd2, 1, 1), "bf16"))


def test_pwdw_stride2_is_stride1_subsampled():
    rng = _rng(34)
    x = oracle.round_to(rng.standard_normal((1, 9, 8, 8)), "f16")
    wp = oracle.round_to(rng.standard_normal((16, 8)) * 0.3, "f16")
    wd = oracle.round_to(rng.standard_normal((16, 3, 3)) * 0.3, "f16")
    kw = dict(bias1=rng.standard_normal(16) * 0.1, act1="relu6", scale2=rng.uniform(
        0.5, 1.5, 16), act2="relu", dtype="f16")
    y1 = oracle.pwdw(x, wp, wd, (1, 1), (1, 1), **kw)
    y2 = oracle.pwdw(x, wp, wd, (2, 2), (1, 1), **kw)
    assert np.array_equal(y2, y1[:, ::2, ::2, :])


def test_pwdw_sampled_rows_equal_full_outputs():
    for name in ("pwdw_f16_32x56x56_c24_k144", "pwdw_f16_32x112x112_c16_k96_s2"):
        wl = fcm_inputs.WORKLOADS[name].replace(N=2, H=11, W=19)
        inp = fcm_inputs.make_inputs(wl)
        kw = dict(stride=(wl.stride,) * 2, pad=(1, 1), scale1=inp["scale1"],
                  bias1=inp["bias1"], act1=wl.act1, scale2=inp["scale2"], bias2=inp["bias2"],
                  act2=wl.act2, dtype=wl.dtype)
        full = oracle.pwdw(inp["x"], inp["w1"], inp["w2"], **kw)
        pix = fcm_inputs.sample_pixels(wl, 40)
        rows = oracle.pwdw_at(inp["x"], inp["w1"], inp["w2"], pix, **kw)
        assert np.array_equal(rows, full[pix[:, 0], pix[:, 1], pix[:, 2]])


def _brute_force_recompute(H, W, th, tw, stride, pad=1, filt=3):
    # count, pixel by pixel, how many output tiles' windows need each intermediate
    # value (windows clipped to the image)
    Ho = (H + 2 * pad - filt) // stride + 1
    Wo = (W + 2 * pad - filt) // stride + 1
    need = np.zeros((H, W), np.int64)
    for t0 in range(0, Ho, th):
        for u0 in range(0, Wo, tw):
            m = np.zeros((H, W), bool)
            for oh in range(t0, min(t0 + th, Ho)):
                for ow in range(u0, min(u0 + tw, Wo)):
                    for r in range(filt):
                        for s_ in range(filt):
                            ih, iw = oh * stride - pad + r, ow * stride - pad + s_
                            if 0 <= ih < H and 0 <= iw < W:
                                m[ih, iw] = True
            need += m
    return need


@pytest.mark.parametrize("H,W,th,tw,stride", [(56, 56, 8, 16, 1), (17, 23, 4, 16, 1),
                                              (112, 112, 4, 16, 2), (9, 9, 3, 5, 2),
                                              (14, 14, 14, 14, 1)])
def test_pwdw_redundancy_equals_brute_force(H, W, th, tw, stride):
    need = _brute_force_recompute(H, W, th, tw, stride)
    expect = need.sum() / (H * W) - 1.0
    assert abs(accounting.pwdw_redundancy(H, W, th, tw, stride) - expect) < 1e-12


def test_page_pwdw_without_tiling_has_no_redundancy():
    # Table II: the PWDW cases (no spatial tiling) recompute nothing
    g = _golden()["pwdw_no_redundant_compute"]
    for H, W, s in [(56, 56, 1), (28, 28, 2), (7, 7, 1)]:
        Ho, Wo = (H - 1) // s + 1, (W - 1) // s + 1
        assert accounting.pwdw_redundancy(H, W, Ho, Wo, s) == g["pwdw_redundancy"]
        assert _brute_force_recompute(H, W, Ho, Wo, s).max() == 1


def test_pwdw_accounting_closed_forms():
    wl = fcm_inputs.WORKLOADS["pwdw_f16_32x56x56_c24_k144"]
    s = accounting.sizes(wl)
    # the intermediate is the pointwise layer's output at the input resolution
    assert s["t"] == 32 * 56 * 56 * 144 * 2
    assert accounting.alg_bytes(wl) == (32 * 56 * 56 * 24 * 2 + 32 * 56 * 56 * 144 * 2 +
                                        144 * 24 * 2 + 144 * 9 * 2 + 4 * 4 * 144)
    assert accounting.alg_bytes(wl, False) - accounting.alg_bytes(wl) == 2 * s["t"]
    assert accounting.flops(wl) == 2 * 32 * 56 * 56 * (24 * 144 + 144 * 9)
    wl2 = fcm_inputs.WORKLOADS["pwdw_f16_32x112x112_c16_k96_s2"]
    assert (wl2.Ho, wl2.Wo) == (56, 56)
    assert accounting.sizes(wl2)["t"] == 32 * 112 * 112 * 96 * 2


# ---------------------------------------------------------------------------------
# the pages' own facts
# ---------------------------------------------------------------------------------
def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_page_dw_tile_shape():
    g = _golden()["dw_tile_shape"]
    x = np.ones((1,) + tuple(g["ifm_hw"]) + (1,))
    w = np.ones((1,) + tuple(g["filter_rs"]))
    t = oracle.dw(x, w, (g["stride"],) * 2, (g["pad"],) * 2)
    assert list(t.shape[1:3]) == g["ofm_hw"]


def test_page_b2b_and_cifar_extents():
    g = _golden()
    b = g["b2b_example"]
    h = oracle.out_size(b["conv1"]["in_hwc"][0], 1, b["conv1"]["filter_rs"][0], 1)
    assert h == b["conv1"]["out_hwc"][0]
    assert oracle.out_size(b["conv2"]["in_hwc"][0], 0, 1, 1) == b["conv2"]["out_hwc"][0]
    c = g["cifar_net_extents"]
    assert oracle.out_size(c["input_hw"], c["dw_pad"], c["dw_kernel"], 1) == c["after_dw"]
    p1 = oracle.out_size(c["after_dw"], 0, c["pool_kernel"], c["pool_stride"])
    assert p1 == c["after_pool1"]
    assert oracle.out_size(p1, 0, c["pool_kernel"], c["pool_stride"]) == c["after_pool2"]


def test_page_fusion_saves_half_and_writes_half():
    g = _golden()
    # C = K, stride 1: the unfused pair moves X, T, T, Y; the fused module X, Y.
    wl = fcm_inputs.Workload("t", "dwpw", "f16", N=64, H=112, W=112, C=32, K=32, K1=32)
    s = accounting.sizes(wl)
    no_w = (s["x"] + s["y"]) / (s["x"] + 2 * s["t"] + s["y"])
    assert 1.0 - no_w == g["fusion_saves_half"]["saving"]
    assert abs(accounting.fused_savings(wl) - g["fusion_saves_half"]["saving"]) < 1e-4
    # writes: unfused writes T and Y, fused only Y
    assert (s["t"] + s["y"]) / s["y"] == g["separable_writes_twice"][
        "write_ratio_unfused_over_fused"]


def test_accounting_of_the_five_workloads():
    # closed forms: X + Y + weights + epilogue arrays; unfused adds 2|T|
    for name, wl in fcm_inputs.WORKLOADS.items():
        s = accounting.sizes(wl)
        e = fcm_inputs.ELEM_BYTES[wl.dtype]
        assert s["x"] == wl.N * wl.H * wl.W * wl.C * e
        assert s["y"] == wl.N * wl.Ho * wl.Wo * wl.K * e
        # (the three-layer block's shortcut reads the input again when run layer by layer)
        extra = s["x"] if wl.kind == "pwdwpw" and wl.residual else 0
        assert (accounting.alg_bytes(wl, False) - accounting.alg_bytes(wl, True)
                == 2 * s["t"] + extra)
        if wl.kind == "pwdwpw":
            # two intermediates: the expansion at the input extent, the depthwise output at
            # the output extent
            assert s["t"] == (wl.N * wl.H * wl.W + wl.N * wl.Ho * wl.Wo) * wl.K1 * e
    assert accounting.alg_bytes(fcm_inputs.WORKLOADS["tiny_f32_1x16x16_c32"]) == 70912
    assert accounting.alg_bytes(fcm_inputs.WORKLOADS["mbv1_f16_8x112x112_c64_k128"]) == 38554240
    assert fcm_inputs.WORKLOADS["down_f16_64x56x56_c256_k512_s2"].Ho == 28


# ---------------------------------------------------------------------------------
# FusePlanner equations
# ---------------------------------------------------------------------------------
@pytest.mark.parametrize("cw,ch,tw,th,f,s", [
    (16, 16, 4, 16, 3, 1), (17, 9, 5, 9, 3, 1), (32, 8, 8, 8, 3, 2), (12, 12, 12, 3, 3, 1),
    (20, 20, 7, 20, 5, 1), (9, 9, 2, 9, 3, 3)])
def test_eq1_overlap_one_direction_equals_brute_force(cw, ch, tw, th, f, s):
    # tiles that split only one direction: Eq. 1 counts exactly the repeated loads
    assert accounting.eq1_overlap(cw, ch, tw, th, f, f, s) == \
        accounting.brute_force_overlap(cw, ch, tw, th, f, s)


@pytest.mark.parametrize("cw,ch,tw,th", [(16, 16, 4, 4), (17, 11, 5, 3), (8, 8, 3, 5)])
def test_eq1_overlap_two_directions_misses_only_corners(cw, ch, tw, th):
    # with both directions split, each border crossing's corner block is loaded by
    # four tiles; Eq. 1 charges it twice, so the brute force exceeds it by one per
    # corner element
    f, s = 3, 1
    corners = (-(-cw // tw) - 1) * (-(-ch // th) - 1) * (f - s) ** 2
    assert accounting.brute_force_overlap(cw, ch, tw, th, f, s) == \
        accounting.eq1_overlap(cw, ch, tw, th, f, f, s) + corners


def test_eq2_eq3_reduce_to_compulsory_traffic_without_tiling():
    # one weight tile, one output tile per SM, no spatial split: every tensor once
    W, I, O = 1000, 5000, 7000
    assert accounting.eq2_pw_gma(W, W, I, O, O, I, I + O + W, 1) == I + O + W
    assert accounting.eq3_dw_gma(8, 0, I, O, 100, 100, W, I, O, W, 1, I + O + W, 1) == \
        I + O + W
    # the weight tile count multiplies IFM reads; the OFM tile count multiplies weights
    assert accounting.eq2_pw_gma(W, W // 4, I, O, O // 2, 1, 10 ** 9, 1) == \
        4 * I + O + 2 * W


def test_equations_mark_infeasible_tilings_infinite():
    assert accounting.eq2_pw_gma(10, 10, 10, 10, 10, 10, 29, 1) == float("inf")
    assert accounting.eq2_pw_gma(10, 10, 10, 100, 10, 10, 1000, 11) == float("inf")
    assert accounting.dwpw_gma(8, 0, 10, 1, 1, 1, 10, 10, 100, 4, 99, 1) == float("inf")
    assert accounting.eq4_pwdw_gma(1, 0, 1, 1, 1, 1, 1, 1, 1, 1, 1, 5, 1, 4, 1) == \
        float("inf")


# ---------------------------------------------------------------------------------
# the sampled back-to-back checker (used at full size on the GPU) against the full one
# ---------------------------------------------------------------------------------
@pytest.mark.parametrize("stride,pad,H,W", [(1, 1, 9, 20), (2, 0, 11, 13), (2, 1, 10, 17),
                                            (1, 0, 7, 6)])
def test_b2b_sampled_rows_equal_full_outputs(stride, pad, H, W):
    # the back-to-back workload's recipe (channels, epilogues, distributions) on a
    # reduced plane; the sampled form sums in another order, but every value here is
    # computed in fp64 and rounded once per storage point, so rows must agree exactly
    wl = fcm_inputs.WORKLOADS["b2b_f16_32x56x56_c64"].replace(N=2, H=H, W=W, stride=stride,
                                                             pad=pad)
    inp = fcm_inputs.make_inputs(wl)
    kw = dict(stride=(stride, stride), pad=(pad, pad), scale1=inp["scale1"],
              bias1=inp["bias1"], act1=wl.act1, scale2=inp["scale2"], bias2=inp["bias2"],
              act2=wl.act2, dtype=wl.dtype)
    full = oracle.b2b(inp["x"], inp["w1"], inp["w2"], **kw)
    assert full.shape == (2, wl.Ho, wl.Wo, wl.K)
    pix = fcm_inputs.sample_pixels(wl, 40)
    rows = oracle.b2b_at(inp["x"], inp["w1"], inp["w2"], pix, **kw)
    assert np.array_equal(rows, full[pix[:, 0], pix[:, 1], pix[:, 2]])
    # and every pixel of one image, so the borders of a stride/pad combination are covered
    every = np.array([(1, h, w) for h in range(wl.Ho) for w in range(wl.Wo)], np.int32)
    assert np.array_equal(oracle.b2b_at(inp["x"], inp["w1"], inp["w2"], every, **kw),
                          full[1].reshape(-1, wl.K))


def test_b2b_sampled_rows_match_library_pipeline():
    # independent of the full C checker: the sampled rows against torch's fp64 conv2d
    # pipeline with the same storage rounding
    wl = fcm_inputs.WORKLOADS["b2b_f16_32x56x56_c64"].replace(N=1, H=8, W=9, C=16, K1=24, K=8)
    inp = fcm_inputs.make_inputs(wl)
    x = torch.from_numpy(inp["x"]).permute(0, 3, 1, 2)
    t = F.conv2d(x, torch.from_numpy(inp["w1"]), padding=1)
    t = t * torch.from_numpy(inp["scale1"])[None, :, None, None] + \
        torch.from_numpy(inp["bias1"])[None, :, None, None]
    t = torch.from_numpy(oracle.round_to(t.clamp(min=0).numpy(), "f16"))
    y = F.conv2d(t, torch.from_numpy(inp["w2"])[:, :, None, None])
    y = y * torch.from_numpy(inp["scale2"])[None, :, None, None] + \
        torch.from_numpy(inp["bias2"])[None, :, None, None]
    y = oracle.round_to(y.clamp(min=0).permute(0, 2, 3, 1).numpy(), "f16")
    pix = np.array([(0, h, w) for h in range(8) for w in range(9)], np.int32)
    rows = oracle.b2b_at(inp["x"], inp["w1"], inp["w2"], pix, scale1=inp["scale1"],
                         bias1=inp["bias1"], act1="relu", scale2=inp["scale2"],
                         bias2=inp["bias2"], act2="relu", dtype="f16")
    # fp64 sums in different orders may differ in the last bit before the rounding to
    # fp16; a flip of one fp16 step is the most that can result
    ref = y.reshape(-1, 8)
    assert np.max(np.abs(rows - ref) / np.maximum(np.abs(ref), 2.0 ** -14)) <= 2.0 ** -10


# ---------------------------------------------------------------------------------
# Eq. 4 and the constructed DW->PW estimate against a simulated tiled execution
# ---------------------------------------------------------------------------------
def _simulate_module_accesses(kind, H, W, C, n1, K, tile_h, tile_w, ct, filt, e):
    """Element-by-element count of the global memory accesses (bytes) of a tiled module
    at stride 1, under the access model the FusePlanner equations describe (FCM paper
    Sec. IV, Fig. 3): the plane is cut into tile_h x tile_w tiles; a tile's input window
    reaches (filt - 1) pixels past every border it shares with another tile (so the
    overlap of each border is fetched by the tiles on both sides of it); the channels
    that a weight tile produces form one work item per spatial tile.  Each work item
    loads its window over all C input channels and the weight tile(s) it needs, and
    writes its output.  kind "dwpw": the channel tile is a slice of ct output channels of
    the pointwise layer, every work item recomputes the whole depthwise layer (all n1 =
    C channels: all depthwise filters) and loads its slice of the pointwise filters.
    kind "pwdw": the channel tile is a slice of ct intermediate channels, carried through
    both layers: its slice of the pointwise filters and of the depthwise filters.
    Returns (total bytes, number of work items)."""
    ext = filt - 1
    loads = np.zeros((H, W), np.int64)
    n_sp = 0
    for y0 in range(0, H, tile_h):
        for x0 in range(0, W, tile_w):
            n_sp += 1
            ya = y0 - (ext if y0 > 0 else 0)
            yb = min(H, y0 + tile_h) + (ext if y0 + tile_h < H else 0)
            xa = x0 - (ext if x0 > 0 else 0)
            xb = min(W, x0 + tile_w) + (ext if x0 + tile_w < W else 0)
            loads[ya:yb, xa:xb] += 1
    n_out = K if kind == "dwpw" else n1
    n_ct = -(-n_out // ct)
    window_bytes = int(loads.sum()) * C * e            # one pass over every window
    total = n_ct * window_bytes
    for c0 in range(0, n_out, ct):
        cw = min(ct, n_out - c0)
        if kind == "dwpw":
            per_item = filt * filt * n1 * e + cw * n1 * e
        else:
            per_item = cw * C * e + filt * filt * cw * e
        total += n_sp * per_item
    total += H * W * n_out * e                          # the module's output, once
    return total, n_sp * n_ct


@pytest.mark.parametrize("H,W,th,tw", [(12, 12, 12, 4), (12, 12, 3, 12), (10, 16, 10, 4),
                                       (9, 9, 9, 9)])
@pytest.mark.parametrize("kind", ["dwpw", "pwdw"])
def test_fcm_estimates_equal_simulated_accesses_without_channel_split(kind, H, W, th, tw):
    # tiles split one direction of the plane (Eq. 1 is exact there) and one channel
    # tile covers every channel: the FCM estimate equals the simulated access count
    C, n1, K, e, filt = 8, 24, 16, 2, 3
    if kind == "dwpw":
        n1 = C
    ch = K if kind == "dwpw" else n1
    sim, items = _simulate_module_accesses(kind, H, W, C, n1, K, th, tw, ch, filt, e)
    ov = accounting.eq1_overlap(W, H, tw, th, filt, filt, 1)
    ifm = H * W * C * e
    ofm = H * W * ch * e
    if kind == "dwpw":
        est = accounting.dwpw_gma(C, ov * e, ifm, 9 * C * e, K * C * e, K * C * e, ofm,
                                  th * tw * K * e, 0, items, 1, 1)
    else:
        est = accounting.eq4_pwdw_gma(C, ov * e, ifm, n1 * C * e, n1 * C * e, 9 * n1 * e,
                                      9 * n1 * e, ofm, th * tw * n1 * e, H * W, th * tw, 0,
                                      items, 1, 1)
    assert est == sim


@pytest.mark.parametrize("ct", [4, 8])
@pytest.mark.parametrize("kind", ["dwpw", "pwdw"])
def test_fcm_estimates_charge_whole_filters_per_output_tile(kind, ct):
    # with the channels split into tiles the printed equations still charge the whole
    # pointwise filter array per output tile (the literal form); the simulation loads
    # only each tile's slice, and every other term agrees exactly
    H, W, th, tw, C, e, filt = 12, 16, 12, 4, 8, 2, 3
    n1 = C if kind == "dwpw" else 16
    K = 16
    ch = K if kind == "dwpw" else n1
    sim, items = _simulate_module_accesses(kind, H, W, C, n1, K, th, tw, ct, filt, e)
    ov = accounting.eq1_overlap(W, H, tw, th, filt, filt, 1)
    ifm, ofm = H * W * C * e, H * W * ch * e
    if kind == "dwpw":
        est = accounting.dwpw_gma(C, ov * e, ifm, 9 * C * e, K * C * e, ct * C * e, ofm,
                                  th * tw * ct * e, 0, items, 1, 1)
        whole, tile = K * C * e, ct * C * e
    else:
        est = accounting.eq4_pwdw_gma(C, ov * e, ifm, n1 * C * e, ct * C * e, 9 * n1 * e,
                                      9 * ct * e, ofm, th * tw * ct * e, H * W, th * tw, 0,
                                      items, 1, 1)
        whole, tile = n1 * C * e, ct * C * e
    assert est - sim == items * (whole - tile)


def test_eq4_weight_tile_count_is_the_larger_layers():
    # the PW input is re-read once per weight tile of whichever layer needs more tiles
    base = dict(pw_ifms_d=4, dw_overlap=10, pw_ifms_sz=1000, pw_weights_sz=64,
                dw_weights_sz=36, dw_ofms_sz=500, dw_ofms_tile_sz=500, dw_ofms_hw=10,
                dw_ofms_tile_hw=10, tiles_sz_sum=0, n_fcm_ofm_tiles=1, l1_sz=1, n_sms=1)
    one = accounting.eq4_pwdw_gma(pw_weights_tile_sz=64, dw_weights_tile_sz=36, **base)
    assert one == (2 * 4 * 10 + 1000) + 64 + 36 + 500
    pw4 = accounting.eq4_pwdw_gma(pw_weights_tile_sz=16, dw_weights_tile_sz=36, **base)
    dw3 = accounting.eq4_pwdw_gma(pw_weights_tile_sz=64, dw_weights_tile_sz=12, **base)
    assert pw4 - one == 3 * (2 * 4 * 10 + 1000)
    assert dw3 - one == 2 * (2 * 4 * 10 + 1000)
    # and without the output term added by reading (iii), the value printed on the page
    assert accounting.eq4_pwdw_gma(pw_weights_tile_sz=64, dw_weights_tile_sz=36,
                                   include_output=False, **base) == one - 500
