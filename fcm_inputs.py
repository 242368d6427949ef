"""Seeded synthetic workloads for the fused depthwise->pointwise module, the
pointwise->depthwise module and the 3x3->1x1 back-to-back pair.

This module only describes shapes and draws random numbers: it holds none of the
method's arithmetic and imports neither the HIP library nor the oracle, so both sides
can take their inputs from it.

Every tensor is drawn in float64 from ``numpy.random.default_rng(seed)`` in the fixed
order X, first-layer weights, scale1, bias1, second-layer weights, scale2, bias2 (and for
the three-layer module the projection's weights, scale3, bias3), then
narrowed to float32 and from there to the storage type with torch's round-to-nearest-
even casts.  The narrowed values *are* the inputs: both the oracle and the GPU see the
same numbers.  Weight layouts are PyTorch's: depthwise [C*mult, R, S], pointwise [K, C],
standard conv [K1, C, 3, 3], second conv [K, K1]; for the pointwise->depthwise module
the first layer is pointwise [K1, C] and the second depthwise [K1, 3, 3] (K = K1); the
three-layer module adds the projection [K, K1].

The workloads stand in for the layer shapes the pages evaluate (MobileNet-style
depthwise-separable blocks, the forum's CIFAR network, ResNet-style 3x3 -> 1x1 pairs,
MobileNetV2-style inverted-residual expansions for the pointwise->depthwise module and
whole inverted-residual blocks for the three-layer module);
no dataset or trained weight is involved.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "dwpw", "b2b", "pwdw", "pwpw" or "pwdwpw"
    dtype: str           # "f32" | "f16" | "bf16" | "i8"
    N: int
    H: int
    W: int
    C: int
    K: int               # output channels of the module (pwdw: == K1)
    K1: int              # b2b: output channels of the 3x3 conv; dwpw: == C;
                         # pwdw, pwdwpw: output channels of the (first) pointwise layer
    stride: int = 1
    pad: int = 1
    R: int = 3
    S: int = 3
    dil: int = 1          # dwpw: dilation of the depthwise taps
    mult: int = 1         # dwpw: depth multiplier (K1 == C * mult)
    act1: str = "none"
    act2: str = "none"
    scale1: bool = False  # whether a per-channel scale / bias array is passed
    bias1: bool = False
    scale2: bool = False
    bias2: bool = False
    act3: str = "none"    # pwdwpw: the projection's activation, scale / bias, and whether
    scale3: bool = False  # the identity shortcut adds the input pixel
    bias3: bool = False
    residual: bool = False
    x_dist: tuple = ("normal", 0.0, 1.0)
    w_dist: tuple = ("normal", 0.0, 0.1)
    scale_dist: tuple = ("uniform", 0.5, 1.5)
    bias_dist: tuple = ("normal", 0.0, 0.1)
    seed: int = 0
    description: str = ""

    @property
    def Ho(self) -> int:
        return (self.H + 2 * self.pad - (self.R - 1) * self.dil - 1) // self.stride + 1

    @property
    def Wo(self) -> int:
        return (self.W + 2 * self.pad - (self.S - 1) * self.dil - 1) // self.stride + 1

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny_f32_1x16x16_c32": Workload(
        "tiny_f32_1x16x16_c32", "dwpw", "f32", N=1, H=16, W=16, C=32, K=32, K1=32,
        bias2=True, x_dist=("normal", 0.0, 1.0), w_dist=("uniform", -0.5, 0.5),
        bias_dist=("zero",), seed=1,
        description="DW 3x3 s1 p1 + PW 1x1, fp32, N=1 16x16 C=32 K=32, bias 0, "
                    "no activation"),
    "mbv1_f16_8x112x112_c64_k128": Workload(
        "mbv1_f16_8x112x112_c64_k128", "dwpw", "f16", N=8, H=112, W=112, C=64, K=128, K1=64,
        act1="relu6", act2="relu6", scale1=True, bias1=True, scale2=True, bias2=True,
        x_dist=("normal", 0.0, 1.0), w_dist=("normal", 0.0, 0.1), seed=2,
        description="MobileNetV1-style block: DW 3x3 s1 C=64 + scale/bias+ReLU6, "
                    "PW 64->128 + scale/bias+ReLU6, fp16, N=8 112x112"),
    "cifar_bf16_256x32x32_c128": Workload(
        "cifar_bf16_256x32x32_c128", "dwpw", "bf16", N=256, H=32, W=32, C=128, K=128, K1=128,
        act2="relu", bias2=True, x_dist=("uniform", -1.0, 1.0),
        w_dist=("normal", 0.0, 0.05), bias_dist=("normal", 0.0, 0.05), seed=3,
        description="CIFAR-style DW+PW pair: DW 3x3 s1 groups=C + PW 128->128, bf16, "
                    "N=256 32x32, bias+ReLU after PW"),
    "down_f16_64x56x56_c256_k512_s2": Workload(
        "down_f16_64x56x56_c256_k512_s2", "dwpw", "f16", N=64, H=56, W=56, C=256, K=512, K1=256, stride=2,
        act1="relu6", act2="relu6", scale1=True, bias1=True, scale2=True, bias2=True,
        w_dist=("normal", 0.0, 0.05), seed=41,
        description="Downsampling FCM: DW 3x3 s2 C=256 + PW 256->512, scale/bias+ReLU6 "
                    "each, fp16, N=64 56x56 -> 28x28"),
    "late_f16_64x7x7_c1024": Workload(
        "late_f16_64x7x7_c1024", "dwpw", "f16", N=64, H=7, W=7, C=1024, K=1024, K1=1024,
        act1="relu6", act2="relu6", scale1=True, bias1=True, scale2=True, bias2=True,
        w_dist=("normal", 0.0, 0.05), seed=42,
        description="Late-stage FCM: DW 3x3 s1 C=1024 + PW 1024->1024, "
                    "scale/bias+ReLU6 each, fp16, N=64 7x7"),
    "b2b_f16_32x56x56_c64": Workload(
        "b2b_f16_32x56x56_c64", "b2b", "f16", N=32, H=56, W=56, C=64, K=64, K1=64,
        act1="relu", act2="relu", scale1=True, bias1=True, scale2=True, bias2=True,
        w_dist=("normal", 0.0, 0.05), seed=5,
        description="Back-to-back: conv 3x3 p1 64->64 + scale_bias_relu, conv 1x1 "
                    "64->64 + scale_bias_relu, fp16, N=32 56x56"),
    "mbv1i8_i8_8x112x112_c32_k64": Workload(
        "mbv1i8_i8_8x112x112_c32_k64", "dwpw", "i8", N=8, H=112, W=112, C=32, K=64, K1=32,
        act1="relu", act2="relu", scale1=True, bias1=True, scale2=True, bias2=True,
        x_dist=("int", -64, 63), w_dist=("int", -127, 127),
        scale_dist=("uniform", 0.002, 0.006), bias_dist=("normal", 0.0, 8.0), seed=8,
        description="INT8 DWPW (MobileNetV1 layers 2-3): DW 3x3 s1 C=32 + requantize+ReLU, "
                    "PW 32->64 + requantize+ReLU, int8 with int32 sums, N=8 112x112"),
    "pwpw_f16_32x56x56_c64_k32_k64": Workload(
        "pwpw_f16_32x56x56_c64_k32_k64", "pwpw", "f16", N=32, H=56, W=56, C=64, K=64, K1=32,
        R=1, S=1, pad=0, act1="relu6", act2="relu6", scale1=True, bias1=True, scale2=True,
        bias2=True, x_dist=("normal", 0.0, 1.0), w_dist=("normal", 0.0, 0.1), seed=9,
        description="PW->PW module (bottleneck pair): PW 64->32 + scale/bias+ReLU6, "
                    "PW 32->64 + scale/bias+ReLU6, fp16, N=32 56x56"),
    "pwdw_f16_32x56x56_c24_k144": Workload(
        "pwdw_f16_32x56x56_c24_k144", "pwdw", "f16", N=32, H=56, W=56, C=24, K=144, K1=144,
        act1="relu6", act2="relu6", scale1=True, bias1=True, scale2=True, bias2=True,
        x_dist=("normal", 0.0, 1.0), w_dist=("normal", 0.0, 0.1), seed=6,
        description="PW->DW module (MobileNetV2-style expansion): PW 24->144 + "
                    "scale/bias+ReLU6, DW 3x3 s1 + scale/bias+ReLU6, fp16, N=32 56x56"),
    "pwdw_f16_32x112x112_c16_k96_s2": Workload(
        "pwdw_f16_32x112x112_c16_k96_s2", "pwdw", "f16", N=32, H=112, W=112, C=16, K=96,
        K1=96, stride=2, act1="relu6", act2="relu6", scale1=True, bias1=True, scale2=True,
        bias2=True, x_dist=("normal", 0.0, 1.0), w_dist=("normal", 0.0, 0.1), seed=7,
        description="Downsampling PW->DW module: PW 16->96 + scale/bias+ReLU6, DW 3x3 s2 "
                    "+ scale/bias+ReLU6, fp16, N=32 112x112 -> 56x56"),
    # the three layers of an inverted-residual block (PW -> DW -> PW)
    "pwdwpw_f16_32x56x56_c24_k144_k24": Workload(
        "pwdwpw_f16_32x56x56_c24_k144_k24", "pwdwpw", "f16", N=32, H=56, W=56, C=24, K=24,
        K1=144, act1="relu6", act2="relu6", act3="none", residual=True, scale1=True,
        bias1=True, scale2=True, bias2=True, scale3=True, bias3=True,
        x_dist=("normal", 0.0, 1.0), w_dist=("normal", 0.0, 0.1), seed=13,
        description="Inverted-residual block (MobileNetV2-style 56x56 stage): PW 24->144 + "
                    "scale/bias+ReLU6, DW 3x3 s1 + scale/bias+ReLU6, PW 144->24 + "
                    "scale/bias (linear), identity shortcut, fp16, N=32 56x56"),
    "pwdwpw_f16_32x112x112_c16_k96_k24_s2": Workload(
        "pwdwpw_f16_32x112x112_c16_k96_k24_s2", "pwdwpw", "f16", N=32, H=112, W=112, C=16,
        K=24, K1=96, stride=2, act1="relu6", act2="relu6", act3="none", scale1=True,
        bias1=True, scale2=True, bias2=True, scale3=True, bias3=True,
        x_dist=("normal", 0.0, 1.0), w_dist=("normal", 0.0, 0.1), seed=14,
        description="Downsampling inverted-residual block: PW 16->96 + scale/bias+ReLU6, "
                    "DW 3x3 s2 + scale/bias+ReLU6, PW 96->24 + scale/bias (linear), fp16, "
                    "N=32 112x112 -> 56x56"),
    # generalised depthwise layers (filter size, dilation, depth multiplier)
    "dw5_f16_32x28x28_c120_k40": Workload(
        "dw5_f16_32x28x28_c120_k40", "dwpw", "f16", N=32, H=28, W=28, C=120, K=40, K1=120,
        R=5, S=5, pad=2, act1="relu", act2="none", scale1=True, bias1=True, scale2=True,
        bias2=True, x_dist=("normal", 0.0, 1.0), w_dist=("normal", 0.0, 0.1), seed=10,
        description="5x5 depthwise block (MobileNetV3-style 28x28 stage): DW 5x5 s1 p2 C=120 "
                    "+ scale/bias+ReLU, PW 120->40 + scale/bias (linear), fp16, N=32 28x28"),
    "dil2_f16_8x33x33_c960_k160": Workload(
        "dil2_f16_8x33x33_c960_k160", "dwpw", "f16", N=8, H=33, W=33, C=960, K=160, K1=960,
        dil=2, pad=2, act1="relu6", act2="none", scale1=True, bias1=True, scale2=True,
        bias2=True, x_dist=("normal", 0.0, 1.0), w_dist=("normal", 0.0, 0.05), seed=11,
        description="Dilated depthwise block (MobileNetV2 backbone at output stride 16): "
                    "DW 3x3 dilation 2 p2 C=960 + scale/bias+ReLU6, PW 960->160 + "
                    "scale/bias (linear), fp16, N=8 33x33"),
    "mult2_f16_8x112x112_c32_k128": Workload(
        "mult2_f16_8x112x112_c32_k128", "dwpw", "f16", N=8, H=112, W=112, C=32, K=128,
        K1=64, mult=2, act1="relu6", act2="relu6", scale1=True, bias1=True, scale2=True,
        bias2=True, x_dist=("normal", 0.0, 1.0), w_dist=("normal", 0.0, 0.1), seed=12,
        description="Depth multiplier 2: DW 3x3 s1 C=32 x2 -> 64 + scale/bias+ReLU6, "
                    "PW 64->128 + scale/bias+ReLU6, fp16, N=8 112x112"),
}


def _draw(rng: np.random.Generator, dist: tuple, shape) -> np.ndarray:
    kind = dist[0]
    if kind == "normal":
        return rng.normal(dist[1], dist[2], size=shape)
    if kind == "uniform":
        return rng.uniform(dist[1], dist[2], size=shape)
    if kind == "zero":
        return np.zeros(shape)
    if kind == "int":          # small integers in [lo, hi]
        return rng.integers(dist[1], dist[2] + 1, size=shape).astype(np.float64)
    if kind == "sparse_sign":  # values in {-1, 0, 1} with P(nonzero) = dist[1]
        mag = rng.random(size=shape) < dist[1]
        sign = np.where(rng.random(size=shape) < 0.5, -1.0, 1.0)
        return np.where(mag, sign, 0.0)
    raise ValueError(f"unknown distribution {dist}")


def _narrow(a: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> float32 -> storage type (torch RNE casts); returned as float64.  int8:
    the nearest integer, saturated."""
    if dtype == "i8":
        return np.clip(np.rint(a), -128, 127).astype(np.float64)
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    return t.to(tdt).to(torch.float64).numpy()


def make_inputs(wl: Workload, seed: Optional[int] = None) -> dict:
    """Draw the workload's tensors.  Returns float64 numpy arrays whose values are
    exactly representable in the storage type (scale/bias are float32 values)."""
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    x = _draw(rng, wl.x_dist, (wl.N, wl.H, wl.W, wl.C))
    if wl.kind == "dwpw":
        w1 = _draw(rng, wl.w_dist, (wl.C * wl.mult, wl.R, wl.S))
        n1 = wl.C * wl.mult
    elif wl.kind in ("pwdw", "pwpw", "pwdwpw"):
        w1 = _draw(rng, wl.w_dist, (wl.K1, wl.C))
        n1 = wl.K1
    else:
        w1 = _draw(rng, wl.w_dist, (wl.K1, wl.C, wl.R, wl.S))
        n1 = wl.K1
    s1 = _draw(rng, wl.scale_dist, (n1,)) if wl.scale1 else None
    b1 = _draw(rng, wl.bias_dist, (n1,)) if wl.bias1 else None
    if wl.kind in ("pwdw", "pwdwpw"):
        w2 = _draw(rng, wl.w_dist, (wl.K1, wl.R, wl.S))
    else:
        w2 = _draw(rng, wl.w_dist, (wl.K, n1))
    n2 = wl.K1 if wl.kind == "pwdwpw" else wl.K
    s2 = _draw(rng, wl.scale_dist, (n2,)) if wl.scale2 else None
    b2 = _draw(rng, wl.bias_dist, (n2,)) if wl.bias2 else None
    w3 = s3 = b3 = None
    if wl.kind == "pwdwpw":
        w3 = _draw(rng, wl.w_dist, (wl.K, wl.K1))
        s3 = _draw(rng, wl.scale_dist, (wl.K,)) if wl.scale3 else None
        b3 = _draw(rng, wl.bias_dist, (wl.K,)) if wl.bias3 else None
    out = {
        "x": _narrow(x, wl.dtype),
        "w1": _narrow(w1, wl.dtype),
        "w2": _narrow(w2, wl.dtype),
        "scale1": None if s1 is None else _narrow(s1, "f32"),
        "bias1": None if b1 is None else _narrow(b1, "f32"),
        "scale2": None if s2 is None else _narrow(s2, "f32"),
        "bias2": None if b2 is None else _narrow(b2, "f32"),
    }
    if wl.kind == "pwdwpw":
        out["w3"] = _narrow(w3, wl.dtype)
        out["scale3"] = None if s3 is None else _narrow(s3, "f32")
        out["bias3"] = None if b3 is None else _narrow(b3, "f32")
    return out


def to_torch(a: Optional[np.ndarray], dtype: str, device=None):
    """Cast a float64 array (already representable) to a torch tensor of the storage
    type, optionally on a device."""
    if a is None:
        return None
    import torch
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
           "i8": torch.int8}[dtype]
    t = torch.from_numpy(np.ascontiguousarray(a)).to(tdt)
    return t.to(device) if device is not None else t


def sample_pixels(wl: Workload, count: int, seed: int = 1234) -> np.ndarray:
    """Output pixels (n, oh, ow) to check at full size: all four image corners and
    edges of the first and last image plus uniformly drawn interior pixels."""
    rng = np.random.default_rng(seed)
    fixed = []
    for n in {0, wl.N - 1}:
        for oh in {0, wl.Ho - 1, wl.Ho // 2}:
            for ow in {0, wl.Wo - 1, wl.Wo // 2}:
                fixed.append((n, oh, ow))
    k = max(0, count - len(fixed))
    rnd = np.stack([rng.integers(0, wl.N, k), rng.integers(0, wl.Ho, k),
                    rng.integers(0, wl.Wo, k)], axis=1) if k else np.zeros((0, 3), int)
    return np.concatenate([np.array(fixed, dtype=np.int64).reshape(-1, 3), rnd]).astype(
        np.int32)
