"""Helpers for the GPU parity tests: run the HIP path through the C ABI and the CPU
oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import numpy as np

import fcm_inputs
import oracle

# int8 codes are decided by the same binary32 steps on both sides: exact
TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2, "i8": 0.0}


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """Normwise max relative error: max|got - ref| / max|ref|."""
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    return num / den if den > 0 else num


MANTISSA = {"f32": 23, "f16": 10, "bf16": 7}


def ulp(a: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the storage type's values at |a| (normal range; subnormal spacing below
    the smallest normal)."""
    m = MANTISSA[dtype]
    emin = {"f32": -126, "f16": -14, "bf16": -126}[dtype]
    e = np.floor(np.log2(np.maximum(np.abs(a), 2.0 ** emin)))
    return 2.0 ** (e - m)


def elementwise_excess(got: np.ndarray, ref: np.ndarray, dtype: str, n_ulp: float = 4.0,
                       floor_ulps: float = 1.0) -> float:
    """Largest |got - ref| / (n_ulp * ulp(ref) + floor_ulps * ulp(max|ref|)) over the
    elements: <= 1 means every element is within a few units of the storage type of the
    oracle's value, plus a floor of one unit at the output's largest magnitude (an
    intermediate value can round to the neighbouring storage value when the fp32 and fp64
    sums straddle a rounding boundary, which moves an output by a fraction of that unit)."""
    if ref.size == 0 or dtype not in ("f16", "bf16"):
        # (fp32 storage: the normwise 1e-5 bar; the fp32 sums of the kernels and the fp64
        # sums of the oracle differ by more than a few output units where terms cancel)
        return 0.0
    top = float(np.max(np.abs(ref)))
    tol = n_ulp * ulp(ref, dtype) + floor_ulps * (ulp(np.array(top), dtype) if top > 0 else 0.0)
    return float(np.max(np.abs(got - ref) / np.maximum(tol, 1e-300)))


def oracle_kwargs(wl, inp) -> dict:
    kw = dict(stride=(wl.stride, wl.stride), pad=(wl.pad, wl.pad), scale1=inp["scale1"],
              bias1=inp["bias1"], act1=wl.act1, scale2=inp["scale2"], bias2=inp["bias2"],
              act2=wl.act2, dtype=wl.dtype)
    if wl.kind == "pwdwpw":
        kw.update(scale3=inp.get("scale3"), bias3=inp.get("bias3"), act3=wl.act3,
                  residual=wl.residual)
    return kw


def final_act(wl) -> str:
    """The activation of the module's last layer."""
    return wl.act3 if wl.kind == "pwdwpw" else wl.act2


def is_gen(wl) -> bool:
    """A DW->PW workload whose depthwise layer is not the plain 3x3 one."""
    return wl.kind == "dwpw" and (wl.R != 3 or wl.S != 3 or wl.dil != 1 or wl.mult != 1)


def oracle_full(wl, inp) -> np.ndarray:
    if is_gen(wl):
        return oracle.dwpw_gen(inp["x"], inp["w1"], inp["w2"],
                               dilation=(wl.dil, wl.dil), **oracle_kwargs(wl, inp))
    if wl.kind == "pwdwpw":
        return oracle.pwdwpw(inp["x"], inp["w1"], inp["w2"], inp["w3"], **oracle_kwargs(wl, inp))
    fn = {"dwpw": oracle.dwpw, "b2b": oracle.b2b, "pwdw": oracle.pwdw,
          "pwpw": oracle.pwpw}[wl.kind]
    return fn(inp["x"], inp["w1"], inp["w2"], **oracle_kwargs(wl, inp))


def oracle_rows(wl, inp, pix) -> np.ndarray:
    if is_gen(wl):  # the whole output (seconds at the workloads' sizes), then the pixels
        full = oracle_full(wl, inp)
        return full[pix[:, 0], pix[:, 1], pix[:, 2]]
    if wl.kind == "pwdwpw":
        return oracle.pwdwpw_at(inp["x"], inp["w1"], inp["w2"], inp["w3"], pix,
                                **oracle_kwargs(wl, inp))
    fn = {"dwpw": oracle.dwpw_at, "b2b": oracle.b2b_at, "pwdw": oracle.pwdw_at,
          "pwpw": oracle.pwpw_at}[wl.kind]
    return fn(inp["x"], inp["w1"], inp["w2"], pix, **oracle_kwargs(wl, inp))


def run_gpu(wl, inp, variant=None, path="fused", tune=False):
    """Run the module on the GPU; returns the output as float64 numpy.  With tune the
    plan is first replaced by the measured choice (fcm_tune), as the benchmark does."""
    import torch
    from depthwise_pointwise_convolution_amd.module import TORCH_DTYPES, from_workload
    mod = from_workload(wl, inp, device="cuda", variant=variant)
    x = torch.from_numpy(inp["x"]).to(TORCH_DTYPES[wl.dtype]).cuda()
    if tune:
        mod.tune(x, iters=3)
        torch.cuda.synchronize()
    y = mod.fused(x) if path == "fused" else mod.unfused(x)
    torch.cuda.synchronize()
    return y.double().cpu().numpy(), mod


def int_inputs(wl, seed: int) -> dict:
    """Small-integer inputs for which every step is exact in every storage type:
    |x| <= 2, filters in {-1, 0, 1} with few non-zeros per output row, scale 1 or 2,
    integer bias.  Intermediates stay below 256 in magnitude, so rounding to bf16,
    fp16 or fp32 never changes a value and the GPU must equal the oracle bit for
    bit whatever its summation order."""
    rng = np.random.default_rng(seed)
    x = rng.integers(-2, 3, size=(wl.N, wl.H, wl.W, wl.C)).astype(np.float64)
    if wl.kind == "pwdw":
        return _int_inputs_pwdw(wl, rng, x)
    if wl.kind == "pwdwpw":
        return _int_inputs_pwdwpw(wl, rng, x)
    n1 = wl.C * wl.mult if wl.kind == "dwpw" else wl.K1
    if is_gen(wl):
        # at most 9 non-zero taps of +-1 per filter, whatever its size
        w1 = np.zeros((n1, wl.R * wl.S))
        for j in range(n1):
            idx = rng.choice(wl.R * wl.S, size=min(9, wl.R * wl.S), replace=False)
            w1[j, idx] = rng.integers(-1, 2, size=idx.size)
        w1 = w1.reshape(n1, wl.R, wl.S)
        acc1 = 9 * 2
    elif wl.kind == "pwpw":
        w1 = np.zeros((wl.K1, wl.C))
        for k in range(wl.K1):
            idx = rng.choice(wl.C, size=min(6, wl.C), replace=False)
            w1[k, idx] = rng.choice([-1.0, 1.0], size=idx.size)
        acc1 = 6 * 2
    elif wl.kind == "dwpw":
        w1 = rng.integers(-1, 2, size=(wl.C, 3, 3)).astype(np.float64)
        acc1 = 9 * 2       # |first-layer sum| <= 9 taps * |x|
    else:
        w1 = np.zeros((wl.K1, wl.C, 3, 3))
        for k in range(wl.K1):
            idx = rng.choice(wl.C * 9, size=min(6, wl.C * 9), replace=False)
            w1[k].reshape(-1)[idx] = rng.choice([-1.0, 1.0], size=idx.size)
        acc1 = 6 * 2
    s1 = rng.choice([1.0, 2.0], size=n1) if wl.scale1 else None
    b1 = rng.integers(-2, 3, size=n1).astype(np.float64) if wl.bias1 else None
    t_max = acc1 * (2 if s1 is not None else 1) + 2
    # second layer: nz non-zeros per output row keep |sum| <= 100, so after a scale
    # of at most 2 and a bias of at most 2 every value is an integer below 256
    nz = max(1, min(n1, 100 // t_max))
    w2 = np.zeros((wl.K, n1))
    for k in range(wl.K):
        idx = rng.choice(n1, size=nz, replace=False)
        w2[k, idx] = rng.choice([-1.0, 1.0], size=nz)
    s2 = rng.choice([1.0, 2.0], size=wl.K) if wl.scale2 else None
    b2 = rng.integers(-2, 3, size=wl.K).astype(np.float64) if wl.bias2 else None
    return {"x": x, "w1": w1, "w2": w2, "scale1": s1, "bias1": b1, "scale2": s2, "bias2": b2}


def _int_inputs_pwdw(wl, rng, x) -> dict:
    """PW->DW module: at most 6 non-zero pointwise filter taps of +-1 per expanded
    channel (|intermediate| <= 2*(2*6)+2 = 26) and at most 4 non-zero depthwise taps
    (|output| <= 2*(4*26)+2 = 210): every value an integer below 256."""
    w1 = np.zeros((wl.K1, wl.C))
    for k in range(wl.K1):
        idx = rng.choice(wl.C, size=min(6, wl.C), replace=False)
        w1[k, idx] = rng.choice([-1.0, 1.0], size=idx.size)
    s1 = rng.choice([1.0, 2.0], size=wl.K1) if wl.scale1 else None
    b1 = rng.integers(-2, 3, size=wl.K1).astype(np.float64) if wl.bias1 else None
    w2 = np.zeros((wl.K1, 9))
    for k in range(wl.K1):
        idx = rng.choice(9, size=4, replace=False)
        w2[k, idx] = rng.choice([-1.0, 1.0], size=4)
    s2 = rng.choice([1.0, 2.0], size=wl.K1) if wl.scale2 else None
    b2 = rng.integers(-2, 3, size=wl.K1).astype(np.float64) if wl.bias2 else None
    return {"x": x, "w1": w1, "w2": w2.reshape(wl.K1, 3, 3), "scale1": s1, "bias1": b1,
            "scale2": s2, "bias2": b2}


def _int_inputs_pwdwpw(wl, rng, x) -> dict:
    """PW->DW->PW module: 2 non-zero expansion taps of +-1 per expanded channel
    (|t1| <= 2*4+2 = 10), 3 non-zero depthwise taps (|t2| <= 2*30+2 = 62), 2 non-zero
    projection taps with scale 1 (|y| <= 124+2, plus 2 for the shortcut): every value an
    integer below 256, exact in every storage type."""
    w1 = np.zeros((wl.K1, wl.C))
    for k in range(wl.K1):
        idx = rng.choice(wl.C, size=min(2, wl.C), replace=False)
        w1[k, idx] = rng.choice([-1.0, 1.0], size=idx.size)
    s1 = rng.choice([1.0, 2.0], size=wl.K1) if wl.scale1 else None
    b1 = rng.integers(-2, 3, size=wl.K1).astype(np.float64) if wl.bias1 else None
    w2 = np.zeros((wl.K1, 9))
    for k in range(wl.K1):
        idx = rng.choice(9, size=3, replace=False)
        w2[k, idx] = rng.choice([-1.0, 1.0], size=3)
    s2 = rng.choice([1.0, 2.0], size=wl.K1) if wl.scale2 else None
    b2 = rng.integers(-2, 3, size=wl.K1).astype(np.float64) if wl.bias2 else None
    w3 = np.zeros((wl.K, wl.K1))
    for k in range(wl.K):
        idx = rng.choice(wl.K1, size=min(2, wl.K1), replace=False)
        w3[k, idx] = rng.choice([-1.0, 1.0], size=idx.size)
    s3 = np.ones(wl.K) if wl.scale3 else None
    b3 = rng.integers(-2, 3, size=wl.K).astype(np.float64) if wl.bias3 else None
    return {"x": x, "w1": w1, "w2": w2.reshape(wl.K1, 3, 3), "scale1": s1, "bias1": b1,
            "scale2": s2, "bias2": b2, "w3": w3, "scale3": s3, "bias3": b3}


def all_variants_for(wl):
    """Indices of every compiled variant able to run the workload."""
    import depthwise_pointwise_convolution_amd as F
    p = F.problem(wl.kind, wl.dtype, wl.N, wl.H, wl.W, wl.C, wl.K,
                  None if wl.kind == "dwpw" else wl.K1, R=wl.R, S=wl.S, stride=wl.stride,
                  pad=wl.pad, act1=wl.act1, act2=wl.act2, dilation=wl.dil, mult=wl.mult,
                  act3=wl.act3, residual=wl.residual)
    out = []
    for v in range(F.fcm_num_variants()):
        try:
            F.fcm_plan_variant(p, v)
            out.append(v)
        except F.FcmError:
            pass
    return out


REDUCED = {
    # ragged spatial tails (not multiples of the tiles) and several tiles per image
    "tiny_f32_1x16x16_c32": dict(),
    "mbv1_f16_8x112x112_c64_k128": dict(N=2, H=29, W=37),
    "cifar_bf16_256x32x32_c128": dict(N=3),
    "down_f16_64x56x56_c256_k512_s2": dict(N=2, H=57, W=45),
    "late_f16_64x7x7_c1024": dict(N=3),
    "b2b_f16_32x56x56_c64": dict(N=2, H=23, W=37),
    "pwdw_f16_32x56x56_c24_k144": dict(N=2, H=29, W=37),
    "mbv1i8_i8_8x112x112_c32_k64": dict(N=2, H=29, W=37),
    "pwpw_f16_32x56x56_c64_k32_k64": dict(N=2, H=29, W=37),
    "pwdw_f16_32x112x112_c16_k96_s2": dict(N=2, H=45, W=57),
    "dw5_f16_32x28x28_c120_k40": dict(N=2, H=29, W=37),
    "dil2_f16_8x33x33_c960_k160": dict(N=2, H=21, W=19),
    "mult2_f16_8x112x112_c32_k128": dict(N=2, H=29, W=37),
    "pwdwpw_f16_32x56x56_c24_k144_k24": dict(N=2, H=29, W=37),
    "pwdwpw_f16_32x112x112_c16_k96_k24_s2": dict(N=2, H=45, W=57),
}


def reduced(name: str):
    return fcm_inputs.WORKLOADS[name].replace(**REDUCED[name])
