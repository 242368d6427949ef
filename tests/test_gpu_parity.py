"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same
seeded inputs.

Bars: bit-exact on integer probes (every step exact, so any index, halo, stride,
padding, tiling or layout mistake shows); normwise max relative error <= 1e-5 for
fp32 storage and <= 2e-2 (fp32 accumulation) for fp16/bf16 otherwise.
"""
import zlib

import numpy as np
import pytest

import fcm_inputs
from gpu_util import (TOL, all_variants_for, elementwise_excess, final_act, gpu_available,
                      int_inputs, oracle_full, oracle_rows, reduced, rel_err, run_gpu)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

NAMES = list(fcm_inputs.WORKLOADS)


def _log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("path", ["fused", "unfused"])
def test_reduced_config_full_compare(name, path):
    wl = reduced(name)
    inp = fcm_inputs.make_inputs(wl)
    _log(f"case {name} reduced {wl.N}x{wl.H}x{wl.W}x{wl.C}->{wl.K} {path}")
    got, mod = run_gpu(wl, inp, path=path)
    ref = oracle_full(wl, inp)
    assert got.shape == ref.shape
    err = rel_err(got, ref)
    ex = elementwise_excess(got, ref, wl.dtype)
    _log(f"  variant {mod.plan.variant} rel err {err:.3e}, elementwise {ex:.3f} of the bound")
    assert np.all(np.isfinite(got))
    assert err <= TOL[wl.dtype], err
    # elementwise: within 4 units of the storage type at each value (plus one unit at the
    # output's largest magnitude) -- rounding-level regressions the normwise bar admits
    assert ex <= 1.0, ex


@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("path", ["fused", "unfused"])
def test_full_size_config_sampled(name, path):
    """BASELINE-size workloads in the launch configuration the benchmark times,
    checked on sampled output pixels (all image corners and edge midpoints of the
    first and last image, plus random pixels), and by properties over the whole
    output."""
    wl = fcm_inputs.WORKLOADS[name]
    inp = fcm_inputs.make_inputs(wl)
    _log(f"case {name} full {path}")
    got, mod = run_gpu(wl, inp, path=path, tune=path == "fused")
    if path == "fused":
        _log(f"  tuned variant {mod.plan.variant} grid {mod.plan.grid} "
             f"{mod.plan.tuned_us:.2f} us")
        assert mod.plan.tuned_us > 0
    pix = fcm_inputs.sample_pixels(wl, 1500)
    rows = oracle_rows(wl, inp, pix)
    sel = got[pix[:, 0], pix[:, 1], pix[:, 2]]
    err = rel_err(sel, rows)
    _log(f"  sampled rel err {err:.3e}")
    assert err <= TOL[wl.dtype], err
    assert np.all(np.isfinite(got))
    if wl.kind == "pwdwpw" and wl.residual:
        pass  # the shortcut moves the output off the activation's range
    elif final_act(wl) == "relu6":
        assert got.min() >= 0 and got.max() <= 6
    elif final_act(wl) == "relu":
        assert got.min() >= 0


CASES_INT = [
    # (kind, dtype, N, H, W, C, K, K1, stride, pad, act1, act2, epilogue flags)
    ("dwpw", "f16", 2, 9, 21, 64, 128, None, 1, 1, "relu6", "relu6", True),
    ("dwpw", "bf16", 2, 11, 17, 128, 128, None, 1, 1, "none", "relu", False),
    ("dwpw", "f16", 1, 13, 15, 256, 512, None, 2, 1, "relu6", "relu6", True),
    ("dwpw", "f16", 2, 7, 7, 1024, 1024, None, 1, 1, "relu6", "relu6", True),
    ("dwpw", "bf16", 2, 10, 13, 192, 136, None, 2, 1, "relu", "relu6", True),
    ("dwpw", "f16", 3, 2, 3, 64, 72, None, 1, 1, "none", "relu", True),
    ("dwpw", "bf16", 2, 12, 10, 40, 24, None, 2, 0, "relu", "none", True),
    ("dwpw", "f32", 1, 16, 16, 32, 32, None, 1, 1, "none", "none", False),
    ("dwpw", "f32", 2, 9, 13, 40, 72, None, 2, 1, "relu6", "relu", True),
    ("b2b", "f16", 2, 9, 19, 64, 64, 64, 1, 1, "relu", "relu", True),
    ("b2b", "bf16", 1, 10, 9, 32, 48, 32, 1, 0, "none", "relu", True),
    ("b2b", "f16", 1, 11, 12, 40, 24, 96, 2, 1, "relu6", "none", True),
    ("dwpw", "i8", 2, 9, 21, 32, 64, None, 1, 1, "relu", "relu", True),
    ("dwpw", "i8", 1, 13, 15, 64, 128, None, 2, 1, "none", "relu6", True),
    ("dwpw", "i8", 2, 7, 7, 16, 48, None, 1, 0, "relu6", "none", False),
    # wider int8 layers in 64-channel slices: four whole slices, and partial last slices
    ("dwpw", "i8", 2, 9, 21, 256, 128, None, 1, 1, "relu", "relu6", True),
    ("dwpw", "i8", 1, 10, 13, 96, 48, None, 2, 1, "none", "relu", True),
    ("dwpw", "i8", 2, 7, 9, 144, 64, None, 1, 0, "relu6", "none", False),
    ("pwpw", "f16", 2, 9, 21, 64, 64, 32, 1, 0, "relu6", "relu6", True),
    ("pwpw", "bf16", 1, 11, 17, 40, 136, 56, 1, 0, "none", "relu", True),
    ("pwpw", "f16", 3, 5, 7, 24, 24, 64, 1, 0, "relu", "none", False),
    # wide bottleneck pairs: intermediate in 64-channel slices (a partial last one), input
    # channels past one slice, 64 and 128 output channels per workgroup
    ("pwpw", "f16", 2, 9, 21, 24, 24, 144, 1, 0, "relu6", "none", True),
    ("pwpw", "bf16", 1, 11, 17, 96, 96, 576, 1, 0, "relu6", "relu", True),
    ("pwpw", "f16", 2, 7, 9, 160, 40, 200, 1, 0, "none", "relu6", False),
    ("pwdw", "f16", 2, 9, 21, 24, 144, 144, 1, 1, "relu6", "relu6", True),
    ("pwdw", "bf16", 1, 11, 17, 64, 48, 48, 1, 1, "none", "relu", False),
    ("pwdw", "f16", 2, 13, 15, 16, 96, 96, 2, 1, "relu", "relu6", True),
    ("pwdw", "bf16", 1, 10, 9, 40, 40, 40, 2, 0, "relu6", "none", True),
    ("pwdw", "f16", 1, 3, 2, 8, 24, 24, 1, 1, "none", "none", True),
    ("pwdw", "f16", 2, 17, 33, 32, 200, 200, 1, 1, "none", "relu", True),
]


def _int_workload(case):
    kind, dtype, N, H, W, C, K, K1, stride, pad, act1, act2, epi = case
    rs = 1 if kind == "pwpw" else 3
    return fcm_inputs.Workload("int", kind, dtype, N=N, H=H, W=W, C=C, K=K,
                               K1=C if K1 is None else K1, stride=stride, pad=pad, act1=act1,
                               act2=act2, scale1=epi, bias1=epi, scale2=epi, bias2=epi, R=rs,
                               S=rs)


@pytest.mark.parametrize("case", CASES_INT, ids=lambda c: "-".join(map(str, c[:10])))
def test_integer_probes_bit_exact_every_variant(case):
    wl = _int_workload(case)
    seed = zlib.crc32(repr(case).encode()) % 1000
    inp = int_inputs(wl, seed=seed)
    ref = oracle_full(wl, inp)
    variants = all_variants_for(wl)
    assert variants, "no variant runs this problem"
    for v in variants:
        _log(f"case int {case} variant {v}")
        got, _ = run_gpu(wl, inp, variant=v)
        bad = np.argwhere(got != ref)
        assert bad.size == 0, (f"variant {v} (input seed {seed}): {len(bad)} mismatches, "
                               f"first {bad[:3].tolist()}")
    got, _ = run_gpu(wl, inp, path="unfused")
    assert np.array_equal(got, ref), f"layer-by-layer path (input seed {seed})"


@pytest.mark.parametrize("name", NAMES)
def test_full_size_integer_exact_every_variant(name):
    """Every variant able to run the full-size workload, on exact integer inputs with the
    activations switched off (a clamp could hide a wrong value), into an output filled
    with NaN first: every element must be written, and equal the oracle's bit for bit."""
    import dataclasses
    import torch
    from depthwise_pointwise_convolution_amd.module import TORCH_DTYPES, from_workload
    wl = dataclasses.replace(fcm_inputs.WORKLOADS[name], act1="none", act2="none",
                             act3="none")
    inp = int_inputs(wl, seed=11)
    ref = oracle_full(wl, inp)
    x = torch.from_numpy(inp["x"]).to(TORCH_DTYPES[wl.dtype]).cuda()
    variants = all_variants_for(wl)
    assert variants
    for v in variants:
        _log(f"case {name} exact variant {v}")
        mod = from_workload(wl, inp, device="cuda", variant=v)
        y = mod.new_output("cuda")
        for rep in range(2):
            # NaN marks unwritten floats; int8 outputs get two different fill codes, so an
            # unwritten element differs from the expected value in at least one run
            y.fill_(float("nan") if wl.dtype != "i8" else (85 if rep == 0 else -86))
            mod.fused(x, y)
            got = y.double().cpu().numpy()
            bad = np.argwhere(~(got == ref))
            assert bad.size == 0, (f"variant {v} run {rep}: {len(bad)} wrong or unwritten, "
                                   f"first {bad[:4].tolist()}")


def _random_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = "b2b" if rng.random() < 0.3 else "dwpw"
        dtype = rng.choice(["f16", "bf16"] + ([] if kind == "b2b" else ["f32"]))
        C = int(rng.choice([8, 16, 24, 40, 64, 72, 136]))
        K = int(rng.choice([8, 24, 40, 64, 136, 200]))
        K1 = int(rng.choice([8, 32, 64, 96])) if kind == "b2b" else C
        out.append(fcm_inputs.Workload(
            f"rnd{i}", kind, str(dtype), N=int(rng.integers(1, 3)), H=int(rng.integers(1, 24)),
            W=int(rng.integers(1, 24)), C=C, K=K, K1=K1, stride=int(rng.integers(1, 3)),
            pad=int(rng.integers(0, 2)), act1=str(rng.choice(["none", "relu", "relu6"])),
            act2=str(rng.choice(["none", "relu", "relu6"])), scale1=bool(rng.random() < .5),
            bias1=bool(rng.random() < .5), scale2=bool(rng.random() < .5),
            bias2=bool(rng.random() < .5), seed=int(rng.integers(1 << 30))))
    return [w for w in out if w.H + 2 * w.pad >= 3 and w.W + 2 * w.pad >= 3]


@pytest.mark.parametrize("wl", _random_cases(24, 7), ids=lambda w: w.name)
def test_random_small_shapes(wl):
    inp = fcm_inputs.make_inputs(wl)
    ref = oracle_full(wl, inp)
    for path in ("fused", "unfused"):
        _log(f"case {wl} {path}")
        got, _ = run_gpu(wl, inp, path=path)
        err = rel_err(got, ref)
        assert err <= TOL[wl.dtype], (path, err)
        ex = elementwise_excess(got, ref, wl.dtype)
        assert ex <= 1.0, (path, "elementwise", ex)


def _random_i8_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        out.append(fcm_inputs.Workload(
            f"q{i}", "dwpw", "i8", N=int(rng.integers(1, 3)), H=int(rng.integers(1, 24)),
            W=int(rng.integers(1, 40)), C=int(rng.choice([16, 32, 48, 64])),
            K=int(rng.choice([16, 32, 64, 80, 128])), K1=0, stride=int(rng.integers(1, 3)),
            pad=int(rng.integers(0, 2)), act1=str(rng.choice(["none", "relu", "relu6"])),
            act2=str(rng.choice(["none", "relu", "relu6"])), scale1=bool(rng.random() < .7),
            bias1=bool(rng.random() < .7), scale2=bool(rng.random() < .7),
            bias2=bool(rng.random() < .7), x_dist=("int", -128, 127),
            w_dist=("int", -127, 127), scale_dist=("uniform", 0.001, 0.01),
            bias_dist=("normal", 0.0, 8.0), seed=int(rng.integers(1 << 30))))
    return [w.replace(K1=w.C) for w in out if w.H + 2 * w.pad >= 3 and w.W + 2 * w.pad >= 3]


@pytest.mark.parametrize("wl", _random_i8_cases(16, 9), ids=lambda w: w.name)
def test_random_small_shapes_i8(wl):
    inp = fcm_inputs.make_inputs(wl)
    ref = oracle_full(wl, inp)
    for path in ("fused", "unfused"):
        _log(f"case {wl} {path}")
        got, _ = run_gpu(wl, inp, path=path)
        bad = np.argwhere(got != ref)
        assert bad.size == 0, (path, len(bad), bad[:3].tolist())


def _random_pwdw_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        C = int(rng.choice([8, 16, 24, 32, 40, 64]))
        K1 = int(rng.choice([8, 16, 24, 48, 96, 136, 144]))
        out.append(fcm_inputs.Workload(
            f"pd{i}", "pwdw", str(rng.choice(["f16", "bf16"])), N=int(rng.integers(1, 3)),
            H=int(rng.integers(1, 24)), W=int(rng.integers(1, 40)), C=C, K=K1, K1=K1,
            stride=int(rng.integers(1, 3)), pad=int(rng.integers(0, 2)),
            act1=str(rng.choice(["none", "relu", "relu6"])),
            act2=str(rng.choice(["none", "relu", "relu6"])), scale1=bool(rng.random() < .5),
            bias1=bool(rng.random() < .5), scale2=bool(rng.random() < .5),
            bias2=bool(rng.random() < .5), seed=int(rng.integers(1 << 30))))
    return [w for w in out if w.H + 2 * w.pad >= 3 and w.W + 2 * w.pad >= 3]


@pytest.mark.parametrize("wl", _random_pwdw_cases(16, 8), ids=lambda w: w.name)
def test_random_small_shapes_pwdw(wl):
    inp = fcm_inputs.make_inputs(wl)
    ref = oracle_full(wl, inp)
    for path in ("fused", "unfused"):
        _log(f"case {wl} {path}")
        got, _ = run_gpu(wl, inp, path=path)
        err = rel_err(got, ref)
        assert err <= TOL[wl.dtype], (path, err)
        ex = elementwise_excess(got, ref, wl.dtype)
        assert ex <= 1.0, (path, "elementwise", ex)


CASES_PWDWPW = [
    # (dtype, N, H, W, C, K1, K, stride, pad, act1, act2, act3, residual, epilogue flags)
    ("f16", 2, 9, 21, 24, 144, 24, 1, 1, "relu6", "relu6", "none", True, True),
    ("bf16", 1, 11, 17, 32, 96, 32, 1, 1, "none", "relu", "relu", True, False),
    ("f16", 2, 13, 15, 16, 96, 24, 2, 1, "relu", "relu6", "none", False, True),
    ("f16", 1, 3, 2, 8, 24, 8, 1, 1, "none", "none", "none", True, True),
    ("f16", 2, 17, 33, 32, 160, 32, 1, 1, "none", "relu", "relu6", False, True),
    ("f16", 1, 10, 9, 24, 40, 16, 2, 0, "relu6", "none", "none", False, True),
    ("bf16", 2, 8, 8, 24, 144, 24, 1, 1, "relu6", "relu6", "none", True, True),
]


def _pwdwpw_workload(case, name="int3"):
    dtype, N, H, W, C, K1, K, stride, pad, act1, act2, act3, res, epi = case
    return fcm_inputs.Workload(name, "pwdwpw", dtype, N=N, H=H, W=W, C=C, K=K, K1=K1,
                               stride=stride, pad=pad, act1=act1, act2=act2, act3=act3,
                               residual=res, scale1=epi, bias1=epi, scale2=epi, bias2=epi,
                               scale3=epi, bias3=epi)


@pytest.mark.parametrize("case", CASES_PWDWPW, ids=lambda c: "-".join(map(str, c[:13])))
def test_pwdwpw_integer_probes_bit_exact_every_variant(case):
    wl = _pwdwpw_workload(case)
    seed = zlib.crc32(repr(case).encode()) % 1000
    inp = int_inputs(wl, seed=seed)
    ref = oracle_full(wl, inp)
    variants = all_variants_for(wl)
    assert variants, "no variant runs this problem"
    for v in variants:
        _log(f"case int pwdwpw {case} variant {v}")
        got, _ = run_gpu(wl, inp, variant=v)
        bad = np.argwhere(got != ref)
        assert bad.size == 0, (f"variant {v} (input seed {seed}): {len(bad)} mismatches, "
                               f"first {bad[:3].tolist()}")
    got, _ = run_gpu(wl, inp, path="unfused")
    assert np.array_equal(got, ref), f"layer-by-layer path (input seed {seed})"


def _random_pwdwpw_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        C = int(rng.choice([8, 16, 24, 32]))
        stride = int(rng.integers(1, 3))
        K1 = int(rng.choice([8, 24, 48, 96] + ([136, 160] if stride == 1 else [])))
        pad = int(rng.integers(0, 2))
        res = stride == 1 and pad == 1 and bool(rng.random() < 0.6)
        K = C if res else int(rng.choice([8, 16, 24, 32]))
        dtype = str(rng.choice(["f16", "bf16"]))
        if stride == 2:
            dtype = "f16"  # (the bf16 build of the three-layer kernel is stride 1 only)
        out.append(fcm_inputs.Workload(
            f"ir{i}", "pwdwpw", dtype, N=int(rng.integers(1, 3)),
            H=int(rng.integers(1, 24)), W=int(rng.integers(1, 40)), C=C, K=K, K1=K1,
            stride=stride, pad=pad, residual=res,
            act1=str(rng.choice(["none", "relu", "relu6"])),
            act2=str(rng.choice(["none", "relu", "relu6"])),
            act3=str(rng.choice(["none", "relu", "relu6"])), scale1=bool(rng.random() < .5),
            bias1=bool(rng.random() < .5), scale2=bool(rng.random() < .5),
            bias2=bool(rng.random() < .5), scale3=bool(rng.random() < .5),
            bias3=bool(rng.random() < .5), seed=int(rng.integers(1 << 30))))
    return [w for w in out if w.H + 2 * w.pad >= 3 and w.W + 2 * w.pad >= 3]


@pytest.mark.parametrize("wl", _random_pwdwpw_cases(16, 5), ids=lambda w: w.name)
def test_random_small_shapes_pwdwpw(wl):
    inp = fcm_inputs.make_inputs(wl)
    ref = oracle_full(wl, inp)
    for path in ("fused", "unfused"):
        _log(f"case {wl} {path}")
        got, _ = run_gpu(wl, inp, path=path)
        err = rel_err(got, ref)
        assert err <= TOL[wl.dtype], (path, err)
        ex = elementwise_excess(got, ref, wl.dtype)
        assert ex <= 1.0, (path, "elementwise", ex)


def test_pwdwpw_output_guard_bands_and_every_output_written():
    import torch
    from depthwise_pointwise_convolution_amd.module import from_workload
    for name in ("pwdwpw_f16_32x56x56_c24_k144_k24", "pwdwpw_f16_32x112x112_c16_k96_k24_s2"):
        wl = reduced(name)
        inp = fcm_inputs.make_inputs(wl)
        x = torch.from_numpy(inp["x"]).half().cuda()
        for v in all_variants_for(wl):
            _log(f"case {name} guard bands variant {v}")
            mod = from_workload(wl, inp, variant=v)
            n = int(np.prod(mod.out_shape))
            guard = 4096
            buf = torch.full((n + 2 * guard,), float("nan"), dtype=torch.float16,
                             device="cuda")
            y = buf[guard:guard + n].view(mod.out_shape)
            mod.fused(x, y)
            torch.cuda.synchronize()
            b = buf.cpu()
            assert torch.isnan(b[:guard]).all() and torch.isnan(b[guard + n:]).all()
            assert not torch.isnan(b[guard:guard + n]).any()


GUARD_NAMES = ["tiny_f32_1x16x16_c32", "mbv1_f16_8x112x112_c64_k128", "cifar_bf16_256x32x32_c128",
               "down_f16_64x56x56_c256_k512_s2", "late_f16_64x7x7_c1024", "b2b_f16_32x56x56_c64",
               "mbv1i8_i8_8x112x112_c32_k64", "pwpw_f16_32x56x56_c64_k32_k64",
               "dw5_f16_32x28x28_c120_k40", "dil2_f16_8x33x33_c960_k160",
               "mult2_f16_8x112x112_c32_k128"]


def _guarded(n, dtype, fill, guard=4096):
    """A tensor of n elements inside a buffer whose guard bands hold `fill`."""
    import torch
    from depthwise_pointwise_convolution_amd.module import TORCH_DTYPES
    buf = torch.full((n + 2 * guard,), fill, dtype=TORCH_DTYPES[dtype], device="cuda")
    return buf, buf[guard:guard + n], guard


def _fills(dtype):
    # NaN marks unwritten floats; int8 gets two different codes in two runs
    return [float("nan")] if dtype != "i8" else [85, -86]


def _check_guarded(buf, guard, n, fill, dtype):
    import torch
    b = buf.float().cpu() if dtype != "i8" else buf.cpu()
    if dtype != "i8":
        assert torch.isnan(b[:guard]).all() and torch.isnan(b[guard + n:]).all(), "guard band written"
        assert not torch.isnan(b[guard:guard + n]).any(), "output element left unwritten"
    else:
        assert (b[:guard] == fill).all() and (b[guard + n:] == fill).all(), "guard band written"
    return b[guard:guard + n].clone()


@pytest.mark.parametrize("name", GUARD_NAMES)
def test_guard_bands_every_kernel_family_and_path(name):
    """Every variant of each workload's module (the generalised, vector-depthwise, fp32, int8,
    chunked and back-to-back kernels included), and the layer-by-layer path with its
    intermediate, write every element of their outputs and nothing around them."""
    import torch
    from depthwise_pointwise_convolution_amd.module import TORCH_DTYPES, from_workload
    wl = reduced(name)
    inp = fcm_inputs.make_inputs(wl)
    x = torch.from_numpy(inp["x"]).to(TORCH_DTYPES[wl.dtype]).cuda()
    for v in all_variants_for(wl) + ["unfused"]:
        _log(f"case {name} guard bands {v}")
        mod = from_workload(wl, inp, variant=None if v == "unfused" else v)
        n = int(np.prod(mod.out_shape))
        nt = int(np.prod(mod.t_shape))
        outs = []
        for fill in _fills(wl.dtype):
            buf, y, g = _guarded(n, wl.dtype, fill)
            if v == "unfused":
                tbuf, t, gt = _guarded(nt, wl.dtype, fill)
                mod.unfused(x, t.view(mod.t_shape), y.view(mod.out_shape))
            else:
                mod.fused(x, y.view(mod.out_shape))
            torch.cuda.synchronize()
            outs.append(_check_guarded(buf, g, n, fill, wl.dtype))
            if v == "unfused":
                _check_guarded(tbuf, gt, nt, fill, wl.dtype)
        if len(outs) == 2:
            assert torch.equal(outs[0], outs[1]), "output depends on the buffer's old contents"


def test_pwdw_output_guard_bands_and_every_output_written():
    import torch
    from depthwise_pointwise_convolution_amd.module import from_workload
    wl = reduced("pwdw_f16_32x56x56_c24_k144")
    inp = fcm_inputs.make_inputs(wl)
    x = torch.from_numpy(inp["x"]).half().cuda()
    for v in all_variants_for(wl):
        _log(f"case pwdw guard bands variant {v}")
        mod = from_workload(wl, inp, variant=v)
        n = int(np.prod(mod.out_shape))
        guard = 4096
        buf = torch.full((n + 2 * guard,), float("nan"), dtype=torch.float16, device="cuda")
        y = buf[guard:guard + n].view(mod.out_shape)
        mod.fused(x, y)
        torch.cuda.synchronize()
        b = buf.cpu()
        assert torch.isnan(b[:guard]).all() and torch.isnan(b[guard + n:]).all()
        assert not torch.isnan(b[guard:guard + n]).any()


def test_output_guard_bands_and_every_output_written():
    import torch
    from depthwise_pointwise_convolution_amd.module import from_workload
    wl = reduced("mbv1_f16_8x112x112_c64_k128")
    inp = fcm_inputs.make_inputs(wl)
    mod = from_workload(wl, inp)
    x = torch.from_numpy(inp["x"]).half().cuda()
    n = int(np.prod(mod.out_shape))
    guard = 4096
    buf = torch.full((n + 2 * guard,), float("nan"), dtype=torch.float16, device="cuda")
    y = buf[guard:guard + n].view(mod.out_shape)
    mod.fused(x, y)
    torch.cuda.synchronize()
    b = buf.cpu()
    assert torch.isnan(b[:guard]).all() and torch.isnan(b[guard + n:]).all()
    assert not torch.isnan(b[guard:guard + n]).any()


def test_repeated_runs_are_bitwise_identical():
    import torch
    from depthwise_pointwise_convolution_amd.module import from_workload
    wl = fcm_inputs.WORKLOADS["mbv1_f16_8x112x112_c64_k128"]
    inp = fcm_inputs.make_inputs(wl)
    mod = from_workload(wl, inp)
    x = torch.from_numpy(inp["x"]).half().cuda()
    first = mod.fused(x).clone()
    for _ in range(20):
        assert torch.equal(mod.fused(x), first)


def test_device_argument_errors_enqueue_nothing():
    import torch
    import depthwise_pointwise_convolution_amd as F
    from depthwise_pointwise_convolution_amd.module import from_workload
    wl = reduced("mbv1_f16_8x112x112_c64_k128")
    inp = fcm_inputs.make_inputs(wl)
    mod = from_workload(wl, inp)
    x = torch.from_numpy(inp["x"]).half().cuda()
    y = mod.new_output("cuda")
    with pytest.raises(F.FcmError) as ei:
        F.fcm_dwpw_fwd(mod.plan, x.data_ptr() + 2, mod.w1p, None, None, mod.w2p, None, None, y)
    assert ei.value.status == F.FCM_ERR_INVALID_ARG
    with pytest.raises(F.FcmError) as ei:
        F.fcm_b2b_conv_fwd(mod.plan, x, mod.w1p, None, None, mod.w2p, None, None, y)
    assert ei.value.status == F.FCM_ERR_INVALID_ARG
    torch.cuda.synchronize()


@pytest.mark.parametrize("H,W,stride,pad", [(1, 1, 1, 1), (2, 3, 2, 1), (3, 3, 1, 0),
                                             (5, 2, 2, 0), (1, 40, 1, 1)])
def test_degenerate_extents(H, W, stride, pad):
    for kind, dtype in (("dwpw", "f16"), ("dwpw", "f32"), ("pwdw", "f16"), ("pwdwpw", "f16")):
        wl = fcm_inputs.Workload("deg", kind, dtype, N=1, H=H, W=W, C=8, K=8, K1=8,
                                 stride=stride, pad=pad, bias1=kind == "pwdw", bias2=True,
                                 act1="relu" if kind == "pwdw" else "none", seed=H * 7 + W)
        if H + 2 * pad < 3 or W + 2 * pad < 3:
            continue
        inp = fcm_inputs.make_inputs(wl)
        got, _ = run_gpu(wl, inp)
        assert rel_err(got, oracle_full(wl, inp)) <= TOL[dtype]
