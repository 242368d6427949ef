"""GPU parity of the DW->PW module with a generalised depthwise layer (R x S filters,
dilation, depth multiplier; PyTorch forum "Using optimised depthwise convolutions")
against the CPU oracle, through the C ABI: bit-exact integer probes on every compiled
variant and on the layer-by-layer pair, ragged shapes, several chunks and K tiles,
stride 2, padding other than "same", and random small shapes within the tolerance of
the storage type.  (The three generalised benchmark workloads also run in
test_gpu_parity.py: reduced, full size sampled, full size integer-exact.)"""
import zlib

import numpy as np
import pytest

import fcm_inputs
from gpu_util import (TOL, all_variants_for, elementwise_excess, gpu_available, int_inputs,
                      oracle_full, rel_err,
                      run_gpu)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


def _log(msg):
    print(msg, flush=True)


# (dtype, N, H, W, C, K, filter, dilation, multiplier, stride, pad, act1, act2, epilogues)
CASES = [
    ("f16", 2, 13, 21, 40, 48, 5, 1, 1, 1, 2, "relu", "none", True),
    ("f16", 1, 9, 35, 64, 136, 5, 1, 1, 2, 2, "relu6", "relu6", True),
    ("f16", 2, 11, 7, 24, 40, 5, 1, 1, 1, 0, "none", "relu", False),
    ("f16", 1, 15, 17, 72, 64, 7, 1, 1, 1, 3, "relu", "relu", True),
    ("f16", 2, 9, 18, 120, 40, 5, 1, 1, 1, 1, "relu", "none", True),
    ("f16", 1, 10, 29, 128, 72, 5, 1, 1, 1, 2, "relu6", "relu6", True),
    ("f16", 2, 12, 19, 96, 264, 3, 2, 1, 1, 2, "relu6", "none", True),
    ("f16", 1, 8, 9, 32, 40, 3, 2, 1, 1, 1, "none", "none", True),
    ("f16", 1, 11, 21, 128, 72, 3, 2, 1, 1, 2, "relu6", "relu", True),
    ("f16", 2, 10, 23, 32, 128, 3, 1, 2, 1, 1, "relu6", "relu6", True),
    ("f16", 1, 17, 13, 48, 72, 3, 1, 2, 2, 1, "relu", "none", True),
    ("f16", 1, 9, 37, 24, 72, 3, 1, 2, 1, 0, "relu", "relu", True),
    ("f16", 2, 6, 40, 8, 24, 3, 1, 2, 1, 1, "relu", "relu6", True),
    ("bf16", 2, 13, 14, 40, 56, 5, 1, 1, 1, 2, "relu", "relu6", True),
    ("bf16", 1, 9, 11, 64, 64, 3, 2, 1, 1, 2, "none", "relu", True),
    ("bf16", 2, 7, 20, 16, 136, 3, 1, 2, 1, 1, "relu6", "none", False),
]


def _wl(c, name="gen"):
    dt, N, H, W, C, K, f, d, m, s, p, a1, a2, epi = c
    return fcm_inputs.Workload(name, "dwpw", dt, N=N, H=H, W=W, C=C, K=K, K1=C * m, R=f, S=f,
                               dil=d, mult=m, stride=s, pad=p, act1=a1, act2=a2, scale1=epi,
                               bias1=epi, scale2=epi, bias2=epi)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c[:11])))
def test_gen_integer_probes_bit_exact_every_variant(case):
    wl = _wl(case)
    seed = zlib.crc32(repr(case).encode()) % 1000
    inp = int_inputs(wl, seed=seed)
    ref = oracle_full(wl, inp)
    variants = all_variants_for(wl)
    assert variants, "no variant runs this problem"
    for v in variants:
        _log(f"case gen int {case} variant {v}")
        got, _ = run_gpu(wl, inp, variant=v)
        bad = np.argwhere(got != ref)
        assert bad.size == 0, (f"variant {v} (input seed {seed}): {len(bad)} mismatches, "
                               f"first {bad[:3].tolist()}")
    _log(f"case gen int {case} layer by layer")
    got, _ = run_gpu(wl, inp, path="unfused")
    assert np.array_equal(got, ref), f"layer-by-layer path (input seed {seed})"


def _random_gen_cases(n, seed):
    rng = np.random.default_rng(seed)
    forms = [(5, 1, 1, 1), (5, 1, 1, 2), (7, 1, 1, 1), (3, 2, 1, 1), (3, 1, 2, 1), (3, 1, 2, 2)]
    out = []
    for i in range(n):
        f, d, m, s = forms[int(rng.integers(len(forms)))]
        ext = (f - 1) * d + 1
        dtype = "f16" if (f, d, m, s) not in ((5, 1, 1, 1), (3, 2, 1, 1), (3, 1, 2, 1)) \
            else str(rng.choice(["f16", "bf16"]))
        H, W = int(rng.integers(1, 26)), int(rng.integers(1, 26))
        pad = int(rng.integers(0, ext))
        if H + 2 * pad < ext or W + 2 * pad < ext:
            pad = ext - 1
        out.append(fcm_inputs.Workload(
            f"rgen{i}", "dwpw", dtype, N=int(rng.integers(1, 3)), H=H, W=W,
            C=(C := int(rng.choice([8, 16, 40, 64, 72]))), K=int(rng.choice([8, 24, 64, 136])),
            K1=C * m, R=f, S=f, dil=d, mult=m, stride=s, pad=pad,
            act1=str(rng.choice(["none", "relu", "relu6"])),
            act2=str(rng.choice(["none", "relu", "relu6"])), scale1=bool(rng.random() < .5),
            bias1=bool(rng.random() < .5), scale2=bool(rng.random() < .5),
            bias2=bool(rng.random() < .5), seed=int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("wl", _random_gen_cases(16, 5), ids=lambda w: w.name)
def test_gen_random_small_shapes(wl):
    inp = fcm_inputs.make_inputs(wl)
    ref = oracle_full(wl, inp)
    for path in ("fused", "unfused"):
        _log(f"case {wl} {path}")
        got, _ = run_gpu(wl, inp, path=path)
        assert got.shape == ref.shape
        err = rel_err(got, ref)
        assert np.all(np.isfinite(got))
        assert err <= TOL[wl.dtype], (path, err)
        ex = elementwise_excess(got, ref, wl.dtype)
        assert ex <= 1.0, (path, "elementwise", ex)
