"""CPU oracle for the fused depthwise->pointwise module, the pointwise->depthwise
module and the 3x3->1x1 pair.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code with
the HIP library and never imports it.

The arithmetic lives in ``fcm_oracle.c`` (plain C, double precision, direct loops);
this module only builds and loads it and marshals numpy arrays.  The cost-model and
byte-accounting definitions are in :mod:`oracle.accounting`.

Array conventions (PyTorch layouts, float64 holding values already representable in
the storage type):

* ``x``      [N, H, W, C]
* ``w_dw``   [C, R, S]            depthwise filters
* ``w_pw``   [K, C]               pointwise filters
* ``w1``     [K1, C, R, S]        first (standard) conv of the back-to-back pair
* ``w2``     [K, K1]              second (1x1) conv of the pair
* PW->DW module: ``w_pw`` [K1, C] then ``w_dw`` [K1, R, S]; output channels K1
* ``scale*``/``bias*`` per channel, or ``None`` (identity)

``dtype="i8"`` is the INT8 module: integer operands, exact sums, and at each storage
point the binary32 requantization fmaf(scale, acc, bias) -> activation clamp -> nearest
integer (ties to even) -> saturation to [-128, 127] (see fcm_oracle.c).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fcm_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

DTYPES = {"f32": 0, "f16": 1, "bf16": 2, "i8": 3}
ACTS = {"none": 0, "relu": 1, "relu6": 2}

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile fcm_oracle.c with gcc (OpenMP, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
               "-Wall", "-o", tmp, SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(LIB)
            dp = ctypes.POINTER(ctypes.c_double)
            i32, i64 = ctypes.c_int32, ctypes.c_int64
            lib.fcm_oracle_threads.restype = ctypes.c_int
            lib.fcm_oracle_threads.argtypes = []
            lib.fcm_oracle_set_threads.restype = None
            lib.fcm_oracle_set_threads.argtypes = [ctypes.c_int]
            lib.fcm_oracle_round.restype = ctypes.c_double
            lib.fcm_oracle_round.argtypes = [ctypes.c_double, ctypes.c_int]
            lib.fcm_oracle_round_array.argtypes = [dp, i64, ctypes.c_int]
            lib.fcm_oracle_f16_bits.restype = ctypes.c_uint16
            lib.fcm_oracle_f16_bits.argtypes = [ctypes.c_double]
            lib.fcm_oracle_bf16_bits.restype = ctypes.c_uint16
            lib.fcm_oracle_bf16_bits.argtypes = [ctypes.c_double]
            lib.fcm_oracle_dw.argtypes = [dp, i32, i32, i32, i32, dp, i32, i32, i32, i32,
                                          i32, i32, dp]
            lib.fcm_oracle_pw.argtypes = [dp, i64, i32, dp, i32, dp]
            lib.fcm_oracle_conv.argtypes = [dp, i32, i32, i32, i32, dp, i32, i32, i32, i32,
                                            i32, i32, i32, dp]
            lib.fcm_oracle_epilogue.argtypes = [dp, i64, i32, dp, dp, ctypes.c_int]
            ci = ctypes.c_int
            # x, N, H, W, C, w1, [K1,] R, S, sh, sw, ph, pw, scale1, bias1, act1,
            # w2, K, scale2, bias2, act2, dtype
            tail = [i32] * 6 + [dp, dp, ci, dp, i32, dp, dp, ci, ci]
            mod_dw = [dp, i32, i32, i32, i32, dp] + tail
            mod_b2b = [dp, i32, i32, i32, i32, dp, i32] + tail
            lib.fcm_oracle_dwpw.argtypes = mod_dw + [dp, dp]
            lib.fcm_oracle_dwpw.restype = ctypes.c_int
            lib.fcm_oracle_b2b.argtypes = mod_b2b + [dp, dp]
            lib.fcm_oracle_b2b.restype = ctypes.c_int
            ip = ctypes.POINTER(ctypes.c_int32)
            lib.fcm_oracle_dwpw_at.argtypes = mod_dw + [ip, i64, dp]
            lib.fcm_oracle_dwpw_at.restype = ctypes.c_int
            lib.fcm_oracle_b2b_at.argtypes = mod_b2b + [ip, i64, dp]
            lib.fcm_oracle_b2b_at.restype = ctypes.c_int
            # x, N, H, W, C, w_pw, K1, scale1, bias1, act1, w_dw, R, S, sh, sw, ph, pw,
            # scale2, bias2, act2, dtype
            mod_pd = [dp, i32, i32, i32, i32, dp, i32, dp, dp, ci, dp] + [i32] * 6 + \
                [dp, dp, ci, ci]
            lib.fcm_oracle_pwdw.argtypes = mod_pd + [dp, dp]
            lib.fcm_oracle_pwdw.restype = ctypes.c_int
            lib.fcm_oracle_pwdw_at.argtypes = mod_pd + [ip, i64, dp]
            lib.fcm_oracle_pwdw_at.restype = ctypes.c_int
            # the PW -> DW arguments up to act2, then w3, K, scale3, bias3, act3, residual,
            # dtype, and (t1, t2, y) or (pix, P, y_rows)
            mod_pdp = mod_pd[:-1] + [dp, i32, dp, dp, ci, ci, ci]
            lib.fcm_oracle_pwdwpw.argtypes = mod_pdp + [dp, dp, dp]
            lib.fcm_oracle_pwdwpw.restype = ctypes.c_int
            lib.fcm_oracle_pwdwpw_at.argtypes = mod_pdp + [ip, i64, dp]
            lib.fcm_oracle_pwdwpw_at.restype = ctypes.c_int
            # x, M, C, w1, K1, scale1, bias1, act1, w2, K, scale2, bias2, act2, dtype, t, y
            lib.fcm_oracle_pwpw.argtypes = [dp, i64, i32, dp, i32, dp, dp, ci, dp, i32, dp, dp,
                                            ci, ci, dp, dp]
            lib.fcm_oracle_pwpw.restype = ctypes.c_int
            # x, N, H, W, C, w, R, S, sh, sw, ph, pw, dh, dw, M, t
            lib.fcm_oracle_dw_gen.argtypes = [dp, i32, i32, i32, i32, dp] + [i32] * 9 + [dp]
            # x, N, H, W, C, w_dw, R, S, sh, sw, ph, pw, dh, dw, M, scale1, bias1, act1,
            # w_pw, K, scale2, bias2, act2, dtype, t, y
            lib.fcm_oracle_dwpw_gen.argtypes = [dp, i32, i32, i32, i32, dp] + [i32] * 9 + \
                [dp, dp, ci, dp, i32, dp, dp, ci, ci, dp, dp]
            lib.fcm_oracle_dwpw_gen.restype = ctypes.c_int
            _lib = lib
    return _lib


def threads() -> int:
    """OpenMP threads the oracle's loops run on."""
    return int(_load().fcm_oracle_threads())


def set_threads(n: int) -> None:
    """Run the oracle's later loops on n OpenMP threads."""
    _load().fcm_oracle_set_threads(int(n))


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def out_size(n: int, pad: int, filt: int, stride: int) -> int:
    """floor((n + 2*pad - filt) / stride) + 1."""
    return (n + 2 * pad - filt) // stride + 1


# ---------------------------------------------------------------------------------
# rounding
# ---------------------------------------------------------------------------------
def round_to(a, dtype: str) -> np.ndarray:
    """Round every element to the nearest value of the storage type (RNE)."""
    out = _f64(a).copy()
    _load().fcm_oracle_round_array(_p(out), out.size, DTYPES[dtype])
    return out


def f16_bits(v: float) -> int:
    return int(_load().fcm_oracle_f16_bits(float(v)))


def bf16_bits(v: float) -> int:
    return int(_load().fcm_oracle_bf16_bits(float(v)))


# ---------------------------------------------------------------------------------
# single layers (no epilogue, no rounding)
# ---------------------------------------------------------------------------------
def dw(x, w_dw, stride=(1, 1), pad=(1, 1)) -> np.ndarray:
    x, w = _f64(x), _f64(w_dw)
    N, H, W, C = x.shape
    Cw, R, S = w.shape
    assert Cw == C
    Ho, Wo = out_size(H, pad[0], R, stride[0]), out_size(W, pad[1], S, stride[1])
    t = np.empty((N, Ho, Wo, C), np.float64)
    _load().fcm_oracle_dw(_p(x), N, H, W, C, _p(w), R, S, stride[0], stride[1], pad[0],
                          pad[1], _p(t))
    return t


def pw(t, w_pw) -> np.ndarray:
    t, w = _f64(t), _f64(w_pw)
    C = t.shape[-1]
    K, Cw = w.shape
    assert Cw == C
    y = np.empty(t.shape[:-1] + (K,), np.float64)
    _load().fcm_oracle_pw(_p(t), t.size // C, C, _p(w), K, _p(y))
    return y


def conv(x, w, stride=(1, 1), pad=(1, 1)) -> np.ndarray:
    x, w = _f64(x), _f64(w)
    N, H, W, C = x.shape
    K, Cw, R, S = w.shape
    assert Cw == C
    Ho, Wo = out_size(H, pad[0], R, stride[0]), out_size(W, pad[1], S, stride[1])
    y = np.empty((N, Ho, Wo, K), np.float64)
    _load().fcm_oracle_conv(_p(x), N, H, W, C, _p(w), K, R, S, stride[0], stride[1],
                            pad[0], pad[1], _p(y))
    return y


def epilogue(a, scale=None, bias=None, act="none") -> np.ndarray:
    out = _f64(a).copy()
    C = out.shape[-1]
    s = None if scale is None else _f64(scale)
    b = None if bias is None else _f64(bias)
    _load().fcm_oracle_epilogue(_p(out), out.size // C, C, _p(s), _p(b), ACTS[act])
    return out


# ---------------------------------------------------------------------------------
# the two modules
# ---------------------------------------------------------------------------------
def _module(fn, x, w1, w2, stride, pad, scale1, bias1, act1, scale2, bias2, act2, dtype,
            return_t, depthwise):
    x, w1, w2 = _f64(x), _f64(w1), _f64(w2)
    N, H, W, C = x.shape
    if depthwise:
        C1, R, S = w1.shape
        K1 = C
        assert C1 == C
    else:
        K1, C1, R, S = w1.shape
        assert C1 == C
    K, K1w = w2.shape
    assert K1w == K1
    Ho, Wo = out_size(H, pad[0], R, stride[0]), out_size(W, pad[1], S, stride[1])
    t = np.empty((N, Ho, Wo, K1), np.float64) if return_t else None
    y = np.empty((N, Ho, Wo, K), np.float64)
    s1 = None if scale1 is None else _f64(scale1)
    b1 = None if bias1 is None else _f64(bias1)
    s2 = None if scale2 is None else _f64(scale2)
    b2 = None if bias2 is None else _f64(bias2)
    args = [_p(x), N, H, W, C, _p(w1)]
    if not depthwise:
        args.append(K1)
    args += [R, S, stride[0], stride[1], pad[0], pad[1], _p(s1), _p(b1), ACTS[act1],
             _p(w2), K, _p(s2), _p(b2), ACTS[act2], DTYPES[dtype], _p(t), _p(y)]
    rc = fn(*args)
    if rc != 0:
        raise MemoryError("oracle could not allocate the intermediate")
    return (y, t) if return_t else y


def dwpw(x, w_dw, w_pw, stride=(1, 1), pad=(1, 1), scale1=None, bias1=None, act1="none",
         scale2=None, bias2=None, act2="none", dtype="f32", return_t=False):
    """Layer-by-layer DW conv -> epilogue -> round -> PW conv -> epilogue -> round."""
    return _module(_load().fcm_oracle_dwpw, x, w_dw, w_pw, stride, pad, scale1, bias1,
                   act1, scale2, bias2, act2, dtype, return_t, True)


def b2b(x, w1, w2, stride=(1, 1), pad=(1, 1), scale1=None, bias1=None, act1="none",
        scale2=None, bias2=None, act2="none", dtype="f32", return_t=False):
    """Layer-by-layer standard conv -> epilogue -> round -> 1x1 conv -> epilogue -> round."""
    return _module(_load().fcm_oracle_b2b, x, w1, w2, stride, pad, scale1, bias1, act1,
                   scale2, bias2, act2, dtype, return_t, False)


def _module_at(fn, x, w1, w2, pix, stride, pad, scale1, bias1, act1, scale2, bias2, act2,
               dtype, depthwise):
    x, w1, w2 = _f64(x), _f64(w1), _f64(w2)
    N, H, W, C = x.shape
    if depthwise:
        _, R, S = w1.shape
        K1 = C
    else:
        K1, _, R, S = w1.shape
    K = w2.shape[0]
    pix = np.ascontiguousarray(pix, dtype=np.int32).reshape(-1, 3)
    P = pix.shape[0]
    y = np.empty((P, K), np.float64)
    s1 = None if scale1 is None else _f64(scale1)
    b1 = None if bias1 is None else _f64(bias1)
    s2 = None if scale2 is None else _f64(scale2)
    b2 = None if bias2 is None else _f64(bias2)
    args = [_p(x), N, H, W, C, _p(w1)]
    if not depthwise:
        args.append(K1)
    args += [R, S, stride[0], stride[1], pad[0], pad[1], _p(s1), _p(b1), ACTS[act1],
             _p(w2), K, _p(s2), _p(b2), ACTS[act2], DTYPES[dtype],
             pix.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), P, _p(y)]
    fn(*args)
    return y


def dwpw_at(x, w_dw, w_pw, pix, stride=(1, 1), pad=(1, 1), scale1=None, bias1=None,
            act1="none", scale2=None, bias2=None, act2="none", dtype="f32"):
    """Rows y[n, oh, ow, :] of :func:`dwpw` at the listed output pixels only."""
    return _module_at(_load().fcm_oracle_dwpw_at, x, w_dw, w_pw, pix, stride, pad, scale1,
                      bias1, act1, scale2, bias2, act2, dtype, True)


def b2b_at(x, w1, w2, pix, stride=(1, 1), pad=(1, 1), scale1=None, bias1=None,
           act1="none", scale2=None, bias2=None, act2="none", dtype="f32"):
    """Rows y[n, oh, ow, :] of :func:`b2b` at the listed output pixels only."""
    return _module_at(_load().fcm_oracle_b2b_at, x, w1, w2, pix, stride, pad, scale1,
                      bias1, act1, scale2, bias2, act2, dtype, False)


# ---------------------------------------------------------------------------------
# the pointwise -> depthwise module
# ---------------------------------------------------------------------------------
def _pwdw_args(x, w_pw, w_dw, stride, pad, scale1, bias1, act1, scale2, bias2, act2, dtype):
    x, wp, wd = _f64(x), _f64(w_pw), _f64(w_dw)
    N, H, W, C = x.shape
    K1, Cw = wp.shape
    K1d, R, S = wd.shape
    assert Cw == C and K1d == K1
    s1 = None if scale1 is None else _f64(scale1)
    b1 = None if bias1 is None else _f64(bias1)
    s2 = None if scale2 is None else _f64(scale2)
    b2 = None if bias2 is None else _f64(bias2)
    keep = (x, wp, wd, s1, b1, s2, b2)
    args = [_p(x), N, H, W, C, _p(wp), K1, _p(s1), _p(b1), ACTS[act1], _p(wd), R, S,
            stride[0], stride[1], pad[0], pad[1], _p(s2), _p(b2), ACTS[act2], DTYPES[dtype]]
    return args, keep, (N, H, W, C, K1, R, S)


def pwdw(x, w_pw, w_dw, stride=(1, 1), pad=(1, 1), scale1=None, bias1=None, act1="none",
         scale2=None, bias2=None, act2="none", dtype="f32", return_t=False):
    """Layer-by-layer PW conv -> epilogue -> round -> DW conv -> epilogue -> round.
    ``w_pw`` [K1, C], ``w_dw`` [K1, R, S]; returns y [N, Ho, Wo, K1] (and the rounded
    intermediate [N, H, W, K1] with ``return_t``)."""
    args, keep, (N, H, W, C, K1, R, S) = _pwdw_args(x, w_pw, w_dw, stride, pad, scale1, bias1,
                                                     act1, scale2, bias2, act2, dtype)
    Ho, Wo = out_size(H, pad[0], R, stride[0]), out_size(W, pad[1], S, stride[1])
    t = np.empty((N, H, W, K1), np.float64) if return_t else None
    y = np.empty((N, Ho, Wo, K1), np.float64)
    rc = _load().fcm_oracle_pwdw(*args, _p(t), _p(y))
    del keep
    if rc != 0:
        raise MemoryError("oracle could not allocate the intermediate")
    return (y, t) if return_t else y


def pwdw_at(x, w_pw, w_dw, pix, stride=(1, 1), pad=(1, 1), scale1=None, bias1=None,
            act1="none", scale2=None, bias2=None, act2="none", dtype="f32"):
    """Rows y[n, oh, ow, :] of :func:`pwdw` at the listed output pixels only."""
    args, keep, (N, H, W, C, K1, R, S) = _pwdw_args(x, w_pw, w_dw, stride, pad, scale1, bias1,
                                                     act1, scale2, bias2, act2, dtype)
    pix = np.ascontiguousarray(pix, dtype=np.int32).reshape(-1, 3)
    y = np.empty((pix.shape[0], K1), np.float64)
    _load().fcm_oracle_pwdw_at(*args, pix.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                               pix.shape[0], _p(y))
    del keep
    return y


# ---------------------------------------------------------------------------------
# the pointwise -> depthwise -> pointwise module (inverted-residual block)
# ---------------------------------------------------------------------------------
def _pwdwpw_args(x, w1, w2, w3, stride, pad, scale1, bias1, act1, scale2, bias2, act2,
                 scale3, bias3, act3, residual, dtype):
    args, keep, dims = _pwdw_args(x, w1, w2, stride, pad, scale1, bias1, act1, scale2, bias2,
                                  act2, dtype)
    w3 = _f64(w3)
    K, K1b = w3.shape
    assert K1b == dims[4]
    s3 = None if scale3 is None else _f64(scale3)
    b3 = None if bias3 is None else _f64(bias3)
    args = args[:-1] + [_p(w3), K, _p(s3), _p(b3), ACTS[act3], int(bool(residual)),
                        DTYPES[dtype]]
    return args, keep + (w3, s3, b3), dims + (K,)


def pwdwpw(x, w1, w2, w3, stride=(1, 1), pad=(1, 1), scale1=None, bias1=None, act1="none",
           scale2=None, bias2=None, act2="none", scale3=None, bias3=None, act3="none",
           residual=False, dtype="f32", return_t=False):
    """Layer by layer: PW (w1 [K1, C]) -> epilogue 1 -> round -> DW (w2 [K1, R, S]) ->
    epilogue 2 -> round -> PW (w3 [K, K1]) -> epilogue 3 (+ the input pixel when
    ``residual``) -> round.  Returns y [N, Ho, Wo, K] (and the two rounded
    intermediates with ``return_t``)."""
    args, keep, (N, H, W, C, K1, R, S, K) = _pwdwpw_args(
        x, w1, w2, w3, stride, pad, scale1, bias1, act1, scale2, bias2, act2, scale3, bias3,
        act3, residual, dtype)
    Ho, Wo = out_size(H, pad[0], R, stride[0]), out_size(W, pad[1], S, stride[1])
    t1 = np.empty((N, H, W, K1), np.float64) if return_t else None
    t2 = np.empty((N, Ho, Wo, K1), np.float64) if return_t else None
    y = np.empty((N, Ho, Wo, K), np.float64)
    rc = _load().fcm_oracle_pwdwpw(*args, _p(t1), _p(t2), _p(y))
    del keep
    if rc == -2:
        raise ValueError("the shortcut needs an unchanged extent and K == C; int8 storage "
                         "is not defined for this module")
    if rc != 0:
        raise MemoryError("oracle could not allocate the intermediate")
    return (y, t1, t2) if return_t else y


def pwdwpw_at(x, w1, w2, w3, pix, stride=(1, 1), pad=(1, 1), scale1=None, bias1=None,
              act1="none", scale2=None, bias2=None, act2="none", scale3=None, bias3=None,
              act3="none", residual=False, dtype="f32"):
    """Rows y[n, oh, ow, :] of :func:`pwdwpw` at the listed output pixels only."""
    args, keep, (N, H, W, C, K1, R, S, K) = _pwdwpw_args(
        x, w1, w2, w3, stride, pad, scale1, bias1, act1, scale2, bias2, act2, scale3, bias3,
        act3, residual, dtype)
    pix = np.ascontiguousarray(pix, dtype=np.int32).reshape(-1, 3)
    y = np.empty((pix.shape[0], K), np.float64)
    rc = _load().fcm_oracle_pwdwpw_at(*args, pix.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                      pix.shape[0], _p(y))
    del keep
    if rc == -2:
        raise ValueError("the shortcut needs an unchanged extent and K == C; int8 storage "
                         "is not defined for this module")
    if rc != 0:
        raise MemoryError("oracle could not allocate the intermediate")
    return y


# ---------------------------------------------------------------------------------
# the pointwise -> pointwise module
# ---------------------------------------------------------------------------------
def pwpw(x, w1, w2, scale1=None, bias1=None, act1="none", scale2=None, bias2=None,
         act2="none", dtype="f32", return_t=False, **_):
    """Layer-by-layer PW conv -> epilogue -> round -> PW conv -> epilogue -> round over
    every pixel of x [..., C]; w1 [K1, C], w2 [K, K1].  (Stride and padding keywords are
    accepted and ignored: a 1x1 layer has neither.)"""
    x, w1, w2 = _f64(x), _f64(w1), _f64(w2)
    C = x.shape[-1]
    K1, C1 = w1.shape
    K, K1b = w2.shape
    assert C1 == C and K1b == K1
    M = x.size // C
    t = np.empty(x.shape[:-1] + (K1,), np.float64)
    y = np.empty(x.shape[:-1] + (K,), np.float64)
    arrs = [None if a is None else _f64(a) for a in (scale1, bias1, scale2, bias2)]
    rc = _load().fcm_oracle_pwpw(_p(x), M, C, _p(w1), K1, _p(arrs[0]), _p(arrs[1]), ACTS[act1],
                                 _p(w2), K, _p(arrs[2]), _p(arrs[3]), ACTS[act2], DTYPES[dtype],
                                 _p(t), _p(y))
    if rc != 0:
        raise MemoryError("oracle could not allocate the intermediate")
    return (y, t) if return_t else y


def pwpw_at(x, w1, w2, pix, **kw):
    """Rows y[n, h, w, :] of :func:`pwpw` at the listed pixels (each pixel is
    independent, so this is the module on those pixels alone)."""
    x = _f64(x)
    pix = np.asarray(pix).reshape(-1, 3)
    return pwpw(x[pix[:, 0], pix[:, 1], pix[:, 2]], w1, w2, **kw)


# ---------------------------------------------------------------------------------
# generalised depthwise layer: R x S filters, dilation, depth multiplier
# (PyTorch forum "Using optimised depthwise convolutions": a grouped convolution with
# one group per input channel and k outputs per group, any filter size, and the
# dilation the thread's separable module gives it)
# ---------------------------------------------------------------------------------
def dw_gen(x, w_dw, stride=(1, 1), pad=(1, 1), dilation=(1, 1)) -> np.ndarray:
    """Depthwise layer with w_dw [C*M][R][S]: output channel j reads input channel j // M."""
    x, w = _f64(x), _f64(w_dw)
    N, H, W, C = x.shape
    CM, R, S = w.shape
    assert CM % C == 0
    M = CM // C
    Ho = out_size(H, pad[0], (R - 1) * dilation[0] + 1, stride[0])
    Wo = out_size(W, pad[1], (S - 1) * dilation[1] + 1, stride[1])
    t = np.empty((N, Ho, Wo, CM), np.float64)
    _load().fcm_oracle_dw_gen(_p(x), N, H, W, C, _p(w), R, S, stride[0], stride[1], pad[0],
                              pad[1], dilation[0], dilation[1], M, _p(t))
    return t


def dwpw_gen(x, w_dw, w_pw, stride=(1, 1), pad=(1, 1), dilation=(1, 1), scale1=None,
             bias1=None, act1="none", scale2=None, bias2=None, act2="none", dtype="f32",
             return_t=False):
    """Layer by layer: generalised DW (w_dw [C*M][R][S]) -> epilogue -> round ->
    PW (w_pw [K][C*M]) -> epilogue -> round."""
    x, w1, w2 = _f64(x), _f64(w_dw), _f64(w_pw)
    N, H, W, C = x.shape
    CM, R, S = w1.shape
    assert CM % C == 0
    M = CM // C
    K, CMw = w2.shape
    assert CMw == CM
    Ho = out_size(H, pad[0], (R - 1) * dilation[0] + 1, stride[0])
    Wo = out_size(W, pad[1], (S - 1) * dilation[1] + 1, stride[1])
    t = np.empty((N, Ho, Wo, CM), np.float64) if return_t else None
    y = np.empty((N, Ho, Wo, K), np.float64)
    s1 = None if scale1 is None else _f64(scale1)
    b1 = None if bias1 is None else _f64(bias1)
    s2 = None if scale2 is None else _f64(scale2)
    b2 = None if bias2 is None else _f64(bias2)
    rc = _load().fcm_oracle_dwpw_gen(
        _p(x), N, H, W, C, _p(w1), R, S, stride[0], stride[1], pad[0], pad[1], dilation[0],
        dilation[1], M, _p(s1), _p(b1), ACTS[act1], _p(w2), K, _p(s2), _p(b2), ACTS[act2],
        DTYPES[dtype], _p(t), _p(y))
    if rc != 0:
        raise MemoryError("oracle could not allocate the intermediate")
    return (y, t) if return_t else y
