"""Python binding of libfcm.so, the MI355X (gfx950) fused convolution module library.

Argument marshalling only: every step of the computation runs in the library's HIP
kernels.  The functions carry the C ABI's names (see ``include/fcm.h``):

    plan = fcm_plan(problem(...))
    fcm_pack_weights(plan, w1_src, w1_dst, w2_src, w2_dst)
    fcm_dwpw_fwd(plan, x, w_dw, scale1, bias1, w_pw, scale2, bias2, y)
    fcm_b2b_conv_fwd(plan, x, w1, scale1, bias1, w2, scale2, bias2, y)
    fcm_pwdw_fwd(plan, x, w_pw, scale1, bias1, w_dw, scale2, bias2, y)
    fcm_pwpw_fwd(plan, x, w1, scale1, bias1, w2, scale2, bias2, y)
    fcm_pwdwpw_fwd(plan, x, w1, scale1, bias1, w2, scale2, bias2, w3, scale3, bias3, y)
    fcm_dw_fwd / fcm_pw_fwd / fcm_conv_fwd / fcm_pwdwpw_lbl   (layer-by-layer baselines)
    fcm_pwdwpw_lbl_noalloc   (the three-layer baseline with the library's static scratch)

Tensor arguments are torch tensors on the GPU (or raw integer device addresses, or
None where the ABI allows NULL); PyTorch only provides device memory and the stream
(``torch.cuda.current_stream()`` unless one is passed).  A non-OK status raises
:class:`FcmError`.  If ``libfcm.so`` has not been built the first call raises: there
is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfcm.so")

FCM_OK, FCM_ERR_INVALID_ARG, FCM_ERR_UNSUPPORTED, FCM_ERR_HIP = 0, 1, 2, 3
FCM_F32, FCM_F16, FCM_BF16, FCM_I8 = 0, 1, 2, 3
FCM_ACT_NONE, FCM_ACT_RELU, FCM_ACT_RELU6 = 0, 1, 2
FCM_KIND_DWPW, FCM_KIND_B2B, FCM_KIND_PWDW, FCM_KIND_PWPW, FCM_KIND_PWDWPW = 0, 1, 2, 3, 4
FCM_PLAN_VERSION = 4

DTYPE_CODES = {"f32": FCM_F32, "f16": FCM_F16, "bf16": FCM_BF16, "i8": FCM_I8}
ACT_CODES = {"none": FCM_ACT_NONE, "relu": FCM_ACT_RELU, "relu6": FCM_ACT_RELU6}
KIND_CODES = {"dwpw": FCM_KIND_DWPW, "b2b": FCM_KIND_B2B, "pwdw": FCM_KIND_PWDW,
              "pwpw": FCM_KIND_PWPW, "pwdwpw": FCM_KIND_PWDWPW}


class FcmError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {_STATUS.get(status, status)}: {detail}")


_STATUS = {0: "FCM_OK", 1: "FCM_ERR_INVALID_ARG", 2: "FCM_ERR_UNSUPPORTED", 3: "FCM_ERR_HIP"}

_i32, _i64, _f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double


class fcm_problem(ctypes.Structure):
    _fields_ = [(n, _i32) for n in ("kind", "dtype", "N", "H", "W", "C", "K1", "K", "R", "S",
                                    "stride_h", "stride_w", "pad_h", "pad_w", "act1", "act2",
                                    "dil_h", "dil_w", "mult", "act3", "residual")]


class fcm_device_spec(ctypes.Structure):
    _fields_ = [("num_cus", _i32), ("num_xcds", _i32), ("simds_per_cu", _i32),
                ("wave_size", _i32), ("max_waves_per_simd", _i32),
                ("vgprs_per_simd_lane", _i32), ("lds_bytes_per_cu", _i32),
                ("lds_bytes_per_wg", _i32), ("l2_bytes_per_xcd", _i64),
                ("hbm_bytes_per_s", _f64), ("mfma_f16_flops", _f64),
                ("mfma_f32_flops", _f64), ("valu_f32_flops", _f64)]


class fcm_plan_t(ctypes.Structure):
    _fields_ = [("version", _i32), ("prob", fcm_problem), ("Ho", _i32), ("Wo", _i32),
                ("variant", _i32), ("tile_h", _i32), ("tile_w", _i32), ("k_tile", _i32),
                ("c_chunk", _i32), ("waves_per_wg", _i32), ("wgs_per_cu", _i32),
                ("num_tiles", _i32), ("grid", _i32), ("lds_bytes", _i32), ("fuse", _i32),
                ("w1_packed_bytes", _i64), ("w2_packed_bytes", _i64),
                ("workspace_bytes", _i64), ("alg_bytes_fused", _i64),
                ("alg_bytes_unfused", _i64), ("pred_bytes_fused", _i64),
                ("pred_bytes_unfused", _i64), ("gma_paper_fused", _f64),
                ("gma_paper_unfused", _f64), ("flops", _f64), ("pred_us_fused", _f64),
                ("tuned_us", _f64)]

    def as_dict(self) -> dict:
        d = {}
        for name, _ in self._fields_:
            v = getattr(self, name)
            if isinstance(v, fcm_problem):
                v = {n: getattr(v, n) for n, _ in fcm_problem._fields_}
            d[name] = v
        return d


FCM_LAYER_DW, FCM_LAYER_PW = 0, 1


class fcm_layer(ctypes.Structure):
    _fields_ = [(n, _i32) for n in ("type", "C", "K", "stride", "act")]


class fcm_chain_group(ctypes.Structure):
    _fields_ = [("first", _i32), ("count", _i32), ("kind", _i32), ("variant", _i32),
                ("gma", _f64)]


# every symbol include/fcm.h declares
EXPORTS = ("fcm_default_device_spec", "fcm_query_device_spec", "fcm_plan", "fcm_plan_variant",
           "fcm_plan_chain",
           "fcm_num_variants", "fcm_variant_name", "fcm_pack_weights", "fcm_dwpw_fwd",
           "fcm_tune",
           "fcm_b2b_conv_fwd", "fcm_pwdw_fwd", "fcm_pwpw_fwd", "fcm_dw_fwd", "fcm_pw_fwd",
           "fcm_conv_fwd", "fcm_pwdwpw_fwd", "fcm_pwdwpw_lbl", "fcm_pwdwpw_lbl_noalloc",
           "fcm_tune_pwdwpw",
           "fcm_status_str",
           "fcm_last_error")

_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    """Load libfcm.so (built in-tree by ``build.py``); raise if it is missing."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise FcmError(FCM_ERR_HIP, "load",
                               f"{LIB_PATH} is not built; run "
                               "`python -m depthwise_pointwise_convolution_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            vp, fp = ctypes.c_void_p, ctypes.c_void_p
            P = ctypes.POINTER
            L.fcm_default_device_spec.argtypes = [P(fcm_device_spec)]
            L.fcm_query_device_spec.argtypes = [ctypes.c_int, P(fcm_device_spec)]
            L.fcm_plan.argtypes = [P(fcm_problem), P(fcm_device_spec), P(fcm_plan_t)]
            L.fcm_plan_variant.argtypes = [P(fcm_problem), P(fcm_device_spec), _i32,
                                           P(fcm_plan_t)]
            L.fcm_plan_chain.argtypes = [P(fcm_layer), _i32, _i32, _i32, _i32, _i32,
                                         P(fcm_device_spec), P(fcm_chain_group), P(_i32),
                                         P(_f64), P(_f64)]
            L.fcm_plan_chain.restype = ctypes.c_int
            L.fcm_num_variants.restype = _i32
            L.fcm_num_variants.argtypes = []
            L.fcm_variant_name.restype = ctypes.c_char_p
            L.fcm_variant_name.argtypes = [_i32]
            L.fcm_pack_weights.argtypes = [P(fcm_plan_t), vp, vp, vp, vp, vp]
            L.fcm_dwpw_fwd.argtypes = [P(fcm_plan_t), vp, vp, fp, fp, vp, fp, fp, vp, vp]
            L.fcm_b2b_conv_fwd.argtypes = [P(fcm_plan_t), vp, vp, fp, fp, vp, fp, fp, vp, vp]
            L.fcm_pwdw_fwd.argtypes = [P(fcm_plan_t), vp, vp, fp, fp, vp, fp, fp, vp, vp]
            L.fcm_pwpw_fwd.argtypes = [P(fcm_plan_t), vp, vp, fp, fp, vp, fp, fp, vp, vp]
            L.fcm_tune.argtypes = [P(fcm_problem), P(fcm_device_spec), _i32, P(vp), vp, fp, fp,
                                   vp, fp, fp, P(vp), vp, _i32, P(fcm_plan_t)]
            L.fcm_pwdwpw_fwd.argtypes = [P(fcm_plan_t), vp, vp, fp, fp, vp, fp, fp, vp, fp, fp,
                                         vp, vp]
            L.fcm_pwdwpw_lbl.argtypes = [P(fcm_plan_t), vp, vp, fp, fp, vp, fp, fp, vp, fp, fp,
                                         vp, vp, vp, vp]
            L.fcm_pwdwpw_lbl_noalloc.argtypes = [P(fcm_plan_t), vp, vp, fp, fp, vp, fp, fp, vp,
                                                 fp, fp, vp, vp]
            L.fcm_tune_pwdwpw.argtypes = [P(fcm_problem), P(fcm_device_spec), _i32, P(vp), vp,
                                          fp, fp, vp, fp, fp, vp, fp, fp, P(vp), vp, _i32,
                                          P(fcm_plan_t)]
            L.fcm_dw_fwd.argtypes = [P(fcm_plan_t), vp, vp, fp, fp, vp, vp]
            L.fcm_pw_fwd.argtypes = [P(fcm_plan_t), vp, vp, fp, fp, vp, vp]
            L.fcm_conv_fwd.argtypes = [P(fcm_plan_t), vp, vp, fp, fp, vp, vp]
            L.fcm_status_str.restype = ctypes.c_char_p
            L.fcm_status_str.argtypes = [ctypes.c_int]
            L.fcm_last_error.restype = ctypes.c_char_p
            L.fcm_last_error.argtypes = []
            for name in ("fcm_default_device_spec", "fcm_query_device_spec", "fcm_plan",
                         "fcm_plan_variant", "fcm_pack_weights", "fcm_dwpw_fwd",
                         "fcm_b2b_conv_fwd", "fcm_pwdw_fwd", "fcm_pwpw_fwd", "fcm_dw_fwd",
                         "fcm_pw_fwd", "fcm_conv_fwd", "fcm_pwdwpw_fwd", "fcm_pwdwpw_lbl",
                         "fcm_pwdwpw_lbl_noalloc", "fcm_tune_pwdwpw", "fcm_tune"):
                getattr(L, name).restype = ctypes.c_int
            _lib = L
    return _lib


def _check(status: int, where: str):
    if status != FCM_OK:
        detail = lib().fcm_last_error().decode(errors="replace")
        raise FcmError(status, where, detail)


def _ptr(t) -> Optional[int]:
    """Device address of a tensor (or an int address); None stays NULL."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------------------------------
# host-side calls
# ------------------------------------------------------------------------------------
def problem(kind="dwpw", dtype="f16", N=1, H=1, W=1, C=8, K=8, K1=None, R=3, S=3,
            stride=1, pad=1, act1="none", act2="none", dilation=1, mult=1, act3="none",
            residual=False) -> fcm_problem:
    """Build an fcm_problem; K1 defaults to C*mult (depthwise first layer).  For the
    PW->DW module ("pwdw") K1 is the pointwise layer's output and K must equal it; for the
    PW->DW->PW module ("pwdwpw") K1 is the expansion's output, K the projection's, act3
    the projection's activation and residual the identity shortcut.
    dilation / mult: the depthwise layer's tap spacing and depth multiplier (DWPW)."""
    p = fcm_problem()
    p.kind = KIND_CODES[kind] if isinstance(kind, str) else kind
    p.dtype = DTYPE_CODES[dtype] if isinstance(dtype, str) else dtype
    p.N, p.H, p.W, p.C, p.K = N, H, W, C, K
    p.K1 = C * mult if K1 is None else K1
    p.R, p.S = R, S
    dh, dw = (dilation, dilation) if isinstance(dilation, int) else dilation
    p.dil_h, p.dil_w, p.mult = dh, dw, mult
    sh, sw = (stride, stride) if isinstance(stride, int) else stride
    ph, pw = (pad, pad) if isinstance(pad, int) else pad
    p.stride_h, p.stride_w, p.pad_h, p.pad_w = sh, sw, ph, pw
    p.act1 = ACT_CODES[act1] if isinstance(act1, str) else act1
    p.act2 = ACT_CODES[act2] if isinstance(act2, str) else act2
    p.act3 = ACT_CODES[act3] if isinstance(act3, str) else act3
    p.residual = int(bool(residual))
    return p


def fcm_default_device_spec() -> fcm_device_spec:
    s = fcm_device_spec()
    _check(lib().fcm_default_device_spec(ctypes.byref(s)), "fcm_default_device_spec")
    return s


def fcm_query_device_spec(device: int = 0) -> fcm_device_spec:
    s = fcm_device_spec()
    _check(lib().fcm_query_device_spec(device, ctypes.byref(s)), "fcm_query_device_spec")
    return s


def fcm_plan(prob: fcm_problem, spec: Optional[fcm_device_spec] = None) -> fcm_plan_t:
    out = fcm_plan_t()
    _check(lib().fcm_plan(ctypes.byref(prob), ctypes.byref(spec) if spec else None,
                          ctypes.byref(out)), "fcm_plan")
    return out


def fcm_plan_variant(prob: fcm_problem, variant: int,
                     spec: Optional[fcm_device_spec] = None) -> fcm_plan_t:
    out = fcm_plan_t()
    _check(lib().fcm_plan_variant(ctypes.byref(prob), ctypes.byref(spec) if spec else None,
                                  variant, ctypes.byref(out)), "fcm_plan_variant")
    return out


def fcm_plan_chain(layers, N: int, H: int, W: int, dtype="f16",
                   spec: Optional[fcm_device_spec] = None):
    """FusePlanner over a chain of layers given as (type, C, K, stride, act) tuples with type
    "dw" or "pw".  Returns (groups, gma_chain, gma_layer_by_layer); each group is a dict
    with first, count, kind (-1: a single layer), variant and gma."""
    n = len(layers)
    arr = (fcm_layer * n)()
    for i, (t, C, K, s, act) in enumerate(layers):
        arr[i].type = {"dw": FCM_LAYER_DW, "pw": FCM_LAYER_PW}[t] if isinstance(t, str) else t
        arr[i].C, arr[i].K, arr[i].stride = C, K, s
        arr[i].act = ACT_CODES[act] if isinstance(act, str) else act
    out = (fcm_chain_group * n)()
    ng, gc, gl = _i32(), _f64(), _f64()
    _check(lib().fcm_plan_chain(arr, n, N, H, W,
                                DTYPE_CODES[dtype] if isinstance(dtype, str) else dtype,
                                ctypes.byref(spec) if spec else None, out, ctypes.byref(ng),
                                ctypes.byref(gc), ctypes.byref(gl)), "fcm_plan_chain")
    groups = [{"first": out[i].first, "count": out[i].count, "kind": out[i].kind,
               "variant": out[i].variant, "gma": out[i].gma} for i in range(ng.value)]
    return groups, gc.value, gl.value


def fcm_num_variants() -> int:
    return int(lib().fcm_num_variants())


def fcm_variant_name(variant: int) -> str:
    return lib().fcm_variant_name(variant).decode()


def fcm_status_str(status: int) -> str:
    return lib().fcm_status_str(status).decode()


def fcm_last_error() -> str:
    return lib().fcm_last_error().decode(errors="replace")


# ------------------------------------------------------------------------------------
# device calls (asynchronous on the stream)
# ------------------------------------------------------------------------------------
def fcm_pack_weights(plan, w1_src, w1_dst, w2_src=None, w2_dst=None, stream=None):
    _check(lib().fcm_pack_weights(ctypes.byref(plan), _ptr(w1_src), _ptr(w1_dst),
                                  _ptr(w2_src), _ptr(w2_dst), _stream(stream)),
           "fcm_pack_weights")


def fcm_dwpw_fwd(plan, x, w_dw, scale1, bias1, w_pw, scale2, bias2, y, stream=None):
    _check(lib().fcm_dwpw_fwd(ctypes.byref(plan), _ptr(x), _ptr(w_dw), _ptr(scale1),
                              _ptr(bias1), _ptr(w_pw), _ptr(scale2), _ptr(bias2), _ptr(y),
                              _stream(stream)), "fcm_dwpw_fwd")


def fcm_b2b_conv_fwd(plan, x, w1, scale1, bias1, w2, scale2, bias2, y, stream=None):
    _check(lib().fcm_b2b_conv_fwd(ctypes.byref(plan), _ptr(x), _ptr(w1), _ptr(scale1),
                                  _ptr(bias1), _ptr(w2), _ptr(scale2), _ptr(bias2), _ptr(y),
                                  _stream(stream)), "fcm_b2b_conv_fwd")


def fcm_pwdw_fwd(plan, x, w_pw, scale1, bias1, w_dw, scale2, bias2, y, stream=None):
    _check(lib().fcm_pwdw_fwd(ctypes.byref(plan), _ptr(x), _ptr(w_pw), _ptr(scale1),
                              _ptr(bias1), _ptr(w_dw), _ptr(scale2), _ptr(bias2), _ptr(y),
                              _stream(stream)), "fcm_pwdw_fwd")


def fcm_pwpw_fwd(plan, x, w1, scale1, bias1, w2, scale2, bias2, y, stream=None):
    _check(lib().fcm_pwpw_fwd(ctypes.byref(plan), _ptr(x), _ptr(w1), _ptr(scale1),
                              _ptr(bias1), _ptr(w2), _ptr(scale2), _ptr(bias2), _ptr(y),
                              _stream(stream)), "fcm_pwpw_fwd")


def fcm_pwdwpw_fwd(plan, x, w1, scale1, bias1, w2, scale2, bias2, w3, scale3, bias3, y,
                   stream=None):
    _check(lib().fcm_pwdwpw_fwd(ctypes.byref(plan), _ptr(x), _ptr(w1), _ptr(scale1),
                                _ptr(bias1), _ptr(w2), _ptr(scale2), _ptr(bias2), _ptr(w3),
                                _ptr(scale3), _ptr(bias3), _ptr(y), _stream(stream)),
           "fcm_pwdwpw_fwd")


def fcm_pwdwpw_lbl(plan, x, w1, scale1, bias1, w2, scale2, bias2, w3, scale3, bias3, t1, t2,
                   y, stream=None):
    _check(lib().fcm_pwdwpw_lbl(ctypes.byref(plan), _ptr(x), _ptr(w1), _ptr(scale1),
                                _ptr(bias1), _ptr(w2), _ptr(scale2), _ptr(bias2), _ptr(w3),
                                _ptr(scale3), _ptr(bias3), _ptr(t1), _ptr(t2), _ptr(y),
                                _stream(stream)), "fcm_pwdwpw_lbl")


# largest plan->workspace_bytes fcm_pwdwpw_lbl_noalloc takes (FCM_NOALLOC_SCRATCH_BYTES)
FCM_NOALLOC_SCRATCH_BYTES = 32 << 20


def fcm_pwdwpw_lbl_noalloc(plan, x, w1, scale1, bias1, w2, scale2, bias2, w3, scale3, bias3,
                           y, stream=None):
    _check(lib().fcm_pwdwpw_lbl_noalloc(ctypes.byref(plan), _ptr(x), _ptr(w1), _ptr(scale1),
                                        _ptr(bias1), _ptr(w2), _ptr(scale2), _ptr(bias2),
                                        _ptr(w3), _ptr(scale3), _ptr(bias3), _ptr(y),
                                        _stream(stream)), "fcm_pwdwpw_lbl_noalloc")


def fcm_tune_pwdwpw(prob, x, w1, scale1, bias1, w2, scale2, bias2, w3, scale3, bias3, y,
                    iters=20, spec=None, stream=None) -> "fcm_plan_t":
    """As :func:`fcm_tune`, for the PW->DW->PW module."""
    xs = list(x) if isinstance(x, (list, tuple)) else [x]
    ys = list(y) if isinstance(y, (list, tuple)) else [y]
    if len(xs) != len(ys):
        raise ValueError("x and y need the same number of tensors")
    xa = (ctypes.c_void_p * len(xs))(*[_ptr(t) for t in xs])
    ya = (ctypes.c_void_p * len(ys))(*[_ptr(t) for t in ys])
    out = fcm_plan_t()
    _check(lib().fcm_tune_pwdwpw(ctypes.byref(prob), ctypes.byref(spec) if spec else None,
                                 len(xs), xa, _ptr(w1), _ptr(scale1), _ptr(bias1), _ptr(w2),
                                 _ptr(scale2), _ptr(bias2), _ptr(w3), _ptr(scale3),
                                 _ptr(bias3), ya, _stream(stream), int(iters),
                                 ctypes.byref(out)), "fcm_tune_pwdwpw")
    return out


def fcm_tune(prob, x, w1, scale1, bias1, w2, scale2, bias2, y, iters=20, spec=None,
             stream=None) -> "fcm_plan_t":
    """x, y: one tensor each, or equal-length sequences of tensors to rotate over."""
    xs = list(x) if isinstance(x, (list, tuple)) else [x]
    ys = list(y) if isinstance(y, (list, tuple)) else [y]
    if len(xs) != len(ys):
        raise ValueError("x and y need the same number of tensors")
    xa = (ctypes.c_void_p * len(xs))(*[_ptr(t) for t in xs])
    ya = (ctypes.c_void_p * len(ys))(*[_ptr(t) for t in ys])
    out = fcm_plan_t()
    _check(lib().fcm_tune(ctypes.byref(prob), ctypes.byref(spec) if spec else None, len(xs),
                          xa, _ptr(w1), _ptr(scale1), _ptr(bias1), _ptr(w2), _ptr(scale2),
                          _ptr(bias2), ya, _stream(stream), int(iters), ctypes.byref(out)),
           "fcm_tune")
    return out


def fcm_dw_fwd(plan, x, w_dw, scale1, bias1, t, stream=None):
    _check(lib().fcm_dw_fwd(ctypes.byref(plan), _ptr(x), _ptr(w_dw), _ptr(scale1),
                            _ptr(bias1), _ptr(t), _stream(stream)), "fcm_dw_fwd")


def fcm_pw_fwd(plan, t, w_pw, scale2, bias2, y, stream=None):
    _check(lib().fcm_pw_fwd(ctypes.byref(plan), _ptr(t), _ptr(w_pw), _ptr(scale2),
                            _ptr(bias2), _ptr(y), _stream(stream)), "fcm_pw_fwd")


def fcm_conv_fwd(plan, x, w1, scale1, bias1, t, stream=None):
    _check(lib().fcm_conv_fwd(ctypes.byref(plan), _ptr(x), _ptr(w1), _ptr(scale1),
                              _ptr(bias1), _ptr(t), _stream(stream)), "fcm_conv_fwd")
