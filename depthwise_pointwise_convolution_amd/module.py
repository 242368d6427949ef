"""Convenience wrapper over the C ABI for one module instance: plans the problem,
packs the PyTorch-layout weights once (the offline packing step), allocates outputs
with torch, and runs the fused kernel or the layer-by-layer pair.  Marshalling only.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (fcm_b2b_conv_fwd, fcm_conv_fwd, fcm_dw_fwd, fcm_dwpw_fwd, fcm_pack_weights,
               fcm_plan, fcm_plan_variant, fcm_pw_fwd, fcm_pwdw_fwd, fcm_pwdwpw_fwd,
               fcm_pwdwpw_lbl, fcm_pwpw_fwd, fcm_tune, fcm_tune_pwdwpw, problem, FCM_KIND_B2B,
               FCM_KIND_PWDW, FCM_KIND_PWDWPW, FCM_KIND_PWPW)

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
                "i8": torch.int8}


class FcmModule:
    """w1: depthwise [C*mult,R,S], standard [K1,C,3,3] or (PW->DW, PW->DW->PW) pointwise
    [K1,C]; w2: [K,C*mult], [K,K1] or (PW->DW, PW->DW->PW) depthwise [K1,3,3]; w3 (PW->DW->PW
    only): the projection [K,K1] (torch, on the GPU, storage dtype); scale/bias: float32
    per-channel tensors or None."""

    def __init__(self, kind: str, dtype: str, N: int, H: int, W: int, C: int, K: int,
                 K1: Optional[int], stride: int, pad: int, act1: str, act2: str, w1, w2,
                 scale1=None, bias1=None, scale2=None, bias2=None,
                 variant: Optional[int] = None, stream=None, R: int = 3, S: int = 3,
                 dilation: int = 1, mult: int = 1, w3=None, scale3=None, bias3=None,
                 act3: str = "none", residual: bool = False):
        self.prob = problem(kind, dtype, N, H, W, C, K, K1, R=R, S=S, stride=stride, pad=pad,
                            act1=act1, act2=act2, dilation=dilation, mult=mult, act3=act3,
                            residual=residual)
        self.plan = fcm_plan(self.prob) if variant is None else fcm_plan_variant(self.prob,
                                                                                 variant)
        self.dtype = dtype
        self.tdtype = TORCH_DTYPES[dtype]
        dev = w1.device
        e = torch.empty((), dtype=self.tdtype).element_size()
        self.w1p = torch.empty(self.plan.w1_packed_bytes // e, dtype=self.tdtype, device=dev)
        self.w2p = torch.empty(self.plan.w2_packed_bytes // e, dtype=self.tdtype, device=dev)
        fcm_pack_weights(self.plan, w1.contiguous(), self.w1p, w2.contiguous(), self.w2p,
                         stream)
        self.s1, self.b1, self.s2, self.b2 = scale1, bias1, scale2, bias2
        self.out_shape = (N, self.plan.Ho, self.plan.Wo, K)
        self.t_shape = (N, self.plan.Ho, self.plan.Wo, self.prob.K1)
        self.b2b = self.prob.kind == FCM_KIND_B2B
        self.pwdw = self.prob.kind == FCM_KIND_PWDW
        if self.pwdw:  # the intermediate is the pointwise layer's output
            self.t_shape = (N, H, W, K1)
        # a PW->PW module runs its layers through the first-conv / 1x1 entry points
        self.pwpw = self.prob.kind == FCM_KIND_PWPW
        self.b2b = self.b2b or self.pwpw
        # the three-layer module: the projection's filters are used unpacked; its
        # layer-by-layer run takes one workspace holding both intermediates
        self.pwdwpw = self.prob.kind == FCM_KIND_PWDWPW
        if self.pwdwpw:
            self.w3 = w3.contiguous()
            self.s3, self.b3 = scale3, bias3
            self.t_shape = (self.plan.workspace_bytes // e,)
            self.t1_shape = (N, H, W, K1)
            self.t2_shape = (N, self.plan.Ho, self.plan.Wo, K1)

    def new_output(self, device) -> torch.Tensor:
        return torch.empty(self.out_shape, dtype=self.tdtype, device=device)

    def fused(self, x, y=None, stream=None) -> torch.Tensor:
        y = self.new_output(x.device) if y is None else y
        if self.pwdwpw:
            fcm_pwdwpw_fwd(self.plan, x, self.w1p, self.s1, self.b1, self.w2p, self.s2, self.b2,
                           self.w3, self.s3, self.b3, y, stream)
            return y
        fn = (fcm_pwpw_fwd if self.pwpw else fcm_b2b_conv_fwd if self.b2b else
              fcm_pwdw_fwd if self.pwdw else fcm_dwpw_fwd)
        fn(self.plan, x, self.w1p, self.s1, self.b1, self.w2p, self.s2, self.b2, y, stream)
        return y

    def tune(self, x, y=None, iters: int = 20, stream=None) -> None:
        """Replace the plan by the fastest measured variant and grid (fcm_tune); the
        packed weights serve every variant of the module kind.  x (and y) may be lists
        of tensors to rotate over."""
        if y is None:
            y = ([self.new_output(t.device) for t in x] if isinstance(x, (list, tuple))
                 else self.new_output(x.device))
        if self.pwdwpw:
            self.plan = fcm_tune_pwdwpw(self.prob, x, self.w1p, self.s1, self.b1, self.w2p,
                                        self.s2, self.b2, self.w3, self.s3, self.b3, y, iters,
                                        stream=stream)
            return
        self.plan = fcm_tune(self.prob, x, self.w1p, self.s1, self.b1, self.w2p, self.s2,
                             self.b2, y, iters, stream=stream)

    def first_layer(self, x, t=None, stream=None) -> torch.Tensor:
        t = torch.empty(self.t_shape, dtype=self.tdtype, device=x.device) if t is None else t
        if self.pwdw:
            fcm_pw_fwd(self.plan, x, self.w1p, self.s1, self.b1, t, stream)
            return t
        fn = fcm_conv_fwd if self.b2b else fcm_dw_fwd
        fn(self.plan, x, self.w1p, self.s1, self.b1, t, stream)
        return t

    def second_layer(self, t, y=None, stream=None) -> torch.Tensor:
        y = self.new_output(t.device) if y is None else y
        if self.pwdw:
            fcm_dw_fwd(self.plan, t, self.w2p, self.s2, self.b2, y, stream)
            return y
        fcm_pw_fwd(self.plan, t, self.w2p, self.s2, self.b2, y, stream)
        return y

    def unfused(self, x, t=None, y=None, stream=None) -> torch.Tensor:
        if self.pwdwpw:
            t = torch.empty(self.t_shape, dtype=self.tdtype, device=x.device) if t is None else t
            y = self.new_output(x.device) if y is None else y
            n1 = 1
            for d in self.t1_shape:
                n1 *= d
            t1 = t[:n1].view(self.t1_shape)
            t2 = t[n1:].view(self.t2_shape)
            fcm_pwdwpw_lbl(self.plan, x, self.w1p, self.s1, self.b1, self.w2p, self.s2, self.b2,
                           self.w3, self.s3, self.b3, t1, t2, y, stream)
            return y
        return self.second_layer(self.first_layer(x, t, stream), y, stream)


def from_workload(wl, tensors: dict, device="cuda", variant=None) -> "FcmModule":
    """Build a module from a workload description and float64 numpy inputs."""
    tdt = TORCH_DTYPES[wl.dtype]

    def dev(a, dt):
        return None if a is None else torch.from_numpy(a).to(dt).to(device)

    three = wl.kind == "pwdwpw"
    return FcmModule(wl.kind, wl.dtype, wl.N, wl.H, wl.W, wl.C, wl.K,
                     None if wl.kind == "dwpw" else wl.K1, wl.stride, wl.pad, wl.act1,
                     wl.act2, dev(tensors["w1"], tdt), dev(tensors["w2"], tdt),
                     dev(tensors["scale1"], torch.float32), dev(tensors["bias1"], torch.float32),
                     dev(tensors["scale2"], torch.float32), dev(tensors["bias2"], torch.float32),
                     variant=variant, R=wl.R, S=wl.S, dilation=wl.dil, mult=wl.mult,
                     w3=dev(tensors["w3"], tdt) if three else None,
                     scale3=dev(tensors.get("scale3"), torch.float32) if three else None,
                     bias3=dev(tensors.get("bias3"), torch.float32) if three else None,
                     act3=wl.act3, residual=wl.residual)
