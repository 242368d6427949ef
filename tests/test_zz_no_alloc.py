"""fcm_pwdwpw_lbl_noalloc (the layer-by-layer PW->DW->PW baseline with its two
intermediates in the library's static device scratch, for callers that cannot allocate)
against fcm_pwdwpw_lbl with caller workspaces, through the C ABI: the same kernels in the
same order, so the outputs must be identical.  Two calls in a row, the second on a smaller
problem (the scratch keeps the first call's contents), and a repeat of the first."""
import dataclasses

import numpy as np
import pytest

import fcm_inputs
from gpu_util import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


def _case(name, **sizes):
    return dataclasses.replace(fcm_inputs.WORKLOADS[name], **sizes)


def _run(wl, seed):
    import torch
    import depthwise_pointwise_convolution_amd as F
    from depthwise_pointwise_convolution_amd.module import TORCH_DTYPES, from_workload
    inp = fcm_inputs.make_inputs(wl, seed=seed)
    mod = from_workload(wl, inp, device="cuda")
    assert mod.plan.workspace_bytes <= F.FCM_NOALLOC_SCRATCH_BYTES
    x = torch.from_numpy(inp["x"]).to(TORCH_DTYPES[wl.dtype]).cuda()
    ref = mod.unfused(x)
    y = torch.full_like(ref, float("nan"))
    F.fcm_pwdwpw_lbl_noalloc(mod.plan, x, mod.w1p, mod.s1, mod.b1, mod.w2p, mod.s2, mod.b2,
                             mod.w3, mod.s3, mod.b3, y)
    torch.cuda.synchronize()
    return y.cpu(), ref.cpu()


def test_noalloc_matches_the_workspace_entry_point_on_consecutive_calls():
    big = _case("pwdwpw_f16_32x56x56_c24_k144_k24", N=2, H=29, W=37)
    small = _case("pwdwpw_f16_32x112x112_c16_k96_k24_s2", N=1, H=13, W=21)
    for i, (wl, seed) in enumerate(((big, 5), (small, 6), (big, 7))):
        print(f"no-alloc call {i}: {wl.name} N={wl.N} H={wl.H} W={wl.W} seed {seed}",
              flush=True)
        y, ref = _run(wl, seed)
        assert not y.isnan().any(), f"call {i}: output not fully written"
        assert np.array_equal(y.numpy(), ref.numpy()), f"call {i}: differs from fcm_pwdwpw_lbl"
