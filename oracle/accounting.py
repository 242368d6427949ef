"""Byte/flop accounting and the FusePlanner global-memory-access (GMA) equations.

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle/``).

Two kinds of quantity live here, both plain integers:

* **Algorithmic (compulsory) bytes** of one module invocation: the input feature maps
  read once, the output feature maps written once, each weight and per-channel
  epilogue array read once.  A layer-by-layer (unfused) execution also writes the
  intermediate feature maps and reads them back.  This is the accounting behind the
  FCM paper's Fig. 1 remark that fusing saves half of the DW+PW off-chip accesses
  ("Fusing Depthwise and Pointwise Convolutions for Efficient Inference on GPUs",
  Sec. I) and the forum's "twice as much memory" argument ("Using optimised depthwise
  convolutions").

* **FusePlanner GMA estimates** (FCM paper Sec. IV, Eq. 1-4), transcribed from the
  equations with the garbled typesetting cleaned up.  Units are bytes; tile sizes are
  bytes of the respective tile; "#SMs" is the number of compute units.  A tiling that
  violates a constraint costs +inf, and a selector must compare with ``< inf`` (the
  TVM profiler thread's invalid-candidate lesson).  Readings:
    - Eq. 4 as printed has no term for the module's own output write; the FCM
      estimates here add it, by analogy with "the OFMs are written once" (Sec. IV-A).
    - The DWPW estimate is not printed ("constructed similarly", Sec. IV-B); it is
      built here from Eq. 2 and 3 the way Eq. 4 is built: the depthwise input (with its
      overlap) is read once per pointwise weight tile, because the intermediate is
      recomputed for each; depthwise weights are read once per output tile; pointwise
      weights as in Eq. 2; the intermediate contributes nothing.
"""
from __future__ import annotations

import math

ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1}
INF = float("inf")


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


# ---------------------------------------------------------------------------------
# algorithmic bytes and flops of one invocation
# ---------------------------------------------------------------------------------
def sizes(wl) -> dict:
    """Element counts and byte sizes of every tensor of one invocation."""
    e = ELEM_BYTES[wl.dtype]
    Ho, Wo = wl.Ho, wl.Wo
    # a depthwise layer with depth multiplier m has C*m outputs (one filter per output)
    n1 = wl.C * wl.mult if wl.kind == "dwpw" else wl.K1
    x = wl.N * wl.H * wl.W * wl.C
    y = wl.N * Ho * Wo * wl.K
    if wl.kind == "pwdwpw":
        # two intermediates: the expansion at the input resolution, the depthwise output
        # at the output resolution; three filter arrays and three epilogues
        t = wl.N * wl.H * wl.W * n1 + wl.N * Ho * Wo * n1
        epi = 4 * (n1 * (int(wl.scale1) + int(wl.bias1) + int(wl.scale2) + int(wl.bias2))
                   + wl.K * (int(wl.scale3) + int(wl.bias3)))
        return {"x": x * e, "t": t * e, "y": y * e, "w1": wl.K1 * wl.C * e,
                "w2": wl.K1 * wl.R * wl.S * e, "w3": wl.K * wl.K1 * e, "epi": epi, "elem": e,
                "pixels_out": wl.N * Ho * Wo}
    if wl.kind == "pwdw":
        # the intermediate is the pointwise layer's output, at the input resolution
        t = wl.N * wl.H * wl.W * n1
        w1 = wl.K1 * wl.C
        w2 = wl.K1 * wl.R * wl.S
    else:
        t = wl.N * Ho * Wo * n1
        w1 = n1 * wl.R * wl.S if wl.kind == "dwpw" else wl.K1 * wl.C * wl.R * wl.S
        w2 = wl.K * n1
    epi = 4 * (n1 * (int(wl.scale1) + int(wl.bias1)) + wl.K * (int(wl.scale2) + int(wl.bias2)))
    return {"x": x * e, "t": t * e, "y": y * e, "w1": w1 * e, "w2": w2 * e, "epi": epi,
            "elem": e, "pixels_out": wl.N * Ho * Wo}


def alg_bytes(wl, fused: bool = True) -> int:
    """Fused: input, output, filters and epilogue arrays once.  Layer by layer: each
    intermediate also written and read back, and (three-layer module with the identity
    shortcut) the input read a second time by the last layer."""
    s = sizes(wl)
    b = s["x"] + s["y"] + s["w1"] + s["w2"] + s.get("w3", 0) + s["epi"]
    if not fused:
        b += 2 * s["t"]
        if wl.kind == "pwdwpw" and wl.residual:
            b += s["x"]
    return b


def flops(wl) -> int:
    """Multiply-adds counted as 2 flops; the epilogue is not counted."""
    P = wl.N * wl.Ho * wl.Wo
    if wl.kind == "dwpw":
        n1 = wl.C * wl.mult
        return 2 * P * n1 * wl.R * wl.S + 2 * P * n1 * wl.K
    if wl.kind == "pwdw":
        return 2 * wl.N * wl.H * wl.W * wl.C * wl.K1 + 2 * P * wl.K1 * wl.R * wl.S
    if wl.kind == "pwdwpw":
        return (2 * wl.N * wl.H * wl.W * wl.C * wl.K1 + 2 * P * wl.K1 * wl.R * wl.S
                + 2 * P * wl.K1 * wl.K)
    return 2 * P * wl.K1 * wl.C * wl.R * wl.S + 2 * P * wl.K1 * wl.K


def fused_savings(wl) -> float:
    """Fraction of the unfused algorithmic bytes that fusion removes."""
    return 1.0 - alg_bytes(wl, True) / alg_bytes(wl, False)


# ---------------------------------------------------------------------------------
# FusePlanner equations (FCM paper Sec. IV)
# ---------------------------------------------------------------------------------
def eq1_overlap(ch_w: int, ch_h: int, tile_w: int, tile_h: int, filt_w: int, filt_h: int,
                stride: int) -> int:
    """Eq. 1: input elements per channel loaded more than once because of tiling.
    Each of the ceil(ChannelW/TileW)-1 interior vertical tile borders repeats
    (FilterW - Strides) columns over the whole channel height, and likewise for rows.
    (FilterW - Strides) is clamped at 0 for strides larger than the filter."""
    ow = max(filt_w - stride, 0)
    oh = max(filt_h - stride, 0)
    return ((_ceil_div(ch_w, tile_w) - 1) * ow * ch_h
            + (_ceil_div(ch_h, tile_h) - 1) * oh * ch_w)


def eq2_pw_gma(weights_sz: int, weights_tile_sz: int, ifms_sz: int, ofms_sz: int,
               ofms_tile_sz: int, ifms_tile_sz: int, l1_sz: int, n_sms: int) -> float:
    """Eq. 2: pointwise GMA.  Every IFM is read once per weight tile, OFMs are written
    once, and the weights are read once per OFM tile."""
    if l1_sz < ifms_tile_sz + ofms_tile_sz + weights_tile_sz:
        return INF
    if _ceil_div(ofms_sz, ofms_tile_sz) < n_sms:
        return INF
    return (_ceil_div(weights_sz, weights_tile_sz) * ifms_sz + ofms_sz
            + _ceil_div(ofms_sz, ofms_tile_sz) * weights_sz)


def eq3_dw_gma(ifms_d: int, overlap: int, ifms_sz: int, ofms_sz: int, ofms_hw: int,
               ofms_tile_hw: int, weights_sz: int, ifms_tile_sz: int, ofms_tile_sz: int,
               weights_tile_sz: int, n_ofm_tiles: int, l1_sz: int, n_sms: int) -> float:
    """Eq. 3: depthwise GMA.  Input read once plus the overlap (counted twice, once
    per side of a border, over all IFM channels), OFMs once, weights once per spatial
    output tile."""
    if l1_sz < ifms_tile_sz + ofms_tile_sz + weights_tile_sz:
        return INF
    if n_ofm_tiles < n_sms:
        return INF
    return (2 * ifms_d * overlap + ifms_sz + ofms_sz
            + _ceil_div(ofms_hw, ofms_tile_hw) * weights_sz)


def eq4_pwdw_gma(pw_ifms_d: int, dw_overlap: int, pw_ifms_sz: int, pw_weights_sz: int,
                 pw_weights_tile_sz: int, dw_weights_sz: int, dw_weights_tile_sz: int,
                 dw_ofms_sz: int, dw_ofms_tile_sz: int, dw_ofms_hw: int,
                 dw_ofms_tile_hw: int, tiles_sz_sum: int, n_fcm_ofm_tiles: int,
                 l1_sz: int, n_sms: int, include_output: bool = True) -> float:
    """Eq. 4: PW->DW module GMA.  The PW input (with the DW overlap carried over to
    it, since the intermediate overlap is recomputed) is read once per weight tile of
    whichever layer has more; weights as in Eq. 2/3; the intermediate is free.
    ``tiles_sz_sum`` = PwIFMsTile + DwOFMsTile + PwWeightsTile + DwWeightsTile +
    CommBuffer.  ``include_output`` adds the module's own output write."""
    if l1_sz < tiles_sz_sum:
        return INF
    if n_fcm_ofm_tiles < n_sms:
        return INF
    g = ((2 * pw_ifms_d * dw_overlap + pw_ifms_sz)
         * max(_ceil_div(pw_weights_sz, pw_weights_tile_sz),
               _ceil_div(dw_weights_sz, dw_weights_tile_sz))
         + _ceil_div(dw_ofms_sz, dw_ofms_tile_sz) * pw_weights_sz
         + _ceil_div(dw_ofms_hw, dw_ofms_tile_hw) * dw_weights_sz)
    if include_output:
        g += dw_ofms_sz
    return g


def dwpw_gma(dw_ifms_d: int, dw_overlap: int, dw_ifms_sz: int, dw_weights_sz: int,
             pw_weights_sz: int, pw_weights_tile_sz: int, pw_ofms_sz: int,
             pw_ofms_tile_sz: int, tiles_sz_sum: int, n_fcm_ofm_tiles: int, l1_sz: int,
             n_sms: int) -> float:
    """DW->PW module GMA built from Eq. 2 and 3 as Eq. 4 is (see module docstring)."""
    if l1_sz < tiles_sz_sum:
        return INF
    if n_fcm_ofm_tiles < n_sms:
        return INF
    n_out_tiles = _ceil_div(pw_ofms_sz, pw_ofms_tile_sz)
    return ((2 * dw_ifms_d * dw_overlap + dw_ifms_sz)
            * _ceil_div(pw_weights_sz, pw_weights_tile_sz)
            + n_out_tiles * (pw_weights_sz + dw_weights_sz)
            + pw_ofms_sz)


def pwdwpw_gma(pw_ifms_d: int, dw_overlap: int, pw_ifms_sz: int, w1_sz: int, w2_sz: int,
               w3_sz: int, ofms_sz: int, ofms_tile_sz: int, tiles_sz_sum: int,
               n_fcm_ofm_tiles: int, l1_sz: int, n_sms: int) -> float:
    """Three-layer PW->DW->PW module.  The pages print no estimate for three layers; this
    one takes Eq. 4's form for a module whose workgroup holds every expanded channel (a
    single weight tile): the first layer's input with the depthwise overlap once, the
    three layers' filters once per output tile, the intermediates free, the output once."""
    if l1_sz < tiles_sz_sum:
        return INF
    if n_fcm_ofm_tiles < n_sms:
        return INF
    return ((2 * pw_ifms_d * dw_overlap + pw_ifms_sz)
            + _ceil_div(ofms_sz, ofms_tile_sz) * (w1_sz + w2_sz + w3_sz) + ofms_sz)


def pwdw_redundancy(H: int, W: int, tile_h: int, tile_w: int, stride: int = 1,
                    pad: int = 1, filt: int = 3) -> float:
    """Redundant pointwise work of a tiled PW->DW module (the _R of PWDW_R, FCM paper
    Sec. II-D and Table II): every output tile of tile_h x tile_w depthwise outputs
    recomputes the intermediate over its whole input window, clipped to the image, so
    the pointwise layer runs on sum(window pixels) instead of H * W pixels.  Returns
    sum(window pixels) / (H * W) - 1; zero when one tile covers the whole plane (the
    PWDW case without redundancy)."""
    Ho = (H + 2 * pad - filt) // stride + 1
    Wo = (W + 2 * pad - filt) // stride + 1

    def inside(n_out, tile, n_in):
        tot = 0
        for t in range(_ceil_div(n_out, tile)):
            lo = t * tile * stride - pad
            hi = lo + (min(tile, n_out - t * tile) - 1) * stride + filt
            tot += max(0, min(hi, n_in) - max(lo, 0))
        return tot

    return inside(Ho, tile_h, H) * inside(Wo, tile_w, W) / (H * W) - 1.0


def brute_force_overlap(ch_w: int, ch_h: int, tile_w: int, tile_h: int, filt: int,
                        stride: int) -> int:
    """Count, for one channel, how many input elements are loaded in total beyond the
    first load when the output plane is cut into tiles whose input windows extend
    (filt - stride) elements past each interior border (Fig. 3(a) of the FCM paper:
    overlap regions are loaded once per tile that shares them).  Returns
    sum over elements of (loads - 1) for loaded elements."""
    ext = max(filt - stride, 0)
    loads = [[0] * ch_w for _ in range(ch_h)]
    for ty in range(_ceil_div(ch_h, tile_h)):
        for tx in range(_ceil_div(ch_w, tile_w)):
            y0, x0 = ty * tile_h, tx * tile_w
            y1 = min(ch_h, y0 + tile_h + (ext if y0 + tile_h < ch_h else 0))
            x1 = min(ch_w, x0 + tile_w + (ext if x0 + tile_w < ch_w else 0))
            for yy in range(y0, y1):
                row = loads[yy]
                for xx in range(x0, x1):
                    row[xx] += 1
    return sum(v - 1 for row in loads for v in row if v > 0)


def is_finite(v: float) -> bool:
    return not math.isinf(v)
