// plan.cpp -- FusePlanner for gfx950 ("Fusing Depthwise and Pointwise Convolutions for
// Efficient Inference on GPUs", Sec. IV), host only.
//
// Inputs are the problem and the device's compute-unit count and on-chip memory
// sizes.  The candidates are the fused kernel variants compiled into the library
// (variants.def); for each one that can run the problem the planner
//   - checks the two constraints of Eq. 2-4: the workgroup's tiles fit the on-chip
//     memory (here: LDS per workgroup; registers are budgeted separately) and the
//     module has at least as many output tiles as there are compute units;
//   - computes the bytes the variant requests from the memory hierarchy with its
//     real tile geometry (exact halo footprint clipped at the image border, input
//     re-read once per output-channel tile, weights once per tile or once per
//     workgroup when they stay in registers, output once);
//   - computes the pages' own Eq. 1-3 estimate for the same tiling;
// and keeps the feasible variant with the shortest roofline time (the slowest of
// HBM, on-chip traffic, matrix and vector work, each counting recomputation; within
// 1%: fewer bytes, less redundant arithmetic, more occupancy).  A
// variant that breaks a constraint costs +infinity and is never preferred to a
// finite one.  It then compares against the layer-by-layer kernels with the same
// models and sets `fuse` when the fused module needs fewer global memory accesses
// (Sec. IV-B, last paragraph).
#include "plan.h"

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <stdlib.h>

#include <algorithm>
#include <initializer_list>
#include <cmath>
#include <vector>

#include "lbl_tiles.h"

namespace fcm {

const VariantDesc kVariants[] = {
#define FCM_V_DWPW(name, dt, CT, S, TH, TW, KT, CC, WRES, OCC) \
    {#name, VK_DWPW, dt, S, TH, TW, KT, CC, WRES ? 1 : 0, 0, 0, OCC, 4, 0, 0},
#define FCM_V_DWPW32(name, S, TH, TW, KT, CC) \
    {#name, VK_DWPW32, FCM_F32, S, TH, TW, KT, CC, 0, 0, 0, 1, 4, 0, 0},
#define FCM_V_B2B(name, dt, CT, S, TH, TW, K1, KT, CC) \
    {#name, VK_B2B, dt, S, TH, TW, KT, CC, 1, 0, K1, 1, 4, 0, 0},
#define FCM_V_DWPW_MM(name, dt, CT, S, TH, TW, KT, CC, NW, OCC) \
    {#name, VK_DWPW_MM, dt, S, TH, TW, KT, CC, 1, 2, 0, OCC, NW, 0, 0},
#define FCM_V_B2B_MM(name, dt, CT, S, OCC) \
    {#name, VK_B2B_MM, dt, S, 4, 16, 64, 64, 1, 2, 64, OCC, 4, 0, 0},
#define FCM_V_DWPW_MMW(name, dt, CT, S, TH, TW, KT, CMAX, NW, OCC) \
    {#name, VK_DWPW_MMW, dt, S, TH, TW, KT, 64, 0, 3, 0, OCC, NW, CMAX, 0},
#define FCM_V_DWPW_MMWD(name, dt, CT, S, D, TH, TW, KT, CMAX, NW, OCC) \
    {#name, VK_DWPW_MMW, dt, S, TH, TW, KT, 64, 0, 3, 0, OCC, NW, CMAX, 0, 3, D, 1},
#define FCM_V_DWPW_MMM(name, dt, CT, S, M, TH, TW, KT, CC, NW, OCC) \
    {#name, VK_DWPW_MM, dt, S, TH, TW, KT, CC, 1, 2, 0, OCC, NW, 0, 0, 3, 1, M},
#define FCM_V_DWPW_MMF(name, dt, CT, S, FS, TH, TW, KT, CC, NW, OCC) \
    {#name, VK_DWPW_MM, dt, S, TH, TW, KT, CC, 1, 2, 0, OCC, NW, 0, 0, FS, 1, 1},
#define FCM_V_DWPW_WS(name, dt, CTy, S, TH, TW, CT, KT, NW) \
    {#name, VK_DWPW_WS, dt, S, TH, TW, KT, CT, 1, 2, 0, NW / 4, NW, CT, 0},
#define FCM_V_DWPW_WSL(name, dt, CT, S, TH, TW, KT, CMAX, NW) \
    {#name, VK_DWPW_WSL, dt, S, TH, TW, KT, 64, 0, 4, 0, NW / 4, NW, CMAX, 0},
#define FCM_V_PWDW_MM(name, dt, CT, S, TH, CMAX, NW, BPW, OCC) \
    {#name, VK_PWDW_MM, dt, S, TH, 16, NW * BPW * 16, CMAX, 1, 2, 0, OCC, NW, CMAX, BPW},
#define FCM_V_PWDWPW_MM(name, dt, CT, S, TH, CMAX, NW, BPW, KB, OCC) \
    {#name, VK_PWDWPW_MM, dt, S, TH, 16, KB * 16, CMAX, 1, 2, NW * BPW * 16, OCC, NW, CMAX, BPW},
#define FCM_V_DWPW_I8(name, S, OCC, CMAX) \
    {#name, VK_DWPW_I8, FCM_I8, S, 4, 16, 64, 64, 1, 2, 0, OCC, 4, CMAX, 0},
#define FCM_V_PWPW_MM(name, dt, CT, PB, OCC, CMAX, KT) \
    {#name, VK_PWPW_MM, dt, 1, PB, 16, KT, CMAX, 1, 2, CMAX == 64 ? 64 : 1 << 20, OCC, 4, CMAX, 0},
#define FCM_V_DWPW_GEN(name, dt, CT, S, FS, D, M, TH, TW, KT, CC, NG) \
    {#name, VK_DWPW_GEN, dt, S, TH, TW, KT, CC, 0, 1, 0, 2, 4 * NG, 0, 0, FS, D, M},
#include "variants.def"
#undef FCM_V_DWPW
#undef FCM_V_DWPW32
#undef FCM_V_B2B
#undef FCM_V_DWPW_MM
#undef FCM_V_B2B_MM
#undef FCM_V_DWPW_MMW
#undef FCM_V_DWPW_MMWD
#undef FCM_V_DWPW_MMM
#undef FCM_V_DWPW_MMF
#undef FCM_V_PWDW_MM
#undef FCM_V_PWDWPW_MM
#undef FCM_V_DWPW_WS
#undef FCM_V_DWPW_WSL
#undef FCM_V_DWPW_I8
#undef FCM_V_PWPW_MM
#undef FCM_V_DWPW_GEN
};
const int kNumVariants = (int)(sizeof(kVariants) / sizeof(kVariants[0]));

namespace {

int elem_bytes(int dtype) { return dtype == FCM_F32 ? 4 : dtype == FCM_I8 ? 1 : 2; }

// Product of sizes for the range checks, saturated at 2^61 (the checks compare it with
// bounds far below, and an unvalidated problem may hold sizes whose product overflows);
// 0 if any factor is not positive.
int64_t sat_mul(std::initializer_list<int64_t> xs) {
    const int64_t cap = (int64_t)1 << 61;
    int64_t r = 1;
    for (int64_t x : xs) {
        if (x <= 0) return 0;
        if (r > cap / x) return cap;
        r *= x;
    }
    return r;
}
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Rows (or columns) of the input that the halo window of output tile `t` (extent
// `tile` outputs, stride s, 3 taps, padding pad) covers inside [0, in).
int64_t window_inside(int t, int tile, int s, int pad, int in, int ext = 3) {
    const int64_t lo = (int64_t)t * tile * s - pad;
    const int64_t hi = lo + (int64_t)(tile - 1) * s + ext;  // exclusive
    const int64_t a = std::max<int64_t>(lo, 0), b = std::min<int64_t>(hi, in);
    return b > a ? b - a : 0;
}

// Sum over all output tiles of an image of the input pixels their halo windows
// load (clipped to the image): the exact per-image footprint of a tiled
// 3x3 stencil, overlaps counted once per tile that loads them.
int64_t halo_pixels(int Ho, int Wo, int H, int W, int th, int tw, int s, int ph, int pw,
                    int ext_h = 3, int ext_w = 3) {
    int64_t rows = 0, cols = 0;
    for (int t = 0; t < cdiv(Ho, th); ++t) rows += window_inside(t, th, s, ph, H, ext_h);
    for (int t = 0; t < cdiv(Wo, tw); ++t) cols += window_inside(t, tw, s, pw, W, ext_w);
    return rows * cols;
}

// FCM paper Eq. 1 over the input plane, with the tile extents in input pixels.
double eq1_overlap(int chw, int chh, int tilew, int tileh, int filt, int stride) {
    const int o = std::max(filt - stride, 0);
    return (double)(cdiv(chw, tilew) - 1) * o * chh + (double)(cdiv(chh, tileh) - 1) * o * chw;
}

}  // namespace

// A multiple of ktiles (a workgroup keeps one output-channel slice for all its tiles),
// no more workgroups than tiles, and never above capacity: a workgroup that has to
// wait for a free slot would run after all the others.
int64_t persistent_grid(int64_t ptiles, int ktiles, int64_t capacity) {
    const int64_t work = ptiles * ktiles;
    const int64_t g = std::min(work, std::max<int64_t>(capacity, ktiles));
    return std::max<int64_t>(g / ktiles, 1) * ktiles;
}

void default_spec(fcm_device_spec* out) {
    memset(out, 0, sizeof(*out));
    out->num_cus = 256;
    out->num_xcds = 8;
    out->simds_per_cu = 4;
    out->wave_size = 64;
    out->max_waves_per_simd = 8;
    out->vgprs_per_simd_lane = 512;
    out->lds_bytes_per_cu = 160 * 1024;
    out->lds_bytes_per_wg = 160 * 1024;
    out->l2_bytes_per_xcd = 4LL * 1024 * 1024;
    out->hbm_bytes_per_s = 8.0e12;
    out->mfma_f16_flops = 2.5e15;
    out->mfma_f32_flops = 157.3e12;
    // 256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz, no packed fp32 math
    out->valu_f32_flops = 256.0 * 4 * 16 * 2 * 2.4e9;
}

int variant_lds_bytes(const VariantDesc& v) {
    const int e = elem_bytes(v.dtype);
    if (v.vkind == VK_DWPW_GEN) {
        // input window chunk, intermediate chunk (C*M channels), fp32 depthwise filters and
        // epilogue-1 constants of the chunk, epilogue-2 constants of the K tile
        // (per channel group), plus the partial sums one group hands to another
        const int ext = (v.fs - 1) * v.dil + 1, cm = v.cc * v.mult, ng = v.waves / 4;
        const int IHg = (v.th - 1) * v.stride + ext, IWg = (v.tw - 1) * v.stride + ext;
        const int red = ng > 1 ? v.th * v.tw * v.kt * 4 : 16;
        return ng * (IHg * IWg * (v.cc + 8) * e + v.th * v.tw * (cm + 8) * e +
                     v.fs * v.fs * cm * 4 + 2 * cm * 4) +
               2 * v.kt * 4 + red;
    }
    // (a variant compiled for another filter size or dilated taps spans (fs - 1) dil + 1
    // pixels per window side)
    const int ext = v.fs > 0 ? (v.fs - 1) * std::max(v.dil, 1) + 1 : 3;
    const int IH = (v.th - 1) * v.stride + ext, IW = (v.tw - 1) * v.stride + ext;
    const int P = v.th * v.tw;
    switch (v.vkind) {
    case VK_DWPW:
        return IH * IW * (v.cc + 8) * e + P * (v.cc + 8) * e + 9 * v.cc * 4 + 2 * v.cc * 4 +
               2 * v.kt * 4;
    case VK_DWPW32:
        return IH * IW * (v.cc + 4) * 4 + P * (v.cc + 4) * 4 + 9 * v.cc * 4 + 2 * v.cc * 4 +
               2 * v.kt * 4;
    case VK_DWPW_MM:
    case VK_B2B_MM: {
        // input tile (or chunk) buffers and as many intermediate tiles (one direct-load
        // round is one 16-byte piece per thread)
        // (a depth multiplier m: the window holds cc / m input channels)
        const int nt = 64 * v.waves;
        const int slots = IH * IW * (v.cc / (8 * std::max(v.mult, 1)));
        const int slots_p = (slots + nt - 1) / nt * nt;
        const int tls = v.th * (v.cc / 32) * 64 * 16;
        return v.nbuf * (slots_p * 16 + tls);
    }
    case VK_DWPW_MMW: {
        // three input chunk buffers (rounded to whole 512-thread load rounds), two
        // intermediate chunks of 16-pixel blocks, epilogue-2 constants of the K tile
        const int nt = 64 * v.waves;
        const int slots = IH * IW * (v.cc / 8);
        const int slots_p = (slots + nt - 1) / nt * nt;
        const int mb = (P + 15) / 16;
        return v.nbuf * slots_p * 16 + 2 * mb * (v.cc / 32) * 64 * 16 + 2 * v.kt * 4 +
               v.cmax * (9 * 2 + 2 * 4);
    }
    case VK_DWPW_WSL: {
        // four input windows (whole load rounds of the depthwise waves), two
        // intermediate slices of 16-pixel blocks, epilogue-2 constants of the K tile,
        // depthwise filters and epilogue-1 constants of every channel
        const int nt = 32 * v.waves;
        const int slots = IH * IW * (v.cc / 8);
        const int slots_p = (slots + nt - 1) / nt * nt;
        const int mb = (P + 15) / 16;
        return v.nbuf * slots_p * 16 + 2 * mb * (v.cc / 32) * 64 * 16 + 2 * v.kt * 4 +
               v.cmax * (9 * 2 + 2 * 4);
    }
    case VK_DWPW_WS: {
        // three input windows (whole direct-load rounds of the depthwise half of the
        // waves, plus one wave's landing slots for the partial round) and three
        // intermediate blocks of 16 pixels x cc channels
        const int nt = 64 * (v.waves / 2);
        const int slots = IH * IW * (v.cc / 8);
        const int rf = slots / nt, rem = slots - rf * nt;
        const int slots_b = rf * nt + (rem + 63) / 64 * 64 + (rem > 0 ? 64 : 0);
        return 3 * slots_b * 16 + 3 * (v.cc / 32) * 1024;
    }
    case VK_PWDWPW_MM: {
        // two input-window buffers (whole load rounds of 16-pixel blocks), one expansion
        // tile per expanded-channel block ((IH + 1) rows x 2 chunks x IW x 16 bytes), and
        // the depthwise tile: th x 16 pixels x (k1 + 8) channels
        const int nt = 64 * v.waves;
        const int iw = 15 * v.stride + 3;
        const int np = IH * iw, npb = (np + 15) / 16;
        const int slots = npb * 16 * (v.cmax / 8);
        const int slots_p = (slots + nt - 1) / nt * nt;
        const int nb = v.k1 / 16;
        return 2 * slots_p * 16 + nb * (IH + 1) * 2 * iw * 16 + v.th * 16 * (v.k1 + 8) * 2;
    }
    case VK_PWPW_MM: {
        // two input tiles of th x 16 pixels x cmax channels, two intermediate tiles of
        // th x 16 pixels x 64 channels
        return 2 * v.th * 16 * v.cmax * e + 2 * v.th * 16 * 64 * e;
    }
    case VK_DWPW_I8: {
        // two input tile buffers (16-byte chunks of 16 channels, whole 256-thread load
        // rounds) and two 4-row intermediate tiles of 1 KB per row
        // (the sliced build: depthwise filters [9][cmax] bytes and epilogue-1 constants
        // of every channel as well)
        const int slots = IH * IW * 4;
        const int slots_p = (slots + 255) / 256 * 256;
        return 2 * slots_p * 16 + 2 * 4 * 1024 + (v.cmax > 64 ? v.cmax * (9 + 8) : 0);
    }
    case VK_PWDW_MM: {
        // two input-window buffers (whole load rounds of 16-pixel blocks) and one
        // intermediate tile per owned channel block: (IH + 1) rows x 2 chunks x IW
        // columns x 16 bytes
        const int nt = 64 * v.waves;
        const int npb = (IH * IW + 15) / 16;
        const int slots = npb * 16 * (v.cmax / 8);
        const int slots_p = (slots + nt - 1) / nt * nt;
        return 2 * slots_p * 16 + v.waves * v.bpw * (IH + 1) * 2 * IW * 16;
    }
    default:
        return IH * IW * (v.cc + 8) * e + 2 * v.k1 * 4 + 2 * v.kt * 4;
    }
}

int variant_vgpr_estimate(const VariantDesc& v) {
    const int P = v.th * v.tw;
    const int MBW = P / 64;
    switch (v.vkind) {
    case VK_DWPW_GEN: {
        // accumulators, the chunk's pointwise operands, the next chunk's input and
        // depthwise constants in flight, one depthwise item's sums
        const int KB = v.kt / 16, ext = (v.fs - 1) * v.dil + 1;
        const int slots = ((v.th - 1) * v.stride + ext) * ((v.tw - 1) * v.stride + ext) *
                          (v.cc / 8);
        const int consts = (v.fs * v.fs * v.cc * v.mult + 255) / 256;
        return 40 + MBW * KB * 4 + (v.cc * v.mult / 32) * KB * 4 + 4 * ((slots + 255) / 256) +
               consts + 8 * v.mult + 24;
    }
    case VK_DWPW: {
        const int KB = v.kt / 16, KS = v.cc / 32;
        const int cg = v.cc / 8;
        int vb = (v.th * v.tw * cg) / 256;
        if (vb < 1) vb = 1;
        return 40 + MBW * KB * 4 + (v.wres ? KS * KB * 4 : 12) + vb * 8 + 24;
    }
    case VK_DWPW32:
        // accumulators of the wave's pixel blocks, the chunk's weight operands, the
        // depthwise work item, staging and addressing
        return 40 + MBW * (v.kt / 16) * 4 + (v.cc / 16) * (v.kt / 16) * 4 + 24 + 24;
    case VK_DWPW_MM: {
        // per wave: pointwise operands of its KT/4 output channels and their epilogue
        // constants, its depthwise operands and epilogue-1 constants, the direct-load
        // plan, accumulators of its rows, staging and addressing
        // (a depth multiplier: three depthwise operands per channel block, not five)
        const int cbw = v.cc / 64, nks = v.cc / 32, kbw = v.kt / 64, nt = 64 * v.waves;
        // (a 5x5 filter: 13 compact operands per block and one block's operand reads)
        const int rw = v.th * 4 / v.waves, m = std::max(v.mult, 1), fs = v.fs > 0 ? v.fs : 3;
        const int slots = ((v.th - 1) * v.stride + fs) * ((v.tw - 1) * v.stride + fs) * (v.cc / (8 * m));
        const int dwops = fs == 5 ? cbw * 13 + 3 * ((rw - 1) * v.stride + fs) * 4
                                  : cbw * (m > 1 ? 12 : 20);
        (void)MBW;
        return nks * kbw * 4 + v.kt / 8 + dwops + cbw * 8 + 2 * ((slots + nt - 1) / nt) +
               rw * 4 + rw * kbw * 4 + 24 + 16;
    }
    case VK_B2B_MM: {
        // per wave: 18 resident 3x3 operands, 8 resident 1x1 operands, 32 epilogue-2
        // constants, input-operand offsets, the direct-load plan, accumulators
        const int slots = ((v.th - 1) * v.stride + 3) * ((v.tw - 1) * v.stride + 3) * 8;
        return 72 + 32 + 32 + 8 + 18 + 2 * ((slots + 255) / 256) + 32 + 16 + 20;
    }
    case VK_DWPW_MMW: {
        // per wave: accumulators of its KT/8 output channels for every 16-pixel block,
        // two sets of pointwise operands, depthwise operands and operand offsets, the
        // direct-load plan, staging and addressing
        const int mb = (P + 15) / 16, kbw = v.kt / (16 * v.waves), nt = 64 * v.waves;
        const int ppw = mb * 4 / v.waves, ext = v.dil > 1 ? 2 * v.dil + 1 : 3;
        const int slots = ((v.th - 1) * v.stride + ext) * ((v.tw - 1) * v.stride + ext) * 8;
        return 4 * mb * kbw + 16 * kbw + 28 + 5 * ppw + 2 * ((slots + nt - 1) / nt) + 36 + 24;
    }
    case VK_DWPW_WSL: {
        // the larger of the two roles: a pointwise wave holds its KT/4 output channels'
        // accumulators for every pixel block, two sets of one step's filters and the step's
        // intermediate operands; a depthwise wave every pixel block's window operands, the
        // diagonal operand, accumulators, read offsets and the direct-load plan
        const int half = v.waves / 2;
        const int mb = (P + 15) / 16, kbw = v.kt / (16 * half), nks = v.cc / 32;
        const int mbw = mb * 4 / half;
        const int slots = ((v.th - 1) * v.stride + 3) * ((v.tw - 1) * v.stride + 3) * 8;
        const int r = (slots + 64 * half - 1) / (64 * half);
        const int pw_regs = 4 * mb * kbw + 2 * 4 * nks * kbw + 4 * mb * nks + 24;
        const int dw_regs = 20 * mbw + 4 + 4 * mbw + 5 * mbw + 3 * r + 8 + 30;
        return std::max(pw_regs, dw_regs) + 16;
    }
    case VK_DWPW_WS: {
        // the larger of the two roles: a pointwise wave holds its output channels'
        // operands over all cc inputs, one step's intermediate operands, accumulators and
        // epilogue constants; a depthwise wave its channel blocks' diagonal operands (5 x 4
        // registers each), epilogue constants, two blocks' window operands and the
        // direct-load plan
        const int npw = v.waves / 2, kbw = v.kt / (16 * npw), nks = v.cc / 32;
        const int cbw = v.cc / 16 / npw;
        const int slots = ((v.th - 1) * v.stride + 3) * ((v.tw - 1) * v.stride + 3) * (v.cc / 8);
        const int r = (slots + 64 * npw - 1) / (64 * npw);
        const int pw_regs = nks * kbw * 4 + 4 * nks + 4 * kbw + 4 * kbw * 2 + 24;
        const int dw_regs = 20 * cbw + 8 * cbw + 40 + r + (r + 1) / 2 + 10 + 24;
        return pw_regs > dw_regs ? pw_regs : dw_regs;
    }
    case VK_PWDWPW_MM: {
        // expansion, depthwise and projection operands (the projection's for every
        // output block), the three epilogues' constants, the reads in flight, the
        // depthwise accumulators of the tile's rows, per-pixel-block offsets, the
        // direct-load plan and addressing
        const int bpw = v.bpw, nkc = v.cmax / 32, nk3 = v.k1 / 32, kb = v.kt / 16;
        const int iw = 15 * v.stride + 3, ih = (v.th - 1) * v.stride + 3;
        const int npb = (ih * iw + 15) / 16;
        const int slots = npb * 16 * (v.cmax / 8), nt = 64 * v.waves;
        return 4 * bpw * nkc + 20 * bpw + 16 * bpw + 4 * kb * nk3 + 8 * kb + 12 * nkc +
               16 * bpw + 4 * v.th + 2 * npb + 2 * ((slots + nt - 1) / nt) + 4 * nk3 + 30;
    }
    case VK_PWPW_MM: {
        // first-layer operands, 8 second-layer operands, 4 + 16 epilogue constants, the
        // direct-load plan, operands and accumulators of the tile, addressing; the wide
        // build: a slice's first-layer operands over cmax inputs, its second-layer
        // operands and accumulators of KT outputs, epilogue-2 constants, the load plan
        if (v.cmax > 64)
            return 4 * (v.cmax / 32) + 8 * (v.kt / 16) + 4 * (v.kt / 16) + v.kt / 2 +
                   v.cmax / 32 + 16 + 40;
        return 8 + 32 + 8 + 32 + v.th * 2 / 4 * 8 + v.th * 8 + (v.th / 4) * 16 + 40;
    }
    case VK_DWPW_I8: {
        // depthwise and pointwise operands, both epilogues' constants (4 + 16 channels),
        // the direct-load plan, operands of the input rows, accumulators, addressing
        // (the sliced build: two operand sets, and the accumulators live across steps)
        const int IH = (v.th - 1) * v.stride + 3, IW = 15 * v.stride + 3;
        return 12 + 16 + 8 + 32 + 2 * ((IH * IW * 4 + 255) / 256) + 4 * IH + 16 + 16 + 40 +
               (v.cmax > 64 ? 16 + 8 : 0);
    }
    case VK_PWDW_MM: {
        // per owned block: pointwise operands, five depthwise operands, both epilogues'
        // constants; window offsets and positions per pixel block, the direct-load plan,
        // the output rows' accumulators, operands in flight, addressing
        const int IH = (v.th - 1) * v.stride + 3, IW = 15 * v.stride + 3;
        const int npb = (IH * IW + 15) / 16, nt = 64 * v.waves;
        const int slots = npb * 16 * (v.cmax / 8);
        return v.bpw * (4 * (v.cmax / 32) + 20 + 16) + 2 * npb + 2 * ((slots + nt - 1) / nt) +
               4 * v.th + 16 + 48;
    }
    default: {
        const int KB1 = v.k1 / 16, KB2 = v.kt / 16, KS2 = v.k1 / 32;
        return 40 + MBW * KB1 * 4 + KS2 * KB2 * 4 + KB2 * 4 + MBW * 4 + 24;
    }
    }
}

fcm_status validate_problem(const fcm_problem* p, std::string* err) {
    if (!p) {
        *err = "problem pointer is NULL";
        return FCM_ERR_INVALID_ARG;
    }
    if (p->kind != FCM_KIND_DWPW && p->kind != FCM_KIND_B2B && p->kind != FCM_KIND_PWDW &&
        p->kind != FCM_KIND_PWPW && p->kind != FCM_KIND_PWDWPW) {
        *err = "unknown kind";
        return FCM_ERR_INVALID_ARG;
    }
    if (p->kind != FCM_KIND_PWDWPW && (p->act3 != 0 || p->residual != 0)) {
        *err = "act3 and residual describe the third layer of a PW->DW->PW module";
        return FCM_ERR_INVALID_ARG;
    }
    if (p->act3 < FCM_ACT_NONE || p->act3 > FCM_ACT_RELU6 || p->residual < 0 ||
        p->residual > 1) {
        *err = "unknown third activation, or residual not 0 or 1";
        return FCM_ERR_INVALID_ARG;
    }
    if (p->dtype < FCM_F32 || p->dtype > FCM_I8) {
        *err = "unknown dtype";
        return FCM_ERR_INVALID_ARG;
    }
    if (p->act1 < FCM_ACT_NONE || p->act1 > FCM_ACT_RELU6 || p->act2 < FCM_ACT_NONE ||
        p->act2 > FCM_ACT_RELU6) {
        *err = "unknown activation";
        return FCM_ERR_INVALID_ARG;
    }
    if (p->N <= 0 || p->H <= 0 || p->W <= 0 || p->C <= 0 || p->K <= 0 || p->K1 <= 0 ||
        p->R <= 0 || p->S <= 0 || p->stride_h <= 0 || p->stride_w <= 0 || p->pad_h < 0 ||
        p->pad_w < 0) {
        *err = "sizes, filter extent and strides must be positive, padding non-negative";
        return FCM_ERR_INVALID_ARG;
    }
    if (p->dil_h < 0 || p->dil_w < 0 || p->mult < 0) {
        *err = "dilation and depth multiplier must be non-negative (0 means 1)";
        return FCM_ERR_INVALID_ARG;
    }
    if (p->kind != FCM_KIND_DWPW && (p->dil_h > 1 || p->dil_w > 1 || p->mult > 1)) {
        *err = "dilation and depth multiplier describe the depthwise layer of a DW->PW module";
        return FCM_ERR_INVALID_ARG;
    }
    if (p->kind == FCM_KIND_DWPW && (int64_t)p->K1 != (int64_t)p->C * prob_mult(*p)) {
        *err = "a depthwise layer has C * mult outputs: K1 must equal C * mult";
        return FCM_ERR_INVALID_ARG;
    }
    if (p->kind == FCM_KIND_PWDW && p->K != p->K1) {
        *err = "the depthwise layer of a PW->DW module keeps the channel count: K must equal K1";
        return FCM_ERR_INVALID_ARG;
    }
    if (p->kind == FCM_KIND_PWDWPW && p->residual &&
        (p->K != p->C ||
         conv_out(p->H, p->pad_h, p->R, p->stride_h) != p->H ||
         conv_out(p->W, p->pad_w, p->S, p->stride_w) != p->W || p->stride_h != 1 ||
         p->stride_w != 1)) {
        *err = "the identity shortcut needs stride 1, K == C and an unchanged extent";
        return FCM_ERR_INVALID_ARG;
    }
    if (p->R > 64 || p->S > 64 || prob_dil_h(*p) > 64 || prob_dil_w(*p) > 64) {
        *err = "filter extent and dilation must be at most 64";
        return FCM_ERR_UNSUPPORTED;
    }
    if (p->pad_h >= prob_ext_h(*p) || p->pad_w >= prob_ext_w(*p)) {
        *err = "padding must be smaller than the filter's (dilated) extent";
        return FCM_ERR_INVALID_ARG;
    }
    if (p->H + 2 * p->pad_h < prob_ext_h(*p) || p->W + 2 * p->pad_w < prob_ext_w(*p)) {
        *err = "padded input is smaller than the filter";
        return FCM_ERR_INVALID_ARG;
    }
    const int64_t big = (int64_t)1 << 31;
    if (sat_mul({p->N, p->H, p->W, p->C}) >= big || sat_mul({p->N, p->H, p->W, p->K}) >= big ||
        sat_mul({p->N, p->H, p->W, p->K1}) >= big) {
        *err = "tensor element counts must stay below 2^31";
        return FCM_ERR_UNSUPPORTED;
    }
    if (p->kind == FCM_KIND_PWPW) {
        // two 1x1 layers: no filter extent, stride or padding to choose
        if (p->R != 1 || p->S != 1 || p->stride_h != 1 || p->stride_w != 1 || p->pad_h != 0 ||
            p->pad_w != 0) {
            *err = "a PW->PW module is two 1x1 layers: R = S = 1, stride 1, no padding";
            return FCM_ERR_INVALID_ARG;
        }
        if (p->C % 8 || p->K % 8 || p->K1 % 8) {
            *err = "channel counts must be multiples of 8 (16-byte NHWC vectors)";
            return FCM_ERR_UNSUPPORTED;
        }
        if (p->dtype == FCM_F32 || p->dtype == FCM_I8) {
            *err = "the PW->PW kernels need 16-bit storage (fp16 or bf16)";
            return FCM_ERR_UNSUPPORTED;
        }
        const int64_t big = (int64_t)1 << 31;
        if (sat_mul({p->N, p->H, p->W, std::max(std::max(p->C, p->K), p->K1)}) >= big) {
            *err = "tensor element counts must stay below 2^31";
            return FCM_ERR_UNSUPPORTED;
        }
        return FCM_OK;
    }
    if (prob_is_gen(*p)) {
        if (p->R != p->S || (p->R != 3 && p->R != 5 && p->R != 7)) {
            *err = "generalised depthwise kernels take square 3x3, 5x5 or 7x7 filters";
            return FCM_ERR_UNSUPPORTED;
        }
        if (prob_dil_h(*p) != prob_dil_w(*p)) {
            *err = "generalised depthwise kernels take the same dilation in both directions";
            return FCM_ERR_UNSUPPORTED;
        }
        if (p->stride_h != p->stride_w || (p->stride_h != 1 && p->stride_h != 2)) {
            *err = "stride must be 1 or 2 in both directions";
            return FCM_ERR_UNSUPPORTED;
        }
        if (p->dtype != FCM_F16 && p->dtype != FCM_BF16) {
            *err = "generalised depthwise kernels need 16-bit storage (fp16 or bf16)";
            return FCM_ERR_UNSUPPORTED;
        }
        if (p->C % 8 || p->K % 8 || p->K1 % 8) {
            *err = "channel counts must be multiples of 8 (16-byte NHWC vectors)";
            return FCM_ERR_UNSUPPORTED;
        }
        return FCM_OK;
    }
    if (p->R != 3 || p->S != 3) {
        *err = "only 3x3 first-layer filters have kernels";
        return FCM_ERR_UNSUPPORTED;
    }
    if (p->stride_h != p->stride_w || (p->stride_h != 1 && p->stride_h != 2)) {
        *err = "stride must be 1 or 2 in both directions";
        return FCM_ERR_UNSUPPORTED;
    }
    if (p->pad_h > 1 || p->pad_w > 1) {
        *err = "padding must be 0 or 1";
        return FCM_ERR_UNSUPPORTED;
    }
    if (p->C % 8 || p->K % 8 || p->K1 % 8) {
        *err = "channel counts must be multiples of 8 (16-byte NHWC vectors)";
        return FCM_ERR_UNSUPPORTED;
    }
    if (p->kind == FCM_KIND_B2B && p->dtype == FCM_F32) {
        *err = "the back-to-back kernels need 16-bit storage (fp16 or bf16)";
        return FCM_ERR_UNSUPPORTED;
    }
    if (p->kind == FCM_KIND_PWDW && p->dtype == FCM_F32) {
        *err = "the PW->DW kernels need 16-bit storage (fp16 or bf16)";
        return FCM_ERR_UNSUPPORTED;
    }
    if (p->kind == FCM_KIND_PWDWPW && (p->dtype == FCM_F32 || p->dtype == FCM_I8)) {
        *err = "the PW->DW->PW kernels need 16-bit storage (fp16 or bf16)";
        return FCM_ERR_UNSUPPORTED;
    }
    if (p->dtype == FCM_I8 && p->kind != FCM_KIND_DWPW) {
        *err = "int8 storage is provided for the DW->PW module only";
        return FCM_ERR_UNSUPPORTED;
    }
    if (p->dtype == FCM_I8 && (p->C % 16 || p->K % 16)) {
        *err = "int8 kernels need channel counts that are multiples of 16 (16-byte vectors)";
        return FCM_ERR_UNSUPPORTED;
    }
    return FCM_OK;
}

bool variant_runs(const VariantDesc& v, const fcm_problem& p, std::string* why) {
    // the chunked matrix-core variants compiled for dilated 3x3 taps run the generalised
    // problems with that dilation (and multiplier 1), nothing else
    const bool dil_mmw = v.vkind == VK_DWPW_MMW && v.dil > 1;
    if (dil_mmw) {
        if (!prob_is_gen(p) || v.dtype != p.dtype || p.R != 3 || p.S != 3 ||
            prob_dil_h(p) != v.dil || prob_dil_w(p) != v.dil || prob_mult(p) != 1 ||
            v.stride != p.stride_h) {
            if (why) *why = "dilated matrix-core variant is for a 3x3 depthwise layer with its "
                            "dilation, multiplier 1, its stride and storage type";
            return false;
        }
        if (p.C % 64 != 0 || p.C > v.cmax) {
            if (why) *why = "chunked matrix-core variant needs C a multiple of 64 up to its "
                            "compiled channel count";
            return false;
        }
        const int Ho = conv_out(p.H, p.pad_h, prob_ext_h(p), p.stride_h);
        const int Wo = conv_out(p.W, p.pad_w, prob_ext_w(p), p.stride_w);
        if (sat_mul({p.N, p.H, p.W, p.C, 2}) >= ((int64_t)1 << 31) ||
            sat_mul({p.N, Ho, Wo, p.K, 2}) >= ((int64_t)1 << 31)) {
            if (why) *why = "matrix-core depthwise variant addresses whole tensors below 2 GiB";
            return false;
        }
        return true;
    }
    // the matrix-core variants compiled for a depth multiplier or another filter size run
    // the generalised problems with an undilated layer of that filter size and multiplier,
    // C * M intermediate channels in one pass
    if (v.vkind == VK_DWPW_MM && (v.mult > 1 || v.fs > 3)) {
        if (!prob_is_gen(p) || v.dtype != p.dtype || p.R != v.fs || p.S != v.fs ||
            prob_dil_h(p) != 1 || prob_dil_w(p) != 1 || prob_mult(p) != std::max(v.mult, 1) ||
            v.stride != p.stride_h) {
            if (why) *why = "matrix-core generalised variant is for an undilated depthwise layer "
                            "with its filter size and multiplier, its stride and storage type";
            return false;
        }
        if ((int64_t)p.C * std::max(v.mult, 1) > v.cc) {
            if (why) *why = "matrix-core generalised variant needs C * mult <= its channel chunk";
            return false;
        }
        const int Ho = conv_out(p.H, p.pad_h, v.fs, p.stride_h);
        const int Wo = conv_out(p.W, p.pad_w, v.fs, p.stride_w);
        if (sat_mul({p.N, p.H, p.W, p.C, 2}) >= ((int64_t)1 << 31) ||
            sat_mul({p.N, Ho, Wo, p.K, 2}) >= ((int64_t)1 << 31)) {
            if (why) *why = "matrix-core depthwise variant addresses whole tensors below 2 GiB";
            return false;
        }
        return true;
    }
    if (v.vkind == VK_DWPW_GEN || prob_is_gen(p)) {
        if (v.vkind != VK_DWPW_GEN || p.kind != FCM_KIND_DWPW || v.dtype != p.dtype) {
            if (why) *why = "variant is for another module kind, depthwise form or storage type";
            return false;
        }
        if (v.stride != p.stride_h || v.fs != p.R || v.fs != p.S || v.dil != prob_dil_h(p) ||
            v.mult != prob_mult(p)) {
            if (why) *why = "variant is compiled for another stride, filter size, dilation or "
                            "depth multiplier";
            return false;
        }
        // whole tensors through 32-bit buffer offsets (the output is bounded by the
        // padded input extent at stride 1)
        const int64_t e = p.dtype == FCM_F32 ? 4 : 2;
        if (sat_mul({p.N, p.H, p.W, p.C, e}) >= ((int64_t)1 << 31) ||
            sat_mul({p.N, (int64_t)p.H + 2 * p.pad_h, (int64_t)p.W + 2 * p.pad_w, p.K, e}) >=
                ((int64_t)1 << 31)) {
            if (why) *why = "generalised variant addresses whole tensors below 2 GiB";
            return false;
        }
        return true;
    }
    if (v.vkind == VK_PWPW_MM || p.kind == FCM_KIND_PWPW) {
        if (v.vkind != VK_PWPW_MM || p.kind != FCM_KIND_PWPW || v.dtype != p.dtype) {
            if (why) *why = "variant is for another module kind or storage type";
            return false;
        }
        if (p.C > v.cmax || p.K1 > v.k1) {
            if (why) *why = v.cmax == 64 ? "single-pass PW->PW variant takes at most 64 input "
                                           "and 64 intermediate channels"
                                         : "wide PW->PW variant stages at most its compiled "
                                           "input channel count";
            return false;
        }
        if (v.cmax > 64 && p.C <= 64 && p.K1 <= 64) {
            if (why) *why = "wide PW->PW variant is for more than 64 input or intermediate "
                            "channels (the single-pass kernel's case)";
            return false;
        }
        const int64_t M = sat_mul({p.N, p.H, p.W});
        if (sat_mul({M, p.C, 2}) >= ((int64_t)1 << 31) || sat_mul({M, p.K, 2}) >= ((int64_t)1 << 30)) {
            if (why) *why = "PW->PW variant addresses inputs below 2 GiB and outputs below 1 GiB";
            return false;
        }
        return true;
    }
    if (v.vkind == VK_DWPW_I8 || p.dtype == FCM_I8) {
        if (v.vkind != VK_DWPW_I8 || p.dtype != FCM_I8 || p.kind != FCM_KIND_DWPW) {
            if (why) *why = "variant is for another module kind or storage type";
            return false;
        }
        if (v.stride != p.stride_h) {
            if (why) *why = "variant is compiled for another stride";
            return false;
        }
        if (p.C > v.cmax) {
            if (why) *why = v.cmax == 64 ? "single-pass int8 variant takes at most 64 input channels"
                                         : "sliced int8 variant stages at most its compiled "
                                           "channel count of depthwise filters in LDS";
            return false;
        }
        if (v.cmax > 64 && p.C <= 64) {
            if (why) *why = "sliced int8 variant is for more than 64 input channels (one slice "
                            "is the single-pass kernel's case)";
            return false;
        }
        const int Ho = conv_out(p.H, p.pad_h, p.R, p.stride_h);
        const int Wo = conv_out(p.W, p.pad_w, p.S, p.stride_w);
        if (sat_mul({p.N, p.H, p.W, p.C}) >= ((int64_t)1 << 31) ||
            sat_mul({p.N, Ho, Wo, p.K}) >= ((int64_t)1 << 30)) {
            if (why) *why = "int8 variant addresses inputs below 2 GiB and outputs below 1 GiB";
            return false;
        }
        return true;
    }
    if (v.vkind == VK_PWDWPW_MM || p.kind == FCM_KIND_PWDWPW) {
        if (v.vkind != VK_PWDWPW_MM || p.kind != FCM_KIND_PWDWPW || v.dtype != p.dtype) {
            if (why) *why = "variant is for another module kind or storage type";
            return false;
        }
        if (v.stride != p.stride_h) {
            if (why) *why = "variant is compiled for another stride";
            return false;
        }
        if (p.C > v.cmax || p.K1 > v.k1 || p.K > v.kt) {
            if (why) *why = "PW->DW->PW variant holds at most its compiled input, expanded and "
                            "output channel counts";
            return false;
        }
        const int Ho = conv_out(p.H, p.pad_h, p.R, p.stride_h);
        const int Wo = conv_out(p.W, p.pad_w, p.S, p.stride_w);
        if (sat_mul({p.N, p.H, p.W, p.C, 2}) >= ((int64_t)1 << 31) ||
            sat_mul({p.N, Ho, Wo, p.K, 2}) >= ((int64_t)1 << 30)) {
            if (why) *why = "PW->DW->PW variant addresses inputs below 2 GiB and outputs below "
                            "1 GiB";
            return false;
        }
        return true;
    }
    if ((v.vkind == VK_PWDW_MM) != (p.kind == FCM_KIND_PWDW) || v.dtype != p.dtype) {
        if (why) *why = "variant is for another module kind or storage type";
        return false;
    }
    if (v.vkind == VK_PWDW_MM) {
        if (v.stride != p.stride_h) {
            if (why) *why = "variant is compiled for another stride";
            return false;
        }
        if (p.C > v.cmax) {
            if (why) *why = "PW->DW variant stages at most its compiled input channel count";
            return false;
        }
        const int Ho = conv_out(p.H, p.pad_h, p.R, p.stride_h);
        const int Wo = conv_out(p.W, p.pad_w, p.S, p.stride_w);
        if (sat_mul({p.N, p.H, p.W, p.C, 2}) >= ((int64_t)1 << 31) ||
            sat_mul({p.N, Ho, Wo, p.K1, 2}) >= ((int64_t)1 << 30)) {
            if (why) *why = "PW->DW variant addresses inputs below 2 GiB and outputs below 1 GiB";
            return false;
        }
        return true;
    }
    const int want = p.kind == FCM_KIND_B2B ? VK_B2B : (p.dtype == FCM_F32 ? VK_DWPW32 : VK_DWPW);
    const int kind = (v.vkind == VK_DWPW_MM || v.vkind == VK_DWPW_MMW || v.vkind == VK_DWPW_WS ||
                      v.vkind == VK_DWPW_WSL)
                         ? VK_DWPW
                     : v.vkind == VK_B2B_MM                           ? VK_B2B
                                                                      : v.vkind;
    if (kind != want || v.dtype != p.dtype) {
        if (why) *why = "variant is for another module kind or storage type";
        return false;
    }
    if (v.stride != p.stride_h) {
        if (why) *why = "variant is compiled for another stride";
        return false;
    }
    if (v.wres && v.vkind == VK_DWPW && p.C > v.cc) {
        if (why) *why = "register-resident pointwise weights need C <= channel chunk";
        return false;
    }
    if (v.vkind == VK_B2B_MM && (p.C > 64 || p.K1 > 64 || p.K > 64)) {
        if (why) *why = "matrix-core back-to-back variant takes at most 64 channels per layer";
        return false;
    }
    if (v.vkind == VK_DWPW_WS && p.C != v.cc) {
        if (why) *why = "register-resident wide variant is compiled for exactly its channel "
                        "count";
        return false;
    }
    if (v.vkind == VK_DWPW_MM || v.vkind == VK_B2B_MM || v.vkind == VK_DWPW_MMW ||
        v.vkind == VK_DWPW_WS || v.vkind == VK_DWPW_WSL) {
        if (v.vkind == VK_DWPW_MM && p.C > v.cc) {
            if (why) *why = "matrix-core depthwise variant needs C <= its channel chunk";
            return false;
        }
        if (v.cmax > 0 && p.C > v.cmax) {
            if (why) *why = "wide matrix-core variant keeps at most its compiled channel count "
                            "of depthwise filters in LDS";
            return false;
        }
        if ((v.vkind == VK_DWPW_MMW || v.vkind == VK_DWPW_WSL) && p.C % 64 != 0) {
            if (why) *why = "chunked matrix-core variant needs C a multiple of 64";
            return false;
        }
        const int Ho = conv_out(p.H, p.pad_h, p.R, p.stride_h);
        const int Wo = conv_out(p.W, p.pad_w, p.S, p.stride_w);
        const int64_t e = p.dtype == FCM_F32 ? 4 : 2;
        if (sat_mul({p.N, p.H, p.W, p.C, e}) >= ((int64_t)1 << 31) ||
            sat_mul({p.N, Ho, Wo, p.K, e}) >= ((int64_t)1 << 31)) {
            if (why) *why = "matrix-core depthwise variant addresses whole tensors below 2 GiB";
            return false;
        }
    }
    if (v.vkind == VK_B2B && p.K1 > v.k1) {
        if (why) *why = "variant is compiled for fewer intermediate channels";
        return false;
    }
    return true;
}

namespace {

struct Estimate {
    double t_us;      // time model (see finish_time)
    int64_t pred;     // bytes requested from the memory hierarchy
    double waste;     // arithmetic done beyond the module's own (recompute, padding)
    double gma;       // pages' Eq.-style estimate (inf when infeasible)
    int wgs_per_cu;
    int num_tiles;
    int grid;
    bool feasible;
    // the time model's terms, seconds: compulsory HBM bytes, bytes requested from the
    // on-chip caches, matrix-core work as executed, vector work; fraction of CUs busy
    double t_hbm, t_l2, t_mat, t_vec, busy;
};

// The time model: the roofline terms of a variant (each at the machine's peak rate) and the
// fraction of the CUs its tiles keep busy, scaled to what the kernels achieve.
void finish_time(Estimate& r, double t_hbm, double t_l2, double t_mat, double t_vec,
                 double busy) {
    r.t_hbm = t_hbm;
    r.t_l2 = t_l2;
    r.t_mat = t_mat;
    r.t_vec = t_vec;
    r.busy = busy;
    // Calibrated on MI355X against every compiled variant of the fifteen benchmark
    // workloads (one measured table, graph-replayed launches streaming from HBM): a launch
    // costs a fixed ~4 us (prologue, pipeline fill and drain, launch spacing) plus its
    // slowest term at the fraction of the peak rate these issue- and latency-bound kernels
    // reach -- HBM 50%, cache requests 20% (of the 4x-HBM rate the terms assume), matrix
    // cores 20%, vector ALUs 15%.  With these factors the cheapest modelled variant is the
    // measured fastest on all fifteen workloads.
    constexpr double kFixedUs = 4.0, kHbm = 0.5, kL2 = 0.2, kMat = 0.2, kVec = 0.15;
    r.t_us = kFixedUs + std::max(std::max(t_hbm / kHbm, t_l2 / kL2),
                                 std::max(t_mat / kMat, t_vec / kVec)) /
                            std::max(busy, 1e-9) * 1e6;
}

// Modelled HBM bytes of a run: its compulsory bytes, plus its filters fetched once per XCD
// (each XCD's L2 serves that XCD's further re-reads of them; the kernels' input-window
// overlaps and K-tile re-reads are served by the L2 the same way).
int64_t modelled_hbm(int64_t alg, int64_t filters, const fcm_device_spec& d) {
    return alg + (int64_t)std::max(d.num_xcds - 1, 0) * filters;
}

// The plan's fuse flag: the fused module's modelled HBM bytes below the layer-by-layer
// kernels' (which also write the intermediate and read it back).  The FusePlanner
// equations count every tile's requests to global memory, re-reads included; on gfx950
// those re-reads hit the XCD's 4 MB L2, so the equations' figures are reported
// (gma_paper_*) but the flag follows the bytes that reach HBM.
int fuse_flag(int64_t alg_fused, int64_t alg_unfused, int64_t filters,
              const fcm_device_spec& d) {
    return modelled_hbm(alg_fused, filters, d) < modelled_hbm(alg_unfused, filters, d) ? 1 : 0;
}

Estimate estimate(const VariantDesc& v, const fcm_problem& p, const fcm_device_spec& d, int Ho,
                  int Wo) {
    Estimate r{};
    const int e = elem_bytes(p.dtype);
    const int lds = variant_lds_bytes(v);
    int vg = variant_vgpr_estimate(v);
    vg = (vg + 7) / 8 * 8;
    // workgroups per CU: a workgroup puts waves/4 waves on each of the 4 SIMDs
    const int wps = std::max(v.waves / 4, 1);
    int occ_lds = lds > 0 ? d.lds_bytes_per_cu / lds : 8;
    int occ_vgpr = std::max(d.vgprs_per_simd_lane / std::max(vg, 1), v.occ) / wps;
    int occ = std::min(std::min(occ_lds, occ_vgpr), d.max_waves_per_simd / wps);
    // the workgroups per CU the kernel's register allocation was tuned for
    if (v.vkind == VK_DWPW_MM || v.vkind == VK_B2B_MM || v.vkind == VK_DWPW_MMW ||
        v.vkind == VK_DWPW_WS || v.vkind == VK_DWPW_WSL)
        occ = std::min(occ, std::max(v.occ / wps, 1));
    if (lds > d.lds_bytes_per_wg) occ = 0;
    r.wgs_per_cu = occ;
    const int tiles_h = (int)cdiv(Ho, v.th), tiles_w = (int)cdiv(Wo, v.tw);
    const int64_t ptiles = (int64_t)p.N * tiles_h * tiles_w;
    const int ktiles = (int)cdiv(p.K, v.kt);
    r.num_tiles = (int)std::min<int64_t>(ptiles * ktiles, INT32_MAX);
    const int64_t grid = persistent_grid(ptiles, ktiles, (int64_t)d.num_cus * std::max(occ, 1));
    r.grid = (int)grid;

    // (window extent from the problem: a dilated layer on a variant compiled for it)
    const int64_t halo = halo_pixels(Ho, Wo, p.H, p.W, v.th, v.tw, p.stride_h, p.pad_h, p.pad_w,
                                     prob_ext_h(p), prob_ext_w(p));
    const int64_t x_reads = halo * p.N * p.C * e * ktiles;
    const int64_t y_bytes = (int64_t)p.N * Ho * Wo * p.K * e;
    // (first-layer outputs: K1 for B2B, C * mult for DW->PW)
    const int n1 = p.kind == FCM_KIND_B2B ? p.K1 : p.C * prob_mult(p);
    const int64_t w1_bytes =
        (int64_t)(p.kind == FCM_KIND_B2B ? (int64_t)p.K1 * 9 * p.C : (int64_t)p.R * p.S * n1) * e;
    const int64_t w2_slice = (int64_t)std::min(v.kt, p.K) * n1 * e;
    const int64_t epi = (int64_t)4 * 2 * (n1 + v.kt);
    int64_t w_reads;
    if (v.vkind == VK_B2B) {
        // 3x3 filters are streamed for every tile, 1x1 filters stay in registers
        w_reads = (int64_t)r.num_tiles * w1_bytes + grid * (w2_slice + epi);
    } else if (v.wres || v.vkind == VK_DWPW_MM) {
        w_reads = grid * (w2_slice + w1_bytes + epi);
    } else {
        w_reads = (int64_t)r.num_tiles * (w2_slice + w1_bytes) + grid * epi;
    }
    r.pred = x_reads + y_bytes + w_reads;
    // redundant work: the first layer is recomputed once per output-channel tile
    // (no redundancy at all with a single tile, as the DWPW module promises) and
    // channels the variant is compiled for but the problem lacks are computed as 0
    r.waste = (double)ktiles * (v.vkind == VK_B2B ? (double)v.k1 / p.K1 : 1.0) *
              ((double)tiles_h * v.th * tiles_w * v.tw) / ((double)Ho * Wo);

    // Roofline time: the slowest of compulsory HBM traffic, traffic requested from
    // the on-chip caches (modelled at 4x HBM), matrix-core work and vector work, each
    // with the variant's redundancy; divided by the fraction of CUs the grid covers.
    const double P = (double)p.N * Ho * Wo;
    const double pad_px = (double)tiles_h * v.th * tiles_w * v.tw / ((double)Ho * Wo);
    const double alg = (double)p.N * p.H * p.W * p.C * e + (double)y_bytes + (double)w1_bytes +
                       (double)p.K * n1 * e;
    // vector work in lane-operations per output pixel (fma + clamp + conversion per
    // epilogue value; 9 multiply-adds per depthwise value on the vector path; 5 mask
    // operations per value when the depthwise matrix operand is rebuilt each use);
    // matrix work as executed (the block-diagonal depthwise product runs at 1/16 of
    // the dense rate: 5 16x16x32 instructions per 16 channels x 16 pixels)
    const double lane_ops_per_s = d.valu_f32_flops / 2.0;
    double t_mat, t_vec;
    const double epi_ops = 3.0 * ((double)n1 * ktiles + p.K);
    if (v.vkind == VK_B2B || v.vkind == VK_B2B_MM) {
        t_mat = 2.0 * P * pad_px * ((double)v.k1 * 9 * p.C * ktiles + (double)v.k1 * p.K) /
                d.mfma_f16_flops;
        t_vec = P * pad_px * epi_ops / lane_ops_per_s;
    } else if (v.vkind == VK_DWPW) {
        t_mat = 2.0 * P * pad_px * (double)p.C * p.K / d.mfma_f16_flops;
        t_vec = P * pad_px * (9.0 * p.C * ktiles + epi_ops) / lane_ops_per_s;
    } else if (v.vkind == VK_DWPW_MMW || v.vkind == VK_DWPW_WSL) {
        // block-diagonal depthwise products (320 flop-equivalents per channel and
        // pixel) recomputed for every K tile
        t_mat = P * pad_px * (2.0 * p.C * p.K + 320.0 * p.C * ktiles) / d.mfma_f16_flops;
        t_vec = P * pad_px * (epi_ops + 1.25 * p.C * ktiles) / lane_ops_per_s;
    } else if (v.vkind == VK_DWPW_WS) {
        // the block-diagonal depthwise products run once per pixel and K tile
        t_mat = P * pad_px * (2.0 * p.C * p.K + 320.0 * p.C * ktiles) / d.mfma_f16_flops;
        t_vec = P * pad_px * epi_ops / lane_ops_per_s;
    } else if (v.vkind == VK_DWPW_I8) {
        // int8 matrix rate is twice the fp16 one; the block-diagonal depthwise product is
        // 3 16x16x64 instructions per 16 channels x 16 pixels (384 op-equivalents per
        // channel and pixel), the pointwise reduction padded to 64 channels; vector work:
        // about five operations per requantized value
        // (the reduction is padded to whole 64-channel slices)
        const double c64 = 64.0 * (double)cdiv(p.C, 64);
        t_mat = P * pad_px * (2.0 * c64 * p.K + 384.0 * c64 * ktiles) / (2.0 * d.mfma_f16_flops);
        t_vec = P * pad_px * 5.0 * ((double)n1 * ktiles + p.K) / lane_ops_per_s;
    } else if (v.vkind == VK_DWPW_MM) {
        // (64 flop-equivalents per intermediate channel and pixel for each of the ntp
        // instructions per 16 channels x 16 pixels: 5 for 3x3, 3 with multiplier 2, 13 for
        // 5x5)
        const int fs = v.fs > 0 ? v.fs : 3;
        const int ntp = v.mult > 1 ? 3 : fs * (fs / 2) + (fs + 1) / 2;
        t_mat = P * pad_px * (2.0 * n1 * p.K + 64.0 * ntp * v.cc * ktiles) / d.mfma_f16_flops;
        // operand expansion when a wave owns several depthwise channel blocks
        t_vec = P * pad_px * (epi_ops + (v.cc > 64 ? 1.25 * v.cc * ktiles : 0.0)) /
                lane_ops_per_s;
    } else {
        // fp32: pointwise products on the fp32 matrix instruction, depthwise on the VALU
        t_mat = 2.0 * P * pad_px * (double)p.C * p.K / d.mfma_f32_flops;
        t_vec = P * pad_px * (9.0 * p.C * ktiles + epi_ops) / lane_ops_per_s;
    }
    const double t_hbm = alg / d.hbm_bytes_per_s;
    const double t_l2 = (double)r.pred / (4.0 * d.hbm_bytes_per_s);
    const double busy = std::min(1.0, (double)r.num_tiles / d.num_cus);
    finish_time(r, t_hbm, t_l2, t_mat, t_vec, busy);

    // Eq.-style estimate (FCM paper Sec. IV): DW->PW constructed from Eq. 2 and 3.
    const double overlap = eq1_overlap(p.W, p.H, v.tw * p.stride_w, v.th * p.stride_h, prob_ext_h(p),
                                       p.stride_h);
    const double ifm = (double)p.N * p.H * p.W * p.C * e;
    const double w_pw = (double)p.K * n1 * e;
    const double w_pw_tile = (double)std::min(v.kt, p.K) * n1 * e;
    const double ofm = (double)y_bytes;
    const double ofm_tile = (double)v.th * v.tw * std::min(v.kt, p.K) * e;
    const bool fits = lds <= d.lds_bytes_per_wg && occ > 0;
    const bool enough = r.num_tiles >= d.num_cus;
    r.feasible = fits && enough;
    if (!fits || !enough) {
        r.gma = INFINITY;
    } else {
        r.gma = (2.0 * p.C * overlap * p.N * e + ifm) * ceil(w_pw / w_pw_tile) +
                ceil(ofm / ofm_tile) * (w_pw + (double)w1_bytes) + ofm;
    }
    return r;
}

// PW->DW module (FCM paper Sec. II-D, Fig. 3(b); Eq. 4).  The pointwise layer runs on
// every tile's whole input window (clipped to the image), so the intermediate on the
// windows' overlap is computed once per tile that needs it; the depthwise layer runs
// once per output pixel.
Estimate estimate_pwdw(const VariantDesc& v, const fcm_problem& p, const fcm_device_spec& d,
                       int Ho, int Wo) {
    Estimate r{};
    const int e = elem_bytes(p.dtype);
    const int lds = variant_lds_bytes(v);
    int vg = (variant_vgpr_estimate(v) + 7) / 8 * 8;
    const int wps = std::max(v.waves / 4, 1);
    const int occ_lds = lds > 0 ? d.lds_bytes_per_cu / lds : 8;
    const int occ_vgpr = std::max(d.vgprs_per_simd_lane / std::max(vg, 1), v.occ) / wps;
    int occ = std::min(std::min(occ_lds, occ_vgpr), d.max_waves_per_simd / wps);
    occ = std::min(occ, std::max(v.occ / wps, 1));
    if (lds > d.lds_bytes_per_wg) occ = 0;
    r.wgs_per_cu = occ;
    const int tiles_h = (int)cdiv(Ho, v.th), tiles_w = (int)cdiv(Wo, v.tw);
    const int64_t ptiles = (int64_t)p.N * tiles_h * tiles_w;
    const int ktiles = (int)cdiv(p.K1, v.kt);
    r.num_tiles = (int)std::min<int64_t>(ptiles * ktiles, INT32_MAX);
    const int64_t grid = persistent_grid(ptiles, ktiles, (int64_t)d.num_cus * std::max(occ, 1));
    r.grid = (int)grid;

    // input windows: the exact clipped footprint, once per channel slice
    const int64_t win = halo_pixels(Ho, Wo, p.H, p.W, v.th, v.tw, p.stride_h, p.pad_h, p.pad_w);
    const int64_t x_reads = win * p.N * p.C * e * ktiles;
    const int64_t y_bytes = (int64_t)p.N * Ho * Wo * p.K1 * e;
    const int kt = std::min(v.kt, p.K1);
    const int64_t w_slice = (int64_t)kt * p.C * e + 9LL * kt * e + 4LL * 4 * kt;
    r.pred = x_reads + y_bytes + grid * w_slice;
    // pointwise pixels computed per pixel of the intermediate (1 = no recomputation)
    r.waste = (double)win / ((double)p.H * p.W) *
              ((double)tiles_h * v.th * tiles_w * v.tw) / ((double)Ho * Wo);

    const double alg = (double)p.N * p.H * p.W * p.C * e + (double)y_bytes +
                       (double)p.K1 * p.C * e + 9.0 * p.K1 * e;
    // window pixels the pointwise layer runs on (each K slice for its own channels)
    const double pw_px = (double)win * p.N;
    const double out_px = (double)p.N * tiles_h * v.th * tiles_w * v.tw;
    const double c_pad = (double)cdiv(p.C, 32) * 32;
    // matrix work as executed: the pointwise product padded to 32 input channels, the
    // block-diagonal depthwise product (320 flop-equivalents per channel and pixel)
    const double t_mat = (pw_px * 2.0 * c_pad * p.K1 + out_px * 320.0 * p.K1) / d.mfma_f16_flops;
    // vector work: an epilogue (fma, clamp, conversion) per intermediate and output value
    const double t_vec = 3.0 * p.K1 * (pw_px + out_px) / (d.valu_f32_flops / 2.0);
    const double t_hbm = alg / d.hbm_bytes_per_s;
    const double t_l2 = (double)r.pred / (4.0 * d.hbm_bytes_per_s);
    const double busy = std::min(1.0, (double)r.num_tiles / d.num_cus);
    finish_time(r, t_hbm, t_l2, t_mat, t_vec, busy);

    // Eq. 4 as printed, plus the module's own output write (the OFMs are written once):
    // the PW input with its overlap (Eq. 1 over the input plane with the tile extents in
    // input pixels, times the PW input depth) once per weight tile of whichever layer
    // has more, PW filters once per output tile, DW filters once per spatial tile.
    const double overlap = eq1_overlap(p.W, p.H, v.tw * p.stride_w, v.th * p.stride_h, 3,
                                       p.stride_h);
    const double ifm = (double)p.N * p.H * p.W * p.C * e;
    const double w_pw = (double)p.K1 * p.C * e, w_pw_tile = (double)kt * p.C * e;
    const double w_dw = 9.0 * p.K1 * e, w_dw_tile = 9.0 * kt * e;
    const double ofm = (double)y_bytes, ofm_tile = (double)v.th * v.tw * kt * e;
    const bool fits = lds <= d.lds_bytes_per_wg && occ > 0;
    const bool enough = r.num_tiles >= d.num_cus;
    r.feasible = fits && enough;
    if (!r.feasible) {
        r.gma = INFINITY;
    } else {
        r.gma = (2.0 * p.C * overlap * p.N * e + ifm) *
                    std::max(ceil(w_pw / w_pw_tile), ceil(w_dw / w_dw_tile)) +
                ceil(ofm / ofm_tile) * w_pw +
                ceil((double)p.N * Ho * Wo / ((double)v.th * v.tw)) * w_dw + ofm;
    }
    return r;
}

// PW->DW->PW module (the three layers of an inverted-residual block): the PW->DW tiling
// (the expansion recomputed on every tile's input window, the depthwise layer once per
// output pixel) with all K1 expanded channels in one workgroup, then the projection on
// the depthwise tile.  No estimate for three layers is printed on the pages; the Eq.-style
// figure takes Eq. 4's form: the input with its overlap once (a single weight tile), the
// three layers' filters once per output tile, the output once.
void estimate_unfused_pwdw(const fcm_problem& p, int Ho, int Wo, int64_t* pred, double* gma);

Estimate estimate_pwdwpw(const VariantDesc& v, const fcm_problem& p, const fcm_device_spec& d,
                         int Ho, int Wo) {
    Estimate r{};
    const int e = elem_bytes(p.dtype);
    const int lds = variant_lds_bytes(v);
    const int vg = (variant_vgpr_estimate(v) + 7) / 8 * 8;
    const int wps = std::max((v.waves + 3) / 4, 1);
    const int occ_lds = lds > 0 ? d.lds_bytes_per_cu / lds : 8;
    const int occ_vgpr = std::max(d.vgprs_per_simd_lane / std::max(vg, 1), v.occ) / wps;
    int occ = std::min(std::min(occ_lds, occ_vgpr), d.max_waves_per_simd / wps);
    if (lds > d.lds_bytes_per_wg) occ = 0;
    r.wgs_per_cu = occ;
    const int tiles_h = (int)cdiv(Ho, v.th), tiles_w = (int)cdiv(Wo, v.tw);
    const int64_t ptiles = (int64_t)p.N * tiles_h * tiles_w;
    r.num_tiles = (int)std::min<int64_t>(ptiles, INT32_MAX);
    const int64_t grid = persistent_grid(ptiles, 1, (int64_t)d.num_cus * std::max(occ, 1));
    r.grid = (int)grid;

    const int64_t win = halo_pixels(Ho, Wo, p.H, p.W, v.th, v.tw, p.stride_h, p.pad_h, p.pad_w);
    const int64_t x_reads = win * p.N * p.C * e;
    const int64_t y_bytes = (int64_t)p.N * Ho * Wo * p.K * e;
    const int64_t w_all = ((int64_t)p.K1 * p.C + 9LL * p.K1 + (int64_t)p.K * p.K1) * e +
                          4LL * 2 * (2 * p.K1 + p.K);
    r.pred = x_reads + y_bytes + grid * w_all;
    r.waste = (double)win / ((double)p.H * p.W) *
              ((double)tiles_h * v.th * tiles_w * v.tw) / ((double)Ho * Wo) *
              ((double)v.k1 / p.K1);

    const double alg = (double)p.N * p.H * p.W * p.C * e + (double)y_bytes + (double)w_all;
    const double pw_px = (double)win * p.N;
    const double out_px = (double)p.N * tiles_h * v.th * tiles_w * v.tw;
    const double c_pad = (double)cdiv(p.C, 32) * 32;
    // matrix work as executed: the expansion padded to 32 input channels over the
    // window, the block-diagonal depthwise product (320 flop-equivalents per channel and
    // pixel), the projection over the held channels and its 16-channel output blocks
    const double t_mat = (pw_px * 2.0 * c_pad * v.k1 + out_px * 320.0 * v.k1 +
                          out_px * 2.0 * v.k1 * (double)cdiv(p.K, 16) * 16) /
                         d.mfma_f16_flops;
    const double t_vec = 3.0 * ((double)v.k1 * (pw_px + out_px) + (double)p.K * out_px) /
                         (d.valu_f32_flops / 2.0);
    const double t_hbm = alg / d.hbm_bytes_per_s;
    const double t_l2 = (double)r.pred / (4.0 * d.hbm_bytes_per_s);
    const double busy = std::min(1.0, (double)r.num_tiles / d.num_cus);
    finish_time(r, t_hbm, t_l2, t_mat, t_vec, busy);

    const double overlap = eq1_overlap(p.W, p.H, v.tw * p.stride_w, v.th * p.stride_h, 3,
                                       p.stride_h);
    const double ifm = (double)p.N * p.H * p.W * p.C * e;
    const double w1 = (double)p.K1 * p.C * e, w2 = 9.0 * p.K1 * e, w3 = (double)p.K * p.K1 * e;
    const double ofm = (double)y_bytes, ofm_tile = (double)v.th * v.tw * p.K * e;
    const bool fits = lds <= d.lds_bytes_per_wg && occ > 0;
    const bool enough = r.num_tiles >= d.num_cus;
    r.feasible = fits && enough;
    r.gma = r.feasible ? (2.0 * p.C * overlap * p.N * e + ifm) +
                             ceil(ofm / ofm_tile) * (w1 + w2 + w3) + ofm
                       : INFINITY;
    return r;
}

// Layer-by-layer PW->DW->PW: the expansion over every input pixel writes t1, the
// depthwise kernel reads it and writes t2, the projection reads t2 (and the input again
// for the shortcut) and writes the output.  Bytes with the baseline kernels' tilings,
// and Eq. 2 (expansion) + Eq. 3 (depthwise) + Eq. 2 (projection).
void estimate_unfused_pwdwpw(const fcm_problem& p, int Ho, int Wo, int64_t* pred, double* gma) {
    int64_t pu = 0;
    double gu = 0;
    // the first two layers are the PW->DW module's layer-by-layer pair with its output
    // (the depthwise layer's K1 channels) as the intermediate t2
    fcm_problem q = p;
    q.kind = FCM_KIND_PWDW;
    q.K = p.K1;
    estimate_unfused_pwdw(q, Ho, Wo, &pu, &gu);
    const int e = elem_bytes(p.dtype);
    const int64_t t2 = (int64_t)p.N * Ho * Wo * p.K1 * e;
    const int64_t y_bytes = (int64_t)p.N * Ho * Wo * p.K * e;
    const int64_t w3 = (int64_t)p.K * p.K1 * e;
    const int64_t m = (int64_t)p.N * Ho * Wo;
    const int mt = lbl::PW_MT16, kt = lbl::PW_KT16;
    const int64_t res = p.residual ? (int64_t)p.N * p.H * p.W * p.C * e : 0;
    const int64_t third = t2 * cdiv(p.K, kt) + cdiv(m, mt) * w3 + y_bytes + res;
    *pred = pu + third;
    const double g3 = ceil((double)w3 / ((double)std::min(kt, p.K) * p.K1 * e)) * (double)t2 +
                      (double)y_bytes + (double)res +
                      ceil((double)y_bytes / ((double)mt * std::min(kt, p.K) * e)) * (double)w3;
    *gma = gu + g3;
}

// PW->PW module: tiles of th x 16 consecutive pixels, both layers on the matrix cores, the
// first layer recomputed once per 64-channel output tile; Eq. 2 for each layer with the
// intermediate removed from the global-memory accesses (FCM paper Sec. IV-B).
// DW->PW module with a generalised depthwise layer (filter FS x FS, dilation D, depth
// multiplier M; PyTorch forum "Using optimised depthwise convolutions").  The same
// tiling as the plain module, with the window extent (FS-1)*D + 1 in place of 3 and
// C*M intermediate channels; the depthwise layer runs on the vector ALU (FS*FS
// multiply-adds per intermediate value) once per output-channel tile, the pointwise
// layer on the matrix cores.  Filters are streamed per tile and chunk.
Estimate estimate_gen(const VariantDesc& v, const fcm_problem& p, const fcm_device_spec& d,
                      int Ho, int Wo) {
    Estimate r{};
    const int e = elem_bytes(p.dtype);
    const int lds = variant_lds_bytes(v);
    int vg = (variant_vgpr_estimate(v) + 7) / 8 * 8;
    // workgroups per CU: a workgroup of NG channel groups puts NG waves on each SIMD
    const int ng = std::max(v.waves / 4, 1);
    int occ = std::min(std::min(lds > 0 ? d.lds_bytes_per_cu / lds : 8,
                                std::max(d.vgprs_per_simd_lane / std::max(vg, 1), v.occ) / ng),
                       d.max_waves_per_simd / ng);
    if (lds > d.lds_bytes_per_wg) occ = 0;
    r.wgs_per_cu = occ;
    const int tiles_h = (int)cdiv(Ho, v.th), tiles_w = (int)cdiv(Wo, v.tw);
    const int64_t ptiles = (int64_t)p.N * tiles_h * tiles_w;
    const int ktiles = (int)cdiv(p.K, v.kt);
    r.num_tiles = (int)std::min<int64_t>(ptiles * ktiles, INT32_MAX);
    const int64_t grid = persistent_grid(ptiles, ktiles, (int64_t)d.num_cus * std::max(occ, 1));
    r.grid = (int)grid;
    const int ext_h = prob_ext_h(p), ext_w = prob_ext_w(p);
    const int64_t halo =
        halo_pixels(Ho, Wo, p.H, p.W, v.th, v.tw, p.stride_h, p.pad_h, p.pad_w, ext_h, ext_w);
    const int64_t y_bytes = (int64_t)p.N * Ho * Wo * p.K * e;
    const int64_t w1_bytes = (int64_t)p.R * p.S * p.K1 * e;
    const int64_t w2_slice = (int64_t)std::min(v.kt, p.K) * p.K1 * e;
    const int64_t epi = (int64_t)4 * 2 * (p.K1 + v.kt);
    r.pred = halo * p.N * p.C * e * ktiles + y_bytes + (int64_t)r.num_tiles * (w2_slice + w1_bytes) +
             grid * epi;
    const double pad_px = (double)tiles_h * v.th * tiles_w * v.tw / ((double)Ho * Wo);
    r.waste = (double)ktiles * pad_px;
    const double P = (double)p.N * Ho * Wo;
    const double alg = (double)p.N * p.H * p.W * p.C * e + (double)y_bytes + (double)w1_bytes +
                       (double)p.K * p.K1 * e;
    const double lane_ops_per_s = d.valu_f32_flops / 2.0;
    const double t_mat = 2.0 * P * pad_px * (double)p.K1 * p.K / d.mfma_f16_flops;
    const double t_vec = P * pad_px *
                         ((double)p.R * p.S * p.K1 * ktiles + 3.0 * ((double)p.K1 * ktiles + p.K)) /
                         lane_ops_per_s;
    const double t_hbm = alg / d.hbm_bytes_per_s;
    const double t_l2 = (double)r.pred / (4.0 * d.hbm_bytes_per_s);
    const double busy = std::min(1.0, (double)r.num_tiles / d.num_cus);
    finish_time(r, t_hbm, t_l2, t_mat, t_vec, busy);
    // each (tile, channel chunk) step of this kernel also pays a fixed latency (two
    // barriers and its loads' round trip, ~1 us measured): the chunks of a workgroup's
    // tiles run one after another
    // (the channel groups of a workgroup take a tile's chunks in turn)
    const int64_t steps =
        cdiv(r.num_tiles, std::max<int64_t>(grid, 1)) * cdiv(cdiv(p.C, v.cc), ng);
    r.t_us += 1.0 * (double)steps;
    // constructed DW->PW estimate (Eq. 1 with the window extent as the filter size)
    const double overlap = eq1_overlap(p.W, p.H, v.tw * p.stride_w, v.th * p.stride_h, ext_h,
                                       p.stride_h);
    const double ifm = (double)p.N * p.H * p.W * p.C * e;
    const double w_pw = (double)p.K * p.K1 * e;
    const double ofm_tile = (double)v.th * v.tw * std::min(v.kt, p.K) * e;
    const bool fits = lds <= d.lds_bytes_per_wg && occ > 0;
    const bool enough = r.num_tiles >= d.num_cus;
    r.feasible = fits && enough;
    r.gma = r.feasible ? (2.0 * p.C * overlap * p.N * e + ifm) * ceil(w_pw / (double)w2_slice) +
                             ceil((double)y_bytes / ofm_tile) * (w_pw + (double)w1_bytes) +
                             (double)y_bytes
                       : INFINITY;
    return r;
}

// Layer-by-layer pair for the generalised module: the depthwise kernel with the
// variant's chunk (input once per tile, filters once per tile and chunk, intermediate
// written), then the pointwise baseline over C*M channels.  Eq. 3 + Eq. 2.
void estimate_unfused_gen(const fcm_problem& p, int cc, int Ho, int Wo, int64_t* pred,
                          double* gma) {
    const int e = elem_bytes(p.dtype);
    const int th = lbl::DWG_TH, tw = lbl::DWG_TW;
    const int64_t t_bytes = (int64_t)p.N * Ho * Wo * p.K1 * e;
    const int64_t y_bytes = (int64_t)p.N * Ho * Wo * p.K * e;
    const int64_t w2 = (int64_t)p.K * p.K1 * e;
    const int ext_h = prob_ext_h(p), ext_w = prob_ext_w(p);
    const int64_t halo =
        halo_pixels(Ho, Wo, p.H, p.W, th, tw, p.stride_h, p.pad_h, p.pad_w, ext_h, ext_w);
    const int64_t tiles = (int64_t)p.N * cdiv(Ho, th) * cdiv(Wo, tw);
    const int64_t first = halo * p.N * p.C * e +
                          tiles * cdiv(p.C, cc) * (int64_t)p.R * p.S * cc * prob_mult(p) * e +
                          t_bytes;
    const int64_t m = (int64_t)p.N * Ho * Wo;
    const int64_t second =
        t_bytes * cdiv(p.K, lbl::PW_KT16) + cdiv(m, lbl::PW_MT16) * w2 + y_bytes;
    *pred = first + second;
    const double ifm = (double)p.N * p.H * p.W * p.C * e;
    const double overlap = eq1_overlap(p.W, p.H, tw * p.stride_w, th * p.stride_h, ext_h,
                                       p.stride_h);
    const double w1 = (double)p.R * p.S * p.K1 * e;
    const double g1 = 2.0 * p.C * overlap * p.N * e + ifm + (double)t_bytes +
                      ceil((double)p.N * Ho * Wo / (th * tw)) * w1;
    const double kt2 = (double)std::min(lbl::PW_KT16, p.K);
    const double g2 = ceil(w2 / (kt2 * p.K1 * e)) * t_bytes + (double)y_bytes +
                      ceil((double)y_bytes / ((double)lbl::PW_MT16 * kt2 * e)) * w2;
    *gma = g1 + g2;
}

Estimate estimate_pwpw(const VariantDesc& v, const fcm_problem& p, const fcm_device_spec& d) {
    Estimate r{};
    const int e = elem_bytes(p.dtype);
    const int lds = variant_lds_bytes(v);
    const int vg = (variant_vgpr_estimate(v) + 7) / 8 * 8;
    const int occ_lds = lds > 0 ? d.lds_bytes_per_cu / lds : 8;
    const int occ_vgpr = std::max(d.vgprs_per_simd_lane / std::max(vg, 1), v.occ);
    int occ = std::min(std::min(occ_lds, occ_vgpr), d.max_waves_per_simd);
    occ = std::min(occ, std::max(v.occ, 1));
    if (lds > d.lds_bytes_per_wg) occ = 0;
    r.wgs_per_cu = occ;
    const int64_t M = (int64_t)p.N * p.H * p.W;
    const int mp = v.th * v.tw;
    const int64_t ptiles = cdiv(M, mp);
    const int ktiles = (int)cdiv(p.K, v.kt);
    r.num_tiles = (int)std::min<int64_t>(ptiles * ktiles, INT32_MAX);
    const int64_t grid = persistent_grid(ptiles, ktiles, (int64_t)d.num_cus * std::max(occ, 1));
    r.grid = (int)grid;
    const int64_t x_bytes = M * p.C * e, y_bytes = M * p.K * e;
    const int64_t w_bytes = ((int64_t)p.K1 * p.C + (int64_t)std::min(v.kt, p.K) * p.K1) * e;
    // (the single-pass build keeps its filters in registers for the workgroup's whole
    // run; the wide build reads both layers' filters again for every tile)
    const bool wide = v.cmax > 64;
    r.pred = x_bytes * ktiles + y_bytes +
             (wide ? (int64_t)r.num_tiles : grid) * (w_bytes + 4LL * 2 * (p.K1 + v.kt));
    r.waste = (double)ktiles * ((double)ptiles * mp / (double)M);
    const double alg = (double)x_bytes + y_bytes + ((double)p.K1 * p.C + (double)p.K * p.K1) * e;
    const double c_pad = wide ? 32.0 * cdiv(p.C, 32) : 64.0;
    const double k1_pad = wide ? 64.0 * cdiv(p.K1, 64) : 64.0;
    const double t_mat = (double)ptiles * mp *
                         (2.0 * c_pad * k1_pad * ktiles + 2.0 * k1_pad * std::min(v.kt, p.K) * ktiles) /
                         d.mfma_f16_flops;
    const double t_vec = (double)ptiles * mp * 3.0 * (k1_pad * ktiles + p.K) /
                         (d.valu_f32_flops / 2.0);
    const double busy = std::min(1.0, (double)r.num_tiles / d.num_cus);
    finish_time(r, alg / d.hbm_bytes_per_s, (double)r.pred / (4.0 * d.hbm_bytes_per_s), t_mat,
                t_vec, busy);
    const bool fits = lds <= d.lds_bytes_per_wg && occ > 0;
    r.feasible = fits && r.num_tiles >= d.num_cus;
    if (!r.feasible) {
        r.gma = INFINITY;
    } else {
        // first layer's input once per weight tile of the second layer, the first
        // layer's filters once per output tile, the second layer's likewise, output once
        const double w1 = (double)p.K1 * p.C * e, w2 = (double)p.K * p.K1 * e;
        const double ofm_tile = (double)mp * std::min(v.kt, p.K) * e;
        r.gma = (double)x_bytes * ceil(w2 / ((double)std::min(v.kt, p.K) * p.K1 * e)) +
                ceil((double)y_bytes / ofm_tile) * (w1 + w2) + (double)y_bytes;
    }
    return r;
}

// Layer-by-layer PW->DW: the 1x1 kernel over every input pixel writes the intermediate,
// the depthwise kernel reads it back.  Bytes with the baseline kernels' tilings, and
// Eq. 2 (PW) + Eq. 3 (DW).
void estimate_unfused_pwdw(const fcm_problem& p, int Ho, int Wo, int64_t* pred, double* gma) {
    const int e = elem_bytes(p.dtype);
    const int64_t x_bytes = (int64_t)p.N * p.H * p.W * p.C * e;
    const int64_t t_bytes = (int64_t)p.N * p.H * p.W * p.K1 * e;
    const int64_t y_bytes = (int64_t)p.N * Ho * Wo * p.K1 * e;
    const int64_t w_pw = (int64_t)p.K1 * p.C * e;
    const int mt = lbl::PW_MT16, kt = lbl::PW_KT16;
    const int64_t m = (int64_t)p.N * p.H * p.W;
    const int64_t first = x_bytes * cdiv(p.K1, kt) + cdiv(m, mt) * w_pw + t_bytes;
    const int th = lbl::DW_TH, tw = lbl::DW_TW, cc = lbl::DW_CC16;
    const int64_t halo = halo_pixels(Ho, Wo, p.H, p.W, th, tw, p.stride_h, p.pad_h, p.pad_w);
    const int64_t tiles_px = (int64_t)p.N * cdiv(Ho, th) * cdiv(Wo, tw);
    const int64_t second = halo * p.N * p.K1 * e + tiles_px * cdiv(p.K1, cc) * 9LL * cc * e +
                           y_bytes;
    *pred = first + second;
    const double g1 = ceil((double)w_pw / ((double)std::min(kt, p.K1) * p.C * e)) * x_bytes +
                      (double)t_bytes +
                      ceil((double)t_bytes / ((double)mt * std::min(kt, p.K1) * e)) * w_pw;
    const double overlap = eq1_overlap(p.W, p.H, tw * p.stride_w, th * p.stride_h, 3, p.stride_h);
    const double g2 = 2.0 * p.K1 * overlap * p.N * e + (double)t_bytes + (double)y_bytes +
                      ceil((double)p.N * Ho * Wo / (double)(th * tw)) * 9.0 * p.K1 * e;
    *gma = g1 + g2;
}

// Layer-by-layer bytes with the baseline kernels' fixed tilings, and the pages'
// Eq. 3 (first layer) + Eq. 2 (1x1 layer) estimate.
void estimate_unfused(const fcm_problem& p, const fcm_device_spec& d, int Ho, int Wo,
                      int64_t* pred, double* gma) {
    const int e = elem_bytes(p.dtype);
    const int n1 = p.kind == FCM_KIND_B2B ? p.K1 : p.C;
    const int64_t t_bytes = (int64_t)p.N * Ho * Wo * n1 * e;
    const int64_t y_bytes = (int64_t)p.N * Ho * Wo * p.K * e;
    const int64_t w2 = (int64_t)p.K * n1 * e;
    int th, tw, l1_kt;
    if (p.kind == FCM_KIND_B2B) {
        th = lbl::CV_TH;
        tw = lbl::CV_TW;
        l1_kt = lbl::CV_KT;
    } else {
        th = lbl::DW_TH;
        tw = lbl::DW_TW;
        l1_kt = p.C;  // depthwise: channels split, no re-read of the input
    }
    const int64_t halo = halo_pixels(Ho, Wo, p.H, p.W, th, tw, p.stride_h, p.pad_h, p.pad_w);
    const int64_t l1_tiles_px = (int64_t)p.N * cdiv(Ho, th) * cdiv(Wo, tw);
    int64_t first;
    if (p.kind == FCM_KIND_B2B) {
        const int64_t kts = cdiv(p.K1, lbl::CV_KT);
        const int64_t w1 = (int64_t)p.K1 * 9 * p.C * e;
        first = halo * p.N * p.C * e * kts + l1_tiles_px * w1 + t_bytes;
    } else {
        const int cc = p.dtype == FCM_F32 ? lbl::DW_CC32 : lbl::DW_CC16;
        const int64_t chunks = cdiv(p.C, cc);
        first = halo * p.N * p.C * e + l1_tiles_px * chunks * 9LL * cc * e + t_bytes;
    }
    (void)l1_kt;
    const int mt = p.dtype == FCM_F32 ? lbl::PW_MT32 : lbl::PW_MT16;
    const int kt = p.dtype == FCM_F32 ? lbl::PW_KT32 : lbl::PW_KT16;
    const int64_t m = (int64_t)p.N * Ho * Wo;
    const int64_t pw_tiles_m = cdiv(m, mt), pw_tiles_k = cdiv(p.K, kt);
    const int64_t second = t_bytes * pw_tiles_k + pw_tiles_m * w2 + y_bytes;
    *pred = first + second;

    // Eq. 3 for the depthwise layer (or Eq. 2-style for the 3x3 conv) + Eq. 2.
    const double ifm = (double)p.N * p.H * p.W * p.C * e;
    const double overlap = eq1_overlap(p.W, p.H, tw * p.stride_w, th * p.stride_h, 3, p.stride_h);
    double g1;
    if (p.kind == FCM_KIND_B2B) {
        const double w1 = (double)p.K1 * 9 * p.C * e;
        g1 = (2.0 * p.C * overlap * p.N * e + ifm) * ceil((double)p.K1 / lbl::CV_KT) +
             (double)t_bytes + ceil((double)t_bytes / ((double)th * tw * lbl::CV_KT * e)) * w1;
    } else {
        g1 = 2.0 * p.C * overlap * p.N * e + ifm + (double)t_bytes +
             ceil((double)p.N * Ho * Wo / (double)(th * tw)) * 9.0 * p.C * e;
    }
    const double g2 = ceil((double)w2 / ((double)std::min(kt, p.K) * n1 * e)) * (double)t_bytes +
                      (double)y_bytes + ceil((double)y_bytes / ((double)mt * std::min(kt, p.K) * e)) *
                                            (double)w2;
    *gma = g1 + g2;
    (void)d;
}

}  // namespace

// FCM_LOG=1 in the environment: every candidate variant's estimate goes to stderr.
bool plan_log_enabled() {
    static const bool on = [] {
        const char* e = getenv("FCM_LOG");
        return e && *e && strcmp(e, "0") != 0;
    }();
    return on;
}

fcm_status plan_problem(const fcm_problem* p, const fcm_device_spec* spec, int forced,
                        fcm_plan_t* out, std::string* err) {
    if (!out) {
        *err = "plan output pointer is NULL";
        return FCM_ERR_INVALID_ARG;
    }
    fcm_status st = validate_problem(p, err);
    if (st != FCM_OK) return st;
    fcm_device_spec d;
    if (spec) {
        d = *spec;
    } else {
        default_spec(&d);
    }
    if (d.num_cus <= 0 || d.lds_bytes_per_cu <= 0 || d.lds_bytes_per_wg <= 0 ||
        d.vgprs_per_simd_lane <= 0 || d.max_waves_per_simd <= 0) {
        *err = "device spec has a non-positive field";
        return FCM_ERR_INVALID_ARG;
    }
    const int Ho = conv_out(p->H, p->pad_h, prob_ext_h(*p), p->stride_h);
    const int Wo = conv_out(p->W, p->pad_w, prob_ext_w(*p), p->stride_w);

    int best = -1;
    Estimate be{};
    std::string why;
    for (int i = 0; i < kNumVariants; ++i) {
        if (forced >= 0 && i != forced) continue;
        const VariantDesc& v = kVariants[i];
        if (!variant_runs(v, *p, forced >= 0 ? &why : nullptr)) continue;
        Estimate e = v.vkind == VK_DWPW_GEN        ? estimate_gen(v, *p, d, Ho, Wo)
                     : p->kind == FCM_KIND_PWDW   ? estimate_pwdw(v, *p, d, Ho, Wo)
                     : p->kind == FCM_KIND_PWDWPW ? estimate_pwdwpw(v, *p, d, Ho, Wo)
                     : p->kind == FCM_KIND_PWPW ? estimate_pwpw(v, *p, d)
                                                : estimate(v, *p, d, Ho, Wo);
        if (plan_log_enabled())
            fprintf(stderr,
                    "fcm plan: %-40s feasible %d wgs/cu %d grid %6d tiles %7d  t %8.3f us "
                    "(hbm %.3f l2 %.3f mat %.3f vec %.3f busy %.2f)  bytes %lld waste %.3f gma %.4g\n",
                    v.name, (int)e.feasible, e.wgs_per_cu, e.grid, e.num_tiles, e.t_us,
                    e.t_hbm * 1e6, e.t_l2 * 1e6, e.t_mat * 1e6, e.t_vec * 1e6, e.busy,
                    (long long)e.pred, e.waste, e.gma);
        if (e.wgs_per_cu <= 0) {
            if (forced >= 0) why = "variant's LDS or registers exceed the device budget";
            continue;
        }
        // (The pages' second constraint, at least as many output tiles as compute units,
        // makes a tiling's Eq.-style estimate infinite; the ranking itself goes by the time
        // model, which already charges the idle CUs of such a tiling.  The first
        // constraint, LDS and registers, excluded the variant above.)
        auto specialised = [](int vk) { return vk == VK_DWPW_WS || vk == VK_DWPW_WSL; };
        bool better;
        if (best < 0) {
            better = true;
        } else if (fabs(e.t_us - be.t_us) > 0.01 * std::min(e.t_us, be.t_us)) {
            better = e.t_us < be.t_us;  // modelled time decides unless within 1%
        } else if (specialised(v.vkind) != specialised(kVariants[best].vkind)) {
            // wave-specialised builds run the two layers' instruction streams on
            // different waves of a SIMD, which overlaps them; the roofline terms are the
            // same
            better = specialised(v.vkind);
        } else if (std::min(e.wgs_per_cu * v.waves, 12) !=
                   std::min(be.wgs_per_cu * kVariants[best].waves, 12)) {
            // resident waves per CU, up to three per SIMD: more hide more latency (the
            // kernels are latency and issue bound, which the roofline terms do not see);
            // beyond that the measured builds gained nothing (mbv1: three workgroups of
            // four waves per CU 9.44 us against two 9.80 us)
            better = std::min(e.wgs_per_cu * v.waves, 12) >
                     std::min(be.wgs_per_cu * kVariants[best].waves, 12);
        } else if (e.pred != be.pred) {
            better = e.pred < be.pred;
        } else if (e.waste != be.waste) {
            better = e.waste < be.waste;
        } else {
            better = e.wgs_per_cu > be.wgs_per_cu;
        }
        if (better) {
            best = i;
            be = e;
        }
    }
    if (best < 0) {
        *err = forced >= 0 ? ("variant cannot run this problem: " + why)
                           : std::string("no compiled kernel variant fits this problem");
        return (forced >= 0 && (forced >= kNumVariants)) ? FCM_ERR_INVALID_ARG
                                                         : FCM_ERR_UNSUPPORTED;
    }
    const VariantDesc& v = kVariants[best];
    fcm_plan_t pl;
    memset(&pl, 0, sizeof(pl));
    pl.version = FCM_PLAN_VERSION;
    pl.prob = *p;
    pl.Ho = Ho;
    pl.Wo = Wo;
    pl.variant = best;
    pl.tile_h = v.th;
    pl.tile_w = v.tw;
    pl.k_tile = v.kt;
    pl.c_chunk = v.cc;
    pl.waves_per_wg = v.waves;
    pl.wgs_per_cu = be.wgs_per_cu;
    pl.num_tiles = be.num_tiles;
    pl.grid = be.grid;
    pl.lds_bytes = variant_lds_bytes(v);
    const int e = elem_bytes(p->dtype);
    if (p->kind == FCM_KIND_PWPW) {
        // first layer [K1][C] as is; second [K][K1] and its blocked copy
        const int64_t M = (int64_t)p->N * p->H * p->W;
        pl.w1_packed_bytes = (int64_t)p->K1 * p->C * e;
        pl.w2_packed_bytes = ((int64_t)p->K * p->K1 + pw_blocked_elems(p->K, p->K1)) * e;
        pl.workspace_bytes = M * p->K1 * e;
        pl.alg_bytes_fused = M * p->C * e + M * p->K * e + (int64_t)p->K1 * p->C * e +
                             (int64_t)p->K * p->K1 * e + (int64_t)4 * 2 * (p->K1 + p->K);
        pl.alg_bytes_unfused = pl.alg_bytes_fused + 2 * pl.workspace_bytes;
        pl.pred_bytes_fused = be.pred;
        // layer by layer: each 1x1 layer with the baseline's tiling (Eq. 2 for each)
        const int mt = lbl::PW_MT16, kt = lbl::PW_KT16;
        const int64_t l1 = M * p->C * e * cdiv(p->K1, kt) + cdiv(M, mt) * p->K1 * p->C * e +
                           pl.workspace_bytes;
        const int64_t l2 = pl.workspace_bytes * cdiv(p->K, kt) + cdiv(M, mt) * p->K * p->K1 * e +
                           M * p->K * e;
        pl.pred_bytes_unfused = l1 + l2;
        pl.gma_paper_fused = be.gma;
        pl.gma_paper_unfused = (double)(l1 + l2);
        pl.fuse = fuse_flag(pl.alg_bytes_fused, pl.alg_bytes_unfused,
                            pl.w1_packed_bytes + (int64_t)p->K * p->K1 * e, d);
        pl.pred_us_fused = be.t_us;
        pl.flops = 2.0 * M * p->C * p->K1 + 2.0 * M * p->K1 * p->K;
        *out = pl;
        return FCM_OK;
    }
    if (p->kind == FCM_KIND_PWDWPW) {
        // expansion [K1][C] as is; depthwise [R*S][K1]; the projection's [K][K1] filters
        // are read unpacked
        pl.w1_packed_bytes = (int64_t)p->K1 * p->C * e;
        pl.w2_packed_bytes = (int64_t)p->R * p->S * p->K1 * e;
        const int64_t t1 = (int64_t)p->N * p->H * p->W * p->K1 * e;
        const int64_t t2 = (int64_t)p->N * Ho * Wo * p->K1 * e;
        pl.workspace_bytes = t1 + t2;
        const int64_t x_bytes = (int64_t)p->N * p->H * p->W * p->C * e;
        const int64_t y_bytes = (int64_t)p->N * Ho * Wo * p->K * e;
        pl.alg_bytes_fused = x_bytes + y_bytes + pl.w1_packed_bytes + pl.w2_packed_bytes +
                             (int64_t)p->K * p->K1 * e + (int64_t)4 * 2 * (2 * p->K1 + p->K);
        // layer by layer: each intermediate written and read back, and the shortcut
        // reads the input a second time
        pl.alg_bytes_unfused = pl.alg_bytes_fused + 2 * (t1 + t2) + (p->residual ? x_bytes : 0);
        pl.pred_bytes_fused = be.pred;
        int64_t pu = 0;
        double gu = 0;
        estimate_unfused_pwdwpw(*p, Ho, Wo, &pu, &gu);
        pl.pred_bytes_unfused = pu;
        pl.gma_paper_fused = be.gma;
        pl.gma_paper_unfused = gu;
        pl.fuse = fuse_flag(pl.alg_bytes_fused, pl.alg_bytes_unfused,
                            pl.w1_packed_bytes + pl.w2_packed_bytes + (int64_t)p->K * p->K1 * e,
                            d);
        pl.pred_us_fused = be.t_us;
        pl.flops = 2.0 * p->N * p->H * p->W * p->C * p->K1 +
                   2.0 * p->N * Ho * Wo * p->K1 * p->R * p->S +
                   2.0 * p->N * Ho * Wo * p->K1 * p->K;
        *out = pl;
        return FCM_OK;
    }
    if (p->kind == FCM_KIND_PWDW) {
        // first layer: pointwise [K1][C] as is; second: depthwise [R*S][K1]
        pl.w1_packed_bytes = (int64_t)p->K1 * p->C * e;
        pl.w2_packed_bytes = (int64_t)p->R * p->S * p->K1 * e;
        pl.workspace_bytes = (int64_t)p->N * p->H * p->W * p->K1 * e;
        const int64_t x_bytes = (int64_t)p->N * p->H * p->W * p->C * e;
        const int64_t y_bytes = (int64_t)p->N * Ho * Wo * p->K1 * e;
        pl.alg_bytes_fused = x_bytes + y_bytes + pl.w1_packed_bytes + pl.w2_packed_bytes +
                             (int64_t)4 * 2 * (p->K1 + p->K1);
        pl.alg_bytes_unfused = pl.alg_bytes_fused + 2 * pl.workspace_bytes;
        pl.pred_bytes_fused = be.pred;
        int64_t pu = 0;
        double gu = 0;
        estimate_unfused_pwdw(*p, Ho, Wo, &pu, &gu);
        pl.pred_bytes_unfused = pu;
        pl.gma_paper_fused = be.gma;
        pl.gma_paper_unfused = gu;
        pl.fuse = fuse_flag(pl.alg_bytes_fused, pl.alg_bytes_unfused,
                            pl.w1_packed_bytes + pl.w2_packed_bytes, d);
        pl.pred_us_fused = be.t_us;
        pl.flops = 2.0 * p->N * p->H * p->W * p->C * p->K1 +
                   2.0 * p->N * Ho * Wo * p->K1 * p->R * p->S;
        *out = pl;
        return FCM_OK;
    }
    // the first layer's outputs: K1 (B2B), C * mult (DW->PW: K1 as validated)
    const int n1 = p->K1;
    pl.w1_packed_bytes =
        (int64_t)(p->kind == FCM_KIND_B2B ? (int64_t)p->K1 * p->R * p->S * p->C
                                          : (int64_t)p->R * p->S * p->K1) * e;
    pl.w2_packed_bytes = (int64_t)p->K * n1 * e;
    if (p->dtype == FCM_I8) {
        // int8: the 1x1 filters again in 64 x 64 blocks (k tile, 64-channel slice) in the
        // int8 matrix-operand order
        pl.w2_packed_bytes += (int64_t)((p->K + 63) / 64) * ((p->C + 63) / 64) * 64 * 64;
    } else if (p->dtype != FCM_F32) {
        // 16-bit storage: the 1x1 filters again in 32 x 32 blocks in matrix-operand order
        // (pw_blocked_elems), and for B2B the 3x3 filters in 16 x 32 blocks
        // (conv_blocked_elems), each after the plain array
        pl.w2_packed_bytes += pw_blocked_elems(p->K, n1) * e;
        if (p->kind == FCM_KIND_B2B) pl.w1_packed_bytes += conv_blocked_elems(p->K1, p->C) * e;
    }
    pl.workspace_bytes = (int64_t)p->N * Ho * Wo * n1 * e;
    const int64_t x_bytes = (int64_t)p->N * p->H * p->W * p->C * e;
    const int64_t y_bytes = (int64_t)p->N * Ho * Wo * p->K * e;
    // epilogue arrays are counted as passed: scale and bias for both layers
    const int64_t epi = (int64_t)4 * 2 * (n1 + p->K);
    const int64_t w1_bytes = (int64_t)(p->kind == FCM_KIND_B2B ? (int64_t)p->K1 * p->R * p->S * p->C
                                                               : (int64_t)p->R * p->S * p->K1) * e;
    pl.alg_bytes_fused = x_bytes + y_bytes + w1_bytes + (int64_t)p->K * n1 * e + epi;
    pl.alg_bytes_unfused = pl.alg_bytes_fused + 2 * pl.workspace_bytes;
    pl.pred_bytes_fused = be.pred;
    int64_t pu = 0;
    double gu = 0;
    if (prob_is_gen(*p))
        estimate_unfused_gen(*p, lbl::DWG_CC, Ho, Wo, &pu, &gu);
    else
        estimate_unfused(*p, d, Ho, Wo, &pu, &gu);
    pl.pred_bytes_unfused = pu;
    pl.gma_paper_fused = be.gma;
    pl.gma_paper_unfused = gu;
    pl.fuse = fuse_flag(pl.alg_bytes_fused, pl.alg_bytes_unfused,
                      w1_bytes + (int64_t)p->K * n1 * e, d);
    pl.pred_us_fused = be.t_us;
    const double P = (double)p->N * Ho * Wo;
    pl.flops = p->kind == FCM_KIND_B2B
                   ? 2.0 * P * p->K1 * p->C * p->R * p->S + 2.0 * P * p->K1 * p->K
                   : 2.0 * P * p->K1 * p->R * p->S + 2.0 * P * p->K1 * p->K;
    *out = pl;
    return FCM_OK;
}

namespace {

// Layer-by-layer estimate of one layer alone (the pages' Eq. 3 for a depthwise layer,
// Eq. 2 for a pointwise layer), with the baseline kernels' tilings.
double single_layer_gma(const fcm_layer& l, int N, int H, int W, int e) {
    if (l.type == FCM_LAYER_DW) {
        const int Ho = conv_out(H, 1, 3, l.stride), Wo = conv_out(W, 1, 3, l.stride);
        const int th = lbl::DW_TH, tw = lbl::DW_TW;
        const double ifm = (double)N * H * W * l.C * e, ofm = (double)N * Ho * Wo * l.C * e;
        const double overlap = eq1_overlap(W, H, tw * l.stride, th * l.stride, 3, l.stride);
        return 2.0 * l.C * overlap * N * e + ifm + ofm +
               ceil((double)N * Ho * Wo / (double)(th * tw)) * 9.0 * l.C * e;
    }
    const int mt = e == 4 ? lbl::PW_MT32 : lbl::PW_MT16, kt = e == 4 ? lbl::PW_KT32 : lbl::PW_KT16;
    const double ifm = (double)N * H * W * l.C * e, ofm = (double)N * H * W * l.K * e;
    const double w = (double)l.K * l.C * e;
    return ceil(w / ((double)std::min(kt, l.K) * l.C * e)) * ifm + ofm +
           ceil(ofm / ((double)mt * std::min(kt, l.K) * e)) * w;
}

}  // namespace

fcm_status plan_chain(const fcm_layer* layers, int n, int N, int H, int W, int dtype,
                      const fcm_device_spec* spec, fcm_chain_group* groups, int* ngroups,
                      double* gma_chain, double* gma_lbl, std::string* err) {
    if (!layers || !groups || !ngroups || !gma_chain || !gma_lbl) {
        *err = "NULL argument";
        return FCM_ERR_INVALID_ARG;
    }
    if (n < 1 || N <= 0 || H <= 0 || W <= 0) {
        *err = "need at least one layer and a positive input extent";
        return FCM_ERR_INVALID_ARG;
    }
    const int e = elem_bytes(dtype);
    // per-layer input extents, validity
    std::vector<int> hin(n + 1), win(n + 1);
    hin[0] = H;
    win[0] = W;
    for (int i = 0; i < n; ++i) {
        const fcm_layer& l = layers[i];
        if (l.type != FCM_LAYER_DW && l.type != FCM_LAYER_PW) {
            *err = "unknown layer type at layer " + std::to_string(i);
            return FCM_ERR_INVALID_ARG;
        }
        if (l.C <= 0 || l.K <= 0 || (i > 0 && l.C != layers[i - 1].K)) {
            *err = "channel counts do not chain at layer " + std::to_string(i);
            return FCM_ERR_INVALID_ARG;
        }
        if (l.type == FCM_LAYER_DW && (l.K != l.C || (l.stride != 1 && l.stride != 2))) {
            *err = "a depthwise layer keeps its channels and has stride 1 or 2 (layer " +
                   std::to_string(i) + ")";
            return FCM_ERR_INVALID_ARG;
        }
        if (l.type == FCM_LAYER_PW && l.stride != 1) {
            *err = "a pointwise layer has stride 1 (layer " + std::to_string(i) + ")";
            return FCM_ERR_INVALID_ARG;
        }
        if (l.C % 8 || l.K % 8) {
            *err = "channel counts must be multiples of 8 (layer " + std::to_string(i) + ")";
            return FCM_ERR_UNSUPPORTED;
        }
        hin[i + 1] = l.type == FCM_LAYER_DW ? conv_out(hin[i], 1, 3, l.stride) : hin[i];
        win[i + 1] = l.type == FCM_LAYER_DW ? conv_out(win[i], 1, 3, l.stride) : win[i];
    }
    // candidate modules for each pair (i, i+1)
    std::vector<double> single(n), pair(n, INFINITY);
    std::vector<int> pkind(n, -1), pvar(n, -1);
    for (int i = 0; i < n; ++i) single[i] = single_layer_gma(layers[i], N, hin[i], win[i], e);
    for (int i = 0; i + 1 < n; ++i) {
        const fcm_layer &a = layers[i], &b = layers[i + 1];
        fcm_problem p;
        memset(&p, 0, sizeof(p));
        p.dtype = dtype;
        p.N = N;
        p.H = hin[i];
        p.W = win[i];
        p.act1 = a.act;
        p.act2 = b.act;
        if (a.type == FCM_LAYER_DW && b.type == FCM_LAYER_PW) {
            p.kind = FCM_KIND_DWPW;
            p.C = p.K1 = a.C;
            p.K = b.K;
            p.R = p.S = 3;
            p.stride_h = p.stride_w = a.stride;
            p.pad_h = p.pad_w = 1;
        } else if (a.type == FCM_LAYER_PW && b.type == FCM_LAYER_DW) {
            p.kind = FCM_KIND_PWDW;
            p.C = a.C;
            p.K1 = p.K = a.K;
            p.R = p.S = 3;
            p.stride_h = p.stride_w = b.stride;
            p.pad_h = p.pad_w = 1;
        } else if (a.type == FCM_LAYER_PW && b.type == FCM_LAYER_PW) {
            p.kind = FCM_KIND_PWPW;
            p.C = a.C;
            p.K1 = a.K;
            p.K = b.K;
            p.R = p.S = 1;
            p.stride_h = p.stride_w = 1;
        } else {
            continue;  // DW -> DW: no module
        }
        fcm_plan_t pl;
        std::string e2;
        if (plan_problem(&p, spec, -1, &pl, &e2) != FCM_OK) continue;  // no kernel
        if (!std::isfinite(pl.gma_paper_fused)) continue;               // infeasible tiling
        pair[i] = pl.gma_paper_fused;
        pkind[i] = p.kind;
        pvar[i] = pl.variant;
    }
    // dynamic program: best[i] = cheapest schedule of layers 0 .. i-1 (then fewest groups)
    std::vector<double> best(n + 1, INFINITY);
    std::vector<int> cnt(n + 1, 0), take(n + 1, 1);
    best[0] = 0.0;
    for (int i = 1; i <= n; ++i) {
        best[i] = best[i - 1] + single[i - 1];
        cnt[i] = cnt[i - 1] + 1;
        take[i] = 1;
        if (i >= 2 && std::isfinite(pair[i - 2])) {
            const double c = best[i - 2] + pair[i - 2];
            if (c < best[i] || (c == best[i] && cnt[i - 2] + 1 < cnt[i])) {
                best[i] = c;
                cnt[i] = cnt[i - 2] + 1;
                take[i] = 2;
            }
        }
    }
    // read the schedule back
    std::vector<fcm_chain_group> sched;
    for (int i = n; i > 0; i -= take[i]) {
        fcm_chain_group g;
        g.count = take[i];
        g.first = i - take[i];
        g.kind = take[i] == 2 ? pkind[i - 2] : -1;
        g.variant = take[i] == 2 ? pvar[i - 2] : -1;
        g.gma = take[i] == 2 ? pair[i - 2] : single[i - 1];
        sched.push_back(g);
    }
    std::reverse(sched.begin(), sched.end());
    for (size_t k = 0; k < sched.size(); ++k) groups[k] = sched[k];
    *ngroups = (int)sched.size();
    *gma_chain = best[n];
    double lbl_total = 0.0;
    for (int i = 0; i < n; ++i) lbl_total += single[i];
    *gma_lbl = lbl_total;
    return FCM_OK;
}

}  // namespace fcm
