// plan.h -- the gfx950 FusePlanner (host only, no HIP dependency).
#pragma once

#include <stdint.h>

#include <string>

#include "../../include/fcm.h"

namespace fcm {

enum VKind {
    VK_DWPW = 0,
    VK_DWPW32 = 1,
    VK_B2B = 2,
    VK_DWPW_MM = 3,
    VK_B2B_MM = 5,
    VK_DWPW_MMW = 6,
    VK_PWDW_MM = 7,
    VK_DWPW_I8 = 8,
    VK_PWPW_MM = 9,
    VK_DWPW_GEN = 10,
    VK_DWPW_WS = 11,
    VK_PWDWPW_MM = 12,
    VK_DWPW_WSL = 13
};

struct VariantDesc {
    const char* name;
    int vkind;   // VKind
    int dtype;   // fcm_dtype
    int stride;
    int th, tw;  // output tile
    int kt;      // output channels per workgroup
    int cc;      // input channels per LDS pass
    int wres;    // pointwise weights resident in registers
    int nbuf;    // input tile buffers in LDS (matrix-core DW only)
    int k1;      // back-to-back: intermediate channels compiled in; PW->DW->PW: expanded
                 // channels one workgroup holds (0 otherwise)
    int occ;     // waves per SIMD the kernel is compiled to allow (register budget)
    int waves;   // waves per workgroup
    int cmax;    // largest C the variant takes (0: no limit)
    int bpw;     // PW->DW and PW->DW->PW: 16-channel blocks per wave (0 otherwise)
    int fs;      // generalised DW->PW: filter size, dilation, depth multiplier (0 otherwise)
    int dil;
    int mult;
};

// MI355X published figures (256 CUs, 160 KB LDS per CU, 8 TB/s HBM, 2.5 PFLOP/s dense
// fp16/bf16 matrix rate, ...); host only.
void default_spec(fcm_device_spec* out);

extern const VariantDesc kVariants[];
extern const int kNumVariants;

// LDS bytes and a per-lane VGPR estimate of one workgroup of variant v.
int variant_lds_bytes(const VariantDesc& v);
// Workgroup count of a persistent launch over ptiles pixel tiles x ktiles output-
// channel tiles when the GPU holds `capacity` workgroups at once.
int64_t persistent_grid(int64_t ptiles, int ktiles, int64_t capacity);
int variant_vgpr_estimate(const VariantDesc& v);

// Checks every field of the problem (see fcm_plan in fcm.h for the rules).
fcm_status validate_problem(const fcm_problem* p, std::string* err);

// Whether variant v can run problem p (kind, type, stride, channel limits).
bool variant_runs(const VariantDesc& v, const fcm_problem& p, std::string* why);

// FusePlanner over a chain of layers (see fcm_plan_chain in fcm.h).
fcm_status plan_chain(const fcm_layer* layers, int n, int N, int H, int W, int dtype,
                      const fcm_device_spec* spec, fcm_chain_group* groups, int* ngroups,
                      double* gma_chain, double* gma_lbl, std::string* err);

// Fill *out for problem p with variant `forced` (or the cheapest one if forced < 0).
fcm_status plan_problem(const fcm_problem* p, const fcm_device_spec* spec, int forced,
                        fcm_plan_t* out, std::string* err);

// Elements of the blocked copy of [K][C] pointwise filters: K and C rounded up to
// multiples of 32, zero filled.  Block (g, s, h) of 64 lanes x 8 elements holds, for
// lane l = 16 * lg + r and element e, filter [32g + 8(r/4) + 4h + r%4][32s + 8lg + e]:
// the A operand of one v_mfma_f32_16x16x32 for output rows 32g.. and input channels
// 32s.., in one contiguous kilobyte.  Blocks are ordered (g, s, h).
inline int64_t pw_blocked_elems(int K, int C) {
    return (int64_t)((K + 31) / 32 * 32) * ((C + 31) / 32 * 32);
}

// Elements of the blocked copy of 3x3 filters [K1][9][C] (16-bit storage): K1 rounded up
// to a multiple of 16, C to a multiple of 64.  Block (g, t, s) of 64 lanes x 8 elements
// holds, for lane l = 16 * lg + r and element e, filter [16g + r][tap t][32s + 8lg + e]:
// the A operand of one v_mfma_f32_16x16x32 for intermediate channels 16g.. and input
// channels 32s.. of tap t, in one contiguous kilobyte.  Blocks are ordered (g, t, s).
inline int64_t conv_blocked_elems(int K1, int C) {
    return (int64_t)((K1 + 15) / 16 * 16) * 9 * ((C + 63) / 64 * 64);
}

// The generalised depthwise fields of a problem (0 means 1) and the input extent of
// one output's window, (R-1)*dil + 1.
inline int prob_dil_h(const fcm_problem& p) { return p.dil_h > 0 ? p.dil_h : 1; }
inline int prob_dil_w(const fcm_problem& p) { return p.dil_w > 0 ? p.dil_w : 1; }
inline int prob_mult(const fcm_problem& p) { return p.mult > 0 ? p.mult : 1; }
inline int prob_ext_h(const fcm_problem& p) { return (p.R - 1) * prob_dil_h(p) + 1; }
inline int prob_ext_w(const fcm_problem& p) { return (p.S - 1) * prob_dil_w(p) + 1; }
// The depthwise layer's input and output channels: K1 for PW->DW and PW->DW->PW (the
// expanded channels), C for the other modules' first layer.
inline bool prob_has_expansion(const fcm_problem& p) {
    return p.kind == FCM_KIND_PWDW || p.kind == FCM_KIND_PWDWPW;
}
// A DW->PW module whose depthwise layer is not the plain 3x3, undilated, multiplier-1 one.
inline bool prob_is_gen(const fcm_problem& p) {
    return p.kind == FCM_KIND_DWPW && (p.R != 3 || p.S != 3 || prob_dil_h(p) != 1 ||
                                       prob_dil_w(p) != 1 || prob_mult(p) != 1);
}

// Output extent of a convolution.
inline int conv_out(int in, int pad, int filt, int stride) {
    // (64-bit: an unvalidated problem may hold sizes whose sum overflows an int)
    return (int)(((int64_t)in + 2 * (int64_t)pad - filt) / stride + 1);
}

}  // namespace fcm
