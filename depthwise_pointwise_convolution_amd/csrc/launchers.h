// launchers.h -- declarations of the templated kernel launchers.  Their definitions
// and explicit instances live in the kernels/*.hip translation units; this header
// lets the API layer refer to them without seeing any device code.
#pragma once

#include "kargs.h"

namespace fcm {

template <typename T, int S, int TH, int TW, int KT, int CC, bool WRES, int OCC>
int launch_dwpw_mfma(const KArgs& a, int grid, void* stream);
template <typename T, int S, int TH, int TW, int KT, int CC, bool WRES, int OCC>
int occ_dwpw_mfma();

template <int S, int TH, int TW, int KT, int CC>
int launch_dwpw_f32(const KArgs& a, int grid, void* stream);
template <int S, int TH, int TW, int KT, int CC>
int occ_dwpw_f32();

// M: depth multiplier of the depthwise layer (1 or 2); FS: its filter size (3 or 5)
template <typename T, int S, int TH, int TW, int KT, int CC, int NW, int OCC, int M, int FS>
int launch_dwpw_mm(const KArgs& a, int grid, void* stream);
template <typename T, int S, int TH, int TW, int KT, int CC, int NW, int OCC, int M, int FS>
int occ_dwpw_mm();

template <typename T, int S, int TH, int TW, int KT, int CMAX, int NW, int OCC, int D>
int launch_dwpw_mmw(const KArgs& a, int grid, void* stream);
template <typename T, int S, int TH, int TW, int KT, int CMAX, int NW, int OCC, int D>
int occ_dwpw_mmw();

template <typename T, int S, int TH, int TW, int CT, int KT, int NW>
int launch_dwpw_ws(const KArgs& a, int grid, void* stream);
template <typename T, int S, int TH, int TW, int CT, int KT, int NW>
int occ_dwpw_ws();

template <typename T, int S, int TH, int TW, int KT, int CMAX, int NW>
int launch_dwpw_wsl(const KArgs& a, int grid, void* stream);
template <typename T, int S, int TH, int TW, int KT, int CMAX, int NW>
int occ_dwpw_wsl();

template <typename T, int S, int TH, int CMAX, int NW, int BPW, int OCC>
int launch_pwdw_mm(const KArgs& a, int grid, void* stream);
template <typename T, int S, int TH, int CMAX, int NW, int BPW, int OCC>
int occ_pwdw_mm();

template <typename T, int S, int TH, int CMAX, int NW, int BPW, int KB, int OCC>
int launch_pwdwpw_mm(const KArgs& a, int grid, void* stream);
template <typename T, int S, int TH, int CMAX, int NW, int BPW, int KB, int OCC>
int occ_pwdwpw_mm();

template <typename T, int PB, int OCC, int CMAX, int KT>
int launch_pwpw_mm(const KArgs& a, int grid, void* stream);
template <typename T, int PB, int OCC, int CMAX, int KT>
int occ_pwpw_mm();

// generalised DW->PW (dwpw_gen.hip): fused kernel, occupancy, and the matching
// layer-by-layer depthwise kernel (NG: the fused variant's channel groups, which only
// tell the instantiations of variants that differ in it apart)
template <typename T, int S, int FS, int D, int M, int TH, int TW, int KT, int CC, int NG>
int launch_dwpw_gen(const KArgs& a, int grid, void* stream);
template <typename T, int S, int FS, int D, int M, int TH, int TW, int KT, int CC, int NG>
int occ_dwpw_gen();
template <typename T, int S, int FS, int D, int M, int TH, int TW, int KT, int CC, int NG>
int launch_dw_gen_lbl(const KArgs& a, int grid, void* stream);

template <int S, int OCC, int CMAX>
int launch_dwpw_i8(const KArgs& a, int grid, void* stream);
template <int S, int OCC, int CMAX>
int occ_dwpw_i8();
// INT8 layer-by-layer baselines and weight packing (dwpw_i8.hip)
int launch_dw_lbl_i8(int stride, const KArgs& a, void* stream);
int launch_pw_lbl_i8(const KArgs& a, void* stream);
int launch_pack_i8(const void* w_dw, void* dw_dst, const void* w_pw, void* pw_dst, int C, int K,
                   void* stream);

template <typename T, int S, int OCC>
int launch_b2b_mm(const KArgs& a, int grid, void* stream);
template <typename T, int S, int OCC>
int occ_b2b_mm();

template <typename T, int S, int TH, int TW, int K1, int KT, int CC>
int launch_b2b_mfma(const KArgs& a, int grid, void* stream);
template <typename T, int S, int TH, int TW, int K1, int KT, int CC>
int occ_b2b_mfma();

// Layer-by-layer baselines (fixed tilings; see lbl.hip / b2b.hip).
int launch_dw_lbl(int dtype, int stride, const KArgs& a, void* stream);
int launch_pw_lbl(int dtype, const KArgs& a, void* stream);
int launch_conv_lbl(int dtype, int stride, const KArgs& a, void* stream);
// (tilings in lbl_tiles.h; the caller fills KArgs tiles_* / num_ptiles / num_ktiles
// accordingly)

// Weight packing (see pack.hip).
int launch_pack_dw(int elem_bytes, const void* src, void* dst, int C, int RS, void* stream);
int launch_pack_conv(int elem_bytes, const void* src, void* dst, int K1, int C, int RS,
                     void* stream);
int launch_pack_pw_blocked(const void* src, void* dst, int K, int C, void* stream);
int launch_pack_conv_blocked(const void* src, void* dst, int K1, int C, void* stream);
int launch_copy(const void* src, void* dst, long long bytes, void* stream);

}  // namespace fcm
