// lbl_tiles.h -- fixed tilings of the layer-by-layer baseline kernels, shared by their
// launchers (as template arguments) and by the planner's byte estimates.
#pragma once

namespace fcm {
namespace lbl {
constexpr int DW_TH = 4, DW_TW = 16;    // depthwise output tile
constexpr int DW_CC16 = 64;             // channels per workgroup, 16-bit storage
constexpr int DW_CC32 = 32;             // channels per workgroup, fp32
constexpr int PW_KT16 = 128;            // pointwise output channels per workgroup
constexpr int PW_MBW16 = 2;             // 16-pixel blocks per wave (128 pixels / WG)
constexpr int PW_MT16 = 64 * PW_MBW16;  // pixels per workgroup
constexpr int PW_KT32 = 64, PW_MT32 = 4;
constexpr int DWG_TH = 4, DWG_TW = 16;  // generalised depthwise output tile
constexpr int DWG_CC = 32;              // and its input channels per workgroup
constexpr int CV_TH = 4, CV_TW = 16, CV_KT = 64, CV_CC = 64;  // 3x3 conv
}  // namespace lbl
}  // namespace fcm
