// kargs.h -- kernel argument block and the host-side launcher signature shared by
// the API layer and the kernel translation units.
#pragma once

#include <stdint.h>

namespace fcm {

struct KArgs {
    const void* x;     // input feature maps [N][H][W][C] (or the intermediate for PW)
    const void* w1;    // packed first-layer filters
    const float* s1;   // epilogue 1 scale / bias (nullable)
    const float* b1;
    const void* w2;    // packed second-layer filters [K][C or K1]
    const float* s2;   // epilogue 2 scale / bias (nullable)
    const float* b2;
    void* y;           // output feature maps
    const void* w3;    // third layer's filters [K][K1] (PW->DW->PW module; else unused)
    const float* s3;   // epilogue 3 scale / bias (nullable)
    const float* b3;
    const void* res;   // shortcut input added after the last epilogue (nullable)
    int N, H, W, C, K1, K, Ho, Wo;
    int pad_h, pad_w;
    int act1, act2, act3;
    int residual;      // PW->DW->PW module: add the input pixel after epilogue 3
    int tiles_h, tiles_w;  // pixel tiles per image
    int num_ptiles;        // N * tiles_h * tiles_w (or flattened pixel tiles)
    int num_ktiles;        // output-channel tiles
};

// A launcher enqueues one kernel for `grid` workgroups on `stream` and returns the
// hipError_t of the launch (as int so this header stays HIP-free).
typedef int (*launch_fn)(const KArgs& a, int grid, void* stream);
// Occupancy query: workgroups of this kernel one CU can hold (0 on error).
typedef int (*occupancy_fn)(void);

}  // namespace fcm
