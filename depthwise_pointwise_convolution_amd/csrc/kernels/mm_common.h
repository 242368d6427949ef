// mm_common.h -- helpers shared by the matrix-core depthwise->pointwise kernels:
// raw buffer resources, exact vector-memory waits, the out-of-range offset and the
// tile position record.
#pragma once

#include "stages.h"

namespace fcm {

namespace mm {

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    // gfx9 raw buffer: stride 0, range check on `bytes`, dword3 = 0x00020000
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

constexpr uint32_t kOob = 0x80000000u;  // byte offset beyond any range: load 0 / drop

// A tile's image, tile row and tile column, and the byte offsets derived from them:
// input window origin (may be negative at the top/left border) and output tile origin,
// both from the start of the whole tensor.
struct TilePos {
    int n, th, tw;
    int ih0, iw0, oh0, ow0;
    int in_base, out_base;
};

}  // namespace mm

}  // namespace fcm
