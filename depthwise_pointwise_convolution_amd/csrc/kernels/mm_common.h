// mm_common.h -- helpers shared by the matrix-core depthwise->pointwise kernels:
// raw buffer resources, exact vector-memory waits, the out-of-range offset and the
// tile position record.
#pragma once

#include "stages.h"

namespace fcm {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// An 8-byte LDS store as one vector value.  A store of the two-field struct is split and
// re-merged by the compiler, which then no longer knows which LDS array it writes and
// waits for every direct global->LDS load in flight before it.
__device__ __forceinline__ void st8(char* p, uint2 v) {
    *reinterpret_cast<u32x2*>(p) = u32x2{v.x, v.y};
}

namespace mm {

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
#if __HIP_DEVICE_COMPILE__
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
#else
    (void)p;
    return 0;
#endif
}

// Ten 16-byte LDS reads issued back to back and waited for within the same statement
// (gfx950 assembly), for the same reason as lds_read20 below.
__device__ __forceinline__ void lds_read10(const uint32_t (&ad)[10], u32x4 (&o)[10]) {
#if __HIP_DEVICE_COMPILE__
    asm volatile(
        "ds_read_b128 %0, %10\n\t"
        "ds_read_b128 %1, %11\n\t"
        "ds_read_b128 %2, %12\n\t"
        "ds_read_b128 %3, %13\n\t"
        "ds_read_b128 %4, %14\n\t"
        "ds_read_b128 %5, %15\n\t"
        "ds_read_b128 %6, %16\n\t"
        "ds_read_b128 %7, %17\n\t"
        "ds_read_b128 %8, %18\n\t"
        "ds_read_b128 %9, %19\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),
          "=&v"(o[6]), "=&v"(o[7]), "=&v"(o[8]), "=&v"(o[9])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]),
          "v"(ad[7]), "v"(ad[8]), "v"(ad[9])
        : "memory");
#else
    (void)ad;
    for (int i = 0; i < 10; ++i) o[i] = u32x4{0u, 0u, 0u, 0u};
#endif
}
// Twenty 16-byte LDS reads issued back to back and waited for within the same statement
// (gfx950 assembly).  The compiler does not see them as LDS accesses, so it adds no wait
// for the direct global->LDS loads in flight before them; the kernel's own waits and
// barriers order the reads after the loads of the buffer they read.
__device__ __forceinline__ void lds_read20(const uint32_t (&ad)[20], u32x4 (&o)[20]) {
#if __HIP_DEVICE_COMPILE__
    asm volatile(
        "ds_read_b128 %0, %20\n\t"
        "ds_read_b128 %1, %21\n\t"
        "ds_read_b128 %2, %22\n\t"
        "ds_read_b128 %3, %23\n\t"
        "ds_read_b128 %4, %24\n\t"
        "ds_read_b128 %5, %25\n\t"
        "ds_read_b128 %6, %26\n\t"
        "ds_read_b128 %7, %27\n\t"
        "ds_read_b128 %8, %28\n\t"
        "ds_read_b128 %9, %29\n\t"
        "ds_read_b128 %10, %30\n\t"
        "ds_read_b128 %11, %31\n\t"
        "ds_read_b128 %12, %32\n\t"
        "ds_read_b128 %13, %33\n\t"
        "ds_read_b128 %14, %34\n\t"
        "ds_read_b128 %15, %35\n\t"
        "ds_read_b128 %16, %36\n\t"
        "ds_read_b128 %17, %37\n\t"
        "ds_read_b128 %18, %38\n\t"
        "ds_read_b128 %19, %39\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),
          "=&v"(o[6]), "=&v"(o[7]), "=&v"(o[8]), "=&v"(o[9]), "=&v"(o[10]), "=&v"(o[11]),
          "=&v"(o[12]), "=&v"(o[13]), "=&v"(o[14]), "=&v"(o[15]), "=&v"(o[16]), "=&v"(o[17]),
          "=&v"(o[18]), "=&v"(o[19])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]),
          "v"(ad[7]), "v"(ad[8]), "v"(ad[9]), "v"(ad[10]), "v"(ad[11]), "v"(ad[12]),
          "v"(ad[13]), "v"(ad[14]), "v"(ad[15]), "v"(ad[16]), "v"(ad[17]), "v"(ad[18]),
          "v"(ad[19])
        : "memory");
#else
    (void)ad;
    for (int i = 0; i < 20; ++i) o[i] = u32x4{0u, 0u, 0u, 0u};
#endif
}

// An 8-byte LDS write in gfx950 assembly.  The compiler does not see it as an LDS
// access, so it adds no wait for the direct global->LDS loads in flight before it (its
// alias analysis cannot always tell them apart); the kernel's own waits and barriers
// order the write against the reads of the same buffer.  (The host compilation pass
// only needs the function to exist.)
__device__ __forceinline__ void lds_st8(uint32_t addr, uint2 v) {
#if __HIP_DEVICE_COMPILE__
    asm volatile("ds_write_b64 %0, %1" : : "v"(addr), "v"(u32x2{v.x, v.y}) : "memory");
#else
    (void)addr;
    (void)v;
#endif
}

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

// Cache policy (the buffer instruction's aux operand) of whole-line output stores:
// non-temporal (bit 1) at device scope (bit 4).  The L2 of each XCD does not keep the
// finished output for reuse and passes it on while the kernel runs, instead of holding
// dirty lines for the write-back at the kernel's end; on MI355X this took 10-23% off the
// memory-bound layers.  Kernels that fill a 128-byte line only in pieces written at
// different times (8-byte stores, or 16-byte stores of lanes spread over many lines) keep
// the default policy, under which the L2 merges the pieces (streamed, they cost 40-60%
// more there).
constexpr int kStoreStream = 0x12;

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
