// common.h -- device-side building blocks shared by the gfx950 kernels: storage types,
// 16-byte vector moves, the MFMA wrappers, the epilogue, and the workgroup -> tile
// mapping.  Everything here is written for CDNA4 wave64; there is no other target.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fcm {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
template <typename T, int N>
using vec_t = T __attribute__((ext_vector_type(N)));

// Number of storage elements in one 16-byte vector.
template <typename T>
struct Vec {
    static constexpr int N = 16 / (int)sizeof(T);
};

__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Unpack a 16-byte vector of storage elements to fp32 (exact for fp16/bf16).
template <typename T>
__device__ __forceinline__ void unpack16(u32x4 raw, float* out) {
    constexpr int N = Vec<T>::N;
    vec_t<T, N> v = __builtin_bit_cast(vec_t<T, N>, raw);
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = (float)v[i];
}

// Round fp32 values to the storage type (round-to-nearest-even) and pack 16 bytes.
template <typename T>
__device__ __forceinline__ u32x4 pack16(const float* in) {
    constexpr int N = Vec<T>::N;
    vec_t<T, N> v;
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = (T)in[i];
    return __builtin_bit_cast(u32x4, v);
}

// Round four fp32 values to a 16-bit storage type and pack 8 bytes.
template <typename T>
__device__ __forceinline__ uint2 pack8(const float* in) {
    static_assert(sizeof(T) == 2, "8-byte packs of four 16-bit values");
    vec_t<T, 4> v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (T)in[i];
    return __builtin_bit_cast(uint2, v);
}

// Activation as a clamp to [lo, hi]: none (-inf, inf), ReLU (0, inf), ReLU6 (0, 6).
struct Act {
    float lo, hi;
};
__device__ __forceinline__ Act act_bounds(int act) {
    Act a;
    a.lo = act != 0 ? 0.0f : -__builtin_inff();
    a.hi = act == 2 ? 6.0f : __builtin_inff();
    return a;
}

// conv -> normalisation -> activation epilogue on one fp32 accumulator: one fused
// multiply-add and one median-of-three (the clamp), whatever the activation.
__device__ __forceinline__ float epilogue(float acc, float scale, float bias, Act act) {
    return __builtin_amdgcn_fmed3f(__builtin_fmaf(scale, acc, bias), act.lo, act.hi);
}

// D(16x16 fp32) += A(16x32) * B(32x16) on the matrix cores.  Lane l supplies row
// l%16 of A and column l%16 of B, each as 8 consecutive reduction indices of group
// l/16 (the same reduction index set for A and B, which is all the contraction
// needs); it receives D rows 4*(l/16) .. 4*(l/16)+3 of column l%16.
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c, _Float16*) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(vec_t<_Float16, 8>, a),
                                                  __builtin_bit_cast(vec_t<_Float16, 8>, b),
                                                  c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c, __bf16*) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(vec_t<__bf16, 8>, a),
                                                   __builtin_bit_cast(vec_t<__bf16, 8>, b),
                                                   c, 0, 0, 0);
}
template <typename T>
__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return mfma_16x16x32(a, b, c, (T*)nullptr);
}

// Output-channel permutation used for every MFMA accumulator tile: row r of k-block
// kb of a tile of KT output channels holds channel
//     (r / 4) * (KT / 4) + kb * 4 + (r % 4),
// so that lane group g = l/16 ends up holding the KT/4 consecutive channels
// [g*KT/4, (g+1)*KT/4) of its pixel and writes them with 16-byte stores.
template <int KT>
__device__ __forceinline__ int kperm(int kb, int r) {
    return (r >> 2) * (KT / 4) + kb * 4 + (r & 3);
}

// Workgroups are handed to the 8 XCDs round-robin (workgroup b runs on XCD b % 8).
// Renumber them so that each XCD owns a contiguous range of logical ids: adjacent
// tiles (which share input halo rows) are then processed by the same L2.
__device__ __forceinline__ int xcd_logical_id(int b, int G) {
    return (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
}

}  // namespace fcm
