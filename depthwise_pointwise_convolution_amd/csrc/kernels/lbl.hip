// lbl.hip -- layer-by-layer (unfused) baselines and the weight-packing kernels.
//
// The FCM paper isolates the effect of fusion by comparing each fused module with
// layer-by-layer kernels that share its dataflow and access patterns (Sec. V-C).
// These kernels do exactly that: the depthwise kernel runs the same LDS staging and
// stencil stage as the fused kernels but writes the intermediate feature maps to
// HBM; the pointwise kernel reads them back and runs the same matrix-core
// contraction and epilogue.
#include "../launchers.h"
#include "../lbl_tiles.h"
#include "stages.h"

namespace fcm {

// Depthwise layer: one workgroup per (TH x TW output tile, CC-channel chunk).
template <typename T, int S, int TH, int TW, int CC>
__global__ __launch_bounds__(256) void dw_lbl_kernel(KArgs a) {
    constexpr int NT = 256;
    constexpr int VN = Vec<T>::N;
    constexpr int IH = (TH - 1) * S + 3, IW = (TW - 1) * S + 3;
    constexpr int XS = CC + 8;
    constexpr int VB = DwBlocking<TH, TW, CC / VN, NT>::VB;
    __shared__ __attribute__((aligned(16))) T xs[IH * IW * XS];
    __shared__ __attribute__((aligned(16))) float wdw_s[9 * CC];
    __shared__ __attribute__((aligned(16))) float s1s[CC], b1s[CC];

    const int tid = threadIdx.x;

    const Act act1 = act_bounds(a.act1), act2 = act_bounds(a.act2);
    const int nchunks = (a.C + CC - 1) / CC;
    const int b = blockIdx.x;
    const int pt = b / nchunks, c0 = (b - pt * nchunks) * CC;
    const int per_img = a.tiles_h * a.tiles_w;
    const int n = pt / per_img;
    const int rem = pt - n * per_img;
    const int th = rem / a.tiles_w, tw = rem - th * a.tiles_w;
    const int oh0 = th * TH, ow0 = tw * TW;
    const T* __restrict__ x = (const T*)a.x;
    T* __restrict__ t = (T*)a.y;

    stage_input<T, IH, IW, CC, XS, NT>(xs, x, a, n, oh0 * S - a.pad_h, ow0 * S - a.pad_w, c0,
                                       tid);
    stage_dw_weights<T, CC, NT>(wdw_s, s1s, b1s, (const T*)a.w1, a, c0, tid);
    __syncthreads();
    dw_stage<T, S, TH, TW, CC, XS, IW, VB, NT>(
        xs, wdw_s, s1s, b1s, act1, tid, [&](int ohl, int col, int cg, u32x4 v) {
            const int oh = oh0 + ohl, ow = ow0 + col, c = c0 + cg * VN;
            if (oh < a.Ho && ow < a.Wo && c < a.C)
                st16(t + (((int64_t)n * a.Ho + oh) * a.Wo + ow) * a.C + c, v);
        });
}

// Pointwise layer on the matrix cores: the M = N*Ho*Wo pixels form the GEMM rows,
// each wave owns MBW 16-pixel blocks and KT output channels; operands stream from
// global memory 32 channels at a time.
template <typename T, int KT, int MBW>
__global__ __launch_bounds__(256) void pw_lbl_kernel(KArgs a) {
    constexpr int KB = KT / 16;
    __shared__ float s2s[KT], b2s[KT];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const Act act1 = act_bounds(a.act1), act2 = act_bounds(a.act2);
    const int lr = lane & 15, lg = lane >> 4;
    const int64_t M = (int64_t)a.N * a.Ho * a.Wo;
    const int b = blockIdx.x;
    const int kt = b % a.num_ktiles;
    const int64_t mt = b / a.num_ktiles;
    const int k0 = kt * KT;
    const T* __restrict__ t = (const T*)a.x;
    const T* __restrict__ w = (const T*)a.w2;
    T* __restrict__ y = (T*)a.y;
    for (int i = tid; i < KT; i += 256) {
        const int k = k0 + i;
        s2s[i] = (a.s2 && k < a.K) ? a.s2[k] : 1.0f;
        b2s[i] = (a.b2 && k < a.K) ? a.b2[k] : 0.0f;
    }
    __syncthreads();
    f32x4 acc[MBW][KB];
#pragma unroll
    for (int mi = 0; mi < MBW; ++mi)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) acc[mi][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int64_t mbase = mt * 64 * MBW + (int64_t)wave * MBW * 16;
    for (int c0 = 0; c0 < a.C; c0 += 32) {
        const int c = c0 + lg * 8;
        u32x4 bfr[MBW];
#pragma unroll
        for (int mi = 0; mi < MBW; ++mi) {
            const int64_t m = mbase + mi * 16 + lr;
            bfr[mi] = (m < M && c < a.C) ? ld16(t + m * a.C + c) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int ko = k0 + kperm<KT>(kb, lr);
            const u32x4 afr =
                (ko < a.K && c < a.C) ? ld16(w + (int64_t)ko * a.C + c) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int mi = 0; mi < MBW; ++mi) acc[mi][kb] = mfma<T>(afr, bfr[mi], acc[mi][kb]);
        }
    }
#pragma unroll
    for (int mi = 0; mi < MBW; ++mi) {
        const int64_t m = mbase + mi * 16 + lr;
        if (m < M) {
#pragma unroll
            for (int kb = 0; kb < KB; kb += 2) {
                const int kl = lg * (KT / 4) + kb * 4;
                if (k0 + kl < a.K) {
                    float o[8];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        o[i] = epilogue(acc[mi][kb][i], s2s[kl + i], b2s[kl + i], act2);
                        o[4 + i] =
                            epilogue(acc[mi][kb + 1][i], s2s[kl + 4 + i], b2s[kl + 4 + i], act2);
                    }
                    if (a.res) {
                        // shortcut: the same pixel and channels of a [M][K] tensor, added
                        // after the activation, before the one rounding
                        float rv[8];
                        unpack16<T>(ld16((const T*)a.res + m * a.K + k0 + kl), rv);
#pragma unroll
                        for (int i = 0; i < 8; ++i) o[i] += rv[i];
                    }
                    st16(y + m * a.K + k0 + kl, pack16<T>(o));
                }
            }
        }
    }
}

// Pointwise layer in fp32 on the VALU: thread (k, pixel) computes one output; 64
// output channels x 4 pixels per workgroup.
__global__ __launch_bounds__(256) void pw_lbl_f32_kernel(KArgs a) {
    static_assert(lbl::PW_KT32 * lbl::PW_MT32 == 256, "one output per thread");
    const int tid = threadIdx.x;
    const Act act1 = act_bounds(a.act1), act2 = act_bounds(a.act2);
    const int64_t M = (int64_t)a.N * a.Ho * a.Wo;
    const int kt = blockIdx.x % a.num_ktiles;
    const int64_t m = (int64_t)(blockIdx.x / a.num_ktiles) * lbl::PW_MT32 + tid / lbl::PW_KT32;
    const int k = kt * lbl::PW_KT32 + (tid % lbl::PW_KT32);
    if (m >= M || k >= a.K) return;
    const float* t = (const float*)a.x + m * a.C;
    const float* w = (const float*)a.w2 + (int64_t)k * a.C;
    float acc = 0.0f;
    for (int c = 0; c < a.C; ++c) acc = __builtin_fmaf(t[c], w[c], acc);
    const float sc = a.s2 ? a.s2[k] : 1.0f, bi = a.b2 ? a.b2[k] : 0.0f;
    ((float*)a.y)[m * a.K + k] = epilogue(acc, sc, bi, act2);
}

// ------------------------------------------------------------------------------------
// weight packing
// ------------------------------------------------------------------------------------
// depthwise [C][RS] -> [RS][C]
template <typename E>
__global__ void pack_dw_kernel(const E* __restrict__ src, E* __restrict__ dst, int C, int RS) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= C * RS) return;
    const int t = i / C, c = i - t * C;
    dst[i] = src[c * RS + t];
}
// standard conv [K1][C][RS] -> [K1][RS][C]
template <typename E>
__global__ void pack_conv_kernel(const E* __restrict__ src, E* __restrict__ dst, int K1, int C,
                                 int RS) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)K1 * C * RS;
    if (i >= total) return;
    const int c = (int)(i % C);
    const int t = (int)((i / C) % RS);
    const int64_t k = i / ((int64_t)C * RS);
    dst[i] = src[(k * C + c) * RS + t];
}

// ------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------
namespace {
template <typename T>
int dw_lbl_launch(int stride, const KArgs& a, void* stream) {
    using namespace lbl;
    constexpr int CC = sizeof(T) == 4 ? DW_CC32 : DW_CC16;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    dim3 g(a.num_ptiles * ((a.C + CC - 1) / CC));
    if (stride == 1)
        hipLaunchKernelGGL((dw_lbl_kernel<T, 1, DW_TH, DW_TW, CC>), g, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((dw_lbl_kernel<T, 2, DW_TH, DW_TW, CC>), g, dim3(256), 0, s, a);
    return (int)hipGetLastError();
}
}  // namespace

int launch_dw_lbl(int dtype, int stride, const KArgs& a, void* stream) {
    switch (dtype) {
    case 0: return dw_lbl_launch<float>(stride, a, stream);
    case 1: return dw_lbl_launch<_Float16>(stride, a, stream);
    default: return dw_lbl_launch<__bf16>(stride, a, stream);
    }
}

// a.num_ktiles must be set for the kernel's KT (see lbl_shape).
int launch_pw_lbl(int dtype, const KArgs& a, void* stream) {
    const int64_t M = (int64_t)a.N * a.Ho * a.Wo;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    using namespace lbl;
    if (dtype == 0) {
        dim3 g((unsigned)(((M + PW_MT32 - 1) / PW_MT32) * a.num_ktiles));
        hipLaunchKernelGGL(pw_lbl_f32_kernel, g, dim3(256), 0, s, a);
    } else {
        dim3 g((unsigned)(((M + PW_MT16 - 1) / PW_MT16) * a.num_ktiles));
        if (dtype == 1)
            hipLaunchKernelGGL((pw_lbl_kernel<_Float16, PW_KT16, PW_MBW16>), g, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((pw_lbl_kernel<__bf16, PW_KT16, PW_MBW16>), g, dim3(256), 0, s, a);
    }
    return (int)hipGetLastError();
}

int launch_pack_dw(int elem_bytes, const void* src, void* dst, int C, int RS, void* stream) {
    const int total = C * RS;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    if (elem_bytes == 4)
        hipLaunchKernelGGL(pack_dw_kernel<uint32_t>, dim3((total + 255) / 256), dim3(256), 0, s,
                           (const uint32_t*)src, (uint32_t*)dst, C, RS);
    else
        hipLaunchKernelGGL(pack_dw_kernel<uint16_t>, dim3((total + 255) / 256), dim3(256), 0, s,
                           (const uint16_t*)src, (uint16_t*)dst, C, RS);
    return (int)hipGetLastError();
}

int launch_pack_conv(int elem_bytes, const void* src, void* dst, int K1, int C, int RS,
                     void* stream) {
    const int64_t total = (int64_t)K1 * C * RS;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    dim3 g((unsigned)((total + 255) / 256));
    if (elem_bytes == 4)
        hipLaunchKernelGGL(pack_conv_kernel<uint32_t>, g, dim3(256), 0, s, (const uint32_t*)src,
                           (uint32_t*)dst, K1, C, RS);
    else
        hipLaunchKernelGGL(pack_conv_kernel<uint16_t>, g, dim3(256), 0, s, (const uint16_t*)src,
                           (uint16_t*)dst, K1, C, RS);
    return (int)hipGetLastError();
}

// Blocked copy of [K][C] pointwise filters (layout in plan.h, pw_blocked_elems): one
// thread per 16-bit destination element, zero where the row or channel does not exist.
__global__ void pack_pw_blocked_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                       int K, int C, int64_t total) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int e = (int)(i & 7), lane = (int)((i >> 3) & 63), h = (int)((i >> 9) & 1);
    const int64_t blk = i >> 10;  // g * S32 + s
    const int S32 = (C + 31) / 32;
    const int g = (int)(blk / S32), sl = (int)(blk % S32);
    const int lg = lane >> 4, r = lane & 15;
    const int k = 32 * g + 8 * (r >> 2) + 4 * h + (r & 3), c = 32 * sl + 8 * lg + e;
    dst[i] = (k < K && c < C) ? src[(int64_t)k * C + c] : (uint16_t)0;
}

int launch_pack_pw_blocked(const void* src, void* dst, int K, int C, void* stream) {
    const int64_t total = (int64_t)((K + 31) / 32 * 32) * ((C + 31) / 32 * 32);
    (void)hipGetLastError();
    hipLaunchKernelGGL(pack_pw_blocked_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256),
                       0, (hipStream_t)stream, (const uint16_t*)src, (uint16_t*)dst, K, C, total);
    return (int)hipGetLastError();
}

// Blocked copy of 3x3 filters from the PyTorch layout [K1][C][3][3] (layout in plan.h,
// conv_blocked_elems): one thread per 16-bit destination element, zero where the
// intermediate or input channel does not exist.
__global__ void pack_conv_blocked_kernel(const uint16_t* __restrict__ src,
                                         uint16_t* __restrict__ dst, int K1, int C, int64_t total) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int e = (int)(i & 7), lane = (int)((i >> 3) & 63);
    const int64_t blk = i >> 9;  // (g * 9 + t) * S32 + s
    const int S32 = (C + 63) / 64 * 2;
    const int s = (int)(blk % S32), t = (int)((blk / S32) % 9), g = (int)(blk / S32 / 9);
    const int lg = lane >> 4, r = lane & 15;
    const int k1 = 16 * g + r, c = 32 * s + 8 * lg + e;
    dst[i] = (k1 < K1 && c < C) ? src[((int64_t)k1 * C + c) * 9 + t] : (uint16_t)0;
}

int launch_pack_conv_blocked(const void* src, void* dst, int K1, int C, void* stream) {
    const int64_t total = (int64_t)((K1 + 15) / 16 * 16) * 9 * ((C + 63) / 64 * 64);
    (void)hipGetLastError();
    hipLaunchKernelGGL(pack_conv_blocked_kernel, dim3((unsigned)((total + 255) / 256)),
                       dim3(256), 0, (hipStream_t)stream, (const uint16_t*)src, (uint16_t*)dst,
                       K1, C, total);
    return (int)hipGetLastError();
}

int launch_copy(const void* src, void* dst, long long bytes, void* stream) {
    return (int)hipMemcpyAsync(dst, src, (size_t)bytes, hipMemcpyDeviceToDevice,
                               (hipStream_t)stream);
}

}  // namespace fcm
