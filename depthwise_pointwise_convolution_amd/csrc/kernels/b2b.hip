// b2b.hip -- back-to-back standard 3x3 conv -> 1x1 conv on gfx950 matrix cores
// ("Fusing two back-to-back convolutions": block-resident fusion, the second conv
// must be 1x1), plus the layer-by-layer 3x3 conv baseline.
//
// The 3x3 conv is an implicit GEMM whose reduction index runs over (tap, channel):
// for every tap the 16-pixel B operand is read straight from the LDS halo tile,
// and the filter A operand streams from the packed [K1][9][C] filters.  Its fp32
// accumulators land in registers in the matrix unit's output layout; with the
// output-channel permutation of kperm<K1>, lane group g holds the K1/4 consecutive
// intermediate channels [g*K1/4, (g+1)*K1/4) of its pixel, which is exactly the
// operand layout the 1x1 conv needs when its reduction index is permuted the same
// way.  So after epilogue 1 and rounding, the intermediate goes from the first
// conv's accumulators to the second conv's operand registers without touching LDS
// or HBM -- the accumulator-to-operand hand-off the CUTLASS discussion describes for
// tensor cores, done here for the CDNA4 lane layout.
#include "../launchers.h"
#include "../lbl_tiles.h"
#include "stages.h"

namespace fcm {

// One channel chunk of the 3x3 conv for MBW 16-pixel blocks per wave and K1T output
// channels starting at k0.  xs holds the chunk's halo tile [IH][IW][XS].
template <typename T, int S, int TW, int IW, int XS, int K1T, int CC, int MBW>
__device__ __forceinline__ void conv3x3_chunk(f32x4 (&acc)[MBW][K1T / 16], const T* xs,
                                              const T* __restrict__ w1, const KArgs& a,
                                              int k0, int c0, int wave, int lr, int lg) {
    constexpr int KB = K1T / 16, KS = CC / 32;
    int base[MBW];
#pragma unroll
    for (int mi = 0; mi < MBW; ++mi) {
        const int px = (wave + 4 * mi) * 16 + lr;
        base[mi] = ((px / TW) * S * IW + (px % TW) * S) * XS + lg * 8;
    }
#pragma unroll
    for (int r = 0; r < 3; ++r) {
#pragma unroll
        for (int s = 0; s < 3; ++s) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 bfr[MBW];
#pragma unroll
                for (int mi = 0; mi < MBW; ++mi)
                    bfr[mi] = ld16(xs + base[mi] + (r * IW + s) * XS + ks * 32);
                const int c = c0 + ks * 32 + lg * 8;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const int ko = k0 + kperm<K1T>(kb, lr);
                    const u32x4 afr = (ko < a.K1 && c < a.C)
                                          ? ld16(w1 + ((int64_t)ko * 9 + r * 3 + s) * a.C + c)
                                          : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                    for (int mi = 0; mi < MBW; ++mi)
                        acc[mi][kb] = mfma<T>(afr, bfr[mi], acc[mi][kb]);
                }
            }
        }
    }
}

template <typename T, int S, int TH, int TW, int K1, int KT, int CC>
__global__ __launch_bounds__(256) void b2b_mfma_kernel(KArgs a) {
    constexpr int NT = 256;
    constexpr int P = TH * TW;
    static_assert(P % 64 == 0, "tile must give each wave whole 16-pixel blocks");
    constexpr int MBW = P / 64;
    constexpr int IH = (TH - 1) * S + 3, IW = (TW - 1) * S + 3;
    constexpr int XS = CC + 8;
    constexpr int KB1 = K1 / 16, KB2 = KT / 16, KS2 = K1 / 32;
    static_assert(K1 % 32 == 0 && KT % 32 == 0 && CC % 32 == 0, "tile sizes");

    __shared__ __attribute__((aligned(16))) T xs[IH * IW * XS];
    __shared__ float s1s[K1], b1s[K1], s2s[KT], b2s[KT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    const Act act1 = act_bounds(a.act1), act2 = act_bounds(a.act2);
    const int lr = lane & 15, lg = lane >> 4;
    const int G = gridDim.x;
    const int L = xcd_logical_id(blockIdx.x, G);
    const int k0 = (L % a.num_ktiles) * KT;
    const int pstep = G / a.num_ktiles;
    const T* __restrict__ x = (const T*)a.x;
    const T* __restrict__ w1 = (const T*)a.w1;
    const T* __restrict__ w2 = (const T*)a.w2;
    T* __restrict__ y = (T*)a.y;

    for (int i = tid; i < K1; i += NT) {
        s1s[i] = (a.s1 && i < a.K1) ? a.s1[i] : 1.0f;
        b1s[i] = (a.b1 && i < a.K1) ? a.b1[i] : 0.0f;
    }
    for (int i = tid; i < KT; i += NT) {
        const int k = k0 + i;
        s2s[i] = (a.s2 && k < a.K) ? a.s2[k] : 1.0f;
        b2s[i] = (a.b2 && k < a.K) ? a.b2[k] : 0.0f;
    }
    // 1x1 filters of this workgroup's output slice, resident in registers; reduction
    // index of step ks2 for lane group g: intermediate channels g*K1/4 + ks2*8 + [0,8).
    u32x4 w2f[KS2][KB2];
#pragma unroll
    for (int ks2 = 0; ks2 < KS2; ++ks2)
#pragma unroll
        for (int kb = 0; kb < KB2; ++kb) {
            const int ko = k0 + kperm<KT>(kb, lr), c = lg * (K1 / 4) + ks2 * 8;
            w2f[ks2][kb] = (ko < a.K && c < a.K1) ? ld16(w2 + (int64_t)ko * a.K1 + c)
                                                  : u32x4{0u, 0u, 0u, 0u};
        }

    const int per_img = a.tiles_h * a.tiles_w;
    for (int pt = L / a.num_ktiles; pt < a.num_ptiles; pt += pstep) {
        const int n = pt / per_img;
        const int rem = pt - n * per_img;
        const int th = rem / a.tiles_w, tw = rem - th * a.tiles_w;
        const int oh0 = th * TH, ow0 = tw * TW;
        f32x4 acc1[MBW][KB1];
#pragma unroll
        for (int mi = 0; mi < MBW; ++mi)
#pragma unroll
            for (int kb = 0; kb < KB1; ++kb) acc1[mi][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int c0 = 0; c0 < a.C; c0 += CC) {
            __syncthreads();  // every wave is done reading the previous halo tile
            stage_input<T, IH, IW, CC, XS, NT>(xs, x, a, n, oh0 * S - a.pad_h,
                                               ow0 * S - a.pad_w, c0, tid);
            __syncthreads();
            conv3x3_chunk<T, S, TW, IW, XS, K1, CC, MBW>(acc1, xs, w1, a, 0, c0, wave, lr, lg);
        }
#pragma unroll
        for (int mi = 0; mi < MBW; ++mi) {
            // epilogue 1, rounded to the storage type, straight into the 1x1 operand
            u32x4 b2f[KS2];
#pragma unroll
            for (int ks2 = 0; ks2 < KS2; ++ks2) {
                float o[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = lg * (K1 / 4) + ks2 * 8 + i;
                    o[i] = epilogue(acc1[mi][2 * ks2][i], s1s[c], b1s[c], act1);
                    o[4 + i] = epilogue(acc1[mi][2 * ks2 + 1][i], s1s[c + 4], b1s[c + 4], act1);
                }
                b2f[ks2] = pack16<T>(o);
            }
            f32x4 acc2[KB2];
#pragma unroll
            for (int kb = 0; kb < KB2; ++kb) acc2[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks2 = 0; ks2 < KS2; ++ks2)
#pragma unroll
                for (int kb = 0; kb < KB2; ++kb)
                    acc2[kb] = mfma<T>(w2f[ks2][kb], b2f[ks2], acc2[kb]);
            const int px = (wave + 4 * mi) * 16 + lr;
            const int oh = oh0 + px / TW, ow = ow0 + px % TW;
            if (oh < a.Ho && ow < a.Wo) {
                T* yp = y + (((int64_t)n * a.Ho + oh) * a.Wo + ow) * a.K;
#pragma unroll
                for (int kb = 0; kb < KB2; kb += 2) {
                    const int kl = lg * (KT / 4) + kb * 4;
                    if (k0 + kl < a.K) {
                        float o[8];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            o[i] = epilogue(acc2[kb][i], s2s[kl + i], b2s[kl + i], act2);
                            o[4 + i] =
                                epilogue(acc2[kb + 1][i], s2s[kl + 4 + i], b2s[kl + 4 + i], act2);
                        }
                        st16(yp + k0 + kl, pack16<T>(o));
                    }
                }
            }
        }
    }
}

// Layer-by-layer 3x3 conv + epilogue 1 writing the intermediate [N][Ho][Wo][K1]:
// one workgroup per (TH x TW output tile, K1T output channels).
template <typename T, int S, int TH, int TW, int K1T, int CC>
__global__ __launch_bounds__(256) void conv_lbl_kernel(KArgs a) {
    constexpr int NT = 256;
    constexpr int P = TH * TW, MBW = P / 64;
    constexpr int IH = (TH - 1) * S + 3, IW = (TW - 1) * S + 3;
    constexpr int XS = CC + 8;
    constexpr int KB = K1T / 16;
    __shared__ __attribute__((aligned(16))) T xs[IH * IW * XS];
    __shared__ float s1s[K1T], b1s[K1T];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const Act act1 = act_bounds(a.act1), act2 = act_bounds(a.act2);
    const int lr = lane & 15, lg = lane >> 4;
    const int b = blockIdx.x;
    const int k0 = (b % a.num_ktiles) * K1T;
    const int pt = b / a.num_ktiles;
    const int per_img = a.tiles_h * a.tiles_w;
    const int n = pt / per_img;
    const int rem = pt - n * per_img;
    const int th = rem / a.tiles_w, tw = rem - th * a.tiles_w;
    const int oh0 = th * TH, ow0 = tw * TW;
    const T* __restrict__ x = (const T*)a.x;
    T* __restrict__ t = (T*)a.y;
    for (int i = tid; i < K1T; i += NT) {
        const int k = k0 + i;
        s1s[i] = (a.s1 && k < a.K1) ? a.s1[k] : 1.0f;
        b1s[i] = (a.b1 && k < a.K1) ? a.b1[k] : 0.0f;
    }
    f32x4 acc[MBW][KB];
#pragma unroll
    for (int mi = 0; mi < MBW; ++mi)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) acc[mi][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < a.C; c0 += CC) {
        __syncthreads();
        stage_input<T, IH, IW, CC, XS, NT>(xs, x, a, n, oh0 * S - a.pad_h, ow0 * S - a.pad_w,
                                           c0, tid);
        __syncthreads();
        conv3x3_chunk<T, S, TW, IW, XS, K1T, CC, MBW>(acc, xs, (const T*)a.w1, a, k0, c0, wave,
                                                      lr, lg);
    }
#pragma unroll
    for (int mi = 0; mi < MBW; ++mi) {
        const int px = (wave + 4 * mi) * 16 + lr;
        const int oh = oh0 + px / TW, ow = ow0 + px % TW;
        if (oh < a.Ho && ow < a.Wo) {
            T* tp = t + (((int64_t)n * a.Ho + oh) * a.Wo + ow) * a.K1;
#pragma unroll
            for (int kb = 0; kb < KB; kb += 2) {
                const int kl = lg * (K1T / 4) + kb * 4;
                if (k0 + kl < a.K1) {
                    float o[8];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        o[i] = epilogue(acc[mi][kb][i], s1s[kl + i], b1s[kl + i], act1);
                        o[4 + i] = epilogue(acc[mi][kb + 1][i], s1s[kl + 4 + i], b1s[kl + 4 + i],
                                            act1);
                    }
                    st16(tp + k0 + kl, pack16<T>(o));
                }
            }
        }
    }
}

template <typename T, int S, int TH, int TW, int K1, int KT, int CC>
int launch_b2b_mfma(const KArgs& a, int grid, void* stream) {
    (void)hipGetLastError();
    hipLaunchKernelGGL((b2b_mfma_kernel<T, S, TH, TW, K1, KT, CC>), dim3(grid), dim3(256), 0,
                       (hipStream_t)stream, a);
    return (int)hipGetLastError();
}
template <typename T, int S, int TH, int TW, int K1, int KT, int CC>
int occ_b2b_mfma() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, b2b_mfma_kernel<T, S, TH, TW, K1, KT, CC>, 256, 0) != hipSuccess)
        return 0;
    return n;
}

// a.tiles_* / num_ptiles for the CV_TH x CV_TW tile, a.num_ktiles = ceil(K1 / CV_KT).
int launch_conv_lbl(int dtype, int stride, const KArgs& a, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    dim3 g((unsigned)(a.num_ptiles * a.num_ktiles));
    (void)hipGetLastError();
    using namespace lbl;
    if (dtype == 1) {
        if (stride == 1)
            hipLaunchKernelGGL((conv_lbl_kernel<_Float16, 1, CV_TH, CV_TW, CV_KT, CV_CC>), g,
                               dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((conv_lbl_kernel<_Float16, 2, CV_TH, CV_TW, CV_KT, CV_CC>), g,
                               dim3(256), 0, s, a);
    } else {
        if (stride == 1)
            hipLaunchKernelGGL((conv_lbl_kernel<__bf16, 1, CV_TH, CV_TW, CV_KT, CV_CC>), g,
                               dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((conv_lbl_kernel<__bf16, 2, CV_TH, CV_TW, CV_KT, CV_CC>), g,
                               dim3(256), 0, s, a);
    }
    return (int)hipGetLastError();
}

// explicit instances of every back-to-back variant listed in variants.def
#define FCM_V_DWPW(...)
#define FCM_V_DWPW32(...)
#define FCM_V_B2B(name, dt, CT, S, TH, TW, K1, KT, CC)                                   \
    template int launch_b2b_mfma<CT, S, TH, TW, K1, KT, CC>(const KArgs&, int, void*); \
    template int occ_b2b_mfma<CT, S, TH, TW, K1, KT, CC>();
#define FCM_V_DWPW_MM(...)
#define FCM_V_B2B_MM(...)
#define FCM_V_DWPW_MMW(...)
#include "../variants.def"
#undef FCM_V_DWPW
#undef FCM_V_DWPW32
#undef FCM_V_B2B
#undef FCM_V_DWPW_MM
#undef FCM_V_B2B_MM
#undef FCM_V_DWPW_MMW

}  // namespace fcm
