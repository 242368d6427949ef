// dwpw.hip -- fused depthwise 3x3 -> pointwise 1x1 kernels for gfx950 (the FCM DWPW
// module, "Fusing Depthwise and Pointwise Convolutions for Efficient Inference on
// GPUs", Sec. III, Fig. 3(b)).
//
// One workgroup (4 waves) owns a TH x TW output tile and a KT-wide slice of the
// output channels, and loops over such tiles (persistent grid).  Per tile and per
// channel chunk of CC channels it
//   1. stages the input halo tile ((TH-1)*S+3 x (TW-1)*S+3 pixels) in LDS with
//      coalesced 16-byte NHWC loads, zero-filled outside the image;
//   2. runs the depthwise stencil + epilogue 1 on the VALU in fp32 and writes the
//      intermediate tile, rounded to the storage type, to an LDS buffer laid out so
//      that the matrix-core operand reads are bank-conflict free (the FCM paper's
//      commBuffer, Sec. III-B) -- it never reaches HBM;
//   3. contracts it with the pointwise weights on the matrix cores
//      (v_mfma_f32_16x16x32_{f16,bf16}); fp32 accumulators stay in registers
//      across chunks (output stationary);
// and finally applies epilogue 2 and writes the output tile with 16-byte stores.
// When the whole pointwise weight slice fits in registers (C <= CC) it is loaded
// once per workgroup and kept there for every tile (local weight stationary).
//
// The fp32 variant contracts the same kind of LDS intermediate (in fp32) with the
// fp32 matrix instruction, four reduction channels per instruction.
#include "stages.h"

namespace fcm {

template <typename T, int S, int TH, int TW, int KT, int CC, bool WRES, int OCC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC, 8)))
void dwpw_mfma_kernel(KArgs a) {
    constexpr int NT = 256;
    constexpr int VN = Vec<T>::N;
    static_assert(VN == 8, "matrix-core path is for 16-bit storage types");
    constexpr int P = TH * TW;
    static_assert(P % 64 == 0, "tile must give each wave whole 16-pixel blocks");
    constexpr int MBW = P / 64;  // 16-pixel blocks per wave
    constexpr int IH = (TH - 1) * S + 3, IW = (TW - 1) * S + 3;
    constexpr int XS = CC + 8, TS = CC + 8;
    constexpr int KB = KT / 16, KS = CC / 32;
    static_assert(KT % 32 == 0 && CC % 32 == 0, "tile sizes");
    constexpr int VB = DwBlocking<TH, TW, CC / VN, NT>::VB;

    __shared__ __attribute__((aligned(16))) T xs[IH * IW * XS];
    __shared__ __attribute__((aligned(16))) T ts[P * TS];
    __shared__ __attribute__((aligned(16))) float wdw_s[9 * CC];
    __shared__ __attribute__((aligned(16))) float s1s[CC], b1s[CC];
    __shared__ __attribute__((aligned(16))) float s2s[KT], b2s[KT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const Act act1 = act_bounds(a.act1), act2 = act_bounds(a.act2);
    const int lr = lane & 15, lg = lane >> 4;
    const int G = gridDim.x;
    const int L = xcd_logical_id(blockIdx.x, G);
    const int k0 = (L % a.num_ktiles) * KT;
    const int pstep = G / a.num_ktiles;
    const T* __restrict__ x = (const T*)a.x;
    const T* __restrict__ wdw = (const T*)a.w1;
    const T* __restrict__ wpw = (const T*)a.w2;
    T* __restrict__ y = (T*)a.y;
    const int per_img = a.tiles_h * a.tiles_w;
    const int nchunks = (a.C + CC - 1) / CC;

    // the first tile's input is requested before anything else
    HaloTile<T, IH, IW, CC, NT> halo;
    int pt = L / a.num_ktiles;
    auto tile_origin = [&](int t, int* n, int* oh0, int* ow0) {
        *n = t / per_img;
        const int rem = t - *n * per_img;
        const int th = rem / a.tiles_w;
        *oh0 = th * TH;
        *ow0 = (rem - th * a.tiles_w) * TW;
    };
    if (pt < a.num_ptiles) {
        int n, oh0, ow0;
        tile_origin(pt, &n, &oh0, &ow0);
        halo.load(x, a, n, oh0 * S - a.pad_h, ow0 * S - a.pad_w, 0, tid);
    }

    for (int i = tid; i < KT; i += NT) {
        const int k = k0 + i;
        s2s[i] = (a.s2 && k < a.K) ? a.s2[k] : 1.0f;
        b2s[i] = (a.b2 && k < a.K) ? a.b2[k] : 0.0f;
    }
    u32x4 wa[WRES ? KS : 1][WRES ? KB : 1];
    if constexpr (WRES) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int ko = k0 + kperm<KT>(kb, lr), c = ks * 32 + lg * 8;
                wa[ks][kb] = (ko < a.K && c < a.C) ? ld16(wpw + (int64_t)ko * a.C + c)
                                                   : u32x4{0u, 0u, 0u, 0u};
            }
        stage_dw_weights<T, CC, NT>(wdw_s, s1s, b1s, wdw, a, 0, tid);
    }

    for (; pt < a.num_ptiles; pt += pstep) {
        int n, oh0, ow0;
        tile_origin(pt, &n, &oh0, &ow0);
        f32x4 acc[MBW][KB];
#pragma unroll
        for (int mi = 0; mi < MBW; ++mi)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) acc[mi][kb] = f32x4{0.f, 0.f, 0.f, 0.f};

        for (int ci = 0; ci < nchunks; ++ci) {
            const int c0 = ci * CC;
            halo.template store<XS>(xs, tid);
            if constexpr (!WRES) stage_dw_weights<T, CC, NT>(wdw_s, s1s, b1s, wdw, a, c0, tid);
            __syncthreads();
            // software pipelining: request the next chunk (or the next tile's first
            // chunk) now; the loads stay in flight through this chunk's compute
            {
                int nt = pt, nc = c0 + CC;
                if (nc >= a.C) {
                    nt = pt + pstep;
                    nc = 0;
                }
                if (nt < a.num_ptiles) {
                    int nn, noh0, now0;
                    tile_origin(nt, &nn, &noh0, &now0);
                    halo.load(x, a, nn, noh0 * S - a.pad_h, now0 * S - a.pad_w, nc, tid);
                }
            }
            dw_stage<T, S, TH, TW, CC, XS, IW, VB, NT>(
                xs, wdw_s, s1s, b1s, act1, tid, [&](int ohl, int col, int cg, u32x4 v) {
                    st16(ts + (ohl * TW + col) * TS + cg * VN, v);
                });
            __syncthreads();
#pragma unroll
            for (int mi = 0; mi < MBW; ++mi) {
                const int row = (wave + 4 * mi) * 16 + lr;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const u32x4 bfrag = ld16(ts + row * TS + ks * 32 + lg * 8);
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        u32x4 afrag;
                        if constexpr (WRES) {
                            afrag = wa[ks][kb];
                        } else {
                            const int ko = k0 + kperm<KT>(kb, lr), c = c0 + ks * 32 + lg * 8;
                            afrag = (ko < a.K && c < a.C) ? ld16(wpw + (int64_t)ko * a.C + c)
                                                          : u32x4{0u, 0u, 0u, 0u};
                        }
                        acc[mi][kb] = mfma<T>(afrag, bfrag, acc[mi][kb]);
                    }
                }
            }
            // No barrier here: the next chunk's LDS stores (xs, wdw_s) target data last
            // read before the barrier above, and ts is rewritten only after the next
            // staging barrier, which a wave reaches only once it is done reading ts.
        }

#pragma unroll
        for (int mi = 0; mi < MBW; ++mi) {
            const int px = (wave + 4 * mi) * 16 + lr;
            const int oh = oh0 + px / TW, ow = ow0 + px % TW;
            if (oh < a.Ho && ow < a.Wo) {
                T* yp = y + (((int64_t)n * a.Ho + oh) * a.Wo + ow) * a.K + k0;
#pragma unroll
                for (int kb = 0; kb < KB; kb += 2) {
                    const int kl = lg * (KT / 4) + kb * 4;
                    if (k0 + kl < a.K) {
                        float o[8];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            o[i] = epilogue(acc[mi][kb][i], s2s[kl + i], b2s[kl + i], act2);
                            o[4 + i] = epilogue(acc[mi][kb + 1][i], s2s[kl + 4 + i],
                                                b2s[kl + 4 + i], act2);
                        }
                        st16(yp + kl, pack16<T>(o));
                    }
                }
            }
        }
    }
}

// fp32 storage: depthwise stage as above (4 channels per 16-byte vector) into an fp32
// LDS intermediate, pointwise contraction on the matrix cores with the fp32 instruction
// v_mfma_f32_16x16x4_f32 (the FP32 FCMs of the FCM paper, Sec. III-B).  Wave w owns the
// 16-pixel blocks w, w + 4, ... of the tile and all KT output channels of the slice.
// One 16-byte LDS read per lane supplies the pixel operand of four consecutive
// instructions: for a slab of 16 channels, instruction j takes channel 4 * g + j from
// lane group g = l / 16 (and the same channel of the weight operand), so the four
// instructions together reduce over the slab's 16 channels.
template <int S, int TH, int TW, int KT, int CC>
__global__ __launch_bounds__(256) void dwpw_f32_kernel(KArgs a) {
    typedef float T;
    constexpr int NT = 256;
    constexpr int VN = 4;
    constexpr int P = TH * TW;
    static_assert(P % 64 == 0, "tile must give each wave whole 16-pixel blocks");
    constexpr int MBW = P / 64;  // 16-pixel blocks per wave
    constexpr int IH = (TH - 1) * S + 3, IW = (TW - 1) * S + 3;
    // row stride of the intermediate: 36 floats = 4 mod 64 banks times an odd factor,
    // so the 16 rows x 4 lane groups of an operand read hit 64 distinct banks
    constexpr int XS = CC + 4, TS = CC + 4;
    static_assert(KT % 16 == 0 && CC % 16 == 0, "tile sizes");
    constexpr int KB = KT / 16, NSL = CC / 16;
    constexpr int VB = DwBlocking<TH, TW, CC / VN, NT>::VB;

    __shared__ __attribute__((aligned(16))) T xs[IH * IW * XS];
    __shared__ __attribute__((aligned(16))) float ts[P * TS];
    __shared__ __attribute__((aligned(16))) float wdw_s[9 * CC];
    __shared__ float s1s[CC], b1s[CC];
    __shared__ float s2s[KT], b2s[KT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const Act act1 = act_bounds(a.act1), act2 = act_bounds(a.act2);
    const int G = gridDim.x;
    const int L = xcd_logical_id(blockIdx.x, G);
    const int k0 = (L % a.num_ktiles) * KT;
    const int pstep = G / a.num_ktiles;
    const T* __restrict__ x = (const T*)a.x;
    const T* __restrict__ wdw = (const T*)a.w1;
    const T* __restrict__ wpw = (const T*)a.w2;
    T* __restrict__ y = (T*)a.y;
    for (int i = tid; i < KT; i += NT) {
        const int k = k0 + i;
        s2s[i] = (a.s2 && k < a.K) ? a.s2[k] : 1.0f;
        b2s[i] = (a.b2 && k < a.K) ? a.b2[k] : 0.0f;
    }

    const int per_img = a.tiles_h * a.tiles_w;
    for (int pt = L / a.num_ktiles; pt < a.num_ptiles; pt += pstep) {
        const int n = pt / per_img;
        const int rem = pt - n * per_img;
        const int th = rem / a.tiles_w, tw = rem - th * a.tiles_w;
        const int oh0 = th * TH, ow0 = tw * TW;
        f32x4 acc[MBW][KB];
#pragma unroll
        for (int mi = 0; mi < MBW; ++mi)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) acc[mi][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int c0 = 0; c0 < a.C; c0 += CC) {
            __syncthreads();  // previous chunk's readers of xs / ts are done
            stage_input<T, IH, IW, CC, XS, NT>(xs, x, a, n, oh0 * S - a.pad_h,
                                               ow0 * S - a.pad_w, c0, tid);
            stage_dw_weights<T, CC, NT>(wdw_s, s1s, b1s, wdw, a, c0, tid);
            // this chunk's weight operands: row kperm(kb, lr) of the slice, channels
            // c0 + 16 * sl + 4 * lg .. + 3 (zeros beyond K or C)
            u32x4 wa[NSL][KB];
#pragma unroll
            for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const int ko = k0 + kperm<KT>(kb, lr), c = c0 + sl * 16 + lg * 4;
                    wa[sl][kb] = (ko < a.K && c < a.C) ? ld16(wpw + (int64_t)ko * a.C + c)
                                                       : u32x4{0u, 0u, 0u, 0u};
                }
            __syncthreads();
            dw_stage<T, S, TH, TW, CC, XS, IW, VB, NT>(
                xs, wdw_s, s1s, b1s, act1, tid, [&](int ohl, int col, int cg, u32x4 v) {
                    st16(ts + (ohl * TW + col) * TS + cg * VN, v);
                });
            __syncthreads();
#pragma unroll
            for (int mi = 0; mi < MBW; ++mi) {
                const int row = (wave + 4 * mi) * 16 + lr;
#pragma unroll
                for (int sl = 0; sl < NSL; ++sl) {
                    const f32x4 bv = __builtin_bit_cast(f32x4, ld16(ts + row * TS + sl * 16 + lg * 4));
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        const f32x4 av = __builtin_bit_cast(f32x4, wa[sl][kb]);
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            acc[mi][kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                av[j], bv[j], acc[mi][kb], 0, 0, 0);
                    }
                }
            }
        }
        // lane (lr, lg) holds channels lg * KT/4 + 4 * kb + i of pixel row lr
#pragma unroll
        for (int mi = 0; mi < MBW; ++mi) {
            const int px = (wave + 4 * mi) * 16 + lr;
            const int oh = oh0 + px / TW, ow = ow0 + px % TW;
            if (oh < a.Ho && ow < a.Wo) {
                T* yp = y + (((int64_t)n * a.Ho + oh) * a.Wo + ow) * a.K + k0;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const int kl = lg * (KT / 4) + kb * 4;
                    if (k0 + kl < a.K) {
                        f32x4 o;
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            o[i] = epilogue(acc[mi][kb][i], s2s[kl + i], b2s[kl + i], act2);
                        st16(yp + kl, __builtin_bit_cast(u32x4, o));
                    }
                }
            }
        }
    }
}

// ------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------
template <typename T, int S, int TH, int TW, int KT, int CC, bool WRES, int OCC>
int launch_dwpw_mfma(const KArgs& a, int grid, void* stream) {
    (void)hipGetLastError();
    hipLaunchKernelGGL((dwpw_mfma_kernel<T, S, TH, TW, KT, CC, WRES, OCC>), dim3(grid),
                       dim3(256), 0, (hipStream_t)stream, a);
    return (int)hipGetLastError();
}
template <typename T, int S, int TH, int TW, int KT, int CC, bool WRES, int OCC>
int occ_dwpw_mfma() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, dwpw_mfma_kernel<T, S, TH, TW, KT, CC, WRES, OCC>, 256, 0) != hipSuccess)
        return 0;
    return n;
}
template <int S, int TH, int TW, int KT, int CC>
int launch_dwpw_f32(const KArgs& a, int grid, void* stream) {
    (void)hipGetLastError();
    hipLaunchKernelGGL((dwpw_f32_kernel<S, TH, TW, KT, CC>), dim3(grid), dim3(256), 0,
                       (hipStream_t)stream, a);
    return (int)hipGetLastError();
}
template <int S, int TH, int TW, int KT, int CC>
int occ_dwpw_f32() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, dwpw_f32_kernel<S, TH, TW, KT, CC>,
                                                     256, 0) != hipSuccess)
        return 0;
    return n;
}

// explicit instances of every DW->PW variant listed in variants.def
#define FCM_V_DWPW(name, dt, CT, S, TH, TW, KT, CC, WRES, OCC)                \
    template int launch_dwpw_mfma<CT, S, TH, TW, KT, CC, WRES, OCC>(const KArgs&, int, \
                                                                     void*);            \
    template int occ_dwpw_mfma<CT, S, TH, TW, KT, CC, WRES, OCC>();
#define FCM_V_DWPW32(name, S, TH, TW, KT, CC)                                  \
    template int launch_dwpw_f32<S, TH, TW, KT, CC>(const KArgs&, int, void*); \
    template int occ_dwpw_f32<S, TH, TW, KT, CC>();
#define FCM_V_B2B(...)
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
