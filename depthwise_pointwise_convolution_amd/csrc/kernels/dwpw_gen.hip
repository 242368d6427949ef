// dwpw_gen.hip -- fused DW->PW module with a generalised depthwise layer: an FS x FS
// filter (3, 5 or 7), a dilation D between the taps and a depth multiplier M (M filters
// per input channel, so the depthwise layer has C*M outputs and the pointwise layer
// reduces over C*M channels).  The depthwise layer is the one the PyTorch forum thread
// "Using optimised depthwise convolutions" describes: a grouped convolution with one
// group per input channel, k outputs per group and any filter size, which its
// separable-convolution module also builds with a dilation; the fusion is the FCM
// paper's DWPW module ("Fusing Depthwise and Pointwise
// Convolutions for Efficient Inference on GPUs", Sec. III, Fig. 3(b)).
//
// One workgroup (4 waves) owns a TH x TW output tile and a KT-wide slice of the output
// channels and loops over such tiles (persistent grid).  Per tile and per chunk of CC
// input channels it
//   1. stages the input window ((TH-1)*S + (FS-1)*D + 1 rows, likewise columns) in LDS
//      with 16-byte NHWC loads, zero-filled outside the image; the input and depthwise
//      constants of a chunk are requested two chunks ahead (two register sets) and stay
//      in flight through the arithmetic in between, and a chunk's pointwise operands are
//      requested before its depthwise stage;
//   2. runs the depthwise stencil on the vector ALU in fp32: a work item takes 16 bytes
//      of input channels of one column and VB output rows, and produces the CC*M/CC
//      outputs of each of those channels (output channel c*M + i reads input channel
//      c), so every input value read from LDS feeds M filters and every input row
//      shared by the item's output rows is read once; epilogue 1, rounding to the
//      storage type, into the LDS intermediate tile [P][CC*M] -- never to HBM;
//   3. contracts the intermediate chunk with the pointwise filters on the matrix cores
//      (v_mfma_f32_16x16x32), fp32 accumulators in registers across the chunks;
// and finally applies epilogue 2 and writes the output tile with 16-byte stores.
// A layer-by-layer depthwise kernel with the same stencil stage (intermediate written
// to HBM) is the unfused baseline's first layer.
#include "../launchers.h"
#include "../lbl_tiles.h"
#include "stages.h"

namespace fcm {

// Depthwise filters of one chunk as fp32 [FS*FS][CC*M] (from the packed [FS*FS][C*M]
// array) and the chunk's epilogue-1 constants (C*M intermediate channels in all).
template <typename T, int FS, int M, int CC, int NT>
__device__ __forceinline__ void stage_dw_gen_weights(float* wdw_s, float* s1s, float* b1s,
                                                     const T* __restrict__ w, const KArgs& a,
                                                     int c0, int tid) {
    constexpr int CM = CC * M, TAPS = FS * FS;
    const int j0 = c0 * M;
    for (int v = tid; v < TAPS * CM; v += NT) {
        const int t = v / CM, j = j0 + (v - t * CM);
        wdw_s[v] = j < a.K1 ? (float)w[t * a.K1 + j] : 0.0f;
    }
    for (int i = tid; i < CM; i += NT) {
        const int j = j0 + i;
        s1s[i] = (a.s1 && j < a.K1) ? a.s1[j] : 1.0f;
        b1s[i] = (a.b1 && j < a.K1) ? a.b1[j] : 0.0f;
    }
}

// The same constants held in registers between their load and their LDS store, so a
// chunk's filters can be requested one chunk ahead (with its input window) and written
// to LDS at the start of the chunk: no load-wait-store round trip inside a chunk.
template <typename T, int FS, int M, int CC, int NT>
struct DwGenConsts {
    static constexpr int CM = CC * M, NW = FS * FS * CM;
    static constexpr int ITW = (NW + NT - 1) / NT, ITE = (CM + NT - 1) / NT;
    float w[ITW], sc[ITE], bi[ITE];

    __device__ __forceinline__ void load(const T* __restrict__ wg, const KArgs& a, int c0,
                                         int tid) {
        const int j0 = c0 * M;
#pragma unroll
        for (int i = 0; i < ITW; ++i) {
            const int v = tid + i * NT;
            const int t = v / CM, j = j0 + (v - t * CM);
            w[i] = (v < NW && j < a.K1) ? (float)wg[t * a.K1 + j] : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < ITE; ++i) {
            const int j = j0 + tid + i * NT;
            const bool in = tid + i * NT < CM && j < a.K1;
            sc[i] = (a.s1 && in) ? a.s1[j] : 1.0f;
            bi[i] = (a.b1 && in) ? a.b1[j] : 0.0f;
        }
    }
    __device__ __forceinline__ void store(float* wdw_s, float* s1s, float* b1s, int tid) const {
#pragma unroll
        for (int i = 0; i < ITW; ++i)
            if (tid + i * NT < NW) wdw_s[tid + i * NT] = w[i];
#pragma unroll
        for (int i = 0; i < ITE; ++i)
            if (tid + i * NT < CM) {
                s1s[tid + i * NT] = sc[i];
                b1s[tid + i * NT] = bi[i];
            }
    }
};

// Generalised depthwise stencil + epilogue 1 over a TH x TW tile and one CC-channel
// chunk in LDS.  Work item = (16-byte channel vector cg, output column, VB adjacent
// output rows).  Input row rr of the item's window feeds output row v with filter row
// (rr - v*S)/D when that is a whole number below FS; all of it is resolved at compile
// time.  fp32 multiply-adds in the fixed tap order (r, s) row-major.  The M outputs of
// each input channel are contiguous: the item hands M packed vectors to
// sink(ohl, col, cg*M + q, packed).
template <typename T, int S, int FS, int D, int M, int TH, int TW, int CC, int XS, int IW,
          int VB, int NT, typename Sink>
__device__ __forceinline__ void dw_gen_stage(const T* xs, const float* wdw_s, const float* s1s,
                                             const float* b1s, Act act1, int tid, Sink sink) {
    constexpr int VN = Vec<T>::N;
    constexpr int CG = CC / VN;
    constexpr int CM = CC * M;
    constexpr int NITEM = TW * (TH / VB) * CG;
    constexpr int NR = (VB - 1) * S + (FS - 1) * D + 1;
    static_assert(TH % VB == 0, "vertical blocking must divide the tile height");
    for (int it = tid; it < NITEM; it += NT) {
        const int cg = it % CG;
        const int col = (it / CG) % TW;
        const int ohl0 = (it / (CG * TW)) * VB;
        float acc[VB][VN * M];
#pragma unroll
        for (int v = 0; v < VB; ++v)
#pragma unroll
            for (int j = 0; j < VN * M; ++j) acc[v][j] = 0.0f;
        const float* wv = wdw_s + cg * VN * M;
#pragma unroll
        for (int rr = 0; rr < NR; ++rr) {
#pragma unroll
            for (int q = 0; q < FS; ++q) {
                float xv[VN];
                unpack16<T>(ld16(xs + ((ohl0 * S + rr) * IW + col * S + q * D) * XS + cg * VN),
                            xv);
#pragma unroll
                for (int v = 0; v < VB; ++v) {
                    const int rd = rr - v * S;
                    if (rd >= 0 && rd % D == 0 && rd / D < FS) {
                        const int r = rd / D;
#pragma unroll
                        for (int j = 0; j < VN * M; ++j)
                            acc[v][j] =
                                __builtin_fmaf(xv[j / M], wv[(r * FS + q) * CM + j], acc[v][j]);
                    }
                }
            }
        }
#pragma unroll
        for (int v = 0; v < VB; ++v) {
#pragma unroll
            for (int qv = 0; qv < M; ++qv) {
                float o[VN];
#pragma unroll
                for (int e = 0; e < VN; ++e) {
                    const int j = qv * VN + e, jl = cg * VN * M + j;
                    o[e] = epilogue(acc[v][j], s1s[jl], b1s[jl], act1);
                }
                sink(ohl0 + v, col, cg * M + qv, pack16<T>(o));
            }
        }
    }
}

template <typename T, int S, int FS, int D, int M, int TH, int TW, int KT, int CC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 8)))
void dwpw_gen_kernel(KArgs a) {
    constexpr int NT = 256;
    constexpr int VN = Vec<T>::N;
    static_assert(VN == 8, "matrix-core path is for 16-bit storage types");
    constexpr int P = TH * TW;
    static_assert(P % 64 == 0, "tile must give each wave whole 16-pixel blocks");
    constexpr int MBW = P / 64;  // 16-pixel blocks per wave
    constexpr int EXT = (FS - 1) * D + 1;  // input extent of one output's window
    constexpr int IH = (TH - 1) * S + EXT, IW = (TW - 1) * S + EXT;
    constexpr int CM = CC * M;             // intermediate channels per chunk
    constexpr int XS = CC + 8, TS = CM + 8;
    constexpr int KB = KT / 16, KSI = CM / 32;
    static_assert(KT % 32 == 0 && CM % 32 == 0 && CC % VN == 0, "tile sizes");
    constexpr int VB = DwBlocking<TH, TW, CC / VN, NT>::VB;

    __shared__ __attribute__((aligned(16))) T xs[IH * IW * XS];
    __shared__ __attribute__((aligned(16))) T ts[P * TS];
    __shared__ __attribute__((aligned(16))) float wdw_s[FS * FS * CM];
    __shared__ __attribute__((aligned(16))) float s1s[CM], b1s[CM];
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

    // The workgroup's steps are its (tile, chunk) pairs in order.  Two register sets
    // hold the input window and depthwise constants of the next two steps, so every
    // step's loads are issued two steps before it needs them (a step is short next to
    // a memory round trip when the chunks are many, as in wide layers).
    const int first = L / a.num_ktiles;
    const int my_tiles = first < a.num_ptiles ? (a.num_ptiles - 1 - first) / pstep + 1 : 0;
    const int nsteps = my_tiles * nchunks;
    auto tile_origin = [&](int t, int* n, int* oh0, int* ow0) {
        *n = t / per_img;
        const int rem = t - *n * per_img;
        const int th = rem / a.tiles_w;
        *oh0 = th * TH;
        *ow0 = (rem - th * a.tiles_w) * TW;
    };
    HaloTile<T, IH, IW, CC, NT> h0, h1;
    DwGenConsts<T, FS, M, CC, NT> d0, d1;
    auto issue = [&](HaloTile<T, IH, IW, CC, NT>& h, DwGenConsts<T, FS, M, CC, NT>& dc,
                     int st) __attribute__((always_inline)) {
        if (st < nsteps) {
            const int ti = st / nchunks, c0 = (st - ti * nchunks) * CC;
            int n, oh0, ow0;
            tile_origin(first + ti * pstep, &n, &oh0, &ow0);
            h.load(x, a, n, oh0 * S - a.pad_h, ow0 * S - a.pad_w, c0, tid);
            dc.load(wdw, a, c0, tid);
        }
    };
    issue(h0, d0, 0);
    issue(h1, d1, 1);
    for (int i = tid; i < KT; i += NT) {
        const int k = k0 + i;
        s2s[i] = (a.s2 && k < a.K) ? a.s2[k] : 1.0f;
        b2s[i] = (a.b2 && k < a.K) ? a.b2[k] : 0.0f;
    }

    f32x4 acc[MBW][KB];
    auto step = [&](HaloTile<T, IH, IW, CC, NT>& h, DwGenConsts<T, FS, M, CC, NT>& dc,
                    int st) __attribute__((always_inline)) {
        const int ti = st / nchunks, ci = st - ti * nchunks, c0 = ci * CC;
        if (ci == 0) {
#pragma unroll
            for (int mi = 0; mi < MBW; ++mi)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) acc[mi][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        h.template store<XS>(xs, tid);
        dc.store(wdw_s, s1s, b1s, tid);
        __syncthreads();
        // this chunk's pointwise operands are requested before the depthwise stage, which
        // hides their latency; then the loads of the step after next reuse h and dc
        const int j0 = c0 * M;
        u32x4 wa[KSI][KB];
#pragma unroll
        for (int ks = 0; ks < KSI; ++ks) {
            const int j = j0 + ks * 32 + lg * 8;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int ko = k0 + kperm<KT>(kb, lr);
                wa[ks][kb] = (ko < a.K && j < a.K1) ? ld16(wpw + (int64_t)ko * a.K1 + j)
                                                    : u32x4{0u, 0u, 0u, 0u};
            }
        }
        issue(h, dc, st + 2);
        dw_gen_stage<T, S, FS, D, M, TH, TW, CC, XS, IW, VB, NT>(
            xs, wdw_s, s1s, b1s, act1, tid, [&](int ohl, int col, int cgm, u32x4 v) {
                st16(ts + (ohl * TW + col) * TS + cgm * VN, v);
            });
        __syncthreads();
#pragma unroll
        for (int mi = 0; mi < MBW; ++mi) {
            const int row = (wave + 4 * mi) * 16 + lr;
#pragma unroll
            for (int ks = 0; ks < KSI; ++ks) {
                const u32x4 bfrag = ld16(ts + row * TS + ks * 32 + lg * 8);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    acc[mi][kb] = mfma<T>(wa[ks][kb], bfrag, acc[mi][kb]);
            }
        }
        // No barrier here: the next step's LDS stores (xs, wdw_s, s1s, b1s) target data
        // last read before the barrier above, and ts is rewritten only after the next
        // step's first barrier, which a wave reaches only once it is done reading ts.
        if (ci == nchunks - 1) {
            int n, oh0, ow0;
            tile_origin(first + ti * pstep, &n, &oh0, &ow0);
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
    };
    for (int st = 0; st < nsteps; st += 2) {
        step(h0, d0, st);
        if (st + 1 < nsteps) step(h1, d1, st + 1);
    }
}

// Layer-by-layer depthwise layer of the same shape: one workgroup per (tile, chunk),
// the same stencil stage, the C*M intermediate channels written to HBM.
template <typename T, int S, int FS, int D, int M, int TH, int TW, int CC>
__global__ __launch_bounds__(256) void dw_gen_lbl_kernel(KArgs a) {
    constexpr int NT = 256;
    constexpr int VN = Vec<T>::N;
    constexpr int EXT = (FS - 1) * D + 1;
    constexpr int IH = (TH - 1) * S + EXT, IW = (TW - 1) * S + EXT;
    constexpr int CM = CC * M;
    constexpr int XS = CC + 8;
    constexpr int VB = DwBlocking<TH, TW, CC / VN, NT>::VB;
    __shared__ __attribute__((aligned(16))) T xs[IH * IW * XS];
    __shared__ __attribute__((aligned(16))) float wdw_s[FS * FS * CM];
    __shared__ __attribute__((aligned(16))) float s1s[CM], b1s[CM];

    const int tid = threadIdx.x;
    const Act act1 = act_bounds(a.act1);
    const int nchunks = (a.C + CC - 1) / CC;
    const int b = blockIdx.x;
    const int pt = b / nchunks, c0 = (b - pt * nchunks) * CC;
    const int per_img = a.tiles_h * a.tiles_w;
    const int n = pt / per_img;
    const int rem = pt - n * per_img;
    const int th = rem / a.tiles_w, tw = rem - th * a.tiles_w;
    const int oh0 = th * TH, ow0 = tw * TW;
    T* __restrict__ t = (T*)a.y;

    stage_input<T, IH, IW, CC, XS, NT>(xs, (const T*)a.x, a, n, oh0 * S - a.pad_h,
                                       ow0 * S - a.pad_w, c0, tid);
    stage_dw_gen_weights<T, FS, M, CC, NT>(wdw_s, s1s, b1s, (const T*)a.w1, a, c0, tid);
    __syncthreads();
    dw_gen_stage<T, S, FS, D, M, TH, TW, CC, XS, IW, VB, NT>(
        xs, wdw_s, s1s, b1s, act1, tid, [&](int ohl, int col, int cgm, u32x4 v) {
            const int oh = oh0 + ohl, ow = ow0 + col, j = c0 * M + cgm * VN;
            if (oh < a.Ho && ow < a.Wo && j < a.K1)
                st16(t + (((int64_t)n * a.Ho + oh) * a.Wo + ow) * a.K1 + j, v);
        });
}

// ------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------
template <typename T, int S, int FS, int D, int M, int TH, int TW, int KT, int CC>
int launch_dwpw_gen(const KArgs& a, int grid, void* stream) {
    (void)hipGetLastError();
    hipLaunchKernelGGL((dwpw_gen_kernel<T, S, FS, D, M, TH, TW, KT, CC>), dim3(grid), dim3(256),
                       0, (hipStream_t)stream, a);
    return (int)hipGetLastError();
}
template <typename T, int S, int FS, int D, int M, int TH, int TW, int KT, int CC>
int occ_dwpw_gen() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, dwpw_gen_kernel<T, S, FS, D, M, TH, TW, KT, CC>, 256, 0) != hipSuccess)
        return 0;
    return n;
}
// The layer-by-layer depthwise kernel for the variant's (type, stride, filter,
// dilation, multiplier), with the baseline's own fixed tiling whatever the fused
// variant's chunk: the caller sets tiles_h / tiles_w for lbl::DWG_TH x lbl::DWG_TW tiles
// and launches num_ptiles * ceil(C / lbl::DWG_CC) workgroups.
template <typename T, int S, int FS, int D, int M, int TH, int TW, int KT, int CC>
int launch_dw_gen_lbl(const KArgs& a, int grid, void* stream) {
    (void)hipGetLastError();
    hipLaunchKernelGGL((dw_gen_lbl_kernel<T, S, FS, D, M, lbl::DWG_TH, lbl::DWG_TW, lbl::DWG_CC>),
                       dim3(grid),
                       dim3(256), 0, (hipStream_t)stream, a);
    return (int)hipGetLastError();
}

#define FCM_V_DWPW(...)
#define FCM_V_DWPW32(...)
#define FCM_V_B2B(...)
#define FCM_V_DWPW_MM(...)
#define FCM_V_B2B_MM(...)
#define FCM_V_DWPW_MMW(...)
#define FCM_V_DWPW_GEN(name, dt, CT, S, FS, D, M, TH, TW, KT, CC)                          \
    template int launch_dwpw_gen<CT, S, FS, D, M, TH, TW, KT, CC>(const KArgs&, int, void*); \
    template int occ_dwpw_gen<CT, S, FS, D, M, TH, TW, KT, CC>();                           \
    template int launch_dw_gen_lbl<CT, S, FS, D, M, TH, TW, KT, CC>(const KArgs&, int, void*);
#include "../variants.def"
#undef FCM_V_DWPW
#undef FCM_V_DWPW32
#undef FCM_V_B2B
#undef FCM_V_DWPW_MM
#undef FCM_V_B2B_MM
#undef FCM_V_DWPW_MMW
#undef FCM_V_DWPW_GEN

}  // namespace fcm
