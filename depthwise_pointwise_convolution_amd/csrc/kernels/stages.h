// stages.h -- the depthwise stencil stage and the LDS staging steps, shared by the
// fused DWPW kernels and the layer-by-layer depthwise kernel (so the unfused baseline
// runs the same stage code, as the FCM paper's layer-by-layer comparison does,
// Sec. V-C).
#pragma once

#include "../kargs.h"
#include "common.h"

namespace fcm {

// The input halo tile of one channel chunk, global -> registers -> LDS.
// LDS layout: [IH][IW][XS] storage elements (XS >= CC; the tail of each pixel is
// padding that spreads the matrix-operand reads over the LDS banks).  Pixels outside
// the image (the zero padding of the convolution) and channels >= C are zeros.
// Loads are 16-byte vectors along the contiguous channel dimension; splitting the
// load from the LDS store lets a kernel issue the next tile's loads early and keep
// them in flight while it computes the current tile.
template <typename T, int IH, int IW, int CC, int NT>
struct HaloTile {
    static constexpr int VN = Vec<T>::N;
    static constexpr int CG = CC / VN;
    static constexpr int TOTAL = IH * IW * CG;
    static constexpr int ITERS = (TOTAL + NT - 1) / NT;
    u32x4 val[ITERS];

    __device__ __forceinline__ void load(const T* __restrict__ x, const KArgs& a, int n, int ih0,
                                         int iw0, int c0, int tid) {
        const T* xn = x + (int64_t)n * a.H * a.W * a.C;
#pragma unroll
        for (int i = 0; i < ITERS; ++i) {
            const int v = tid + i * NT;
            val[i] = u32x4{0u, 0u, 0u, 0u};
            if (v < TOTAL) {
                const int p = v / CG, cv = v - p * CG;
                const int ihl = p / IW, iwl = p - ihl * IW;
                const int ih = ih0 + ihl, iw = iw0 + iwl, c = c0 + cv * VN;
                if ((unsigned)ih < (unsigned)a.H && (unsigned)iw < (unsigned)a.W && c < a.C)
                    val[i] = ld16(xn + (ih * a.W + iw) * a.C + c);
            }
        }
    }
    template <int XS>
    __device__ __forceinline__ void store(T* xs, int tid) const {
#pragma unroll
        for (int i = 0; i < ITERS; ++i) {
            const int v = tid + i * NT;
            if (v < TOTAL) {
                const int p = v / CG, cv = v - p * CG;
                st16(xs + p * XS + cv * VN, val[i]);
            }
        }
    }
};

template <typename T, int IH, int IW, int CC, int XS, int NT>
__device__ __forceinline__ void stage_input(T* xs, const T* __restrict__ x, const KArgs& a,
                                            int n, int ih0, int iw0, int c0, int tid) {
    HaloTile<T, IH, IW, CC, NT> h;
    h.load(x, a, n, ih0, iw0, c0, tid);
    h.template store<XS>(xs, tid);
}

// Depthwise weights of one chunk as fp32 [9][CC], plus epilogue-1 scale/bias.
// Packed weight layout in memory: [9][C] storage elements.
template <typename T, int CC, int NT>
__device__ __forceinline__ void stage_dw_weights(float* wdw_s, float* s1s, float* b1s,
                                                 const T* __restrict__ w, const KArgs& a,
                                                 int c0, int tid) {
    for (int v = tid; v < 9 * CC; v += NT) {
        const int t = v / CC, c = c0 + (v - t * CC);
        wdw_s[v] = c < a.C ? (float)w[t * a.C + c] : 0.0f;
    }
    for (int i = tid; i < CC; i += NT) {
        const int c = c0 + i;
        s1s[i] = (a.s1 && c < a.C) ? a.s1[c] : 1.0f;
        b1s[i] = (a.b1 && c < a.C) ? a.b1[c] : 0.0f;
    }
}

// Depthwise 3x3 stencil + epilogue 1 over a TH x TW output tile and one CC-channel
// chunk held in LDS.  Work item = (channel vector of VN channels, one output column,
// VB vertically adjacent output rows): the item reads (VB-1)*S+3 input rows x 3
// columns of 16-byte vectors from LDS, so rows shared by its VB outputs are read once.
// fp32 multiply-adds in the fixed tap order (r, s) = (0,0), (0,1), ..., (2,2); the
// result after the epilogue is rounded to the storage type and handed to `sink(ohl,
// col, cg, packed)`.
template <typename T, int S, int TH, int TW, int CC, int XS, int IW, int VB, int NT,
          typename Sink>
__device__ __forceinline__ void dw_stage(const T* xs, const float* wdw_s, const float* s1s,
                                         const float* b1s, Act act1, int tid, Sink sink) {
    constexpr int VN = Vec<T>::N;
    constexpr int CG = CC / VN;
    constexpr int NITEM = TW * (TH / VB) * CG;
    constexpr int NR = (VB - 1) * S + 3;
    static_assert(TH % VB == 0, "vertical blocking must divide the tile height");
    for (int it = tid; it < NITEM; it += NT) {
        const int cg = it % CG;
        const int col = (it / CG) % TW;
        const int ohl0 = (it / (CG * TW)) * VB;
        float acc[VB][VN];
#pragma unroll
        for (int v = 0; v < VB; ++v)
#pragma unroll
            for (int j = 0; j < VN; ++j) acc[v][j] = 0.0f;
        const float* wv = wdw_s + cg * VN;
#pragma unroll
        for (int rr = 0; rr < NR; ++rr) {
#pragma unroll
            for (int s = 0; s < 3; ++s) {
                float xv[VN];
                unpack16<T>(ld16(xs + ((ohl0 * S + rr) * IW + col * S + s) * XS + cg * VN), xv);
#pragma unroll
                for (int v = 0; v < VB; ++v) {
                    const int r = rr - v * S;
                    if (r >= 0 && r < 3) {
#pragma unroll
                        for (int j = 0; j < VN; ++j)
                            acc[v][j] = __builtin_fmaf(xv[j], wv[(r * 3 + s) * CC + j], acc[v][j]);
                    }
                }
            }
        }
        float sc[VN], bi[VN];
#pragma unroll
        for (int j = 0; j < VN; ++j) {
            sc[j] = s1s[cg * VN + j];
            bi[j] = b1s[cg * VN + j];
        }
#pragma unroll
        for (int v = 0; v < VB; ++v) {
            float o[VN];
#pragma unroll
            for (int j = 0; j < VN; ++j) o[j] = epilogue(acc[v][j], sc[j], bi[j], act1);
            sink(ohl0 + v, col, cg, pack16<T>(o));
        }
    }
}

// Vertical blocking that gives each of NT threads about one depthwise work item.
template <int TH, int TW, int CG, int NT>
struct DwBlocking {
    static constexpr int raw = (TH * TW * CG) / NT;
    static constexpr int pick() {
        int vb = raw < 1 ? 1 : raw;
        while (vb > 1 && TH % vb != 0) --vb;
        return vb > TH ? TH : vb;
    }
    static constexpr int VB = pick();
};

}  // namespace fcm
