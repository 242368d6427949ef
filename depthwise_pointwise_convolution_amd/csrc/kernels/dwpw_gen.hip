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
#include "mm_common.h"

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

// The loads of the fused kernel's steps (input window, depthwise constants, pointwise
// operands) are range-checked buffer loads that every lane issues whatever its position:
// positions outside the image, channels past the layer and steps past the workgroup's
// last one get the out-of-range offset and load zeros.  The compiler can then count the
// loads still in flight at each use; a load under a per-lane or per-step condition makes
// it wait for every outstanding load there instead, and the loads issued two steps
// ahead would no longer overlap anything.

// Input window of one channel chunk, global -> registers (-> LDS by store()).
template <typename T, int IH, int IW, int CC, int NT>
struct GenWindow {
    static constexpr int VN = Vec<T>::N;
    static constexpr int CG = CC / VN;
    static constexpr int TOTAL = IH * IW * CG;
    static constexpr int ITERS = (TOTAL + NT - 1) / NT;
    u32x4 val[ITERS];

    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rx, const KArgs& a, bool live,
                                         int n, int ih0, int iw0, int c0, int tid) {
        const int nb = live ? n : 0;
#pragma unroll
        for (int i = 0; i < ITERS; ++i) {
            const int v = tid + i * NT;
            const int p = v / CG, cv = v - p * CG;
            const int ihl = p / IW, iwl = p - ihl * IW;
            const int ih = ih0 + ihl, iw = iw0 + iwl, c = c0 + cv * VN;
            const bool ok = live && v < TOTAL && (unsigned)ih < (unsigned)a.H &&
                            (unsigned)iw < (unsigned)a.W && c < a.C;
            const uint32_t off =
                ok ? (uint32_t)(((nb * a.H + ih) * a.W + iw) * a.C + c) * (uint32_t)sizeof(T)
                   : mm::kOob;
            val[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
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

// Depthwise filters (fp32 [FS*FS][CC*M]) and epilogue-1 constants of one chunk, held in
// registers between their load and their LDS store.  A missing scale or bias array has
// an empty range (every load yields zero) and is replaced by 1 or 0 afterwards.
template <typename T, int FS, int M, int CC, int NT>
struct GenConsts {
    static constexpr int CM = CC * M, NW = FS * FS * CM;
    static constexpr int ITW = (NW + NT - 1) / NT, ITE = (CM + NT - 1) / NT;
    float w[ITW], sc[ITE], bi[ITE];

    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rs,
                                         __amdgpu_buffer_rsrc_t rb, const KArgs& a, int c0,
                                         int tid) {
        const int j0 = c0 * M;
#pragma unroll
        for (int i = 0; i < ITW; ++i) {
            const int v = tid + i * NT;
            const int t = v / CM, j = j0 + (v - t * CM);
            const bool ok = v < NW && j < a.K1;
            const uint32_t off = ok ? (uint32_t)(t * a.K1 + j) * (uint32_t)sizeof(T) : mm::kOob;
            const uint16_t h = __builtin_amdgcn_raw_buffer_load_b16(rw, off, 0, 0);
            w[i] = (float)__builtin_bit_cast(T, h);
        }
#pragma unroll
        for (int i = 0; i < ITE; ++i) {
            const int j = j0 + tid + i * NT;
            const bool in = tid + i * NT < CM && j < a.K1;
            const uint32_t off = in ? (uint32_t)j * 4u : mm::kOob;
            const float s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
            const float b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, off, 0, 0));
            sc[i] = (a.s1 && in) ? s : 1.0f;
            bi[i] = (a.b1 && in) ? b : 0.0f;
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

// NG channel groups of four waves share a workgroup's tile: group g takes the tile's
// chunks g, g + NG, ... with LDS buffers of its own, so a tile's chunk steps are NG
// times fewer and every SIMD holds NG waves of the tile (a wide layer with few tiles
// otherwise leaves one wave per SIMD, which waits out every latency of its steps).  At
// the tile's end the groups' pointwise sums are added into group 0's in group order,
// through LDS, and group 0 applies epilogue 2.
template <typename T, int S, int FS, int D, int M, int TH, int TW, int KT, int CC, int NG>
__global__ __launch_bounds__(256 * NG) __attribute__((amdgpu_waves_per_eu(2, 8)))
void dwpw_gen_kernel(KArgs a) {
    constexpr int NT = 256;  // threads of a channel group
    static_assert(NG == 1 || NG == 2, "one or two channel groups");
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
    constexpr int RED = NG > 1 ? 4 * 64 * MBW * KB : 1;  // partial sums of one group

    __shared__ __attribute__((aligned(16))) T xs[NG][IH * IW * XS];
    __shared__ __attribute__((aligned(16))) T ts[NG][P * TS];
    __shared__ __attribute__((aligned(16))) float wdw_s[NG][FS * FS * CM];
    __shared__ __attribute__((aligned(16))) float s1s[NG][CM], b1s[NG][CM];
    __shared__ __attribute__((aligned(16))) float s2s[KT], b2s[KT];
    __shared__ __attribute__((aligned(16))) f32x4 red[RED];

    const int tid = threadIdx.x, lane = tid & 63;
    const int g = tid / NT, tg = tid - g * NT;     // channel group, thread within it
    const int wave = (tid >> 6) & 3;               // wave within the group
    const Act act1 = act_bounds(a.act1), act2 = act_bounds(a.act2);
    const int lr = lane & 15, lg = lane >> 4;
    const int G = gridDim.x;
    const int L = xcd_logical_id(blockIdx.x, G);
    const int k0 = (L % a.num_ktiles) * KT;
    const int pstep = G / a.num_ktiles;
    const int es = (int)sizeof(T);
    const int per_img = a.tiles_h * a.tiles_w;
    const int nchunks = (a.C + CC - 1) / CC;
    const int nsub = (nchunks + NG - 1) / NG;      // chunk steps per tile
    const __amdgpu_buffer_rsrc_t rx = mm::rsrc(a.x, (uint32_t)(a.N * a.H * a.W * a.C * es));
    const __amdgpu_buffer_rsrc_t rw1 = mm::rsrc(a.w1, (uint32_t)(FS * FS * a.K1 * es));
    const __amdgpu_buffer_rsrc_t rs1 = mm::rsrc(a.s1, a.s1 ? (uint32_t)(a.K1 * 4) : 0u);
    const __amdgpu_buffer_rsrc_t rb1 = mm::rsrc(a.b1, a.b1 ? (uint32_t)(a.K1 * 4) : 0u);
    const __amdgpu_buffer_rsrc_t rw2 = mm::rsrc(a.w2, (uint32_t)(a.K * a.K1 * es));
    const __amdgpu_buffer_rsrc_t ry = mm::rsrc(a.y, (uint32_t)(a.N * a.Ho * a.Wo * a.K * es));
    T* const xsg = xs[g];
    T* const tsg = ts[g];
    float* const wdwg = wdw_s[g];
    float* const s1g = s1s[g];
    float* const b1g = b1s[g];

    // The workgroup's steps are its (tile, chunk step) pairs in order.  Two register
    // sets hold the input window and depthwise constants of the next two steps, so
    // every step's loads are issued two steps before it needs them (a step is short
    // next to a memory round trip when the chunks are many, as in wide layers).
    const int first = L / a.num_ktiles;
    const int my_tiles = first < a.num_ptiles ? (a.num_ptiles - 1 - first) / pstep + 1 : 0;
    const int nsteps = my_tiles * nsub;
    auto tile_origin = [&](int t, int* n, int* oh0, int* ow0) {
        *n = t / per_img;
        const int rem = t - *n * per_img;
        const int th = rem / a.tiles_w;
        *oh0 = th * TH;
        *ow0 = (rem - th * a.tiles_w) * TW;
    };
    GenWindow<T, IH, IW, CC, NT> h0, h1;
    GenConsts<T, FS, M, CC, NT> d0, d1;
    // (steps past the last one, and a group's chunk past the layer's last, load zeros:
    // the same loads on every step)
    auto issue = [&](GenWindow<T, IH, IW, CC, NT>& h, GenConsts<T, FS, M, CC, NT>& dc,
                     int st) __attribute__((always_inline)) {
        const int ti = st / nsub, ci = (st - ti * nsub) * NG + g, c0 = ci * CC;
        const bool live = st < nsteps && ci < nchunks;
        int n, oh0, ow0;
        tile_origin(first + ti * pstep, &n, &oh0, &ow0);
        h.load(rx, a, live, n, oh0 * S - a.pad_h, ow0 * S - a.pad_w, c0, tg);
        dc.load(rw1, rs1, rb1, a, c0, tg);
    };
    issue(h0, d0, 0);
    issue(h1, d1, 1);
    for (int i = tid; i < KT; i += NT * NG) {
        const int k = k0 + i;
        s2s[i] = (a.s2 && k < a.K) ? a.s2[k] : 1.0f;
        b2s[i] = (a.b2 && k < a.K) ? a.b2[k] : 0.0f;
    }

    f32x4 acc[MBW][KB];
    auto step = [&](GenWindow<T, IH, IW, CC, NT>& h, GenConsts<T, FS, M, CC, NT>& dc,
                    int st) __attribute__((always_inline)) {
        const int ti = st / nsub, si = st - ti * nsub, c0 = (si * NG + g) * CC;
        if (si == 0) {
#pragma unroll
            for (int mi = 0; mi < MBW; ++mi)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) acc[mi][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        h.template store<XS>(xsg, tg);
        dc.store(wdwg, s1g, b1g, tg);
        __syncthreads();
        // this chunk's pointwise operands are requested before the depthwise stage, which
        // hides their latency; then the loads of the step after next reuse h and dc
        // (a group whose chunk lies past the layer loads zeros and adds nothing)
        const int j0 = c0 * M;
        u32x4 wa[KSI][KB];
#pragma unroll
        for (int ks = 0; ks < KSI; ++ks) {
            const int j = j0 + ks * 32 + lg * 8;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int ko = k0 + kperm<KT>(kb, lr);
                const uint32_t off =
                    (ko < a.K && j < a.K1) ? (uint32_t)(ko * a.K1 + j) * (uint32_t)es : mm::kOob;
                wa[ks][kb] = __builtin_amdgcn_raw_buffer_load_b128(rw2, off, 0, 0);
            }
        }
        issue(h, dc, st + 2);
        dw_gen_stage<T, S, FS, D, M, TH, TW, CC, XS, IW, VB, NT>(
            xsg, wdwg, s1g, b1g, act1, tg, [&](int ohl, int col, int cgm, u32x4 v) {
                st16(tsg + (ohl * TW + col) * TS + cgm * VN, v);
            });
        __syncthreads();
#pragma unroll
        for (int mi = 0; mi < MBW; ++mi) {
            const int row = (wave + 4 * mi) * 16 + lr;
#pragma unroll
            for (int ks = 0; ks < KSI; ++ks) {
                const u32x4 bfrag = ld16(tsg + row * TS + ks * 32 + lg * 8);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    acc[mi][kb] = mfma<T>(wa[ks][kb], bfrag, acc[mi][kb]);
            }
        }
        // No barrier here: the next step's LDS stores (xs, wdw_s, s1s, b1s) target data
        // last read before the barrier above, and ts is rewritten only after the next
        // step's first barrier, which a wave reaches only once it is done reading ts.
        const bool fin = si == nsub - 1;
        if constexpr (NG > 1) {
            if (fin) {
                // group 1's sums into group 0's (red was last read a tile ago, before
                // the barriers of the steps since)
                if (g == 1) {
#pragma unroll
                    for (int mi = 0; mi < MBW; ++mi)
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb)
                            red[((mi * KB + kb) * 4 + wave) * 64 + lane] = acc[mi][kb];
                }
                __syncthreads();
                if (g == 0) {
#pragma unroll
                    for (int mi = 0; mi < MBW; ++mi)
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb) {
                            const f32x4 o = red[((mi * KB + kb) * 4 + wave) * 64 + lane];
#pragma unroll
                            for (int i = 0; i < 4; ++i) acc[mi][kb][i] += o[i];
                        }
                }
                __syncthreads();
            }
        }
        // The output stores go out on every step and from every group, with the
        // out-of-range offset (dropped) except for group 0 at a tile's last chunk step,
        // so that every step issues the same memory operations.
        const bool out = fin && g == 0;
        int n, oh0, ow0;
        tile_origin(first + ti * pstep, &n, &oh0, &ow0);
#pragma unroll
        for (int mi = 0; mi < MBW; ++mi) {
            const int px = (wave + 4 * mi) * 16 + lr;
            const int oh = oh0 + px / TW, ow = ow0 + px % TW;
            const bool pix_ok = out && oh < a.Ho && ow < a.Wo;
            const int pbase =
                ((n * a.Ho + (pix_ok ? oh : 0)) * a.Wo + (pix_ok ? ow : 0)) * a.K + k0;
#pragma unroll
            for (int kb = 0; kb < KB; kb += 2) {
                const int kl = lg * (KT / 4) + kb * 4;
                u32x4 ov = u32x4{0u, 0u, 0u, 0u};
                if (out) {
                    float o[8];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        o[i] = epilogue(acc[mi][kb][i], s2s[kl + i], b2s[kl + i], act2);
                        o[4 + i] = epilogue(acc[mi][kb + 1][i], s2s[kl + 4 + i],
                                            b2s[kl + 4 + i], act2);
                    }
                    ov = pack16<T>(o);
                }
                const uint32_t off = (pix_ok && k0 + kl < a.K)
                                         ? (uint32_t)(pbase + kl) * (uint32_t)es
                                         : mm::kOob;
                __builtin_amdgcn_raw_buffer_store_b128(ov, ry, off, 0, 0);
                // one wait state before anything may write the store's data registers
                // (the compiler schedules the next step's LDS reads into them otherwise)
                asm volatile("s_nop 0" ::: "memory");
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
template <typename T, int S, int FS, int D, int M, int TH, int TW, int KT, int CC, int NG>
int launch_dwpw_gen(const KArgs& a, int grid, void* stream) {
    (void)hipGetLastError();
    hipLaunchKernelGGL((dwpw_gen_kernel<T, S, FS, D, M, TH, TW, KT, CC, NG>), dim3(grid),
                       dim3(256 * NG), 0, (hipStream_t)stream, a);
    return (int)hipGetLastError();
}
template <typename T, int S, int FS, int D, int M, int TH, int TW, int KT, int CC, int NG>
int occ_dwpw_gen() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, dwpw_gen_kernel<T, S, FS, D, M, TH, TW, KT, CC, NG>, 256 * NG, 0) != hipSuccess)
        return 0;
    return n;
}
// The layer-by-layer depthwise kernel for the variant's (type, stride, filter,
// dilation, multiplier), with the baseline's own fixed tiling whatever the fused
// variant's chunk: the caller sets tiles_h / tiles_w for lbl::DWG_TH x lbl::DWG_TW tiles
// and launches num_ptiles * ceil(C / lbl::DWG_CC) workgroups.
template <typename T, int S, int FS, int D, int M, int TH, int TW, int KT, int CC, int NG>
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
#define FCM_V_DWPW_GEN(name, dt, CT, S, FS, D, M, TH, TW, KT, CC, NG)                          \
    template int launch_dwpw_gen<CT, S, FS, D, M, TH, TW, KT, CC, NG>(const KArgs&, int, void*); \
    template int occ_dwpw_gen<CT, S, FS, D, M, TH, TW, KT, CC, NG>();                           \
    template int launch_dw_gen_lbl<CT, S, FS, D, M, TH, TW, KT, CC, NG>(const KArgs&, int, void*);
#include "../variants.def"
#undef FCM_V_DWPW
#undef FCM_V_DWPW32
#undef FCM_V_B2B
#undef FCM_V_DWPW_MM
#undef FCM_V_B2B_MM
#undef FCM_V_DWPW_MMW
#undef FCM_V_DWPW_GEN

}  // namespace fcm
