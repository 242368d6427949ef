// dwpw_mm.hip -- fused depthwise 3x3 -> pointwise 1x1 with BOTH convolutions on the
// gfx950 matrix cores (16-bit storage, C <= CC channels in one pass).
//
// The FCM DWPW module ("Fusing Depthwise and Pointwise Convolutions for Efficient
// Inference on GPUs", Sec. III, Fig. 3(b)) spends most of its non-memory work in the
// depthwise stencil.  On gfx950 the vector ALU is the scarce unit for that stencil
// (9 fp32 multiply-adds per intermediate value, plus both epilogues), while the matrix
// cores are idle outside the small pointwise GEMM.  This kernel therefore runs the
// depthwise layer as a matrix product too:
//
//   T'[c][p] = sum over (tap t, channel c') of Wdiag[c][(t, c')] * X[p + off_t][c'],
//   Wdiag[c][(t, c')] = w[t][c] if c' == c else 0,
//
// one v_mfma_f32_16x16x32 per 16 channels x 16 pixels x 2 taps (5 per 16x16 block for
// the 9 taps).  The B operand is 16 bytes of the LDS input tile per lane, exactly
// what a vector stencil would load; the block-diagonal A operand is built once from
// the depthwise filters.  Products of two 16-bit values are exact in fp32 and the
// accumulation is fp32, as in the vector version.
//
// Work split of a 4x16-pixel tile over the 4 waves of a workgroup:
//   phase A  wave w computes the depthwise layer of output row w (16 pixels, all CC
//            channels).  The result lands in the matrix unit's output layout -- lane
//            (l%16, l/16) holds channels 16*cb + 4*(l/16) + [0,4) of pixel l%16 -- and
//            two channel blocks give a lane 8 channels of its pixel: exactly the B
//            operand of the pointwise product when its reduction index is permuted the
//            same way.  After epilogue 1 and rounding to the storage type, each lane
//            writes its 16 bytes to the LDS intermediate tile (one contiguous 1 KB
//            block per wave and 32 channels, no bank conflicts).
//   phase B  wave w computes output channels [KT/4*w, KT/4*(w+1)) of the tile for all
//            four rows, reading the intermediate back as ready-made B operands.  Its
//            pointwise weights (the A operands) and epilogue-2 constants stay in
//            registers for the whole kernel.
// The intermediate thus lives only in LDS (the commBuffer of the page's design) and
// never reaches HBM.
//
// Input tiles arrive by direct global->LDS loads (buffer_load_dwordx4 ... lds): the
// next tile's halo is requested as soon as phase A of the current tile has finished
// reading the input buffer, so it streams in during phase B.  Out-of-image pixels (the
// zero padding) come back as zeros from the buffer resource's range check.  Each
// pixel's 16-byte channel chunks are XOR-swizzled so the 16 lanes of an operand read
// (16 consecutive pixels, same chunk) hit distinct LDS banks.  Outputs are written
// with buffer stores whose out-of-range lanes are dropped by the same range check, so
// every wave issues the same number of memory instructions per tile and the wait for
// the next tile's input can count them exactly (gfx9 vector memory operations
// complete in issue order).
#include <type_traits>

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

}  // namespace mm

template <typename T, int S, int TH, int TW, int KT, int CC, bool DWL, int OCC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC, 8)))
void dwpw_mm_kernel(KArgs a) {
    constexpr int NT = 256;
    static_assert(TH == 4 && TW == 16, "one 16-pixel output row per wave");
    constexpr int IH = (TH - 1) * S + 3, IW = (TW - 1) * S + 3, NPIX = IH * IW;
    constexpr int CH = CC / 8;  // 16-byte chunks per pixel
    static_assert(CH == 8 || CH == 16, "swizzle needs 8 or 16 chunks per pixel");
    constexpr int SLOTS = NPIX * CH;
    constexpr int R = (SLOTS + NT - 1) / NT;  // direct-load rounds per tile
    constexpr int SLOTS_P = R * NT;
    constexpr int NCB = CC / 16, NKS = CC / 32, NTP = 5;
    constexpr int KW = KT / 4;    // output channels per wave
    constexpr int KBW = KW / 16;  // 16-channel output blocks per wave
    static_assert(KT % 64 == 0, "each wave owns whole 16-channel output blocks");
    constexpr int NST = TH * (KBW / 2);  // buffer stores per lane per tile
    static_assert(KBW % 2 == 0 && NST < 64, "store count");

    __shared__ __attribute__((aligned(16))) u32x4 xs[SLOTS_P];                 // input tile
    __shared__ __attribute__((aligned(16))) u32x4 tls[TH * NKS * 64];          // intermediate
    __shared__ __attribute__((aligned(16))) u32x4 dwf[DWL ? NCB * NTP * 64 : 1];  // DW operand
    __shared__ __attribute__((aligned(16))) float s1s[CC], b1s[CC];
    __shared__ __attribute__((aligned(16))) T dws[9 * CC];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const Act act1 = act_bounds(a.act1), act2 = act_bounds(a.act2);
    const int G = gridDim.x;
    const int L = xcd_logical_id(blockIdx.x, G);
    const int k0 = (L % a.num_ktiles) * KT;
    const int kw0 = k0 + wave * KW;  // this wave's output channels
    const int pstep = G / a.num_ktiles;
    const int per_img = a.tiles_h * a.tiles_w;
    const T* __restrict__ wdw = (const T*)a.w1;
    const T* __restrict__ wpw = (const T*)a.w2;
    const uint32_t img_in_bytes = (uint32_t)(a.H * a.W * a.C) * (uint32_t)sizeof(T);
    const uint32_t img_out_bytes = (uint32_t)(a.Ho * a.Wo * a.K) * (uint32_t)sizeof(T);

    // ---- direct-load plan (tile invariant): slot -> source offset, window position ---
    int dl_off[R], dl_pos[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int s = r * NT + tid;
        const int p = s / CH, qs = s % CH;
        const int q = qs ^ (p & 7);
        const int ihl = p / IW, iwl = p % IW;
        dl_off[r] = (ihl * a.W + iwl) * a.C + q * 8;
        dl_pos[r] = (s < SLOTS && q * 8 < a.C) ? (ihl << 16) | iwl : 0x7fff7fff;
    }
    auto tile_origin = [&](int t, int* n, int* oh0, int* ow0) {
        *n = t / per_img;
        const int rem = t - *n * per_img;
        const int th = rem / a.tiles_w;
        *oh0 = th * TH;
        *ow0 = (rem - th * a.tiles_w) * TW;
    };
    auto issue_tile = [&](int t) {
        int n, oh0, ow0;
        tile_origin(t, &n, &oh0, &ow0);
        const T* img = (const T*)a.x + (int64_t)n * a.H * a.W * a.C;
        const __amdgpu_buffer_rsrc_t rs = mm::rsrc(img, img_in_bytes);
        const int ih0 = oh0 * S - a.pad_h, iw0 = ow0 * S - a.pad_w;
        const int base = (ih0 * a.W + iw0) * a.C;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int ih = ih0 + (dl_pos[r] >> 16), iw = iw0 + (dl_pos[r] & 0xffff);
            const bool ok = (unsigned)ih < (unsigned)a.H && (unsigned)iw < (unsigned)a.W;
            const uint32_t off = ok ? (uint32_t)(base + dl_off[r]) * (uint32_t)sizeof(T) : mm::kOob;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (__attribute__((address_space(3))) void*)(xs + r * NT + wave * 64), 16, off, 0,
                0, 0);
        }
    };

    // ---- constants ---------------------------------------------------------------------
    // depthwise filters [9][CC] and epilogue-1 arrays via LDS (one coalesced load)
    {
        constexpr int DI = (9 * CC + NT - 1) / NT;
        T tmp[DI];
#pragma unroll
        for (int i = 0; i < DI; ++i) {
            const int v = tid + i * NT;
            const int t = v / CC, c = v % CC;
            const bool ok = v < 9 * CC && c < a.C;
            const T val = wdw[ok ? t * a.C + c : 0];
            tmp[i] = ok ? val : (T)0.0f;
        }
#pragma unroll
        for (int i = 0; i < DI; ++i) {
            const int v = tid + i * NT;
            if (v < 9 * CC) dws[v] = tmp[i];
        }
        for (int i = tid; i < CC; i += NT) {
            const bool ok = i < a.C;
            const float sv = a.s1 ? a.s1[ok ? i : 0] : 1.0f;
            const float bv = a.b1 ? a.b1[ok ? i : 0] : 0.0f;
            s1s[i] = ok ? sv : 1.0f;
            b1s[i] = ok ? bv : 0.0f;
        }
    }
    // pointwise A operand of this wave's slice for reduction step ks, block kb: row
    // kperm<KW>(kb, l%16) of the slice, reduction channels 32ks + 4(l/16) + [0,4) and
    // 32ks + 16 + 4(l/16) + [0,4) (the order the depthwise result arrives in)
    u32x4 wa[NKS][KBW];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) {
            const int ko = kw0 + kperm<KW>(kb, lr), c = ks * 32 + lg * 4;
            const bool ok_lo = ko < a.K && c < a.C, ok_hi = ko < a.K && c + 16 < a.C;
            const T* row = wpw + (int64_t)(ko < a.K ? ko : 0) * a.C;
            const uint2 lo = *reinterpret_cast<const uint2*>(row + (ok_lo ? c : 0));
            const uint2 hi = *reinterpret_cast<const uint2*>(row + (ok_hi ? c + 16 : 0));
            wa[ks][kb] = u32x4{ok_lo ? lo.x : 0u, ok_lo ? lo.y : 0u, ok_hi ? hi.x : 0u,
                               ok_hi ? hi.y : 0u};
        }
    // epilogue-2 constants of the lane's output channels kw0 + (KW/4)(l/16) + [0,KW/4)
    float s2r[KW / 4], b2r[KW / 4];
#pragma unroll
    for (int i = 0; i < KW / 4; ++i) {
        const int k = kw0 + lg * (KW / 4) + i;
        const bool ok = k < a.K;
        const float sv = a.s2 ? a.s2[ok ? k : 0] : 1.0f;
        const float bv = a.b2 ? a.b2[ok ? k : 0] : 0.0f;
        s2r[i] = ok ? sv : 1.0f;
        b2r[i] = ok ? bv : 0.0f;
    }
    __syncthreads();  // dws / s1s / b1s visible
    // depthwise A operand (block diagonal) for channel block cb, tap pair tp: row l%16
    // = channel 16cb + l%16; reduction index 8(l/16) + j = (tap 2tp + (l/16)/2,
    // channel 8((l/16)&1) + j); non-zero only where that channel is the row's.
    const bool dw_active = (lr >> 3) == (lg & 1);
    const int dw_j = lr & 7;
    uint32_t dmask[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) dmask[i] = (i == (dw_j >> 1)) ? 0xffffffffu : 0u;
    auto dw_value = [&](int cb, int tp) -> uint32_t {
        const int t = 2 * tp + (lg >> 1);
        const uint16_t h = __builtin_bit_cast(uint16_t, dws[(t < 9 ? t : 0) * CC + cb * 16 + lr]);
        const uint32_t v = (dw_active && t < 9) ? (uint32_t)h : 0u;
        return (dw_j & 1) ? (v << 16) : v;
    };
    uint32_t wdc[DWL ? 1 : NCB][DWL ? 1 : NTP];
    if constexpr (DWL) {
        for (int f = wave; f < NCB * NTP; f += 4) {
            const uint32_t v = dw_value(f / NTP, f % NTP);
            dwf[f * 64 + lane] = u32x4{v & dmask[0], v & dmask[1], v & dmask[2], v & dmask[3]};
        }
    } else {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int tp = 0; tp < NTP; ++tp) wdc[cb][tp] = dw_value(cb, tp);
    }
    // LDS operand offsets of this lane's pixel (tile invariant): pixel index x chunks
    // and the chunk XOR of its swizzle, per tap pair; the 10th tap (tp 4, upper lanes)
    // reads a valid slot and is zeroed
    int xb_pix[NTP], xb_x[NTP];
    bool xb_ok[NTP];
#pragma unroll
    for (int tp = 0; tp < NTP; ++tp) {
        xb_ok[tp] = 2 * tp + (lg >> 1) < 9;
        const int t = xb_ok[tp] ? 2 * tp + (lg >> 1) : 0;
        const int p_in = (wave * S + t / 3) * IW + lr * S + t % 3;
        xb_pix[tp] = p_in * CH;
        xb_x[tp] = (lg & 1) ^ (p_in & 7);
    }
    __syncthreads();  // dwf visible; every wave is past its reads of dws

    // ---- persistent tile loop -------------------------------------------------------------
    int pt = L / a.num_ktiles;
    if (pt < a.num_ptiles) issue_tile(pt);
    bool first = true;
    for (; pt < a.num_ptiles; pt += pstep) {
        // this tile's input (issued before the previous tile's NST stores) has landed
        if (first) mm::wait_vmcnt<0>(); else mm::wait_vmcnt<NST>();
        first = false;
        __builtin_amdgcn_s_barrier();  // xs complete; every wave is done reading tls
        // phase A: depthwise on the matrix cores for this wave's 16-pixel row, epilogue
        // 1, and the result -- already in pointwise operand order -- to tls
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            f32x4 d[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int tp = 0; tp < NTP; ++tp) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int cb = 2 * ks + h;
                    u32x4 xb = xs[xb_pix[tp] + ((2 * cb) ^ xb_x[tp])];
                    if (!xb_ok[tp]) xb = u32x4{0u, 0u, 0u, 0u};
                    u32x4 wf;
                    if constexpr (DWL) {
                        wf = dwf[(cb * NTP + tp) * 64 + lane];
                    } else {
                        uint32_t v = wdc[cb][tp];
                        asm volatile("" : "+v"(v));  // rebuilt per use, not hoisted
                        wf = u32x4{v & dmask[0], v & dmask[1], v & dmask[2], v & dmask[3]};
                    }
                    d[h] = mfma<T>(wf, xb, d[h]);
                }
            }
            float o[8];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int c = (2 * ks + h) * 16 + lg * 4;
                const f32x4 sc = *reinterpret_cast<const f32x4*>(s1s + c);
                const f32x4 bi = *reinterpret_cast<const f32x4*>(b1s + c);
#pragma unroll
                for (int i = 0; i < 4; ++i) o[4 * h + i] = epilogue(d[h][i], sc[i], bi[i], act1);
            }
            tls[(wave * NKS + ks) * 64 + lane] = pack16<T>(o);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's tls writes done
        __builtin_amdgcn_s_barrier();       // tls complete; xs free
        if (pt + pstep < a.num_ptiles) issue_tile(pt + pstep);
        // phase B: pointwise on the matrix cores, this wave's KW output channels for all
        // TH rows of the tile, epilogue 2, 16-byte stores (64 contiguous bytes per pixel
        // per store instruction; out-of-range lanes dropped by the range check)
        int n, oh0, ow0;
        tile_origin(pt, &n, &oh0, &ow0);
        const __amdgpu_buffer_rsrc_t ry =
            mm::rsrc((const T*)a.y + (int64_t)n * a.Ho * a.Wo * a.K, img_out_bytes);
#pragma unroll
        for (int mb = 0; mb < TH; ++mb) {
            f32x4 acc[KBW];
#pragma unroll
            for (int kb = 0; kb < KBW; ++kb) acc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const u32x4 bfr = tls[(mb * NKS + ks) * 64 + lane];
#pragma unroll
                for (int kb = 0; kb < KBW; ++kb) acc[kb] = mfma<T>(wa[ks][kb], bfr, acc[kb]);
            }
            const int oh = oh0 + mb, ow = ow0 + lr;
            const bool pix_ok = oh < a.Ho && ow < a.Wo;
#pragma unroll
            for (int kb = 0; kb < KBW; kb += 2) {
                float o[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    o[i] = epilogue(acc[kb][i], s2r[kb * 4 + i], b2r[kb * 4 + i], act2);
                    o[4 + i] =
                        epilogue(acc[kb + 1][i], s2r[kb * 4 + 4 + i], b2r[kb * 4 + 4 + i], act2);
                }
                const int k = kw0 + lg * (KW / 4) + kb * 4;
                const bool ok = pix_ok && k < a.K;
                const uint32_t off =
                    ok ? (uint32_t)((oh * a.Wo + ow) * a.K + k) * (uint32_t)sizeof(T) : mm::kOob;
                __builtin_amdgcn_raw_buffer_store_b128(pack16<T>(o), ry, off, 0, 0);
            }
        }
    }
}

template <typename T, int S, int TH, int TW, int KT, int CC, bool DWL, int OCC>
int launch_dwpw_mm(const KArgs& a, int grid, void* stream) {
    (void)hipGetLastError();
    hipLaunchKernelGGL((dwpw_mm_kernel<T, S, TH, TW, KT, CC, DWL, OCC>), dim3(grid), dim3(256), 0,
                       (hipStream_t)stream, a);
    return (int)hipGetLastError();
}
template <typename T, int S, int TH, int TW, int KT, int CC, bool DWL, int OCC>
int occ_dwpw_mm() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, dwpw_mm_kernel<T, S, TH, TW, KT, CC, DWL, OCC>, 256, 0) != hipSuccess)
        return 0;
    return n;
}

#define FCM_V_DWPW(...)
#define FCM_V_DWPW32(...)
#define FCM_V_B2B(...)
#define FCM_V_DWPW_MM(name, dt, CT, S, TH, TW, KT, CC, DWL, OCC)                           \
    template int launch_dwpw_mm<CT, S, TH, TW, KT, CC, DWL, OCC>(const KArgs&, int, void*); \
    template int occ_dwpw_mm<CT, S, TH, TW, KT, CC, DWL, OCC>();
#include "../variants.def"
#undef FCM_V_DWPW
#undef FCM_V_DWPW32
#undef FCM_V_B2B
#undef FCM_V_DWPW_MM

}  // namespace fcm
