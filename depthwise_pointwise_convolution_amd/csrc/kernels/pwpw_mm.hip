// pwpw_mm.hip -- fused pointwise 1x1 -> pointwise 1x1 (the FCM PWPW module) on the gfx950
// matrix cores, 16-bit storage: a single-pass kernel for C <= 64 input and K1 <= 64
// intermediate channels, and a wide kernel (further down) for C <= CMAX and any K1.
//
// The PWPW fusion case of "Fusing Depthwise and Pointwise Convolutions for Efficient
// Inference on GPUs" (Sec. III, Table II) chains two 1x1 layers: two GEMMs over the
// channels of every pixel.  A pixel's output depends on that pixel alone, so a
// workgroup's tile is a run of PB x 16 consecutive pixels of the flattened N x H x W
// extent -- one contiguous block of memory, no halo -- and the intermediate never leaves
// the chip.
//
// Four waves; step i runs phase A of tile i+1 and phase B of tile i (two input and two
// intermediate buffers, one barrier per step, input tiles by direct global->LDS loads
// with exact vector-memory waits), as in the matrix-core DW->PW kernel:
//   phase A  wave w computes intermediate channels 16w .. 16w+15 of all PB pixel blocks:
//            one v_mfma_f32_16x16x32 per 16 channels x 16 pixels x 32 input channels
//            (A = the first layer's filters, register-resident; B = 16 bytes of the LDS
//            input tile per lane), epilogue 1, rounding, and 8 bytes per lane into the
//            LDS intermediate in the second layer's operand order;
//   phase B  wave w computes pixel blocks w*PB/4 .. for the workgroup's 64 output
//            channels with register-resident operands from the blocked filter copy
//            (output rows permuted so a lane ends with 8 consecutive channels), epilogue
//            2, 16-byte stores.
// Pixels past the end of the tensor come back as zeros from the buffer range check and
// their stores fall outside the output's range and are dropped.
#include <type_traits>

#include "mm_common.h"

namespace fcm {

template <typename T, int PB, int OCC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC, 8)))
void pwpw_mm_kernel(KArgs a) {
    constexpr int NT = 256, CC = 64, KT = 64, MP = PB * 16;
    constexpr int CH = CC / 8;                 // 16-byte chunks per pixel
    constexpr int SLOTS = MP * CH;
    constexpr int R = SLOTS / NT;              // direct-load rounds per tile
    static_assert(SLOTS % NT == 0, "whole load rounds");
    constexpr int NKC = CC / 32, NKS = 2;      // reduction steps of the two layers
    constexpr int MBW = PB / 4;                // pixel blocks per wave in phase B
    constexpr int NST = MBW * (KT / 32);       // stores per lane per step
    static_assert(PB % 4 == 0, "phase B splits the pixel blocks over four waves");

    __shared__ __attribute__((aligned(16))) u32x4 xs0[SLOTS];
    __shared__ __attribute__((aligned(16))) u32x4 xs1[SLOTS];
    __shared__ __attribute__((aligned(16))) u32x4 tl0[PB * NKS * 64];
    __shared__ __attribute__((aligned(16))) u32x4 tl1[PB * NKS * 64];
    u32x4* const X0 = xs0;
    u32x4* const X1 = xs1;
    u32x4* const T0 = tl0;
    u32x4* const T1 = tl1;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const Act act1 = act_bounds(a.act1), act2 = act_bounds(a.act2);
    const int G = gridDim.x;
    const int L = xcd_logical_id(blockIdx.x, G);
    const int k0 = (L % a.num_ktiles) * KT;
    const int es = (int)sizeof(T);
    const int64_t M = (int64_t)a.N * a.H * a.W;
    const __amdgpu_buffer_rsrc_t rx = mm::rsrc(a.x, (uint32_t)(M * a.C * es));
    const __amdgpu_buffer_rsrc_t ry = mm::rsrc(a.y, (uint32_t)(M * a.K * es));
    const int ntiles = a.num_ptiles;
    const int pstep = G / a.num_ktiles;

    // ---- direct-load plan: slot s holds chunk position s % CH of tile pixel p = s / CH,
    // i.e. input chunk q = (s % CH) ^ ((p >> 1) & 7), so the 16 lanes of an operand read
    // (16 consecutive pixels, one chunk) hit distinct bank groups; chunks past C load zero
    uint32_t dl_off[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int s = r * NT + tid;
        const int p = s / CH;
        const int q = (s % CH) ^ ((p >> 1) & 7);
        dl_off[r] = q * 8 < a.C ? (uint32_t)((p * a.C + q * 8) * es) : mm::kOob;
    }
    auto issue_tile = [&](int t, auto buf) __attribute__((always_inline)) {
        u32x4* dst = decltype(buf)::value == 0 ? X0 : X1;
        // past the last tile every lane gets the out-of-range offset (same op count)
        const bool live = t < ntiles;
        const int base = live ? t * MP * a.C * es : 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t off = live ? dl_off[r] : mm::kOob;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rx, (__attribute__((address_space(3))) void*)(dst + r * NT + wave * 64), 16, off,
                base, 0, 0);
        }
    };

    int cur = L / a.num_ktiles;
    int nxt = cur + pstep;
    issue_tile(cur, std::integral_constant<int, 0>{});

    // ---- constants -------------------------------------------------------------------
    // first layer, block w: lane (l%16, l/16) holds filter [16w + l%16][32kc + 8(l/16) ..]
    // (16 bytes of the plain [K1][C] filters; zero past K1 or C)
    const T* __restrict__ w1 = (const T*)a.w1;
    const int c1 = 16 * wave + lr;
    u32x4 a1[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
        const int ci = 32 * kc + 8 * lg;
        a1[kc] = *reinterpret_cast<const u32x4*>(w1 + (int64_t)(c1 < a.K1 ? c1 : 0) * a.C +
                                                 (ci < a.C ? ci : 0));
    }
    const float* s1p = a.s1 ? a.s1 : (const float*)a.w2;
    const float* b1p = a.b1 ? a.b1 : (const float*)a.w2;
    const float* s2p = a.s2 ? a.s2 : (const float*)a.w2;
    const float* b2p = a.b2 ? a.b2 : (const float*)a.w2;
    float s1r[4], b1r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = 16 * wave + 4 * lg + i, cc = c < a.K1 ? c : 0;
        s1r[i] = s1p[cc];
        b1r[i] = b1p[cc];
    }
    // second layer: blocked copy after the plain [K][K1] filters, block (32-channel
    // output group, reduction step, half) of 64 lanes x 8 elements, one 16-byte load
    const u32x4* __restrict__ wpb =
        reinterpret_cast<const u32x4*>((const T*)a.w2 + (int64_t)a.K * a.K1);
    const int s32 = (a.K1 + 31) / 32, g32n = (a.K + 31) / 32;
    u32x4 wa[NKS][4];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int g = min(k0 / 32 + kb / 2, g32n - 1);
            wa[ks][kb] = wpb[((g * s32 + min(ks, s32 - 1)) * 2 + (kb & 1)) * 64 + lane];
        }
    // epilogue-2 constants of the lane's output channels k0 + 32 g + 8(l/16) + j
    float s2r[2][8], b2r[2][8];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int k = k0 + 32 * g + 8 * lg + j, kk = k < a.K ? k : 0;
            s2r[g][j] = s2p[kk];
            b2r[g][j] = b2p[kk];
        }
    issue_tile(nxt, std::integral_constant<int, 1>{});

    // now the loaded values are used
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
        if (!(c1 < a.K1 && 32 * kc + 8 * lg < a.C)) a1[kc] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool ok = 16 * wave + 4 * lg + i < a.K1;
        s1r[i] = (a.s1 && ok) ? s1r[i] : 1.0f;
        b1r[i] = (a.b1 && ok) ? b1r[i] : 0.0f;
    }
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool ok = k0 + 32 * g + 8 * lg + j < a.K;
            s2r[g][j] = (a.s2 && ok) ? s2r[g][j] : 1.0f;
            b2r[g][j] = (a.b2 && ok) ? b2r[g][j] : 0.0f;
        }
    // phase A operand read of pixel block pb, step kc: pixel 16pb + l%16, chunk 4kc + l/16
    uint32_t xo[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
        const int q = 4 * kc + lg;
        xo[kc] = (uint32_t)((lr * CH + (q ^ ((lr >> 1) & 7))) * 16);
    }
    // intermediate: channels 16w + 4(l/16) + i of a pixel are channels 16(w%2) + 4(l/16) + i
    // of reduction step w/2, i.e. lane group 2(w%2) + (l/16)/2, bytes 8((l/16)%2) .. + 7
    const uint32_t tls_w = (uint32_t)(((2 * (wave & 1) + (lg >> 1)) * 16 + lr) * 16 + (lg & 1) * 8);
    // output store: lane part (pixel and channel group within a 16-pixel block; out of
    // range past K) plus a wave-uniform block part; any sum with an out-of-range part is
    // past the output (kept below 1 GiB by the planner), so the store is dropped, and no
    // per-lane condition reaches the store itself
    constexpr uint32_t kLaneOob = 0x40000000u, kRowOob = 0x80000000u;
    uint32_t st_lane[2];
#pragma unroll
    for (int g = 0; g < 2; ++g)
        st_lane[g] = k0 + 32 * g + 8 * lg < a.K ? (uint32_t)((lr * a.K + k0 + 32 * g + 8 * lg) * es)
                                                : kLaneOob;

    auto phase_a = [&](const u32x4* src, u32x4* dst) __attribute__((always_inline)) {
        const char* xb = reinterpret_cast<const char*>(src);
        u32x4 bx[PB][NKC];
#pragma unroll
        for (int pb = 0; pb < PB; ++pb)
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
                bx[pb][kc] = *reinterpret_cast<const u32x4*>(xb + pb * 16 * CH * 16 + xo[kc]);
        f32x4 d[PB];
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) {
            d[pb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) d[pb] = mfma<T>(a1[kc], bx[pb][kc], d[pb]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, PB * NKC, 0);  // operand reads
        __builtin_amdgcn_sched_group_barrier(0x008, PB * NKC, 0);  // products
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) {
            float o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = epilogue(d[pb][i], s1r[i], b1r[i], act1);
            st8(reinterpret_cast<char*>(dst) + ((pb * NKS + (wave >> 1)) * 64) * 16 + tls_w,
                pack8<T>(o));
        }
    };
    auto phase_b = [&](const u32x4* src, int t) __attribute__((always_inline)) {
        u32x4 bfr[MBW][NKS];
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                bfr[mb][ks] = src[((wave * MBW + mb) * NKS + ks) * 64 + lane];
        f32x4 acc[MBW][4];
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) acc[mb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    acc[mb][kb] = mfma<T>(wa[ks][kb], bfr[mb][ks], acc[mb][kb]);
        __builtin_amdgcn_sched_group_barrier(0x100, MBW * NKS, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, MBW * NKS * 4, 0);
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) {
            // pixels past the tensor fall past the output's range (below 1 GiB, checked by
            // the planner) and are dropped
            const uint32_t pix0 = t < ntiles
                                      ? (uint32_t)((t * MP + (wave * MBW + mb) * 16) * a.K * es)
                                      : kRowOob;
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                float o[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    o[i] = epilogue(acc[mb][2 * g][i], s2r[g][i], b2r[g][i], act2);
                    o[4 + i] = epilogue(acc[mb][2 * g + 1][i], s2r[g][4 + i], b2r[g][4 + i], act2);
                }
                // the whole offset in the vector operand, scalar offset 0
                __builtin_amdgcn_raw_buffer_store_b128(pack16<T>(o), ry, st_lane[g] + pix0, 0,
                                                       mm::kStoreStream);
            }
        }
    };

    // ---- software-pipelined tile loop -----------------------------------------------
    mm::wait_vmcnt<R>();
    __builtin_amdgcn_s_barrier();
    if (cur < ntiles) phase_a(X0, T0);
    auto step_fn = [&](auto par, bool first) __attribute__((always_inline)) {
        constexpr int P = decltype(par)::value;
        if (first) mm::wait_vmcnt<0>(); else mm::wait_vmcnt<NST>();
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): own intermediate writes done
        __builtin_amdgcn_s_barrier();
        const int nn = nxt + pstep;
        issue_tile(nn, std::integral_constant<int, P>{});
        if (nxt < ntiles) phase_a(P == 0 ? X1 : X0, P == 0 ? T1 : T0);
        phase_b(P == 0 ? T0 : T1, cur);
        cur = nxt;
        nxt = nn;
    };
    bool first = true;
    while (cur < ntiles) {
        step_fn(std::integral_constant<int, 0>{}, first);
        first = false;
        if (cur >= ntiles) break;
        step_fn(std::integral_constant<int, 1>{}, false);
    }
    mm::wait_vmcnt<0>();
}

// Wide PW->PW (MobileNetV2-style bottleneck pairs such as 24 -> 144 -> 24 and
// 96 -> 576 -> 96): C <= CMAX input channels, any number of intermediate channels in
// 64-channel slices, KT = 64 or 128 output channels per workgroup.  Four waves, tiles of
// 64 consecutive pixels; the whole input tile (all C channels) sits in LDS, the next
// tile's by direct global->LDS loads during the current one.  Per intermediate slice j:
//   phase A  wave w: intermediate channels 64j + 16w .. +15 of the four pixel blocks,
//            reduced over C in 32-channel steps (first-layer filters from the plain
//            [K1][C] array, 16 bytes per lane and step), epilogue 1, rounding, 8-byte
//            writes of the slice into an LDS buffer in the second layer's operand order
//            (two buffers, alternating by slice);
//   phase B  wave w: pixel block w, the workgroup's KT output channels: the slice's two
//            32-channel reduction steps accumulated in registers across the slices
//            (blocked filter copy, as in the single-pass kernel).
// One barrier per slice (after phase A); both layers' filters of a slice are requested
// at its start, so the second layer's arrive behind phase A.  After the last slice,
// epilogue 2 and 16-byte stores.  Channels past C or K1 come out as zeros (zero-filled
// input chunks, zero filters), so a partial last slice needs no special case.
template <typename T, int CMAX, int KT, int OCC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC, 8)))
void pwpw_wide_kernel(KArgs a) {
    constexpr int NT = 256, PB = 4, MP = PB * 16, CH = 8;
    constexpr int NSL = CMAX / 64;              // 64-channel slices of the input tile
    constexpr int SLOTS = NSL * MP * CH;
    constexpr int R = SLOTS / NT;               // direct-load rounds per tile
    static_assert(CMAX % 64 == 0 && SLOTS % NT == 0, "whole slices and load rounds");
    constexpr int NKC = CMAX / 32;              // first-layer reduction steps (at most)
    constexpr int NKS = 2;                      // second-layer reduction steps per slice
    constexpr int KBW = KT / 16;                // 16-channel output blocks per wave
    static_assert(KT == 64 || KT == 128, "64 or 128 output channels per workgroup");

    __shared__ __attribute__((aligned(16))) u32x4 xs0[SLOTS];
    __shared__ __attribute__((aligned(16))) u32x4 xs1[SLOTS];
    __shared__ __attribute__((aligned(16))) u32x4 tl0[PB * NKS * 64];
    __shared__ __attribute__((aligned(16))) u32x4 tl1[PB * NKS * 64];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const Act act1 = act_bounds(a.act1), act2 = act_bounds(a.act2);
    const int G = gridDim.x;
    const int L = xcd_logical_id(blockIdx.x, G);
    const int k0 = (L % a.num_ktiles) * KT;
    const int es = (int)sizeof(T);
    const int64_t M = (int64_t)a.N * a.H * a.W;
    const __amdgpu_buffer_rsrc_t rx = mm::rsrc(a.x, (uint32_t)(M * a.C * es));
    const __amdgpu_buffer_rsrc_t ry = mm::rsrc(a.y, (uint32_t)(M * a.K * es));
    const int ntiles = a.num_ptiles;
    const int pstep = G / a.num_ktiles;
    const int nkc = (a.C + 31) / 32;   // first-layer reduction steps of this problem
    const int nj = (a.K1 + 63) / 64;   // intermediate slices

    // ---- direct-load plan: slot s = (slice sl, pixel p, chunk position) holds input
    // chunk q = position ^ ((p >> 1) & 7) of the slice; chunks past C load zero
    uint32_t dl_off[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int s = r * NT + tid;
        const int sl = s / (MP * CH), p = (s / CH) % MP;
        const int q = (s % CH) ^ ((p >> 1) & 7);
        const int c = sl * 64 + q * 8;
        dl_off[r] = c < a.C ? (uint32_t)((p * a.C + c) * es) : mm::kOob;
    }
    auto issue_tile = [&](int t, u32x4* dst) __attribute__((always_inline)) {
        const bool live = t < ntiles;
        const int base = live ? t * MP * a.C * es : 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t off = live ? dl_off[r] : mm::kOob;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rx, (__attribute__((address_space(3))) void*)(dst + r * NT + wave * 64), 16, off,
                base, 0, 0);
        }
    };

    // ---- per-lane constants ------------------------------------------------------------
    const T* __restrict__ w1 = (const T*)a.w1;
    const u32x4* __restrict__ wpb =
        reinterpret_cast<const u32x4*>((const T*)a.w2 + (int64_t)a.K * a.K1);
    const int s32 = (a.K1 + 31) / 32, g32n = (a.K + 31) / 32;
    // epilogue-2 constants of the lane's output channels k0 + 32 g + 8(l/16) + j
    float s2r[KT / 32][8], b2r[KT / 32][8];
#pragma unroll
    for (int g = 0; g < KT / 32; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int k = k0 + 32 * g + 8 * lg + j;
            const bool ok = k < a.K;
            s2r[g][j] = (a.s2 && ok) ? a.s2[k] : 1.0f;
            b2r[g][j] = (a.b2 && ok) ? a.b2[k] : 0.0f;
        }
    // phase A operand read of step kc: pixel 16pb + l%16, chunk 4(kc%2) + l/16 of slice
    // kc/2 (pixel blocks add 16 * CH * 16 bytes, slices MP * CH * 16)
    uint32_t xo[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int q = 4 * h + lg;
        xo[h] = (uint32_t)((lr * CH + (q ^ ((lr >> 1) & 7))) * 16);
    }
    const uint32_t tls_w = (uint32_t)(((2 * (wave & 1) + (lg >> 1)) * 16 + lr) * 16 + (lg & 1) * 8);
    constexpr uint32_t kLaneOob = 0x40000000u, kRowOob = 0x80000000u;
    uint32_t st_lane[KT / 32];
#pragma unroll
    for (int g = 0; g < KT / 32; ++g)
        st_lane[g] = k0 + 32 * g + 8 * lg < a.K ? (uint32_t)((lr * a.K + k0 + 32 * g + 8 * lg) * es)
                                                : kLaneOob;

    // one tile: slices of the intermediate, then epilogue 2 and the stores
    auto tile = [&](int t, const u32x4* xsrc) __attribute__((always_inline)) {
        const char* xb = reinterpret_cast<const char*>(xsrc);
        f32x4 acc[KBW];
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) acc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < nj; ++j) {
            // both layers' filters of the slice
            const int c1 = 64 * j + 16 * wave + lr;
            u32x4 a1[NKC];
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                const int ci = 32 * kc + 8 * lg;
                a1[kc] = (kc < nkc && c1 < a.K1 && ci < a.C)
                             ? *reinterpret_cast<const u32x4*>(w1 + (int64_t)c1 * a.C + ci)
                             : u32x4{0u, 0u, 0u, 0u};
            }
            u32x4 wa[NKS][KBW];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int kb = 0; kb < KBW; ++kb) {
                    const int g = min(k0 / 32 + kb / 2, g32n - 1);
                    wa[ks][kb] = wpb[((g * s32 + min(2 * j + ks, s32 - 1)) * 2 + (kb & 1)) * 64 + lane];
                }
            float s1r[4], b1r[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = 64 * j + 16 * wave + 4 * lg + i;
                const bool ok = c < a.K1;
                s1r[i] = (a.s1 && ok) ? a.s1[c] : 1.0f;
                b1r[i] = (a.b1 && ok) ? a.b1[c] : 0.0f;
            }
            // phase A: the slice of the intermediate for the four pixel blocks
            f32x4 d[PB];
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) d[pb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                if (kc < nkc) {
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb) {
                        const u32x4 bx = *reinterpret_cast<const u32x4*>(
                            xb + (kc >> 1) * (MP * CH * 16) + pb * (16 * CH * 16) + xo[kc & 1]);
                        d[pb] = mfma<T>(a1[kc], bx, d[pb]);
                    }
                }
            }
            u32x4* tdst = (j & 1) ? tl1 : tl0;
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) {
                float o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = epilogue(d[pb][i], s1r[i], b1r[i], act1);
                st8(reinterpret_cast<char*>(tdst) + ((pb * NKS + (wave >> 1)) * 64) * 16 + tls_w,
                    pack8<T>(o));
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): own intermediate writes done
            __builtin_amdgcn_s_barrier();
            // phase B: pixel block `wave`, the slice's two reduction steps
            u32x4 bfr[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) bfr[ks] = tdst[(wave * NKS + ks) * 64 + lane];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int kb = 0; kb < KBW; ++kb) acc[kb] = mfma<T>(wa[ks][kb], bfr[ks], acc[kb]);
        }
        // pixels past the tensor fall past the output's range (below 1 GiB, checked by the
        // planner) and are dropped
        const uint32_t pix0 = t < ntiles ? (uint32_t)((t * MP + wave * 16) * a.K * es) : kRowOob;
#pragma unroll
        for (int g = 0; g < KT / 32; ++g) {
            float o[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                o[i] = epilogue(acc[2 * g][i], s2r[g][i], b2r[g][i], act2);
                o[4 + i] = epilogue(acc[2 * g + 1][i], s2r[g][4 + i], b2r[g][4 + i], act2);
            }
            // the whole offset in the vector operand, scalar offset 0
            __builtin_amdgcn_raw_buffer_store_b128(pack16<T>(o), ry, st_lane[g] + pix0, 0,
                                                   mm::kStoreStream);
        }
    };

    // ---- tile loop: the next tile's input is requested before the current one runs ---
    int cur = L / a.num_ktiles;
    issue_tile(cur, xs0);
    mm::wait_vmcnt<0>();
    int par = 0;
    while (cur < ntiles) {
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_s_barrier();  // every wave is done with the buffers the next
                                       // tile's loads and slices overwrite
        issue_tile(cur + pstep, par ? xs0 : xs1);
        tile(cur, par ? xs1 : xs0);
        mm::wait_vmcnt<0>();  // the next tile's input (and this tile's stores)
        cur += pstep;
        par ^= 1;
    }
}

template <typename T, int PB, int OCC, int CMAX, int KT>
int launch_pwpw_mm(const KArgs& a, int grid, void* stream) {
    (void)hipGetLastError();
    if constexpr (CMAX == 64)
        hipLaunchKernelGGL((pwpw_mm_kernel<T, PB, OCC>), dim3(grid), dim3(256), 0,
                           (hipStream_t)stream, a);
    else
        hipLaunchKernelGGL((pwpw_wide_kernel<T, CMAX, KT, OCC>), dim3(grid), dim3(256), 0,
                           (hipStream_t)stream, a);
    return (int)hipGetLastError();
}
template <typename T, int PB, int OCC, int CMAX, int KT>
int occ_pwpw_mm() {
    int n = 0;
    hipError_t e;
    if constexpr (CMAX == 64)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, pwpw_mm_kernel<T, PB, OCC>, 256, 0);
    else
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, pwpw_wide_kernel<T, CMAX, KT, OCC>,
                                                         256, 0);
    return e == hipSuccess ? n : 0;
}

#define FCM_V_DWPW(...)
#define FCM_V_DWPW32(...)
#define FCM_V_B2B(...)
#define FCM_V_B2B_MM(...)
#define FCM_V_DWPW_MM(...)
#define FCM_V_DWPW_MMW(...)
#define FCM_V_PWDW_MM(...)
#define FCM_V_DWPW_I8(...)
#define FCM_V_PWPW_MM(name, dt, CT, PB, OCC, CMAX, KT)                                  \
    template int launch_pwpw_mm<CT, PB, OCC, CMAX, KT>(const KArgs&, int, void*); \
    template int occ_pwpw_mm<CT, PB, OCC, CMAX, KT>();
#include "../variants.def"
#undef FCM_V_DWPW
#undef FCM_V_DWPW32
#undef FCM_V_B2B
#undef FCM_V_DWPW_MM
#undef FCM_V_B2B_MM
#undef FCM_V_DWPW_MMW
#undef FCM_V_PWDW_MM
#undef FCM_V_DWPW_I8
#undef FCM_V_PWPW_MM

}  // namespace fcm
