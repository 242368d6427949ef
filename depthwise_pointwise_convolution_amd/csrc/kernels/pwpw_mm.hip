// pwpw_mm.hip -- fused pointwise 1x1 -> pointwise 1x1 (the FCM PWPW module) on the gfx950
// matrix cores, 16-bit storage, C <= 64 input and K1 <= 64 intermediate channels.
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
                __builtin_amdgcn_raw_buffer_store_b128(pack16<T>(o), ry, st_lane[g] + pix0, 0, 0);
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

template <typename T, int PB, int OCC>
int launch_pwpw_mm(const KArgs& a, int grid, void* stream) {
    (void)hipGetLastError();
    hipLaunchKernelGGL((pwpw_mm_kernel<T, PB, OCC>), dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       a);
    return (int)hipGetLastError();
}
template <typename T, int PB, int OCC>
int occ_pwpw_mm() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, pwpw_mm_kernel<T, PB, OCC>, 256, 0) !=
        hipSuccess)
        return 0;
    return n;
}

#define FCM_V_DWPW(...)
#define FCM_V_DWPW32(...)
#define FCM_V_B2B(...)
#define FCM_V_B2B_MM(...)
#define FCM_V_DWPW_MM(...)
#define FCM_V_DWPW_MMW(...)
#define FCM_V_PWDW_MM(...)
#define FCM_V_DWPW_I8(...)
#define FCM_V_PWPW_MM(name, dt, CT, PB, OCC)                                  \
    template int launch_pwpw_mm<CT, PB, OCC>(const KArgs&, int, void*); \
    template int occ_pwpw_mm<CT, PB, OCC>();
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
