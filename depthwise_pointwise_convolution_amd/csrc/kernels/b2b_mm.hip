// b2b_mm.hip -- back-to-back standard 3x3 conv -> 1x1 conv ("Fusing two back-to-back
// convolutions": block-resident fusion, the second conv 1x1) for up to 64 channels in
// each layer, both convolutions on the gfx950 matrix cores, with the input pipeline of
// the matrix-core DW->PW kernel (dwpw_mm.hip): direct global->LDS loads of 4x16-pixel
// tiles plus halo, XOR-swizzled chunks, two input and two intermediate buffers, one
// barrier per software-pipelined step.
//
// Step s runs phase A of tile s+1 and phase B of tile s:
//   phase A  the 3x3 conv as an implicit GEMM whose reduction index runs over (tap,
//            32-channel half): 18 steps of v_mfma_f32_16x16x32.  Wave w owns
//            intermediate channels [16w, 16w+16) of all 4 rows; its 18 filter operands
//            stay in registers for the whole kernel (the "weights resident" end of the
//            CUTLASS discussion's design space), the 16-pixel input operands are read
//            from the LDS tile.  Epilogue 1, rounding, and 8 bytes per lane into the LDS
//            intermediate tile in 1x1-operand order (the accumulator -> operand
//            hand-off, through LDS because a wave holds only 16 of the 64 channels).
//   phase B  the 1x1 conv: wave w owns output row w, all (up to 64) output channels,
//            with resident filter operands; epilogue 2; two 16-byte stores per lane.
#include <type_traits>

#include "mm_common.h"

namespace fcm {

// Matrix products of the 3x3 convolution that use input row IR of the tile window:
// six operands (three filter columns, two channel halves), each applied to every output
// row r = (IR - dh) / S it feeds.
template <int S, int TH, int IR>
__device__ constexpr int b2b_row_products() {
    int n = 0;
    for (int dh = 0; dh < 3; ++dh)
        if (IR - dh >= 0 && (IR - dh) % S == 0 && (IR - dh) / S < TH) n += 6;
    return n;
}
// Scheduling groups for phase A (compiler scheduling hints only, no effect on results):
// the six LDS operand reads of row IR + 1, then the products of row IR, for every row,
// so that each row's reads are in flight while the previous row's products run.
template <int S, int TH, int IR, int IH>
__device__ __forceinline__ void b2b_sched_rows() {
    if constexpr (IR + 1 < IH) __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
    if constexpr (b2b_row_products<S, TH, IR>() > 0)
        __builtin_amdgcn_sched_group_barrier(0x008, b2b_row_products<S, TH, IR>(), 0);
    if constexpr (IR + 1 < IH) b2b_sched_rows<S, TH, IR + 1, IH>();
}

template <typename T, int S, int OCC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC, 8)))
void b2b_mm_kernel(KArgs a) {
    constexpr int NT = 256, TH = 4, TW = 16, CC = 64, K1T = 64, KT = 64;
    constexpr int IH = (TH - 1) * S + 3, IW = (TW - 1) * S + 3, NPIX = IH * IW;
    constexpr int CH = CC / 8;
    constexpr int SLOTS = NPIX * CH;
    constexpr int R = (SLOTS + NT - 1) / NT;
    constexpr int SLOTS_P = R * NT;
    constexpr int NK1 = 18;              // reduction steps of the 3x3 conv: 9 taps x 2
    constexpr int NKS2 = K1T / 32;       // reduction steps of the 1x1 conv
    constexpr int KB2 = KT / 16;         // 16-channel output blocks of a wave's row
    constexpr int NST = 2;               // stores per lane per step

    __shared__ __attribute__((aligned(16))) u32x4 xs0[SLOTS_P];
    __shared__ __attribute__((aligned(16))) u32x4 xs1[SLOTS_P];
    __shared__ __attribute__((aligned(16))) u32x4 tl0[TH * NKS2 * 64];
    __shared__ __attribute__((aligned(16))) u32x4 tl1[TH * NKS2 * 64];
    u32x4* const X0 = xs0;
    u32x4* const X1 = xs1;
    u32x4* const T0 = tl0;
    u32x4* const T1 = tl1;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const Act act1 = act_bounds(a.act1), act2 = act_bounds(a.act2);
    const int G = gridDim.x;
    const int L = xcd_logical_id(blockIdx.x, G);
    const T* __restrict__ w1 = (const T*)a.w1;
    const T* __restrict__ w2 = (const T*)a.w2;
    const int es = (int)sizeof(T);
    const __amdgpu_buffer_rsrc_t rx = mm::rsrc(a.x, (uint32_t)(a.N * a.H * a.W * a.C * es));
    const __amdgpu_buffer_rsrc_t ry = mm::rsrc(a.y, (uint32_t)(a.N * a.Ho * a.Wo * a.K * es));
    const int in_img = a.H * a.W * a.C * es, in_row = a.W * a.C * es;
    const int out_img = a.Ho * a.Wo * a.K * es, out_row = a.Wo * a.K * es;

    // ---- tile walk (one output-channel tile: the grid is the pixel-tile step) --------
    const int pstep = G;
    using Pos = mm::TilePos;
    auto derive = [&](Pos& p) {
        p.oh0 = p.th * TH;
        p.ow0 = p.tw * TW;
        p.ih0 = p.oh0 * S - a.pad_h;
        p.iw0 = p.ow0 * S - a.pad_w;
        p.in_base = p.n * in_img + p.ih0 * in_row + p.iw0 * a.C * es;
        p.out_base = p.n * out_img + p.oh0 * out_row + p.ow0 * a.K * es;
    };
    auto split = [&](int t) {
        Pos p;
        const int per_img = a.tiles_h * a.tiles_w;
        p.n = t / per_img;
        const int rem = t - p.n * per_img;
        p.th = rem / a.tiles_w;
        p.tw = rem - p.th * a.tiles_w;
        derive(p);
        return p;
    };
    const Pos step = split(pstep);
    auto advance = [&](Pos p) {
        p.tw += step.tw;
        if (p.tw >= a.tiles_w) {
            p.tw -= a.tiles_w;
            ++p.th;
        }
        p.th += step.th;
        if (p.th >= a.tiles_h) {
            p.th -= a.tiles_h;
            ++p.n;
        }
        p.n += step.n;
        derive(p);
        return p;
    };

    // ---- direct-load plan: slot s = chunk q of window pixel s / CH, s % CH = q ^ (col & 7)
    uint32_t dl_off[R];
    int dl_pos[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int s = r * NT + tid;
        const int p = s / CH, ihl = p / IW, iwl = p % IW;
        const int q = (s % CH) ^ (iwl & 7);
        const bool real = s < SLOTS && q * 8 < a.C;
        dl_off[r] = real ? (uint32_t)((ihl * a.W + iwl) * a.C + q * 8) * (uint32_t)es : mm::kOob;
        dl_pos[r] = real ? (ihl << 16) | iwl : 0;
    }
    auto issue_tile = [&](const Pos& t, auto buf) {
        u32x4* dst = decltype(buf)::value == 0 ? X0 : X1;
        const bool live = t.n < a.N;
        const bool inside = live && t.ih0 >= 0 && t.iw0 >= 0 && t.ih0 + IH <= a.H &&
                            t.iw0 + IW <= a.W;
        if (inside) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t off = dl_off[r];  // (a copy, see dwpw_mm.hip)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rx, (__attribute__((address_space(3))) void*)(dst + r * NT + wave * 64), 16,
                    off, t.in_base, 0, 0);
            }
        } else {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int ih = t.ih0 + (dl_pos[r] >> 16), iw = t.iw0 + (dl_pos[r] & 0xffff);
                const bool ok = live && dl_off[r] != mm::kOob && (unsigned)ih < (unsigned)a.H &&
                                (unsigned)iw < (unsigned)a.W;
                const uint32_t off = ok ? (uint32_t)(t.in_base + (int)dl_off[r]) : mm::kOob;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rx, (__attribute__((address_space(3))) void*)(dst + r * NT + wave * 64), 16,
                    off, 0, 0, 0);
            }
        }
    };

    // the first two tiles' input goes out before anything else, so that its latency
    // overlaps that of the resident operands below
    Pos cur = split(L);
    Pos nxt = advance(cur);
    issue_tile(cur, std::integral_constant<int, 0>{});
    issue_tile(nxt, std::integral_constant<int, 1>{});

    // ---- resident operands -------------------------------------------------------------
    // 3x3 filters of intermediate channels [16w, 16w+16): operand of reduction step
    // ks = (tap ks/2, channel half ks%2) is block (w, ks/2, ks%2) of the blocked copy
    // after the plain [K1][9][C] array (one contiguous kilobyte, zero where the channel
    // does not exist); lane (l%16, l/16): channel 16w + l%16, input channels
    // 32(ks%2) + 8(l/16) + [0,8)
    const u32x4* __restrict__ w1b =
        reinterpret_cast<const u32x4*>(w1 + (int64_t)a.K1 * 9 * a.C);
    // a wave whose 16 channels lie past K1 gets zero operands: its intermediate channels
    // are then exactly 0, which the clamped 1x1 operands below rely on
    const bool w1live = 16 * wave < a.K1;
    const int w1g = w1live ? wave : 0;
    u32x4 wa1[NK1];
#pragma unroll
    for (int ks = 0; ks < NK1; ++ks) wa1[ks] = w1b[(w1g * NK1 + ks) * 64 + lane];
    if (!w1live) {
#pragma unroll
        for (int ks = 0; ks < NK1; ++ks) wa1[ks] = u32x4{0u, 0u, 0u, 0u};
    }
    float s1r[4], b1r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int k1 = 16 * wave + 4 * lg + i;
        const bool ok = k1 < a.K1;
        const float sv = a.s1 ? a.s1[ok ? k1 : 0] : 1.0f;
        const float bv = a.b1 ? a.b1[ok ? k1 : 0] : 0.0f;
        s1r[i] = ok ? sv : 1.0f;
        b1r[i] = ok ? bv : 0.0f;
    }
    // 1x1 filters: operand of step ks2, block kb is block (kb/2, ks2, kb%2) of the
    // blocked copy after the plain [K][K1] array: row 32(kb/2) + 8(r/4) + 4(kb%2) + r%4 for
    // lane row r, intermediate channels 32ks2 + 8(l/16) + [0,8).  Blocks past K or K1 are
    // clamped to existing ones: their rows are never stored, and the intermediate channels
    // they would multiply are zero.
    const u32x4* __restrict__ w2b = reinterpret_cast<const u32x4*>(w2 + (int64_t)a.K * a.K1);
    const int g2max = (a.K + 31) / 32 - 1, s2max = (a.K1 + 31) / 32 - 1;
    const int s32_2 = s2max + 1;
    u32x4 wa2[NKS2][KB2];
#pragma unroll
    for (int ks2 = 0; ks2 < NKS2; ++ks2)
#pragma unroll
        for (int kb = 0; kb < KB2; ++kb) {
            const int g = min(kb >> 1, g2max), sl = min(ks2, s2max);
            wa2[ks2][kb] = w2b[((g * s32_2 + sl) * 2 + (kb & 1)) * 64 + lane];
        }
    // epilogue-2 constants in LDS (read back four at a time per use: registers are
    // the scarce resource of this kernel)
    __shared__ __attribute__((aligned(16))) float s2s[KT], b2s[KT];
    for (int k = tid; k < KT; k += NT) {
        const bool ok = k < a.K;
        const float sv = a.s2 ? a.s2[ok ? k : 0] : 1.0f;
        const float bv = a.b2 ? a.b2[ok ? k : 0] : 0.0f;
        s2s[k] = ok ? sv : 1.0f;
        b2s[k] = ok ? bv : 0.0f;
    }
    const float* const S2 = s2s;
    const float* const B2 = b2s;
    // LDS byte offsets of the lane's 3x3 input operand in input row 0, per filter column
    // dw and channel half (input row ir adds ir * IN_ROW_BYTES)
    constexpr uint32_t IN_ROW_BYTES = (uint32_t)IW * CH * 16;
    uint32_t xoff[3][2];
#pragma unroll
    for (int dw = 0; dw < 3; ++dw)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int col = lr * S + dw, q = 4 * h + lg;
            xoff[dw][h] = (uint32_t)(col * CH + (q ^ (col & 7))) * 16u;
        }
    // intermediate: conv1 output rows 4(l/16)+i of wave w's 16 channels are channels
    // 16(w%2) + 4(l/16) + i of 32-channel slice w/2, i.e. lane group 2(w%2) + (l/16)/2,
    // bytes 8((l/16)%2)..+7 of its 16-byte operand (the 1x1 operand's natural order)
    const uint32_t tls_w =
        (uint32_t)(((2 * (wave & 1) + (lg >> 1)) * 16 + lr) * 16 + (lg & 1) * 8);
    // store offsets of the lane's two 8-channel runs (output channels 8(l/16) and
    // 32 + 8(l/16)) within a pixel row (kOob when the run lies beyond K)
    const uint32_t st0 = 8 * lg < a.K ? (uint32_t)(lr * a.K + 8 * lg) * (uint32_t)es : mm::kOob;
    const uint32_t st1 =
        32 + 8 * lg < a.K ? (uint32_t)(lr * a.K + 32 + 8 * lg) * (uint32_t)es : mm::kOob;

    auto phase_a = [&](const u32x4* src, u32x4* dst) {
        const char* xb = reinterpret_cast<const char*>(src);
        f32x4 d[TH];
#pragma unroll
        for (int r = 0; r < TH; ++r) d[r] = f32x4{0.f, 0.f, 0.f, 0.f};
        // walk the input rows: the operand of input row ir, filter column dw and channel
        // half h is read once and used by every output row r = (ir - dh) / S it feeds
        // (filter row dh), instead of once per (output row, tap).  The six operands of
        // row ir + 1 are requested before the products of row ir, so the LDS latency
        // overlaps matrix work instead of stalling it.
        u32x4 xv[2][6];
        auto load_row = [&](int ir, u32x4* o) {
#pragma unroll
            for (int dw = 0; dw < 3; ++dw)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    o[dw * 2 + h] =
                        *reinterpret_cast<const u32x4*>(xb + xoff[dw][h] + ir * IN_ROW_BYTES);
        };
        load_row(0, xv[0]);
#pragma unroll
        for (int ir = 0; ir < IH; ++ir) {
            if (ir + 1 < IH) load_row(ir + 1, xv[(ir + 1) & 1]);
#pragma unroll
            for (int dw = 0; dw < 3; ++dw)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int dh = 0; dh < 3; ++dh) {
                        const int r = (ir - dh) / S;
                        if (ir - dh >= 0 && (ir - dh) % S == 0 && r < TH)
                            d[r] = mfma<T>(wa1[(dh * 3 + dw) * 2 + h], xv[ir & 1][dw * 2 + h],
                                           d[r]);
                    }
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // row 0's reads
        b2b_sched_rows<S, TH, 0, IH>();
#pragma unroll
        for (int r = 0; r < TH; ++r) {
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = epilogue(d[r][i], s1r[i], b1r[i], act1);
            st8(reinterpret_cast<char*>(dst) + ((r * NKS2 + (wave >> 1)) * 64) * 16 + tls_w,
                pack8<T>(v));
        }
    };
    auto phase_b = [&](const u32x4* src, const Pos& t) {
        f32x4 acc[KB2];
#pragma unroll
        for (int kb = 0; kb < KB2; ++kb) acc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks2 = 0; ks2 < NKS2; ++ks2) {
            const u32x4 bfr = src[(wave * NKS2 + ks2) * 64 + lane];
#pragma unroll
            for (int kb = 0; kb < KB2; ++kb) acc[kb] = mfma<T>(wa2[ks2][kb], bfr, acc[kb]);
        }
        // lane holds output channels 32(kb/2) + 8(l/16) + 4(kb%2) + [0,4) of pixel l%16
        // in row w: runs of 8 at 8(l/16) (kb 0, 1) and 32 + 8(l/16) (kb 2, 3)
        float o[16];
#pragma unroll
        for (int kb = 0; kb < KB2; ++kb) {
            const int ch = 32 * (kb >> 1) + 8 * lg + 4 * (kb & 1);
            const f32x4 sc = *reinterpret_cast<const f32x4*>(S2 + ch);
            const f32x4 bi = *reinterpret_cast<const f32x4*>(B2 + ch);
#pragma unroll
            for (int i = 0; i < 4; ++i) o[4 * kb + i] = epilogue(acc[kb][i], sc[i], bi[i], act2);
        }
        // whole offsets in the vector operand, scalar offset 0 (see dwpw_mm.hip)
        const bool ok = t.oh0 + wave < a.Ho && t.ow0 + lr < a.Wo;
        const uint32_t row = (uint32_t)(t.out_base + wave * out_row);
        __builtin_amdgcn_raw_buffer_store_b128(pack16<T>(o), ry,
                                               ok && st0 != mm::kOob ? row + st0 : mm::kOob, 0,
                                               mm::kStoreStream);
        __builtin_amdgcn_raw_buffer_store_b128(pack16<T>(o + 8), ry,
                                               ok && st1 != mm::kOob ? row + st1 : mm::kOob, 0,
                                               mm::kStoreStream);
    };

    // ---- software-pipelined tile loop (see dwpw_mm.hip): step i waits for tile i+1's
    // input (only step i-1's NST stores were issued after it), barrier, requests tile
    // i+2, phase A of tile i+1, phase B of tile i.  (The first two tiles were requested
    // before the resident operands: both latencies overlap.)
    mm::wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (cur.n < a.N) phase_a(X0, T0);
    auto step_fn = [&](auto par, bool first) {
        constexpr int P = decltype(par)::value;
        if (first) mm::wait_vmcnt<0>(); else mm::wait_vmcnt<NST>();
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): own intermediate writes done
        __builtin_amdgcn_s_barrier();
        const Pos nn = advance(nxt);
        issue_tile(nn, std::integral_constant<int, P>{});
        if (nxt.n < a.N) phase_a(P == 0 ? X1 : X0, P == 0 ? T1 : T0);
        phase_b(P == 0 ? T0 : T1, cur);
        cur = nxt;
        nxt = nn;
    };
    bool first = true;
    while (cur.n < a.N) {
        step_fn(std::integral_constant<int, 0>{}, first);
        first = false;
        if (cur.n >= a.N) break;
        step_fn(std::integral_constant<int, 1>{}, false);
    }
    mm::wait_vmcnt<0>();
}

template <typename T, int S, int OCC>
int launch_b2b_mm(const KArgs& a, int grid, void* stream) {
    (void)hipGetLastError();
    hipLaunchKernelGGL((b2b_mm_kernel<T, S, OCC>), dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       a);
    return (int)hipGetLastError();
}
template <typename T, int S, int OCC>
int occ_b2b_mm() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, b2b_mm_kernel<T, S, OCC>, 256, 0) !=
        hipSuccess)
        return 0;
    return n;
}

#define FCM_V_DWPW(...)
#define FCM_V_DWPW32(...)
#define FCM_V_B2B(...)
#define FCM_V_DWPW_MM(...)
#define FCM_V_B2B_MM(name, dt, CT, S, OCC)                                   \
    template int launch_b2b_mm<CT, S, OCC>(const KArgs&, int, void*); \
    template int occ_b2b_mm<CT, S, OCC>();
#define FCM_V_DWPW_MMW(...)
#include "../variants.def"
#undef FCM_V_DWPW
#undef FCM_V_DWPW32
#undef FCM_V_B2B
#undef FCM_V_DWPW_MM
#undef FCM_V_B2B_MM
#undef FCM_V_DWPW_MMW

}  // namespace fcm
