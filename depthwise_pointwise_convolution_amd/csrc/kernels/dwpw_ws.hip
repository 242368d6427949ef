// dwpw_ws.hip -- fused depthwise 3x3 -> pointwise 1x1 on the gfx950 matrix cores for
// wide layers, pointwise filters stationary in registers (FCM paper "Fusing Depthwise
// and Pointwise Convolutions for Efficient Inference on GPUs", Sec. III, Fig. 3(b): the
// DWPW module, output stationary within a tile; Sec. IV-A: weights read once per tile
// of output feature maps -- here once per workgroup for the whole launch).
//
// A workgroup walks over 16-pixel output blocks (a TH x TW tile, TH * TW = 16) of the
// batch for one K tile of KT output channels; one step is one block with every input
// channel.  Its 8 waves split into two roles, one wave of each on every SIMD, so that
// the two instruction streams overlap:
//   - depthwise waves (0..3): request the input windows ((TH-1)S+3 x (TW-1)S+3 pixels,
//     all C channels) by direct global->LDS loads -- every window row is one contiguous
//     run of whole pixels (all channels of a pixel are adjacent in NHWC) -- and run the
//     depthwise layer as block-diagonal matrix products (v_mfma_f32_16x16x32, a
//     16-channel filter diagonal for two taps against 16 bytes of the window per lane,
//     five per 16 channels; the diagonal operands stay in registers), epilogue 1,
//     rounding, and write the LDS intermediate in pointwise-operand order; wave w owns
//     channel blocks CBW w .. CBW w + CBW - 1;
//   - pointwise waves (4..7): hold the pointwise filters of KT/4 output channels over all
//     C input channels in registers (loaded once from the blocked copy fcm_pack_weights
//     writes), contract the intermediate (C/32 reduction slices, four independent
//     accumulator chains), epilogue 2, 16-byte buffer stores.
// Step s (one barrier): the depthwise waves request window s+3 and compute the
// depthwise layer of block s+1 from window s+1; the pointwise waves compute block s
// from the intermediate written in step s-1.  Three window buffers keep two windows in
// flight; three intermediate buffers make the buffer pattern repeat every three steps,
// and the loops are instantiated for each of those phases so that every LDS buffer is
// named at compile time.
// With one K tile (K <= KT) the depthwise layer runs exactly once per pixel, the DWPW
// module's no-redundancy property; with more, the workgroups of one block's K tiles
// have neighbouring ids (the same XCD) and run the block at the same time, so its
// window comes from HBM once and from that XCD's L2 for the other K tiles.
//
// LDS window layout: 16-byte piece q of window pixel p (row i, column j) sits at slot
// p*C/8 + (q ^ sw(p)), sw = (j/S + TW*(i/S)) & 15 (& C/8 - 1 below 128 channels).  The
// 16 lanes of a depthwise operand read (16 output pixels of the block, one tap, one
// 8-channel piece) then fall into 16 distinct bank groups at either stride.
#include <type_traits>

#include "mm_common.h"

namespace fcm {

namespace ws {
// (The statements below are gfx950 assembly; the host compilation pass of this source
// only needs the functions to exist.)
// Four 16-byte LDS reads at base + 1024 i, likewise.
__device__ __forceinline__ void lds_read4k(uint32_t base, u32x4 (&o)[4]) {
#if __HIP_DEVICE_COMPILE__
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:1024\n\t"
        "ds_read_b128 %2, %4 offset:2048\n\t"
        "ds_read_b128 %3, %4 offset:3072\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
        : "v"(base)
        : "memory");
#endif
}
// Two 8-byte LDS writes at base and base + 512 (the rows of two adjacent channel blocks in
// the intermediate), likewise.
__device__ __forceinline__ void lds_write2x8(uint32_t base, vec_t<uint32_t, 2> d0,
                                             vec_t<uint32_t, 2> d1) {
#if __HIP_DEVICE_COMPILE__
    asm volatile("ds_write2st64_b64 %0, %1, %2 offset1:1" : : "v"(base), "v"(d0), "v"(d1)
                 : "memory");
#endif
}
}  // namespace ws

template <typename T, int S, int TH, int TW, int CT, int KT, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void dwpw_ws_kernel(KArgs a) {
    static_assert(TH * TW == 16, "one 16-pixel matrix block per step");
    static_assert(NW == 8, "four depthwise and four pointwise waves");
    constexpr int NDW = NW / 2, NPW = NW - NDW;
    constexpr int NTD = 64 * NDW;                    // threads issuing the window loads
    constexpr int IH = (TH - 1) * S + 3, IW = (TW - 1) * S + 3, NPIX = IH * IW;
    constexpr int CH = CT / 8;                       // 16-byte pieces per pixel
    constexpr int SWM = (CH < 16 ? CH : 16) - 1;     // swizzle mask (stays within a pixel)
    constexpr int SLOTS = NPIX * CH;
    constexpr int RF = SLOTS / NTD;                  // full direct-load rounds
    constexpr int REM = SLOTS - RF * NTD;            // slots of the last, partial round
    constexpr int RW = (REM + 63) / 64;              // waves that take part in it
    constexpr int R = RF + (REM > 0 ? 1 : 0);        // loads per window and wave
    constexpr int SLOTS_P = RF * NTD + RW * 64;      // (whole waves of the last round)
    constexpr int SLOTS_B = SLOTS_P + (REM > 0 ? 64 : 0);  // + the other waves' landing
    constexpr int NKS = CT / 32;                     // pointwise reduction slices
    static_assert(NKS % 4 == 0, "the intermediate reads go four at a time");
    constexpr int KW = KT / NPW;                     // output channels per pointwise wave
    constexpr int KBW = KW / 16;                     // 16-channel output blocks per wave
    static_assert(KBW % 2 == 0, "each lane stores 16-byte runs of 8 output channels");
    constexpr int NST = KBW / 2;                     // stores per lane per step
    constexpr int NCB = CT / 16;                     // depthwise channel blocks
    static_assert(NCB % (2 * NDW) == 0, "pairs of channel blocks per depthwise wave");
    constexpr int CBW = NCB / NDW;                   // channel blocks per depthwise wave
    constexpr int NTP = 5;                           // tap pairs (the tenth tap is empty)
    static_assert(R < 32, "vmcnt range");

    __shared__ __attribute__((aligned(16))) u32x4 xs0[SLOTS_B];
    __shared__ __attribute__((aligned(16))) u32x4 xs1[SLOTS_B];
    __shared__ __attribute__((aligned(16))) u32x4 xs2[SLOTS_B];
    __shared__ __attribute__((aligned(16))) u32x4 tl0[NKS * 64];
    __shared__ __attribute__((aligned(16))) u32x4 tl1[NKS * 64];
    __shared__ __attribute__((aligned(16))) u32x4 tl2[NKS * 64];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int G = gridDim.x;
    const int L = xcd_logical_id(blockIdx.x, G);
    const int nkt = a.num_ktiles;
    const int k0 = (L % nkt) * KT;   // the workgroup's K tile (fixed: G % nkt == 0)
    const int es = (int)sizeof(T);
    const int per_img = a.tiles_h * a.tiles_w, nblk = a.num_ptiles;
    const int b0 = L / nkt, bstep = G / nkt;

    // ---- the block walk: block b0, b0 + G/nkt, ... ------------------------------------
    using Pos = mm::TilePos;
    const int in_img = a.H * a.W * CT * es, in_row = a.W * CT * es;
    const int out_img = a.Ho * a.Wo * a.K * es, out_row = a.Wo * a.K * es;
    auto block = [&](int b) {
        Pos p;
        p.n = b / per_img;
        const int rem = b - p.n * per_img;
        p.th = rem / a.tiles_w;
        p.tw = rem - p.th * a.tiles_w;
        p.oh0 = p.th * TH;
        p.ow0 = p.tw * TW;
        p.ih0 = p.oh0 * S - a.pad_h;
        p.iw0 = p.ow0 * S - a.pad_w;
        p.in_base = p.n * in_img + p.ih0 * in_row + p.iw0 * CT * es;
        p.out_base = p.n * out_img + p.oh0 * out_row + p.ow0 * a.K * es;
        return p;
    };

    if (wave < NDW) {
        // =============================== depthwise waves ===============================
        const int dtid = tid;  // 0 .. NTD-1
        const Act act1 = act_bounds(a.act1);
        const __amdgpu_buffer_rsrc_t rx =
            mm::rsrc(a.x, (uint32_t)(a.N * a.H * a.W * CT * es));
        // direct-load plan: round r of thread dtid fills slot r*NTD + dtid (waves < RW in
        // the last round); its byte offset from the window origin, and its window row and
        // column packed two rounds per register (8 bits each) for the border path
        static_assert(IH < 256 && IW < 256, "packed window positions");
        uint32_t dl_off[R], dl_pos[(R + 1) / 2];
#pragma unroll
        for (int r = 0; r < (R + 1) / 2; ++r) dl_pos[r] = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int s = r * NTD + dtid;
            const int p = s / CH, ihl = p / IW, iwl = p % IW;
            const int q = (s % CH) ^ ((iwl / S + TW * (ihl / S)) & SWM);
            const bool real = s < SLOTS;
            dl_off[r] = real ? (uint32_t)((ihl * a.W + iwl) * CT + q * 8) * (uint32_t)es
                             : mm::kOob;
            if (real) dl_pos[r / 2] |= (uint32_t)((ihl << 8) | iwl) << (16 * (r & 1));
        }
        const bool last_round = wave < RW;
        // Every depthwise wave issues R loads per window (waves without a slot in the
        // last round load zeros into 64 landing slots past the window, which nothing
        // reads), so the vector-memory waits below are exact.  Outside the image (and
        // for a block past the end) the range check loads zeros.
        auto issue_window = [&](int b, u32x4* dst) {
            const Pos t = block(b);
            const bool live = b < nblk;
            const bool inside = live && t.ih0 >= 0 && t.iw0 >= 0 && t.ih0 + IH <= a.H &&
                                t.iw0 + IW <= a.W;
            // per-lane offset of round r for a window that crosses the image border: the
            // out-of-range offset for pixels outside the image.  (The empty asm statement
            // keeps the unpacking here rather than letting the compiler keep every
            // round's unpacked values alive across the loop.)
            auto border_off = [&](int r) {
                uint32_t pk = dl_pos[r / 2], o = dl_off[r];
                asm volatile("" : "+v"(pk), "+v"(o));
                pk >>= 16 * (r & 1);
                const int ih = t.ih0 + (int)((pk >> 8) & 0xff), iw = t.iw0 + (int)(pk & 0xff);
                const bool ok = live && o != mm::kOob && (unsigned)ih < (unsigned)a.H &&
                                (unsigned)iw < (unsigned)a.W;
                return ok ? (uint32_t)(t.in_base + (int)o) : mm::kOob;
            };
            // (every builtin argument is a plain local: the host compilation pass drops
            // the kernel when a call result is passed straight to the builtin)
            if (inside) {
#pragma unroll
                for (int r = 0; r < RF; ++r) {
                    const uint32_t off = dl_off[r];
                    u32x4* d = dst + r * NTD + wave * 64;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rx, (__attribute__((address_space(3))) void*)d, 16, off, t.in_base, 0, 0);
                }
            } else {
#pragma unroll
                for (int r = 0; r < RF; ++r) {
                    const uint32_t off = border_off(r);
                    u32x4* d = dst + r * NTD + wave * 64;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rx, (__attribute__((address_space(3))) void*)d, 16, off, 0, 0, 0);
                }
            }
            if constexpr (REM > 0) {
                if (last_round) {
                    const uint32_t off = inside ? dl_off[RF] : border_off(RF);
                    const int soff = inside ? t.in_base : 0;
                    u32x4* d = dst + RF * NTD + wave * 64;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rx, (__attribute__((address_space(3))) void*)d, 16, off, soff, 0, 0);
                } else {
                    u32x4* d = dst + SLOTS_P;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rx, (__attribute__((address_space(3))) void*)d, 16, mm::kOob, 0, 0, 0);
                }
            }
        };
        // resident depthwise operands and epilogue-1 constants (filled in the prologue)
        u32x4 dwa[CBW][NTP];
        f32x4 e1s[CBW], e1b[CBW];
        // LDS byte offsets of the lane's window reads relative to a channel block's piece:
        // pixel of (output pixel lr, tap 2tp + lg/2), piece 2cb + (lg&1) swizzled with the
        // pixel's sw
        uint32_t xoff[NTP], xsw[NTP];
        {
            const int r = lr / TW, c = lr % TW;
#pragma unroll
            for (int tp = 0; tp < NTP; ++tp) {
                const int t0 = 2 * tp + (lg >> 1), t = t0 < 9 ? t0 : 0;
                const int ih = r * S + t / 3, iw = c * S + t % 3;
                xoff[tp] = (uint32_t)((ih * IW + iw) * CH) * 16u;
                xsw[tp] = (uint32_t)((iw / S + TW * (ih / S)) & SWM);
            }
        }
        // intermediate: depthwise output rows 4(l/16)+i of channel block cb are channels
        // 16(cb%2) + 4(l/16) + i of slice cb/2: lane group 2(cb%2) + (l/16)/2, bytes
        // 8((l/16)%2)..+7 of its 16-byte operand; blocks 2m and 2m+1 land 512 bytes apart
        const uint32_t tl_lane = (uint32_t)(((lg >> 1) * 16 + lr) * 16 + (lg & 1) * 8);
        // the depthwise layer of one block: window buffer src -> intermediate buffer dst,
        // two channel blocks (two independent product chains) at a time
        auto dw_step = [&](const u32x4* src, u32x4* dst) {
            const uint32_t xb = mm::lds_addr(src), tb = mm::lds_addr(dst);
#pragma unroll
            for (int j0 = 0; j0 < CBW; j0 += 2) {
                uint32_t ad[10];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const uint32_t q = (uint32_t)(2 * (CBW * wave + j0 + j) + (lg & 1));
#pragma unroll
                    for (int tp = 0; tp < NTP; ++tp)
                        ad[j * NTP + tp] = xb + xoff[tp] + ((q ^ xsw[tp]) << 4);
                }
                u32x4 xr[10];
                mm::lds_read10(ad, xr);
                f32x4 d[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) d[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int tp = 0; tp < NTP; ++tp)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        d[j] = mfma<T>(dwa[j0 + j][tp], xr[j * NTP + tp], d[j]);
                vec_t<uint32_t, 2> pk[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    float v[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        v[i] = epilogue(d[j][i], e1s[j0 + j][i], e1b[j0 + j][i], act1);
                    const uint2 pv = pack8<T>(v);
                    pk[j] = vec_t<uint32_t, 2>{pv.x, pv.y};
                }
                const int cb = CBW * wave + j0;  // even: cb and cb + 1 share slice cb / 2
                ws::lds_write2x8(tb + (uint32_t)((cb >> 1) * 1024) + tl_lane, pk[0], pk[1]);
            }
        };

        // prologue: the window of step 0, then the resident operands, then the windows of
        // steps 1 and 2.  The operands are complete before the later windows are
        // requested: the compiler's wait for them counts every load issued before it, so
        // it would otherwise also wait for those windows (at launch, when every
        // workgroup requests its first windows at once, that wait is the longest).
        issue_window(b0, xs0);
        asm volatile("" ::: "memory");
        // resident depthwise operands of the wave's channel blocks cb = CBW wave + j: lane
        // (l%16, l/16) holds reduction index 8(l/16) + e = (tap 2tp + (l/16)/2, channel
        // 16cb + 8((l/16)&1) + e); the one non-zero element (channel 16cb + l%16) sits at
        // e = l%8 of lanes whose channel half matches.  Epilogue-1 constants of the lane's
        // depthwise rows 4(l/16)..+3 of each block.
        const T* __restrict__ wdw = (const T*)a.w1;
        const bool dw_active = (lr >> 3) == (lg & 1);
        const int dw_e = lr & 7;
#pragma unroll
        for (int j = 0; j < CBW; ++j) {
#pragma unroll
            for (int tp = 0; tp < NTP; ++tp) {
                const int t = 2 * tp + (lg >> 1);
                const int c = 16 * (CBW * wave + j) + lr;
                const uint16_t h = (dw_active && t < 9)
                                       ? reinterpret_cast<const uint16_t*>(wdw)[t * CT + c]
                                       : (uint16_t)0;
                const uint32_t v = (dw_e & 1) ? ((uint32_t)h << 16) : (uint32_t)h;
                const int w = dw_e >> 1;
                dwa[j][tp] = u32x4{w == 0 ? v : 0u, w == 1 ? v : 0u, w == 2 ? v : 0u,
                                   w == 3 ? v : 0u};
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = 16 * (CBW * wave + j) + 4 * lg + i;
                e1s[j][i] = a.s1 ? a.s1[c] : 1.0f;
                e1b[j][i] = a.b1 ? a.b1[c] : 0.0f;
            }
        }
#pragma unroll
        for (int j = 0; j < CBW; ++j) {
#pragma unroll
            for (int tp = 0; tp < NTP; ++tp) asm volatile("" : "+v"(dwa[j][tp]));
            asm volatile("" : "+v"(e1s[j]), "+v"(e1b[j]));
        }
        issue_window(b0 + bstep, xs1);
        issue_window(b0 + 2 * bstep, xs2);
        // window 0 is in once at most the last two windows' loads are outstanding
        mm::wait_vmcnt<2 * R>();
        __builtin_amdgcn_s_barrier();
        dw_step(xs0, tl0);
        // step s: window s+1 complete (only window s+2's loads were issued after it);
        // barrier; window s+3 into the buffer of window s; depthwise layer of step s+1
        int b = b0;
        auto step = [&](auto phase) {
            constexpr int P = decltype(phase)::value;
            mm::wait_vmcnt<R>();
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): intermediate writes done
            __builtin_amdgcn_s_barrier();
            issue_window(b + 3 * bstep, P == 0 ? xs0 : P == 1 ? xs1 : xs2);
            dw_step(P == 0 ? xs1 : P == 1 ? xs2 : xs0, P == 0 ? tl1 : P == 1 ? tl2 : tl0);
            b += bstep;
        };
        while (b < nblk) {
            step(std::integral_constant<int, 0>{});
            if (b >= nblk) break;
            step(std::integral_constant<int, 1>{});
            if (b >= nblk) break;
            step(std::integral_constant<int, 2>{});
        }
        // windows of steps past the end may still be in flight into LDS
        mm::wait_vmcnt<0>();
    } else {
        // =============================== pointwise waves ===============================
        const int pw = wave - NDW;
        const Act act2 = act_bounds(a.act2);
        const __amdgpu_buffer_rsrc_t ry =
            mm::rsrc(a.y, (uint32_t)(a.N * a.Ho * a.Wo * a.K * es));
        const int kw0 = k0 + pw * KW;  // this wave's first output channel
        // pointwise A operands of the wave's slice: blocked copy, block (g, s, h) =
        // ((kw0 + 32(kb/2))/32, ks, kb%2); a block past the last output channel is clamped
        // to the last one (its rows belong to channels that are never stored)
        const T* __restrict__ wpw = (const T*)a.w2;
        const u32x4* __restrict__ wpb =
            reinterpret_cast<const u32x4*>(wpw + (int64_t)a.K * CT);
        const int g32 = (a.K + 31) / 32;
        u32x4 apw[NKS][KBW];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int kb = 0; kb < KBW; ++kb) {
                const int g = min((kw0 >> 5) + (kb >> 1), g32 - 1);
                apw[ks][kb] = wpb[((g * NKS + ks) * 2 + (kb & 1)) * 64 + lane];
            }
        // epilogue-2 constants of the lane's 8-channel output runs kw0 + 32 j + 8(l/16)
        f32x4 e2s[NST][2], e2b[NST][2];
#pragma unroll
        for (int j = 0; j < NST; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int k = kw0 + 32 * j + 8 * lg + 4 * h + i;
                    e2s[j][h][i] = (a.s2 && k < a.K) ? a.s2[k] : 1.0f;
                    e2b[j][h][i] = (a.b2 && k < a.K) ? a.b2[k] : 0.0f;
                }
        // pointwise layer of one block, epilogue 2 and its stores (always NST per lane;
        // pixels past the output and 8-channel runs past K get the out-of-range offset,
        // whose stores are dropped)
        auto pw_step = [&](const u32x4* src, int b) {
            const uint32_t tb = mm::lds_addr(src) + lane * 16u;
            u32x4 bv[NKS];
#pragma unroll
            for (int k4 = 0; k4 < NKS; k4 += 4) {
                u32x4 r4[4];
                ws::lds_read4k(tb + k4 * 1024u, r4);
#pragma unroll
                for (int i = 0; i < 4; ++i) bv[k4 + i] = r4[i];
            }
            f32x4 acc[KBW];
#pragma unroll
            for (int kb = 0; kb < KBW; ++kb) acc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int kb = 0; kb < KBW; ++kb) acc[kb] = mfma<T>(apw[ks][kb], bv[ks], acc[kb]);
            const Pos t = block(b);
            const int r = lr / TW, c = lr % TW;
            const bool ok = b < nblk && t.oh0 + r < a.Ho && t.ow0 + c < a.Wo;
            const uint32_t v = (uint32_t)(r * out_row + c * a.K * es);
#pragma unroll
            for (int j = 0; j < NST; ++j) {
                const int kl = kw0 + 32 * j + 8 * lg;  // first channel of the lane's run
                float o[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    o[i] = epilogue(acc[2 * j][i], e2s[j][0][i], e2b[j][0][i], act2);
                    o[4 + i] = epilogue(acc[2 * j + 1][i], e2s[j][1][i], e2b[j][1][i], act2);
                }
                // the whole offset in the vector operand, scalar offset 0 (see dwpw_mm.hip)
                const bool run_ok = ok && kl < a.K;
                __builtin_amdgcn_raw_buffer_store_b128(
                    pack16<T>(o), ry,
                    run_ok ? (uint32_t)t.out_base + v + (uint32_t)(kl * es) : mm::kOob, 0,
                    mm::kStoreStream);
            }
        };
        // the prologue's barrier (the depthwise layer of step 0 is not read before the
        // first step's barrier)
        __builtin_amdgcn_s_barrier();
        int b = b0;
        auto step = [&](auto phase) {
            constexpr int P = decltype(phase)::value;
            __builtin_amdgcn_s_barrier();
            pw_step(P == 0 ? tl0 : P == 1 ? tl1 : tl2, b);
            b += bstep;
        };
        while (b < nblk) {
            step(std::integral_constant<int, 0>{});
            if (b >= nblk) break;
            step(std::integral_constant<int, 1>{});
            if (b >= nblk) break;
            step(std::integral_constant<int, 2>{});
        }
    }
}

template <typename T, int S, int TH, int TW, int CT, int KT, int NW>
int launch_dwpw_ws(const KArgs& a, int grid, void* stream) {
    (void)hipGetLastError();
    hipLaunchKernelGGL((dwpw_ws_kernel<T, S, TH, TW, CT, KT, NW>), dim3(grid), dim3(64 * NW), 0,
                       (hipStream_t)stream, a);
    return (int)hipGetLastError();
}
template <typename T, int S, int TH, int TW, int CT, int KT, int NW>
int occ_dwpw_ws() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, dwpw_ws_kernel<T, S, TH, TW, CT, KT, NW>,
                                                     64 * NW, 0) != hipSuccess)
        return 0;
    return n;
}

#define FCM_V_DWPW(...)
#define FCM_V_DWPW32(...)
#define FCM_V_B2B(...)
#define FCM_V_DWPW_MM(...)
#define FCM_V_B2B_MM(...)
#define FCM_V_DWPW_MMW(...)
#define FCM_V_DWPW_WS(name, dt, CTy, S, TH, TW, CT, KT, NW)                     \
    template int launch_dwpw_ws<CTy, S, TH, TW, CT, KT, NW>(const KArgs&, int, void*); \
    template int occ_dwpw_ws<CTy, S, TH, TW, CT, KT, NW>();
#include "../variants.def"
#undef FCM_V_DWPW
#undef FCM_V_DWPW32
#undef FCM_V_B2B
#undef FCM_V_DWPW_MM
#undef FCM_V_B2B_MM
#undef FCM_V_DWPW_MMW
#undef FCM_V_DWPW_WS

}  // namespace fcm
