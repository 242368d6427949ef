// dwpw_wsl.hip -- fused depthwise 3x3 -> pointwise 1x1 on the gfx950 matrix cores for
// small maps with many channels (late-network layers such as 7x7 maps with C = K = 1024),
// wave-specialised (FCM paper "Fusing Depthwise and Pointwise Convolutions for Efficient
// Inference on GPUs", Sec. III, Fig. 3(b): the DWPW module, output stationary within a
// tile; Sec. IV-A: the pointwise filters of a K tile read once per output tile).
//
// A workgroup owns a TH x TW output tile of at most 64 pixels (a whole 7x7 map is one
// tile of four 16-pixel blocks) and KT output channels; one step is one 64-channel slice
// of the input channels.  Its NW = 8 or 16 waves split into two roles, the same number
// of each on every SIMD, so that the two instruction streams overlap:
//   - depthwise waves (the first NW/2) request the input window of step s+4 by direct
//     global->LDS loads (four window buffers: three windows in flight while one is
//     read) and compute the depthwise layer of step s+1 for channel block w % 4 of the
//     slice and 16 / (NW/2) of the tile's four pixel blocks: block-diagonal matrix
//     products (v_mfma_f32_16x16x32, five per 16 channels x 16 pixels, one independent
//     product chain per pixel block), epilogue 1, rounding, 8-byte writes of the LDS
//     intermediate in pointwise-operand order;
//   - pointwise waves (the other NW/2) request the pointwise filters of step s+1 into the
//     second of two operand register sets (16-byte loads from the blocked copy that
//     fcm_pack_weights writes after the [K][C] filters), contract the intermediate of
//     step s with the filters of step s for KT/(NW/2) output channels of every pixel
//     block, and after a tile's last step apply epilogue 2 and store the tile.
// With 16 waves a depthwise wave reads half as much of the window per step (its product
// chains, LDS reads and epilogue are the step's critical path) and a pointwise wave
// holds half as many output channels.
// One barrier per step.  The roles run separate loops with the same number of barriers;
// the pointwise loop runs two steps per round, so the two operand sets are named at
// compile time and alternate without register copies.  The depthwise filters and
// epilogue constants of all C <= CMAX channels are copied to LDS once per workgroup.
//
// Where a tile is a whole map (one tile per image) every window has the same shape, so
// the direct-load offsets of a lane, with the zero padding as out-of-range offsets, are
// computed once: a step's loads are then one instruction each, based at the image and
// channel slice.  Otherwise the window's border is checked per step.
//
// Channel orders (as in the chunked wide kernel of dwpw_mmw.hip): the reduction index k
// of a 32-channel slice is input channel 32 ks + k (lane group l/16 holds channels
// 8(l/16)..+7 of the intermediate); row r of output block kb holds output channel
// 32(kb/2) + 8(r/4) + 4(kb%2) + r%4 of the wave's slice, so that lane group g ends up
// with 8 consecutive output channels per block pair and writes them with one 16-byte
// store.
#include <type_traits>

#include "mm_common.h"

namespace fcm {

template <typename T, int S, int TH, int TW, int KT, int CMAX, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void dwpw_wsl_kernel(KArgs a) {
    static_assert(NW == 8 || NW == 16, "one or two waves of each role per SIMD");
    constexpr int NT = 64 * NW, NDW = NW / 2, NTD = 64 * NDW;
    constexpr int CC = 64, NBX = 4, NKS = CC / 32, NTP = 5;
    constexpr int NPX = TH * TW, MB = (NPX + 15) / 16;
    static_assert(MB == 4, "tiles of 49 to 64 pixels: four 16-pixel blocks");
    constexpr int MBW = MB * 4 / NDW;  // pixel blocks of a depthwise wave (one channel block)
    constexpr int IH = (TH - 1) * S + 3, IW = (TW - 1) * S + 3, NPIX = IH * IW;
    constexpr int CH = CC / 8;                   // 16-byte pieces per pixel of a slice
    constexpr int SLOTS = NPIX * CH;
    constexpr int R = (SLOTS + NTD - 1) / NTD;  // direct-load rounds per depthwise thread
    constexpr int SLOTS_P = R * NTD;
    constexpr int KW = KT / NDW;  // pointwise output channels per pointwise wave
    constexpr int KBW = KW / 16;  // 16-channel output blocks per pointwise wave
    static_assert(KBW % 2 == 0, "each lane stores 16-byte runs of 8 output channels");
    constexpr int NLD = NKS * KBW;      // pointwise operand loads per lane and step
    constexpr int NST = MB * (KBW / 2);  // buffer stores per lane per finished tile
    static_assert(3 * R < 64 && NLD + NST < 64, "vmcnt range");
    static_assert(CMAX % 64 == 0, "whole slices");

    __shared__ __attribute__((aligned(16))) u32x4 xs[NBX * SLOTS_P];
    __shared__ __attribute__((aligned(16))) u32x4 tl[2 * MB * NKS * 64];
    __shared__ __attribute__((aligned(16))) float s2s[KT];
    __shared__ __attribute__((aligned(16))) float b2s[KT];
    __shared__ __attribute__((aligned(16))) u32x4 wds[9 * CMAX / 8];  // depthwise [9][CMAX]
    __shared__ __attribute__((aligned(16))) float s1s[CMAX];
    __shared__ __attribute__((aligned(16))) float b1s[CMAX];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int G = gridDim.x;
    const int L = xcd_logical_id(blockIdx.x, G);
    const int k0 = (L % a.num_ktiles) * KT;
    const int nch = a.C / CC;
    const int es = (int)sizeof(T);
    const int in_img = a.H * a.W * a.C * es, in_row = a.W * a.C * es;
    const int out_img = a.Ho * a.Wo * a.K * es, out_row = a.Wo * a.K * es;

    // ---- constants: epilogue-2 constants of the K tile, depthwise filters and
    // epilogue-1 constants of every channel (all loads issued before the first write)
    constexpr int I2 = (KT + NT - 1) / NT, IW9 = (9 * CMAX / 8 + NT - 1) / NT;
    constexpr int I1 = (CMAX + NT - 1) / NT;
    const int nw = 9 * (a.C / 8);
    float s2v[I2], b2v[I2], s1v[I1], b1v[I1];
    u32x4 wv[IW9];
    {
        const T* __restrict__ wdw = (const T*)a.w1;
#pragma unroll
        for (int r = 0; r < I2; ++r) {
            const int i = tid + r * NT, k = k0 + i;
            const bool ok = i < KT && k < a.K;
            s2v[r] = (a.s2 && ok) ? a.s2[k] : 1.0f;
            b2v[r] = (a.b2 && ok) ? a.b2[k] : 0.0f;
        }
#pragma unroll
        for (int r = 0; r < IW9; ++r) {
            const int i = tid + r * NT;
            wv[r] = i < nw ? reinterpret_cast<const u32x4*>(wdw)[i] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int r = 0; r < I1; ++r) {
            const int i = tid + r * NT;
            s1v[r] = (a.s1 && i < a.C) ? a.s1[i] : 1.0f;
            b1v[r] = (a.b1 && i < a.C) ? a.b1[i] : 0.0f;
        }
    }
    auto write_constants = [&]() {
#pragma unroll
        for (int r = 0; r < I2; ++r) {
            const int i = tid + r * NT;
            if (i < KT) {
                s2s[i] = s2v[r];
                b2s[i] = b2v[r];
            }
        }
#pragma unroll
        for (int r = 0; r < IW9; ++r) {
            const int i = tid + r * NT;
            if (i < nw) {
                const int t = i / (a.C / 8), c8 = i - t * (a.C / 8);
                wds[t * (CMAX / 8) + c8] = wv[r];
            }
        }
#pragma unroll
        for (int r = 0; r < I1; ++r) {
            const int i = tid + r * NT;
            if (i < a.C) {
                s1s[i] = s1v[r];
                b1s[i] = b1v[r];
            }
        }
    };

    // ---- (tile, slice) walk, identical in both roles -------------------------------
    const int pstep = G / a.num_ktiles;
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
    const Pos pstep_pos = split(pstep);
    auto advance = [&](Pos p) {
        p.tw += pstep_pos.tw;
        if (p.tw >= a.tiles_w) {
            p.tw -= a.tiles_w;
            ++p.th;
        }
        p.th += pstep_pos.th;
        if (p.th >= a.tiles_h) {
            p.th -= a.tiles_h;
            ++p.n;
        }
        p.n += pstep_pos.n;
        derive(p);
        return p;
    };
    struct Step {
        Pos t;
        int c;
    };
    auto next = [&](const Step& s) {
        Step n;
        if (s.c + 1 < nch) {
            n.t = s.t;
            n.c = s.c + 1;
        } else {
            n.t = advance(s.t);
            n.c = 0;
        }
        return n;
    };
    Step s0;
    s0.t = split(L / a.num_ktiles);
    s0.c = 0;
    // the workgroup's step count, known up front (no exit test inside a round of steps)
    const int t_first = L / a.num_ktiles;
    const int n_tiles = t_first < a.num_ptiles ? (a.num_ptiles - 1 - t_first) / pstep + 1 : 0;
    const int n_steps = n_tiles * nch;

    if (wave < NDW) {
        // ================================ depthwise waves ================================
        const int cbw = wave & 3;           // channel block of every slice
        const int jb = (wave >> 2) * MBW;   // first pixel block
        const __amdgpu_buffer_rsrc_t rx =
            mm::rsrc(a.x, (uint32_t)(a.N * a.H * a.W * a.C * es));
        // direct-load plan: slot s holds 16-byte piece q of window pixel p = s / CH,
        // s % CH = q ^ ((column - row) & 7); per lane and round, the offset from the window
        // origin and, where a tile is a whole map, from the image origin (padding out of
        // range).  (With the column alone in the key, 8 lanes of a depthwise read whose
        // output pixels wrap from one row of a 7-wide map into the next hit one bank group
        // twice; column minus row gives them 8 distinct groups in every pixel block.)
        const bool whole = a.tiles_h == 1 && a.tiles_w == 1;
        uint32_t dl_off[R], dl_img[R];
        int dl_pos[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int s = r * NTD + tid;
            const int p = s / CH, ihl = p / IW, iwl = p % IW;
            const int q = (s % CH) ^ ((iwl - ihl) & 7);
            const bool real = s < SLOTS;
            dl_off[r] = real ? (uint32_t)((ihl * a.W + iwl) * a.C + q * 8) * (uint32_t)es : mm::kOob;
            dl_pos[r] = real ? (ihl << 16) | iwl : 0;
            const int ih = ihl - a.pad_h, iw = iwl - a.pad_w;
            dl_img[r] = real && (unsigned)ih < (unsigned)a.H && (unsigned)iw < (unsigned)a.W
                            ? (uint32_t)((ih * a.W + iw) * a.C + q * 8) * (uint32_t)es
                            : mm::kOob;
        }
        // always R loads per lane, whatever the step (zero-filled when outside the image
        // or past the last tile), so the vector-memory counts of the waits are exact
        auto issue_window = [&](const Step& st, u32x4* dst) {
            const Pos& t = st.t;
            const bool live = t.n < a.N;
            const int cbyte = st.c * CC * es;
            if (whole) {
                const int base = live ? t.n * in_img + cbyte : 0;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint32_t off = live ? dl_img[r] : mm::kOob;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rx, (__attribute__((address_space(3))) void*)(dst + r * NTD + wave * 64),
                        16, off, base, 0, 0);
                }
                return;
            }
            const bool inside = live && t.ih0 >= 0 && t.iw0 >= 0 && t.ih0 + IH <= a.H &&
                                t.iw0 + IW <= a.W;
            if (inside) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint32_t off = dl_off[r];
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rx, (__attribute__((address_space(3))) void*)(dst + r * NTD + wave * 64),
                        16, off, t.in_base + cbyte, 0, 0);
                }
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int ih = t.ih0 + (dl_pos[r] >> 16), iw = t.iw0 + (dl_pos[r] & 0xffff);
                    const bool ok = live && dl_off[r] != mm::kOob && (unsigned)ih < (unsigned)a.H &&
                                    (unsigned)iw < (unsigned)a.W;
                    const uint32_t off =
                        ok ? (uint32_t)(t.in_base + cbyte + (int)dl_off[r]) : mm::kOob;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rx, (__attribute__((address_space(3))) void*)(dst + r * NTD + wave * 64),
                        16, off, 0, 0, 0);
                }
            }
        };
        // depthwise operands: matrix operand lane (l%16, l/16) holds channel 16cb + l%16
        // against reduction index 8(l/16) + e = (tap 2tp + (l/16)/2, channel
        // 16cb + 8((l/16)&1) + e): one non-zero 16-bit element per lane
        const bool dw_active = (lr >> 3) == (lg & 1);
        const int dw_e = lr & 7;
        const uint16_t* wds16 = reinterpret_cast<const uint16_t*>(wds);
        auto dw_operand = [&](uint32_t v) {
            const int w = dw_e >> 1;
            return u32x4{w == 0 ? v : 0u, w == 1 ? v : 0u, w == 2 ? v : 0u, w == 3 ? v : 0u};
        };
        // LDS byte offsets of the lane's window reads for pixel block j and tap pair tp;
        // pixels past the tile read the last pixel (their results are never stored; the
        // same address as the block's last real lane, so no further bank group), the
        // empty tenth tap reads the first tap's pixel
        uint32_t xoff[MBW][NTP];
#pragma unroll
        for (int j = 0; j < MBW; ++j) {
            const int p0 = (jb + j) * 16 + lr, p = p0 < NPX ? p0 : NPX - 1;
            const int r = p / TW, c = p % TW;
#pragma unroll
            for (int tp = 0; tp < NTP; ++tp) {
                const int t0 = 2 * tp + (lg >> 1), t = t0 < 9 ? t0 : 0;
                const int ih = r * S + t / 3, iw = c * S + t % 3;
                const int q = 2 * cbw + (lg & 1);
                xoff[j][tp] = (uint32_t)((ih * IW + iw) * CH + (q ^ ((iw - ih) & 7))) * 16u;
            }
        }
        // intermediate: depthwise output rows 4(l/16)+i of channel block cb are channels
        // 16(cb%2) + 4(l/16) + i of slice cb/2, i.e. lane group 2(cb%2) + (l/16)/2, bytes
        // 8((l/16)%2)..+7 of its 16-byte operand
        const uint32_t tls_w =
            (uint32_t)(((2 * (cbw & 1) + (lg >> 1)) * 16 + lr) * 16 + (lg & 1) * 8);
        // one step's depthwise layer: window buffer src, slice c -> intermediate dst
        auto depthwise = [&](const u32x4* src, u32x4* dst, int c) {
            const char* xb = reinterpret_cast<const char*>(src);
            const int cb = c * 4 + cbw;
            uint32_t h[NTP];
#pragma unroll
            for (int tp = 0; tp < NTP; ++tp) {
                const int t = 2 * tp + (lg >> 1);
                h[tp] = wds16[(t < 9 ? t : 0) * CMAX + cb * 16 + lr];
            }
            const f32x4 sc = *reinterpret_cast<const f32x4*>(s1s + cb * 16 + lg * 4);
            const f32x4 bi = *reinterpret_cast<const f32x4*>(b1s + cb * 16 + lg * 4);
            // (one statement for the window reads: the window buffers and the buffer
            // being filled are one LDS array indexed at run time, so reads the compiler
            // saw would wait for every direct load in flight)
            uint32_t ad[NTP * MBW];
            u32x4 xr[NTP * MBW];
            const uint32_t xb0 = mm::lds_addr(xb);
#pragma unroll
            for (int tp = 0; tp < NTP; ++tp)
#pragma unroll
                for (int j = 0; j < MBW; ++j) ad[tp * MBW + j] = xb0 + xoff[j][tp];
            if constexpr (MBW == 4)
                mm::lds_read20(ad, xr);
            else
                mm::lds_read10(ad, xr);
            f32x4 d[MBW];
#pragma unroll
            for (int j = 0; j < MBW; ++j) d[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int tp = 0; tp < NTP; ++tp) {
                const int t = 2 * tp + (lg >> 1);
                const uint32_t v = (dw_active && t < 9) ? h[tp] : 0u;
                const u32x4 wf = dw_operand((dw_e & 1) ? (v << 16) : v);
#pragma unroll
                for (int j = 0; j < MBW; ++j) d[j] = mfma<T>(wf, xr[tp * MBW + j], d[j]);
            }
            const Act act1 = act_bounds(a.act1);
            const uint32_t tb = mm::lds_addr(dst);
#pragma unroll
            for (int j = 0; j < MBW; ++j) {
                float v[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = epilogue(d[j][i], sc[i], bi[i], act1);
                mm::lds_st8(tb + (uint32_t)(((jb + j) * NKS + (cbw >> 1)) * 64 * 16) + tls_w,
                            pack8<T>(v));
            }
        };

        // prologue: windows of steps 0..3, constants to LDS, depthwise layer of step 0
        Step w1 = next(s0);
        Step w2 = next(w1);
        Step w3 = next(w2);
        issue_window(s0, xs);
        issue_window(w1, xs + SLOTS_P);
        issue_window(w2, xs + 2 * SLOTS_P);
        issue_window(w3, xs + 3 * SLOTS_P);
        write_constants();
        mm::wait_vmcnt<3 * R>();  // window 0 (and the constants); windows 1..3 in flight
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): constants written
        __builtin_amdgcn_s_barrier();
        depthwise(xs, tl, 0);
        // step t: window t+1 waited for (t+2, t+3 in flight); barrier; window t+4 into
        // the buffer window t left; depthwise layer of step t+1
        Step sd = w1;         // the step whose depthwise layer this step computes
        Step si = next(w3);   // the step whose window this step requests
        for (int t = 0; t < n_steps; ++t) {
            mm::wait_vmcnt<2 * R>();
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): intermediate written
            __builtin_amdgcn_s_barrier();
            issue_window(si, xs + (t & 3) * SLOTS_P);
            __builtin_amdgcn_sched_barrier(0);  // the loads go out first
            depthwise(xs + ((t + 1) & 3) * SLOTS_P, tl + ((t + 1) & 1) * (MB * NKS * 64),
                      sd.c);
            sd = next(sd);
            si = next(si);
        }
        // windows of steps past the end may still be in flight into LDS
        mm::wait_vmcnt<0>();
    } else {
        // ================================ pointwise waves ================================
        const int p = wave - NDW;
        const int kw0 = k0 + p * KW;  // this wave's output channels
        const __amdgpu_buffer_rsrc_t ry =
            mm::rsrc(a.y, (uint32_t)(a.N * a.Ho * a.Wo * a.K * es));
        // pointwise A operand of this wave's slice for slice c, reduction step ks, block
        // kb: blocked copy, block (g, s, h) = ((kw0 + 32(kb/2))/32, 2c + ks, kb%2); a block
        // past the last output channel is clamped to the last one (its accumulator rows
        // belong to channels that are never stored).  Buffer loads with a 32-bit offset:
        // the destination registers are written by the load alone.
        struct PwOps {
            u32x4 w[NKS][KBW];
        };
        const int s32 = a.C / 32, g32 = (a.K + 31) / 32;
        const __amdgpu_buffer_rsrc_t rw =
            mm::rsrc((const T*)a.w2 + (int64_t)a.K * a.C, (uint32_t)(g32 * 32 * a.C * es));
        auto load_pw = [&](const Step& st, PwOps& o) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int kb = 0; kb < KBW; ++kb) {
                    const int g = min((kw0 >> 5) + (kb >> 1), g32 - 1);
                    const int blk = (g * s32 + 2 * st.c + ks) * 2 + (kb & 1);
                    o.w[ks][kb] = __builtin_bit_cast(
                        u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                   rw, (uint32_t)(blk * 64 + lane) * 16u, 0, 0));
                }
        };
        f32x4 acc[MB][KBW];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int kb = 0; kb < KBW; ++kb) acc[mb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        // epilogue 2 and the tile's stores: always NST per lane; pixels past the tile or
        // the output, and 8-channel runs past K, get the out-of-range offset
        auto finish = [&](const Pos& t) {
            const Act act2 = act_bounds(a.act2);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int px = mb * 16 + lr, r = px / TW, c = px % TW;
                const bool ok = px < NPX && t.oh0 + r < a.Ho && t.ow0 + c < a.Wo;
                const uint32_t v = (uint32_t)(r * out_row + c * a.K * es);
#pragma unroll
                for (int kb = 0; kb < KBW; kb += 2) {
                    const int kl = p * KW + 16 * kb + 8 * lg;  // run start in the K tile
                    const f32x4 sa = *reinterpret_cast<const f32x4*>(s2s + kl);
                    const f32x4 sb = *reinterpret_cast<const f32x4*>(s2s + kl + 4);
                    const f32x4 ba = *reinterpret_cast<const f32x4*>(b2s + kl);
                    const f32x4 bb = *reinterpret_cast<const f32x4*>(b2s + kl + 4);
                    float o[8];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        o[i] = epilogue(acc[mb][kb][i], sa[i], ba[i], act2);
                        o[4 + i] = epilogue(acc[mb][kb + 1][i], sb[i], bb[i], act2);
                    }
                    // the whole offset goes in the vector operand, scalar offset 0 (see
                    // dwpw_mm.hip)
                    const bool run_ok = ok && k0 + kl < a.K;
                    __builtin_amdgcn_raw_buffer_store_b128(
                        pack16<T>(o), ry,
                        run_ok ? (uint32_t)t.out_base + v + (uint32_t)((k0 + kl) * es) : mm::kOob,
                        0, mm::kStoreStream);
                }
#pragma unroll
                for (int kb = 0; kb < KBW; ++kb) acc[mb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        };
        // one step: barrier; filters of the next step into the other operand set;
        // products of this step; after a tile's last slice, epilogue 2 and stores; then
        // the wait for the next step's filters (on the branch that issued or skipped the
        // stores, so the compiler's count of the loads in flight is exact on every path)
        Step cur = s0;
        auto step = [&](const PwOps& use, PwOps& fill, int par) {
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): operand reads done
            __builtin_amdgcn_s_barrier();
            const Step nx = next(cur);
            load_pw(nx, fill);
            // the loads go out before this step's products: both operand sets stay live
            __builtin_amdgcn_sched_barrier(0);
            const u32x4* src = tl + par * (MB * NKS * 64);
            u32x4 bfr[MB][NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) bfr[mb][ks] = src[(mb * NKS + ks) * 64 + lane];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int kb = 0; kb < KBW; ++kb)
                        acc[mb][kb] = mfma<T>(use.w[ks][kb], bfr[mb][ks], acc[mb][kb]);
            if (cur.c == nch - 1) {
                finish(cur.t);
                mm::wait_vmcnt<NST>();
            } else {
                mm::wait_vmcnt<0>();
            }
            cur = nx;
        };
        PwOps pa, pb;
        load_pw(s0, pa);
        write_constants();
        mm::wait_vmcnt<0>();                 // the first step's filters and the constants
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): constants written
        __builtin_amdgcn_s_barrier();
        int t = 0;
        for (; t + 2 <= n_steps; t += 2) {
            step(pa, pb, 0);
            step(pb, pa, 1);
        }
        if (t < n_steps) step(pa, pb, 0);
    }
}

template <typename T, int S, int TH, int TW, int KT, int CMAX, int NW>
int launch_dwpw_wsl(const KArgs& a, int grid, void* stream) {
    (void)hipGetLastError();
    hipLaunchKernelGGL((dwpw_wsl_kernel<T, S, TH, TW, KT, CMAX, NW>), dim3(grid), dim3(64 * NW),
                       0, (hipStream_t)stream, a);
    return (int)hipGetLastError();
}
template <typename T, int S, int TH, int TW, int KT, int CMAX, int NW>
int occ_dwpw_wsl() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, dwpw_wsl_kernel<T, S, TH, TW, KT, CMAX, NW>, 64 * NW, 0) != hipSuccess)
        return 0;
    return n;
}

#define FCM_V_DWPW(...)
#define FCM_V_DWPW32(...)
#define FCM_V_B2B(...)
#define FCM_V_DWPW_MM(...)
#define FCM_V_B2B_MM(...)
#define FCM_V_DWPW_MMW(...)
#define FCM_V_DWPW_WSL(name, dt, CT, S, TH, TW, KT, CMAX, NW)                              \
    template int launch_dwpw_wsl<CT, S, TH, TW, KT, CMAX, NW>(const KArgs&, int, void*); \
    template int occ_dwpw_wsl<CT, S, TH, TW, KT, CMAX, NW>();
#include "../variants.def"
#undef FCM_V_DWPW
#undef FCM_V_DWPW32
#undef FCM_V_B2B
#undef FCM_V_DWPW_MM
#undef FCM_V_B2B_MM
#undef FCM_V_DWPW_MMW
#undef FCM_V_DWPW_WSL

}  // namespace fcm
