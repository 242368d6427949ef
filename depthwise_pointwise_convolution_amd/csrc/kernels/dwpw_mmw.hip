// dwpw_mmw.hip -- fused depthwise 3x3 -> pointwise 1x1 on the gfx950 matrix cores for
// layers with C a multiple of 64 (K up to 512 per workgroup): NW = 4 or 8 waves,
// the input channels streamed in 64-channel chunks with two chunks in flight, the
// pointwise accumulators held in registers across the chunks (output stationary, FCM
// paper "Fusing Depthwise and Pointwise Convolutions for Efficient Inference on GPUs",
// Sec. III, Fig. 3(b)).  With a K tile that covers all output channels the depthwise
// layer is computed exactly once, which is the DWPW module's "no redundant
// computation" property (Sec. III-A).
//
// The output tile is any TH x TW block of pixels, numbered row-major and cut into
// 16-pixel matrix blocks (a whole 7x7 map is one tile of four blocks), so small late-
// network maps do not waste most of a 4x16 tile.
//
// One step processes one (tile, chunk) pair:
//   phase A  the chunk's depthwise layer as block-diagonal matrix products
//            (v_mfma_f32_16x16x32, five per 16 channels x 16 pixels), epilogue 1,
//            rounding, and 8-byte writes of the LDS intermediate chunk in pointwise
//            operand order; the (pixel block, channel block) pairs are spread over
//            the 8 waves;
//   phase B  wave w accumulates output channels [KT/8*w, KT/8*(w+1)) of every pixel
//            block over the chunk; after the last chunk of a tile it applies
//            epilogue 2 and writes the tile with 16-byte buffer stores.
// Steps are software-pipelined with one barrier each: step s runs phase A of step
// s+1 and phase B of step s on three input buffers and two intermediate buffers, and
// requests the input chunk of step s+3 by direct global->LDS loads, so two chunks are
// in flight while the matrix cores work.  The depthwise filters and epilogue
// constants of all C <= CMAX channels are copied to LDS once per workgroup.  The
// pointwise filters of step s+1 are loaded into registers before step s's direct
// loads, one 16-byte load per matrix operand from the blocked copy that
// fcm_pack_weights writes after the [K][C] filters (each operand one contiguous
// kilobyte); the wait at the start of a step then counts exactly the loads of one
// chunk (and the stores of a finished tile).
//
// Channel orders: the reduction index k of a 32-channel slice is input channel
// 32 ks + k (lane group l/16 holds channels 8(l/16)..+7 of the intermediate); row r of
// output block kb holds output channel 32(kb/2) + 8(r/4) + 4(kb%2) + r%4 of the wave's
// slice, so that lane group g ends up with 8 consecutive output channels per block
// pair and writes them with one 16-byte store.
#include <type_traits>

#include "mm_common.h"

namespace fcm {

// D: dilation of the depthwise taps (the window then spans (TH-1)S + 2D + 1 rows)
template <typename T, int S, int TH, int TW, int KT, int CMAX, int NW, int OCC, int D>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(OCC, 8)))
void dwpw_mmw_kernel(KArgs a) {
    static_assert(NW == 4 || NW == 8, "4 or 8 waves");
    constexpr int NT = 64 * NW, CC = 64, NB = 3;
    constexpr int NPX = TH * TW, MB = (NPX + 15) / 16;
    constexpr int IH = (TH - 1) * S + 2 * D + 1, IW = (TW - 1) * S + 2 * D + 1, NPIX = IH * IW;
    constexpr int CH = CC / 8;  // 16-byte pieces per pixel
    constexpr int SLOTS = NPIX * CH;
    constexpr int R = (SLOTS + NT - 1) / NT;  // direct-load rounds per chunk
    constexpr int SLOTS_P = R * NT;
    constexpr int NKS = CC / 32, NTP = 5;
    constexpr int KW = KT / NW;   // pointwise output channels per wave
    constexpr int KBW = KW / 16;  // 16-channel output blocks per wave
    static_assert(KBW % 2 == 0, "each lane stores 16-byte runs of 8 output channels");
    constexpr int PPW = MB * 4 / NW;  // depthwise (pixel block, channel block) pairs per wave
    static_assert(PPW * NW == MB * 4, "pixel blocks must split evenly over the waves");
    constexpr int NST = MB * (KBW / 2);  // buffer stores per lane per finished tile
    static_assert(R + NST < 64 && 2 * R < 64, "vmcnt range");
    static_assert(CMAX % 64 == 0, "whole chunks");
    // phase B's operands can be read before phase A when its accumulators leave room
    constexpr bool EARLY_B = MB * KBW <= 8;

    __shared__ __attribute__((aligned(16))) u32x4 xs[NB * SLOTS_P];
    __shared__ __attribute__((aligned(16))) u32x4 tl0[MB * NKS * 64];
    __shared__ __attribute__((aligned(16))) u32x4 tl1[MB * NKS * 64];
    __shared__ __attribute__((aligned(16))) float s2s[KT];
    __shared__ __attribute__((aligned(16))) float b2s[KT];
    __shared__ __attribute__((aligned(16))) u32x4 wds[9 * CMAX / 8];  // depthwise [9][CMAX]
    __shared__ __attribute__((aligned(16))) float s1s[CMAX];
    __shared__ __attribute__((aligned(16))) float b1s[CMAX];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const Act act1 = act_bounds(a.act1), act2 = act_bounds(a.act2);
    const int G = gridDim.x;
    const int L = xcd_logical_id(blockIdx.x, G);
    const int k0 = (L % a.num_ktiles) * KT;
    const int kw0 = k0 + wave * KW;  // this wave's output channels
    const int nch = a.C / CC;
    const T* __restrict__ wdw = (const T*)a.w1;
    const T* __restrict__ wpw = (const T*)a.w2;
    const int es = (int)sizeof(T);
    const __amdgpu_buffer_rsrc_t rx = mm::rsrc(a.x, (uint32_t)(a.N * a.H * a.W * a.C * es));
    const __amdgpu_buffer_rsrc_t ry = mm::rsrc(a.y, (uint32_t)(a.N * a.Ho * a.Wo * a.K * es));
    const int in_img = a.H * a.W * a.C * es, in_row = a.W * a.C * es;
    const int out_img = a.Ho * a.Wo * a.K * es, out_row = a.Wo * a.K * es;

    // epilogue-2 constants of the workgroup's K tile (read back per finished tile), the
    // depthwise filters and the epilogue-1 constants of every channel.  Every load is
    // issued before the first LDS write (fixed per-thread counts, masked past the end),
    // so the copy costs one memory latency rather than one per loop round; the writes
    // come after the prologue has requested the first chunks and operands.
    constexpr int I2 = (KT + NT - 1) / NT, IW9 = (9 * CMAX / 8 + NT - 1) / NT;
    constexpr int I1 = (CMAX + NT - 1) / NT;
    const int nw = 9 * (a.C / 8);
    float s2v[I2], b2v[I2], s1v[I1], b1v[I1];
    u32x4 wv[IW9];
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
    auto load_constants = [&]() {
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
    };

    // ---- (tile, chunk) walk --------------------------------------------------------
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

    // ---- direct-load plan of one chunk (step invariant) ---------------------------
    // slot s holds 16-byte piece q of window pixel p = s / CH, s % CH = q ^ (column & 7)
    uint32_t dl_off[R];
    int dl_pos[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int s = r * NT + tid;
        const int p = s / CH, ihl = p / IW, iwl = p % IW;
        const int q = (s % CH) ^ (iwl & 7);
        const bool real = s < SLOTS;
        dl_off[r] = real ? (uint32_t)((ihl * a.W + iwl) * a.C + q * 8) * (uint32_t)es : mm::kOob;
        dl_pos[r] = real ? (ihl << 16) | iwl : 0;
    }
    // always R loads per lane, whatever the step (zero-filled when outside the image or
    // past the last tile), so the vector-memory counts of the waits are exact
    auto issue_chunk = [&](const Step& st, u32x4* dst) {
        const Pos& t = st.t;
        const bool live = t.n < a.N;
        const int cbyte = st.c * CC * es;
        const bool inside = live && t.ih0 >= 0 && t.iw0 >= 0 && t.ih0 + IH <= a.H &&
                            t.iw0 + IW <= a.W;
        if (inside) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t off = dl_off[r];  // (a copy, see dwpw_mm.hip)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rx, (__attribute__((address_space(3))) void*)(dst + r * NT + wave * 64), 16,
                    off, t.in_base + cbyte, 0, 0);
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
                    rx, (__attribute__((address_space(3))) void*)(dst + r * NT + wave * 64), 16,
                    off, 0, 0, 0);
            }
        }
    };

    // ---- operands ----------------------------------------------------------------------
    // depthwise: this wave's channel block cb = wave % 4 of the chunk; matrix operand
    // lane (l%16, l/16): channel 16cb + l%16, reduction index 8(l/16) + e = (tap
    // 2tp + (l/16)/2, channel 16cb + 8((l/16)&1) + e): one non-zero 16-bit element per
    // lane, read from the LDS copy of the filters
    const int cbw = wave & 3;
    const bool dw_active = (lr >> 3) == (lg & 1);
    const int dw_e = lr & 7;
    const uint16_t* wds16 = reinterpret_cast<const uint16_t*>(wds);
    // pointwise A operand of this wave's slice for chunk c, reduction step ks, block kb:
    // blocked copy, block (g, s, h) = ((kw0 + 32(kb/2))/32, 2c + ks, kb%2); a block past
    // the last output channel is clamped to the last one (its accumulator rows belong to
    // channels that are never stored)
    struct PwOps {
        u32x4 w[NKS][KBW];
    };
    // (buffer loads with a 32-bit offset: the destination registers are written by the
    // load alone, so reusing them for the next step's operands waits for nothing)
    const int s32 = a.C / 32, g32 = (a.K + 31) / 32;
    const __amdgpu_buffer_rsrc_t rw =
        mm::rsrc(wpw + (int64_t)a.K * a.C, (uint32_t)(g32 * 32 * a.C * es));
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
    auto dw_operand = [&](uint32_t v) {
        const int w = dw_e >> 1;
        return u32x4{w == 0 ? v : 0u, w == 1 ? v : 0u, w == 2 ? v : 0u, w == 3 ? v : 0u};
    };

    // LDS byte offsets of the lane's depthwise operand reads for its pixel blocks
    // mb = wave / 4 + j * (NW / 4); pixels past the tile read pixel 0 (their results
    // are never stored); the empty tenth tap reads the first tap's pixel
    uint32_t xoff[PPW][NTP];
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
        const int mb = (wave >> 2) + j * (NW / 4);
        const int p0 = mb * 16 + lr, p = p0 < NPX ? p0 : 0;
        const int r = p / TW, c = p % TW;
#pragma unroll
        for (int tp = 0; tp < NTP; ++tp) {
            const int t0 = 2 * tp + (lg >> 1), t = t0 < 9 ? t0 : 0;
            const int ih = r * S + (t / 3) * D, iw = c * S + (t % 3) * D;
            const int q = 2 * cbw + (lg & 1);
            xoff[j][tp] = (uint32_t)((ih * IW + iw) * CH + (q ^ (iw & 7))) * 16u;
        }
    }
    // intermediate: DW output rows 4(l/16)+i of channel block cb are channels
    // 16(cb%2) + 4(l/16) + i of slice cb/2, i.e. lane group 2(cb%2) + (l/16)/2, bytes
    // 8((l/16)%2)..+7 of its 16-byte operand
    const uint32_t tls_w =
        (uint32_t)(((2 * (cbw & 1) + (lg >> 1)) * 16 + lr) * 16 + (lg & 1) * 8);

    // phase A of one step: xs chunk c -> intermediate chunk (the LDS reads of the
    // depthwise operands, then the products, epilogue 1 and the intermediate writes)
    struct AIn {
        uint32_t h[NTP];
        f32x4 s, b;
        u32x4 xv[NTP][PPW];
    };
    auto phase_a_load = [&](const u32x4* src, int c, AIn& in) {
        const char* xb = reinterpret_cast<const char*>(src);
        const int cb = c * 4 + cbw;
#pragma unroll
        for (int tp = 0; tp < NTP; ++tp) {
            const int t = 2 * tp + (lg >> 1);
            in.h[tp] = wds16[(t < 9 ? t : 0) * CMAX + cb * 16 + lr];
        }
        in.s = *reinterpret_cast<const f32x4*>(s1s + cb * 16 + lg * 4);
        in.b = *reinterpret_cast<const f32x4*>(b1s + cb * 16 + lg * 4);
#pragma unroll
        for (int tp = 0; tp < NTP; ++tp)
#pragma unroll
            for (int j = 0; j < PPW; ++j)
                in.xv[tp][j] = *reinterpret_cast<const u32x4*>(xb + xoff[j][tp]);
    };
    auto phase_a_compute = [&](const AIn& in, u32x4* dst) {
        u32x4 wf[NTP];
#pragma unroll
        for (int tp = 0; tp < NTP; ++tp) {
            const int t = 2 * tp + (lg >> 1);
            const uint32_t v = (dw_active && t < 9) ? in.h[tp] : 0u;
            wf[tp] = dw_operand((dw_e & 1) ? (v << 16) : v);
        }
        f32x4 d[PPW];
#pragma unroll
        for (int j = 0; j < PPW; ++j) d[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int tp = 0; tp < NTP; ++tp)
#pragma unroll
            for (int j = 0; j < PPW; ++j) d[j] = mfma<T>(wf[tp], in.xv[tp][j], d[j]);
#pragma unroll
        for (int j = 0; j < PPW; ++j) {
            const int mb = (wave >> 2) + j * (NW / 4);
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = epilogue(d[j][i], in.s[i], in.b[i], act1);
            mm::lds_st8(mm::lds_addr(dst) + ((mb * NKS + (cbw >> 1)) * 64) * 16 + tls_w,
                        pack8<T>(v));
        }
    };
    auto phase_a = [&](const u32x4* src, u32x4* dst, int c) {
        AIn in;
        phase_a_load(src, c, in);
        phase_a_compute(in, dst);
    };
    // phase B of one step: acc += pointwise filters x intermediate chunk
    f32x4 acc[MB][KBW];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) acc[mb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // (reduction step outermost: the two updates of an accumulator are MB * KBW matrix
    // instructions apart and each one reads and writes it in place)
    // the intermediate operands of phase B (read before phase A writes the other
    // intermediate buffer, so that the reads can be issued early)
    struct BIn {
        u32x4 v[MB][NKS];
    };
    auto phase_b_load = [&](const u32x4* src, BIn& bfr) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) bfr.v[mb][ks] = src[(mb * NKS + ks) * 64 + lane];
    };
    auto phase_b = [&](const BIn& in, const PwOps& o) {
        const auto& bfr = in.v;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int kb = 0; kb < KBW; ++kb)
                    acc[mb][kb] = mfma<T>(o.w[ks][kb], bfr[mb][ks], acc[mb][kb]);
    };
    // epilogue 2 and the tile's stores: always NST per lane; pixels past the tile or the
    // output, and 8-channel runs past K, get the out-of-range offset
    auto finish = [&](const Pos& t) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int p = mb * 16 + lr, r = p / TW, c = p % TW;
            const bool ok = p < NPX && t.oh0 + r < a.Ho && t.ow0 + c < a.Wo;
            const uint32_t v = (uint32_t)(r * out_row + c * a.K * es);
#pragma unroll
            for (int kb = 0; kb < KBW; kb += 2) {
                const int kl = wave * KW + 16 * kb + 8 * lg;  // run start in the K tile
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

    // ---- prologue: operands of steps 0 and 1, input chunks of steps 0, 1, 2 -------
    Step s0;
    s0.t = split(L / a.num_ktiles);
    s0.c = 0;
    const Step s1 = next(s0);
    const Step s2 = next(s1);
    PwOps pwo0, pwo1;
    load_constants();
    load_pw(s0, pwo0);
    issue_chunk(s0, xs);
    issue_chunk(s1, xs + SLOTS_P);
    issue_chunk(s2, xs + 2 * SLOTS_P);
    write_constants();
    mm::wait_vmcnt<2 * R>();  // chunk 0 and the operands; chunks 1, 2 stay in flight
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): LDS constants written
    __builtin_amdgcn_s_barrier();
    if (s0.t.n < a.N) phase_a(xs, tl0, s0.c);
    mm::wait_vmcnt<R>();  // chunk 1 (chunk 2 stays in flight)

    // ---- pipelined steps ---------------------------------------------------------------
    // step s (P = s % 2, xi = s % 3): barrier (chunk s+1 and the operands of step s were
    // waited for at the end of step s-1: only chunk s+2's loads and step s-1's stores, if
    // it finished a tile, were issued after them); pointwise operands of step s+1 into the
    // other operand set; input chunk of step s+3 into xs[xi]; phase A of s+1 from
    // xs[(xi+1)%3] into tl[1-P]; phase B of s from tl[P]; if s ends its tile, epilogue 2
    // and stores.  The loop runs two steps per round, so the two operand sets and the
    // two intermediate buffers are named at compile time and alternate without register
    // copies (a copy of the operands just requested would wait for those loads); the
    // accumulators stay in the same registers, so every matrix instruction of a chain
    // reads and writes its accumulator in place.
    Step cur = s0, nx = s1, nn = s2;
    int xi = 0;
    auto step = [&](auto parc, const PwOps& use, PwOps& fill) {
        constexpr int par = decltype(parc)::value;
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): own intermediate writes done
        __builtin_amdgcn_s_barrier();
        const Step n3 = next(nn);
        // (every step issues the same loads, so the compiler's count of the loads in
        // flight is the same on every path; with one chunk they repeat the same operands)
        load_pw(nx, fill);
        const int xa = xi == 2 ? 0 : xi + 1;
        issue_chunk(n3, xs + xi * SLOTS_P);
        // phase A runs even for a step past the last tile (its chunk was zero-filled and
        // its intermediate is never read)
        // scheduling groups for the step: the LDS operand reads of a phase before its
        // products; where registers allow (EARLY_B), phase B's intermediate operands
        // (written in the previous step) are read before phase A as well
        BIn bfr;
        if constexpr (EARLY_B) phase_b_load(par ? tl1 : tl0, bfr);
        phase_a(xs + xa * SLOTS_P, par ? tl0 : tl1, nx.c);
        if constexpr (!EARLY_B) phase_b_load(par ? tl1 : tl0, bfr);
        phase_b(bfr, use);
        if constexpr (EARLY_B) {
            __builtin_amdgcn_sched_group_barrier(0x100, NTP + 2 + NTP * PPW + MB * NKS, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, NTP * PPW, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, MB * KBW * NKS, 0);
        } else {
            __builtin_amdgcn_sched_group_barrier(0x100, NTP + 2 + NTP * PPW, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, NTP * PPW, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, MB * NKS, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, MB * KBW * NKS, 0);
        }
        // the wait for the next step sits on the branch that issued (or skipped) the
        // stores, so the compiler's own count of the loads in flight stays exact on
        // every path
        if (cur.c == nch - 1) {
            finish(cur.t);
            mm::wait_vmcnt<R + NST>();
        } else {
            mm::wait_vmcnt<R>();
        }
        cur = nx;
        nx = nn;
        nn = n3;
        xi = xa;
    };
    // the workgroup's step count, known up front: a loop of step pairs and at most one
    // more step, with no exit test between the two steps of a pair (an exit test there
    // lets the compiler merge the two steps into one loop body entered either way, and
    // its count of the loads in flight then has to cover paths that never run)
    const int t_first = L / a.num_ktiles;
    const int n_tiles = t_first < a.num_ptiles ? (a.num_ptiles - 1 - t_first) / pstep + 1 : 0;
    const int n_steps = n_tiles * nch;
    int si = 0;
    for (; si + 2 <= n_steps; si += 2) {
        step(std::integral_constant<int, 0>{}, pwo0, pwo1);
        step(std::integral_constant<int, 1>{}, pwo1, pwo0);
    }
    if (si < n_steps) step(std::integral_constant<int, 0>{}, pwo0, pwo1);
    // chunks of steps past the end may still be in flight into LDS
    mm::wait_vmcnt<0>();
}

template <typename T, int S, int TH, int TW, int KT, int CMAX, int NW, int OCC, int D>
int launch_dwpw_mmw(const KArgs& a, int grid, void* stream) {
    (void)hipGetLastError();
    hipLaunchKernelGGL((dwpw_mmw_kernel<T, S, TH, TW, KT, CMAX, NW, OCC, D>), dim3(grid), dim3(64 * NW), 0,
                       (hipStream_t)stream, a);
    return (int)hipGetLastError();
}
template <typename T, int S, int TH, int TW, int KT, int CMAX, int NW, int OCC, int D>
int occ_dwpw_mmw() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, dwpw_mmw_kernel<T, S, TH, TW, KT, CMAX, NW, OCC, D>,
                                                     64 * NW, 0) != hipSuccess)
        return 0;
    return n;
}

#define FCM_V_DWPW(...)
#define FCM_V_DWPW32(...)
#define FCM_V_B2B(...)
#define FCM_V_DWPW_MM(...)
#define FCM_V_B2B_MM(...)
#define FCM_V_DWPW_MMW(name, dt, CT, S, TH, TW, KT, CMAX, NW, OCC)                           \
    template int launch_dwpw_mmw<CT, S, TH, TW, KT, CMAX, NW, OCC, 1>(const KArgs&, int, void*); \
    template int occ_dwpw_mmw<CT, S, TH, TW, KT, CMAX, NW, OCC, 1>();
#define FCM_V_DWPW_MMWD(name, dt, CT, S, D, TH, TW, KT, CMAX, NW, OCC)                        \
    template int launch_dwpw_mmw<CT, S, TH, TW, KT, CMAX, NW, OCC, D>(const KArgs&, int, void*); \
    template int occ_dwpw_mmw<CT, S, TH, TW, KT, CMAX, NW, OCC, D>();
#include "../variants.def"
#undef FCM_V_DWPW
#undef FCM_V_DWPW32
#undef FCM_V_B2B
#undef FCM_V_DWPW_MM
#undef FCM_V_B2B_MM
#undef FCM_V_DWPW_MMW
#undef FCM_V_DWPW_MMWD

}  // namespace fcm
