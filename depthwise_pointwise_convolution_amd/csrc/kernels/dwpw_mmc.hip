// dwpw_mmc.hip -- fused depthwise 3x3 -> pointwise 1x1 on the gfx950 matrix cores for
// any channel count C that is a multiple of 64: the input channels are streamed in
// 64-channel chunks and the pointwise accumulators stay in registers across chunks
// (output stationary, FCM paper "Fusing Depthwise and Pointwise Convolutions for
// Efficient Inference on GPUs", Sec. III, Fig. 3(b), with the channel dimension tiled
// as in its Eq. 2-4 accounting).
//
// A workgroup of 4 waves owns a 4x16-pixel output tile and a KT-wide slice of the
// output channels.  One step processes one (tile, chunk) pair:
//   phase A  wave w computes the depthwise layer of channel block w of the chunk
//            (16 channels, all 4 rows) as block-diagonal matrix products
//            (v_mfma_f32_16x16x32, five per 16 channels x 16 pixels), epilogue 1,
//            rounds, and writes 8 bytes per lane of the LDS intermediate chunk, in
//            pointwise B-operand order;
//   phase B  wave w accumulates output channels [KT/4*w, KT/4*(w+1)) of all 4 rows
//            over the chunk; after the last chunk of a tile it applies epilogue 2 and
//            writes the tile with 16-byte buffer stores.
// Steps are software-pipelined with one barrier each: step s runs phase A of step s+1
// and phase B of step s, on two input and two intermediate buffers, and requests the
// input chunk of step s+2 -- by direct global->LDS loads -- at its start.  The
// per-chunk operands (depthwise filters, epilogue-1 constants, pointwise filters) are
// loaded one or two steps ahead into registers, before the step's direct loads, so
// the only vector-memory operations issued after a chunk's loads are the previous
// step's stores, and the wait for the chunk counts exactly those.
#include <type_traits>

#include "mm_common.h"

namespace fcm {

template <typename T, int S, int KT, int OCC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC, 8)))
void dwpw_mmc_kernel(KArgs a) {
    constexpr int NT = 256, TH = 4, TW = 16, CC = 64;
    constexpr int IH = (TH - 1) * S + 3, IW = (TW - 1) * S + 3, NPIX = IH * IW;
    constexpr int CH = CC / 8;  // 16-byte chunks per pixel
    constexpr int SLOTS = NPIX * CH;
    constexpr int R = (SLOTS + NT - 1) / NT;  // direct-load rounds per step
    constexpr int SLOTS_P = R * NT;
    constexpr int NKS = CC / 32, NTP = 5;
    constexpr int KW = KT / 4;    // pointwise output channels per wave
    constexpr int KBW = KW / 16;  // 16-channel output blocks per wave
    static_assert(KT % 128 == 0, "each wave stores 16-byte runs of 8 output channels");
    constexpr int NST = TH * (KBW / 2);  // buffer stores per lane per finished tile
    static_assert(NST < 64, "vmcnt range");
    constexpr uint32_t ROW_BYTES = (uint32_t)S * IW * CH * 16;  // one output row down

    __shared__ __attribute__((aligned(16))) u32x4 xs0[SLOTS_P];
    __shared__ __attribute__((aligned(16))) u32x4 xs1[SLOTS_P];
    __shared__ __attribute__((aligned(16))) u32x4 tl0[TH * NKS * 64];
    __shared__ __attribute__((aligned(16))) u32x4 tl1[TH * NKS * 64];
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
    const int kw0 = k0 + wave * KW;  // this wave's output channels
    const int nch = a.C / CC;
    const T* __restrict__ wdw = (const T*)a.w1;
    const T* __restrict__ wpw = (const T*)a.w2;
    const int es = (int)sizeof(T);
    const __amdgpu_buffer_rsrc_t rx = mm::rsrc(a.x, (uint32_t)(a.N * a.H * a.W * a.C * es));
    const __amdgpu_buffer_rsrc_t ry = mm::rsrc(a.y, (uint32_t)(a.N * a.Ho * a.Wo * a.K * es));
    const int in_img = a.H * a.W * a.C * es, in_row = a.W * a.C * es;
    const int out_img = a.Ho * a.Wo * a.K * es, out_row = a.Wo * a.K * es;

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
    // slot s holds 16-byte chunk q of window pixel p = s / CH, s % CH = q ^ (column & 7)
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
    auto issue_chunk = [&](const Step& st, auto buf) {
        u32x4* dst = decltype(buf)::value == 0 ? X0 : X1;
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

    // ---- per-chunk operands, loaded ahead into one of two register sets -----------
    // depthwise: block cb = 4c + wave of chunk c; matrix operand lane (l%16, l/16):
    // channel 16cb + l%16, reduction index 8(l/16) + e = (tap 2tp + (l/16)/2, channel
    // 16cb + 8((l/16)&1) + e), one non-zero 16-bit element per lane (see dwpw_mm.hip);
    // the loads are unconditional (clamped addresses) so their number never varies
    const bool dw_active = (lr >> 3) == (lg & 1);
    const int dw_e = lr & 7;
    struct DwOps {
        uint32_t w[NTP];
        float s[4], b[4];
    };
    const float* s1p = a.s1 ? a.s1 : (const float*)a.w2;
    const float* b1p = a.b1 ? a.b1 : (const float*)a.w2;
    auto load_dw = [&](const Step& st, DwOps& o) {
        const int cb = st.c * 4 + wave;
#pragma unroll
        for (int tp = 0; tp < NTP; ++tp) {
            const int t = 2 * tp + (lg >> 1), c = cb * 16 + lr;
            const bool ok = dw_active && t < 9 && c < a.C;
            const uint16_t h = __builtin_bit_cast(uint16_t, wdw[(t < 9 ? t : 0) * a.C +
                                                                (c < a.C ? c : 0)]);
            const uint32_t v = ok ? (uint32_t)h : 0u;
            o.w[tp] = (dw_e & 1) ? (v << 16) : v;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = cb * 16 + lg * 4 + i;
            const int cc = c < a.C ? c : 0;
            const float sv = s1p[cc], bv = b1p[cc];
            o.s[i] = (a.s1 && c < a.C) ? sv : 1.0f;
            o.b[i] = (a.b1 && c < a.C) ? bv : 0.0f;
        }
    };
    // pointwise A operand of this wave's slice for chunk c, reduction step ks, block kb
    struct PwOps {
        u32x4 w[NKS][KBW];
    };
    auto load_pw = [&](const Step& st, PwOps& o) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int kb = 0; kb < KBW; ++kb) {
                const int ko = kw0 + kperm<KW>(kb, lr);
                const int c = st.c * CC + ks * 32 + lg * 4;
                const bool ok = ko < a.K;
                const T* row = wpw + (int64_t)(ok ? ko : 0) * a.C;
                const uint2 lo = *reinterpret_cast<const uint2*>(row + c);
                const uint2 hi = *reinterpret_cast<const uint2*>(row + c + 16);
                o.w[ks][kb] = u32x4{ok ? lo.x : 0u, ok ? lo.y : 0u, ok ? hi.x : 0u,
                                    ok ? hi.y : 0u};
            }
    };
    auto dw_operand = [&](uint32_t v) {
        const int w = dw_e >> 1;
        return u32x4{w == 0 ? v : 0u, w == 1 ? v : 0u, w == 2 ? v : 0u, w == 3 ? v : 0u};
    };

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
    // LDS byte offsets of the lane's depthwise operand reads in output row 0 (row r
    // adds r * ROW_BYTES); the empty tenth tap reads the first tap's pixel
    uint32_t xoff[NTP];
#pragma unroll
    for (int tp = 0; tp < NTP; ++tp) {
        const int t0 = 2 * tp + (lg >> 1), t = t0 < 9 ? t0 : 0;
        const int col = lr * S + t % 3;
        const int p = (t / 3) * IW + col;
        const int q = 2 * wave + (lg & 1);
        xoff[tp] = (uint32_t)(p * CH + (q ^ (col & 7))) * 16u;
    }
    const uint32_t tls_w = (uint32_t)lane * 16u + (uint32_t)(wave & 1) * 8u;
    const int kl = kw0 + lg * (KW / 4);
    const uint32_t st_lane =
        kl < a.K ? (uint32_t)(lr * a.K + kl) * (uint32_t)sizeof(T) : mm::kOob;

    // phase A of one step: xs -> tl (this wave's 16 channels of the chunk, 4 rows)
    auto phase_a = [&](const u32x4* src, u32x4* dst, const DwOps& o) {
        const char* xb = reinterpret_cast<const char*>(src);
        u32x4 wf[NTP];
#pragma unroll
        for (int tp = 0; tp < NTP; ++tp) wf[tp] = dw_operand(o.w[tp]);
        f32x4 d[TH];
#pragma unroll
        for (int r = 0; r < TH; ++r) d[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int tp = 0; tp < NTP; ++tp) {
            u32x4 xv[TH];
#pragma unroll
            for (int r = 0; r < TH; ++r)
                xv[r] = *reinterpret_cast<const u32x4*>(xb + xoff[tp] + r * ROW_BYTES);
#pragma unroll
            for (int r = 0; r < TH; ++r) d[r] = mfma<T>(wf[tp], xv[r], d[r]);
        }
#pragma unroll
        for (int r = 0; r < TH; ++r) {
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = epilogue(d[r][i], o.s[i], o.b[i], act1);
            *reinterpret_cast<uint2*>(reinterpret_cast<char*>(dst) +
                                      ((r * NKS + (wave >> 1)) * 64) * 16 + tls_w) = pack8<T>(v);
        }
    };
    // phase B of one step: acc += pointwise filters x intermediate chunk
    f32x4 acc[TH][KBW];
#pragma unroll
    for (int mb = 0; mb < TH; ++mb)
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) acc[mb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto phase_b = [&](const u32x4* src, const PwOps& o) {
        u32x4 bfr[TH][NKS];
#pragma unroll
        for (int mb = 0; mb < TH; ++mb)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) bfr[mb][ks] = src[(mb * NKS + ks) * 64 + lane];
#pragma unroll
        for (int mb = 0; mb < TH; ++mb)
#pragma unroll
            for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    acc[mb][kb] = mfma<T>(o.w[ks][kb], bfr[mb][ks], acc[mb][kb]);
    };
    // epilogue 2 and the tile's stores (always NST per lane; rows or lanes outside the
    // output get the out-of-range offset)
    auto finish = [&](const Pos& t) {
        const uint32_t voff = t.ow0 + lr < a.Wo ? st_lane : mm::kOob;
#pragma unroll
        for (int mb = 0; mb < TH; ++mb) {
            const bool row_ok = t.oh0 + mb < a.Ho;
            const uint32_t v = row_ok ? voff : mm::kOob;
            const int srow = row_ok ? t.out_base + mb * out_row : 0;
#pragma unroll
            for (int kb = 0; kb < KBW; kb += 2) {
                float o[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    o[i] = epilogue(acc[mb][kb][i], s2r[kb * 4 + i], b2r[kb * 4 + i], act2);
                    o[4 + i] = epilogue(acc[mb][kb + 1][i], s2r[kb * 4 + 4 + i],
                                        b2r[kb * 4 + 4 + i], act2);
                }
                __builtin_amdgcn_raw_buffer_store_b128(pack16<T>(o), ry, v + kb * 4 * sizeof(T),
                                                       srow, 0);
            }
#pragma unroll
            for (int kb = 0; kb < KBW; ++kb) acc[mb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };

    // ---- prologue: operands of steps 0 and 1, input chunks of steps 0 and 1 --------
    Step s0;
    s0.t = split(L / a.num_ktiles);
    s0.c = 0;
    Step s1 = next(s0);
    DwOps dwo0, dwo1;
    PwOps pwo0, pwo1;
    load_dw(s0, dwo0);
    load_dw(s1, dwo1);
    load_pw(s0, pwo0);
    issue_chunk(s0, std::integral_constant<int, 0>{});
    issue_chunk(s1, std::integral_constant<int, 1>{});
    mm::wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (s0.t.n < a.N) phase_a(X0, T0, dwo0);

    // ---- pipelined steps ---------------------------------------------------------------
    // step s (P = s % 2): wait for chunk s+1 (only the previous step's stores, if it
    // finished a tile, were issued after it); barrier; operands of step s+2 (depthwise)
    // and s+1 (pointwise); input chunk of step s+2 into xs[P]; phase A of s+1; phase B
    // of s; if s ends its tile, epilogue 2 and stores.
    Step cur = s0, nx = s1;
    bool stored = false;
    auto step_fn = [&](auto par, DwOps& dw_this, DwOps& dw_next, PwOps& pw_this,
                       PwOps& pw_next) {
        constexpr int P = decltype(par)::value;
        if (stored) mm::wait_vmcnt<NST>(); else mm::wait_vmcnt<0>();
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): own intermediate writes done
        __builtin_amdgcn_s_barrier();
        const Step nn = next(nx);
        load_dw(nn, dw_this);   // dw_this held step s's filters, used in step s-1
        load_pw(nx, pw_next);   // pw_next held step s-1's filters, used in step s-1
        issue_chunk(nn, std::integral_constant<int, P>{});
        if (nx.t.n < a.N) phase_a(P == 0 ? X1 : X0, P == 0 ? T1 : T0, dw_next);
        phase_b(P == 0 ? T0 : T1, pw_this);
        stored = cur.c == nch - 1;
        if (stored) finish(cur.t);
        cur = nx;
        nx = nn;
    };
    while (cur.t.n < a.N) {
        step_fn(std::integral_constant<int, 0>{}, dwo0, dwo1, pwo0, pwo1);
        if (cur.t.n >= a.N) break;
        step_fn(std::integral_constant<int, 1>{}, dwo1, dwo0, pwo1, pwo0);
    }
    // chunks of steps past the end may still be in flight into LDS
    mm::wait_vmcnt<0>();
}

template <typename T, int S, int KT, int OCC>
int launch_dwpw_mmc(const KArgs& a, int grid, void* stream) {
    (void)hipGetLastError();
    hipLaunchKernelGGL((dwpw_mmc_kernel<T, S, KT, OCC>), dim3(grid), dim3(256), 0,
                       (hipStream_t)stream, a);
    return (int)hipGetLastError();
}
template <typename T, int S, int KT, int OCC>
int occ_dwpw_mmc() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, dwpw_mmc_kernel<T, S, KT, OCC>, 256,
                                                     0) != hipSuccess)
        return 0;
    return n;
}

#define FCM_V_DWPW(...)
#define FCM_V_DWPW32(...)
#define FCM_V_B2B(...)
#define FCM_V_DWPW_MM(...)
#define FCM_V_B2B_MM(...)
#define FCM_V_DWPW_MMC(name, dt, CT, S, KT, OCC)                                 \
    template int launch_dwpw_mmc<CT, S, KT, OCC>(const KArgs&, int, void*); \
    template int occ_dwpw_mmc<CT, S, KT, OCC>();
#include "../variants.def"
#undef FCM_V_DWPW
#undef FCM_V_DWPW32
#undef FCM_V_B2B
#undef FCM_V_DWPW_MM
#undef FCM_V_DWPW_MMC
#undef FCM_V_B2B_MM

}  // namespace fcm
