// pwdwpw_mm.hip -- the three convolutional layers of an inverted-residual block in one
// kernel: pointwise 1x1 expansion -> depthwise 3x3 -> pointwise 1x1 projection, each
// with its epilogue, and the block's identity shortcut (16-bit storage, C <= CMAX).
//
// "Fusing Depthwise and Pointwise Convolutions for Efficient Inference on GPUs" builds
// its modules from the layers of separable convolutions and inverted residuals
// (Sec. II-B: an inverted residual is PW-DW-PW; Fig. 4); its FCMs fuse two of them.
// This module fuses all three, so neither intermediate reaches HBM: the expansion's
// output lives in LDS as in the PW->DW module (PWDW_R, Sec. II-D, Fig. 3(b): the
// expansion is recomputed on the halo that neighbouring tiles share), and the
// depthwise output feeds the projection from LDS as the DW->PW module's intermediate
// does (Sec. III, Fig. 3(b)).  The projection needs every expanded channel of a pixel,
// so one workgroup holds all of them (the DW->PW feasibility rule of Sec. II-D).
//
// Work of a workgroup: one TH x 16 tile of output pixels, all K1 expanded channels
// (NB = NW * BPW 16-channel blocks, wave w owning blocks w * BPW .. + BPW - 1), all K
// output channels (KB 16-channel blocks).  One step per tile:
//   expansion  T^T[c][p] = sum_ci W1[c][ci] * X[p][ci] over every 16-pixel block of the
//              input window (one v_mfma_f32_16x16x32 per 16 channels x 16 pixels x 32
//              input channels); epilogue 1; window pixels outside the image are set to
//              zero (the depthwise layer's zero padding surrounds the intermediate); the
//              rounded values go to the wave's LDS tile;
//   depthwise  the block-diagonal matrix form over the wave's LDS tile (A = the 16-channel
//              filter diagonal for two taps, B = 16 bytes of the intermediate per lane);
//              epilogue 2; the rounded values go to the shared depthwise tile in LDS,
//              [pixel][channel] with one spare 16-byte slot per pixel row so the 16 lanes
//              of a projection operand read (16 pixels, same channels) hit distinct bank
//              groups;
//   barrier;
//   projection Y^T[k][p] = sum_c W3[k][c] * D[p][c]: the TH x KB (row, output block)
//              units are spread over the waves; the W3 operands of all KB blocks stay in
//              registers; epilogue 3, plus the input pixel for the shortcut (read from
//              the input window in LDS: stride 1 and K == C), one rounding, 8-byte
//              buffer stores.
// The input window arrives by direct global->LDS loads into two buffers, the next
// tile's window requested at the start of a step; out-of-image pixels and channels
// past C come back as zeros from the buffer range check; every wave issues the same
// number of memory instructions per step (stores of pixels outside the output get an
// out-of-range offset and are dropped), so the wait for the next window counts them
// exactly.
#include <type_traits>

#include "mm_common.h"

namespace fcm {

template <typename T, int S, int TH, int CMAX, int NW, int BPW, int KB, int OCC>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(OCC, 8)))
void pwdwpw_mm_kernel(KArgs a) {
    constexpr int TW = 16;
    constexpr int NT = 64 * NW;
    constexpr int IH = (TH - 1) * S + 3, IW = (TW - 1) * S + 3, NP = IH * IW;
    constexpr int NPB = (NP + 15) / 16;  // 16-pixel blocks of the window
    constexpr int NCH = CMAX / 8;        // 16-byte chunks per window pixel in LDS
    static_assert(NCH == 4 || NCH == 8, "32 or 64 input channels");
    constexpr int NKC = CMAX / 32;       // reduction steps of the expansion
    constexpr int SLOTS = NPB * 16 * NCH;
    constexpr int R = (SLOTS + NT - 1) / NT;  // direct-load rounds per window
    constexpr int SLOTS_P = R * NT;
    constexpr int NB = NW * BPW;         // expanded-channel blocks of the workgroup
    static_assert(NB % 2 == 0, "the projection reduces over whole 32-channel steps");
    constexpr int K1P = NB * 16;         // expanded channels held (K1 <= K1P)
    constexpr int NK3 = K1P / 32;        // reduction steps of the projection
    constexpr int NU = (TH * KB + NW - 1) / NW;  // projection units per wave
    constexpr int NST = NU;              // buffer stores per lane per step
    static_assert(NST < 64, "vmcnt range");
    static_assert(NPB <= 32, "window validity fits one 32-bit mask");
    // intermediate tile of one channel block: (IH + 1) rows (the extra row takes the
    // pixels of the last, partial pixel block) x 2 chunks x IW columns x 16 bytes
    constexpr int TROW = 2 * IW * 16;
    constexpr int TREG = (IH + 1) * TROW;
    constexpr int IHW = IH;
    // depthwise tile: TH * 16 pixels x (K1P + 8) channels (a spare 16-byte slot per pixel)
    constexpr int DSTR = (K1P + 8) * 2;
    constexpr int DT = TH * 16 * DSTR;

    __shared__ __attribute__((aligned(16))) u32x4 xs0[SLOTS_P];
    __shared__ __attribute__((aligned(16))) u32x4 xs1[SLOTS_P];
    __shared__ __attribute__((aligned(16))) u32x4 tl[NB * TREG / 16];
    __shared__ __attribute__((aligned(16))) u32x4 dt[DT / 16];
    u32x4* const X0 = xs0;
    u32x4* const X1 = xs1;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    char* const tbase = reinterpret_cast<char*>(tl) + wave * BPW * TREG;
    char* const dbase = reinterpret_cast<char*>(dt);
    const Act act1 = act_bounds(a.act1), act2 = act_bounds(a.act2), act3 = act_bounds(a.act3);
    const int G = gridDim.x;
    const int L = xcd_logical_id(blockIdx.x, G);
    const int cb0 = wave * BPW;  // first owned expanded-channel block
    const T* __restrict__ wpw = (const T*)a.w1;   // [K1][C]
    const T* __restrict__ wdw = (const T*)a.w2;   // [9][K1]
    const T* __restrict__ wpj = (const T*)a.w3;   // [K][K1]
    const int es = (int)sizeof(T);
    const __amdgpu_buffer_rsrc_t rx = mm::rsrc(a.x, (uint32_t)(a.N * a.H * a.W * a.C * es));
    const __amdgpu_buffer_rsrc_t ry = mm::rsrc(a.y, (uint32_t)(a.N * a.Ho * a.Wo * a.K * es));
    const int in_img = a.H * a.W * a.C * es, in_row = a.W * a.C * es;
    const int out_img = a.Ho * a.Wo * a.K * es, out_row = a.Wo * a.K * es;

    // ---- tile walk: tiles L, L + G, ... as (image, tile row, tile column), advanced by
    // mixed-radix addition ----------------------------------------------------------------
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
    const Pos step = split(G);
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

    // ---- direct-load plan (tile invariant) ----------------------------------------------
    // LDS slot s holds chunk position s % NCH of window pixel p = s / NCH, i.e. input chunk
    // q = (s % NCH) ^ ((p / (16 / NCH)) % NCH).  dl_off: byte offset of the source from the
    // window origin (kOob for pixels past the window and chunks past C); dl_pos: the
    // pixel's window row and column.
    uint32_t dl_off[R];
    int dl_pos[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int s = r * NT + tid;
        const int p = s / NCH, wr = p / IW, wc = p % IW;
        const int q = (s % NCH) ^ ((p / (16 / NCH)) & (NCH - 1));
        const bool real = p < NP && q * 8 < a.C;
        dl_off[r] = real ? (uint32_t)((wr * a.W + wc) * a.C + q * 8) * (uint32_t)es : mm::kOob;
        dl_pos[r] = real ? (wr << 16) | wc : 0;
    }
    // always R loads per lane (a tile past the end loads nothing), so waits are exact
    auto issue_tile = [&](const Pos& t, auto buf) __attribute__((always_inline)) {
        u32x4* dst = decltype(buf)::value == 0 ? X0 : X1;
        const bool live = t.n < a.N;
        const bool inside = live && t.ih0 >= 0 && t.iw0 >= 0 && t.ih0 + IH <= a.H &&
                            t.iw0 + IW <= a.W;
        if (inside) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t off = dl_off[r];
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

    Pos cur = split(L);
    issue_tile(cur, std::integral_constant<int, 0>{});

    // ---- per-wave constants (requested after the first window) --------------------------
    // expansion A operand of block j, reduction step kc, lane (l%16, l/16): row = expanded
    // channel 16 cb + l%16, reduction index 8(l/16) + e = input channel 32 kc + 8(l/16) + e
    // (16 contiguous bytes of the [K1][C] filters; zero past C or K1)
    u32x4 apw[BPW][NKC];
    // depthwise A operand of block j and tap pair tp: row = channel 16 cb + l%16, reduction
    // index 8(l/16) + e = (tap pair_tap(tp, (l/16)/2), channel 8((l/16)&1) + e); non-zero
    // only where that channel is the row's: one 16-bit element per lane
    auto pair_tap = [](int tp, int hh) { return tp < 3 ? 3 * tp + hh : tp == 3 ? 3 * hh + 2 : 8 + hh; };
    const bool dw_active = (lr >> 3) == (lg & 1);
    uint16_t wdr[BPW][5];
    float s1r[BPW][4], b1r[BPW][4], s2r[BPW][4], b2r[BPW][4];
    // projection A operand of output block kb, reduction step kc: row = output channel
    // 16 kb + l%16, reduction index 8(l/16) + e = expanded channel 32 kc + 8(l/16) + e
    // (16 contiguous bytes of the [K][K1] filters; zero past K or K1)
    u32x4 apj[KB][NK3];
    float s3r[KB][4], b3r[KB][4];
    const float* dflt = (const float*)a.w1;  // any readable address for masked loads
    const float* s1p = a.s1 ? a.s1 : dflt;
    const float* b1p = a.b1 ? a.b1 : dflt;
    const float* s2p = a.s2 ? a.s2 : dflt;
    const float* b2p = a.b2 ? a.b2 : dflt;
    const float* s3p = a.s3 ? a.s3 : dflt;
    const float* b3p = a.b3 ? a.b3 : dflt;
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
        const int c = (cb0 + j) * 16 + lr;
        const int cc = c < a.K1 ? c : 0;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            const int ci = 32 * kc + 8 * lg;
            const int cic = ci < a.C ? ci : 0;
            apw[j][kc] = *reinterpret_cast<const u32x4*>(wpw + (int64_t)cc * a.C + cic);
        }
#pragma unroll
        for (int tp = 0; tp < 5; ++tp) {
            const int t = pair_tap(tp, lg >> 1);
            wdr[j][tp] = __builtin_bit_cast(uint16_t, wdw[(t < 9 ? t : 0) * a.K1 + cc]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = (cb0 + j) * 16 + 4 * lg + i, kk = k < a.K1 ? k : 0;
            s1r[j][i] = s1p[kk];
            b1r[j][i] = b1p[kk];
            s2r[j][i] = s2p[kk];
            b2r[j][i] = b2p[kk];
        }
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int k = kb * 16 + lr;
        const int kk = k < a.K ? k : 0;
#pragma unroll
        for (int kc = 0; kc < NK3; ++kc) {
            const int c = 32 * kc + 8 * lg;
            const int ccl = c < a.K1 ? c : 0;
            apj[kb][kc] = *reinterpret_cast<const u32x4*>(wpj + (int64_t)kk * a.K1 + ccl);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ko = kb * 16 + 4 * lg + i, kq = ko < a.K ? ko : 0;
            s3r[kb][i] = s3p[kq];
            b3r[kb][i] = b3p[kq];
        }
    }
    mm::wait_vmcnt<0>();  // first window and constants
    u32x4 adw[BPW][5];
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
        const int c = (cb0 + j) * 16 + lr;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            const bool ok = c < a.K1 && 32 * kc + 8 * lg < a.C;
            if (!ok) apw[j][kc] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int tp = 0; tp < 5; ++tp) {
            const int t = pair_tap(tp, lg >> 1);
            const bool ok = dw_active && t < 9 && c < a.K1;
            const uint32_t v = ok ? (uint32_t)wdr[j][tp] : 0u;
            const uint32_t h = (lr & 1) ? (v << 16) : v;
            const int w = (lr & 7) >> 1;
            adw[j][tp] = u32x4{w == 0 ? h : 0u, w == 1 ? h : 0u, w == 2 ? h : 0u, w == 3 ? h : 0u};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // channels past K1 leave the depthwise layer as exact zeros (epilogue of 0
            // with scale 1, bias 0), which the projection's zero operands then ignore
            const bool ok = (cb0 + j) * 16 + 4 * lg + i < a.K1;
            s1r[j][i] = (a.s1 && ok) ? s1r[j][i] : 1.0f;
            b1r[j][i] = (a.b1 && ok) ? b1r[j][i] : 0.0f;
            s2r[j][i] = (a.s2 && ok) ? s2r[j][i] : 1.0f;
            b2r[j][i] = (a.b2 && ok) ? b2r[j][i] : 0.0f;
        }
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int kc = 0; kc < NK3; ++kc) {
            const bool ok = kb * 16 + lr < a.K && 32 * kc + 8 * lg < a.K1;
            if (!ok) apj[kb][kc] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = kb * 16 + 4 * lg + i < a.K;
            s3r[kb][i] = (a.s3 && ok) ? s3r[kb][i] : 1.0f;
            b3r[kb][i] = (a.b3 && ok) ? b3r[kb][i] : 0.0f;
        }
    }

    // ---- per-lane offsets (tile invariant) ------------------------------------------------
    // expansion X operand of window block pb, step kc: pixel 16 pb + l%16, chunk
    // 4 kc + l/16 (the swizzle term does not depend on pb)
    uint32_t xo[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
        const int q = 4 * kc + lg;
        xo[kc] = (uint32_t)(lr * NCH + (q ^ ((lr / (16 / NCH)) & (NCH - 1)))) * 16u;
    }
    // intermediate write of window block pb: pixel p = 16 pb + l%16 at (row, column)
    // (p / IW, p % IW) -- pixels past the window go to the spare row IH -- channels
    // 4(l/16) .. + 3 of the block = chunk (l/16)/2, bytes 8((l/16)&1) .. + 7;
    // wpos: the pixel's window row and column (row IH for the spare pixels)
    uint32_t two[NPB];
    int wpos[NPB];
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb) {
        const int p = 16 * pb + lr;
        const int wr = p < NP ? p / IW : IH, wc = p < NP ? p % IW : (p - NP);
        two[pb] = (uint32_t)(wr * TROW + ((lg >> 1) * IW + wc) * 16 + (lg & 1) * 8);
        wpos[pb] = (wr << 16) | wc;
    }
    // depthwise B operand reads: lane (l%16, l/16) reads chunk (l/16)&1 of column
    // l%16 * S + dw; the (dh,0)+(dh,1) pairs take dw = (l/16)/2 from one input row, the
    // dw = 2 pairs take column + 2 from two consecutive rows ((l/16)/2 rows down)
    const int hh = lg >> 1, ch = lg & 1;
    const uint32_t rd_p = (uint32_t)((ch * IW + lr * S + hh) * 16);
    const uint32_t rd_q = (uint32_t)(hh * TROW + (ch * IW + lr * S + 2) * 16);
    const uint32_t rd_qc = (uint32_t)((ch * IW + lr * S + 2) * 16);
    // depthwise tile: the lane's output pixel (row r, column l%16) and channels
    // 16 cb + 4(l/16) .. + 3 (written), or 32 kc + 8(l/16) .. + 7 (read by the projection)
    const uint32_t dw_lane = (uint32_t)(lr * DSTR + 4 * lg * 2);
    const uint32_t dr_lane = (uint32_t)(lr * DSTR + 8 * lg * 2);
    // shortcut: the input pixel under output pixel (r, l%16) is window pixel
    // (r + pad_h, l%16 + pad_w) (stride 1); channels 16 kb + 4(l/16) .. + 3 are chunk
    // 2 kb + (l/16)/2, bytes 8((l/16)&1) .. + 7
    auto res_off = [&](int r, int kb) {
        const int p = (r + a.pad_h) * IW + lr + a.pad_w;
        const int q = 2 * kb + (lg >> 1);
        return (uint32_t)((p * NCH + (q ^ ((p / (16 / NCH)) & (NCH - 1)))) * 16 + (lg & 1) * 8);
    };

    auto q_used = [](int ir) {
        return (ir % S == 0 && ir / S < TH) || (ir >= 2 && (ir - 2) % S == 0 && (ir - 2) / S < TH);
    };

    // one step: expansion over the window of tile t (buffer src) into the wave's
    // intermediate tiles, depthwise over them into the shared depthwise tile, barrier,
    // projection, epilogue 3 and the shortcut, stores
    auto compute = [&](const u32x4* src, const Pos& t) __attribute__((always_inline)) {
        uint32_t valid = 0;
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb) {
            const int ih = t.ih0 + (wpos[pb] >> 16), iw = t.iw0 + (wpos[pb] & 0xffff);
            const bool ok = (wpos[pb] >> 16) < IH && (unsigned)ih < (unsigned)a.H &&
                            (unsigned)iw < (unsigned)a.W;
            valid |= ok ? (1u << pb) : 0u;
        }
        const char* xb = reinterpret_cast<const char*>(src);
        // reads run ahead of their products (window block pb + PDX, input row ir + PDR);
        // scheduling barriers keep the compiler from sinking a read next to its use
        constexpr int PDX = NPB < 2 ? NPB : 2;
        constexpr int PDR = IHW < 2 ? IHW : 2;
        u32x4 bx[NPB][NKC];
        auto read_x = [&](int pb) __attribute__((always_inline)) {
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
                bx[pb][kc] = *reinterpret_cast<const u32x4*>(xb + pb * 16 * NCH * 16 + xo[kc]);
        };
        // expansion over the window
#pragma unroll
        for (int pb = 0; pb < PDX; ++pb) read_x(pb);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb) {
            if (pb + PDX < NPB) read_x(pb + PDX);
            const bool ok = (valid >> pb) & 1u;
            const float lo = ok ? act1.lo : 0.0f, hi = ok ? act1.hi : 0.0f;
#pragma unroll
            for (int j = 0; j < BPW; ++j) {
                f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc) acc = mfma<T>(apw[j][kc], bx[pb][kc], acc);
                float o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    o[i] = __builtin_amdgcn_fmed3f(__builtin_fmaf(acc[i], s1r[j][i], b1r[j][i]),
                                                   lo, hi);
                st8(tbase + j * TREG + two[pb], pack8<T>(o));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // depthwise layer, block by block, into the shared depthwise tile
        u32x4 bp[BPW][IHW], bq[BPW][IHW];
        auto read_row = [&](int j, int ir) __attribute__((always_inline)) {
            const char* tb = tbase + j * TREG;
            bp[j][ir] = *reinterpret_cast<const u32x4*>(tb + ir * TROW + rd_p);
            if (q_used(ir))
                bq[j][ir] = *reinterpret_cast<const u32x4*>(tb + ir * TROW +
                                                            (ir + 1 < IHW ? rd_q : rd_qc));
        };
#pragma unroll
        for (int ir = 0; ir < PDR; ++ir) read_row(0, ir);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < BPW; ++j) {
            f32x4 d[TH];
#pragma unroll
            for (int r = 0; r < TH; ++r) d[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ir = 0; ir < IHW; ++ir) {
                if (ir + PDR < IHW) read_row(j, ir + PDR);
                else if (j + 1 < BPW) read_row(j + 1, ir + PDR - IHW);
#pragma unroll
                for (int dh = 0; dh < 3; ++dh)
                    if (ir >= dh && (ir - dh) % S == 0 && (ir - dh) / S < TH)
                        d[(ir - dh) / S] = mfma<T>(adw[j][dh], bp[j][ir], d[(ir - dh) / S]);
                if (ir % S == 0 && ir / S < TH)
                    d[ir / S] = mfma<T>(adw[j][3], bq[j][ir], d[ir / S]);
                if (ir >= 2 && (ir - 2) % S == 0 && (ir - 2) / S < TH)
                    d[(ir - 2) / S] = mfma<T>(adw[j][4], bq[j][ir], d[(ir - 2) / S]);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int r = 0; r < TH; ++r) {
                float o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = epilogue(d[r][i], s2r[j][i], b2r[j][i], act2);
                st8(dbase + r * 16 * DSTR + dw_lane + (cb0 + j) * 16 * 2, pack8<T>(o));
            }
        }
        // every wave's depthwise outputs are in the shared tile (the empty statements keep
        // the compiler from moving LDS accesses across the barrier, which it does not
        // treat as a memory operation)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        // projection: unit u = wave + NW i is (row u / KB, output block u % KB); units past
        // the tile store to the out-of-range offset.  Store offsets as in the PW->DW kernel:
        // a per-lane part plus a wave-uniform row part, either one out of range drops it.
        constexpr uint32_t kLaneOob = 0x40000000u, kRowOob = 0x80000000u;
        const bool col_ok = t.ow0 + lr < a.Wo;
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int u = wave + NW * i;
            const bool real = u < TH * KB;
            const int r = real ? u / KB : 0, kb = real ? u % KB : 0;
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
            u32x4 bd[NK3];
#pragma unroll
            for (int kc = 0; kc < NK3; ++kc)
                bd[kc] = *reinterpret_cast<const u32x4*>(dbase + r * 16 * DSTR + dr_lane +
                                                         kc * 64);
            // the unit's operands and constants, selected from the resident ones (kb is
            // uniform across the wave)
#pragma unroll
            for (int kc = 0; kc < NK3; ++kc) {
                u32x4 av = apj[0][kc];
#pragma unroll
                for (int kq = 1; kq < KB; ++kq) av = kq == kb ? apj[kq][kc] : av;
                acc = mfma<T>(av, bd[kc], acc);
            }
            float o[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float s3 = s3r[0][q], b3 = b3r[0][q];
#pragma unroll
                for (int kq = 1; kq < KB; ++kq) {
                    s3 = kq == kb ? s3r[kq][q] : s3;
                    b3 = kq == kb ? b3r[kq][q] : b3;
                }
                o[q] = epilogue(acc[q], s3, b3, act3);
            }
            if (a.residual) {
                const uint2 rv = *reinterpret_cast<const uint2*>(
                    reinterpret_cast<const char*>(src) + res_off(r, kb));
                const vec_t<T, 4> xv = __builtin_bit_cast(vec_t<T, 4>, rv);
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] += (float)xv[q];
            }
            const uint32_t lane_off = (col_ok && kb * 16 + 4 * lg < a.K)
                                          ? (uint32_t)(lr * a.K + kb * 16 + 4 * lg) * (uint32_t)es
                                          : kLaneOob;
            const uint32_t row = (real && t.oh0 + r < a.Ho) ? (uint32_t)(t.out_base + r * out_row)
                                                            : kRowOob;
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, pack8<T>(o)), ry,
                                                  lane_off + row, 0, 0);
        }
    };

    // ---- tile loop ------------------------------------------------------------------------
    // Step i (buffer P = i % 2): wait for tile i's window (the memory operations issued
    // after its loads are the NST stores of step i-1); barrier (every wave's share of the
    // window has landed, every wave is done with step i-1: buffer 1-P and the depthwise
    // tile are free); request tile i+1 into buffer 1-P; compute tile i from buffer P.
    auto step_fn = [&](auto par, bool first) __attribute__((always_inline)) {
        constexpr int P = decltype(par)::value;
        if (!first) mm::wait_vmcnt<NST>();
        __builtin_amdgcn_s_barrier();
        const Pos nxt = advance(cur);
        issue_tile(nxt, std::integral_constant<int, 1 - P>{});
        compute(P == 0 ? X0 : X1, cur);
        cur = nxt;
    };
    bool first = true;
    while (cur.n < a.N) {
        step_fn(std::integral_constant<int, 0>{}, first);
        first = false;
        if (cur.n >= a.N) break;
        step_fn(std::integral_constant<int, 1>{}, false);
    }
    // loads of the tile past the end may still be in flight into LDS
    mm::wait_vmcnt<0>();
}

template <typename T, int S, int TH, int CMAX, int NW, int BPW, int KB, int OCC>
int launch_pwdwpw_mm(const KArgs& a, int grid, void* stream) {
    (void)hipGetLastError();
    hipLaunchKernelGGL((pwdwpw_mm_kernel<T, S, TH, CMAX, NW, BPW, KB, OCC>), dim3(grid),
                       dim3(64 * NW), 0, (hipStream_t)stream, a);
    return (int)hipGetLastError();
}
template <typename T, int S, int TH, int CMAX, int NW, int BPW, int KB, int OCC>
int occ_pwdwpw_mm() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, pwdwpw_mm_kernel<T, S, TH, CMAX, NW, BPW, KB, OCC>, 64 * NW, 0) != hipSuccess)
        return 0;
    return n;
}

#define FCM_V_DWPW(...)
#define FCM_V_DWPW32(...)
#define FCM_V_B2B(...)
#define FCM_V_B2B_MM(...)
#define FCM_V_DWPW_MM(...)
#define FCM_V_DWPW_MMW(...)
#define FCM_V_PWDWPW_MM(name, dt, CT, S, TH, CMAX, NW, BPW, KB, OCC)                     \
    template int launch_pwdwpw_mm<CT, S, TH, CMAX, NW, BPW, KB, OCC>(const KArgs&, int,   \
                                                                     void*);              \
    template int occ_pwdwpw_mm<CT, S, TH, CMAX, NW, BPW, KB, OCC>();
#include "../variants.def"
#undef FCM_V_DWPW
#undef FCM_V_DWPW32
#undef FCM_V_B2B
#undef FCM_V_DWPW_MM
#undef FCM_V_B2B_MM
#undef FCM_V_DWPW_MMW
#undef FCM_V_PWDWPW_MM

}  // namespace fcm
