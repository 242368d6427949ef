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
// Work split of a 4x16-pixel tile over the NW = 4 or 8 waves of a workgroup; wave w
// works on channel group g = w % 4 and on rows RW * (w / 4) .. + RW - 1 (RW = 16 / NW):
//   phase A  wave w computes the depthwise layer of channel blocks g, g + 4, ... of
//            its rows.  The result lands in the matrix unit's output layout -- lane
//            (l%16, l/16) holds channels 16*cb + 4*(l/16) + [0,4) of pixel l%16 -- and
//            two channel blocks give a lane 8 channels of its pixel: exactly the B
//            operand of the pointwise product when its reduction index is permuted the
//            same way.  After epilogue 1 and rounding to the storage type, each lane
//            writes its 8 bytes to the LDS intermediate tile (contiguous 1 KB operand
//            blocks, no bank conflicts).
//   phase B  wave w computes output channels [KT/4*g, KT/4*(g+1)) of its rows,
//            reading the intermediate back as ready-made B operands.  Its pointwise
//            weights (the A operands) and epilogue-2 constants stay in registers for
//            the whole kernel.
// Eight waves pay off where the tile buffers leave room for one workgroup per CU (128
// channels): two waves per SIMD instead of one.
// The intermediate thus lives only in LDS (the commBuffer of the page's design) and
// never reaches HBM.
//
// The two phases are software-pipelined over a workgroup's tiles with one barrier per
// step: step i runs phase A of tile i+1 and phase B of tile i (two input tile buffers,
// two intermediate buffers), so the matrix products of one phase interleave with the
// vector epilogue of the other, and tile i+2's input is requested at the start of the
// step and has a whole step to arrive.
//
// Input tiles arrive by direct global->LDS loads (buffer_load_dwordx4 ... lds).
// Out-of-image pixels (the zero padding) come back as zeros from the buffer resource's
// range check.  Each pixel's 16-byte channel chunks are XOR-swizzled so the 16 lanes of
// an operand read (16 consecutive pixels, same chunk) hit distinct LDS banks.  Outputs
// are written with buffer stores whose out-of-range lanes are dropped by the same range
// check, so every wave issues the same number of memory instructions per step and the
// wait for the next tile's input can count them exactly (gfx9 vector memory operations
// complete in issue order).  Per-lane offsets are fixed for the whole kernel; the
// tile's position enters as a scalar offset, so interior tiles need no per-lane
// address arithmetic at all.
//
// Depth multiplier M = 2 (the depthwise layer of the PyTorch forum's "Using optimised
// depthwise convolutions", two outputs per input channel: output channel j reads input
// channel j / 2).  CC then counts intermediate channels, the window holds CC / 2 input
// channels, and the 16 intermediate channels of a block read 8 input channels, one
// 16-byte piece per pixel.  A product then takes one input row's three taps in its four
// 8-channel reduction slots (slot l/16 = tap column, the fourth slot zero-weighted):
// A[row i][(slot s, channel e)] = w[3 dh + s][16 cb + i] where e == i / 2, else 0.  Each
// input row is read once per channel block and serves the (up to three) output rows
// below it, three products per 16 channels x 16 pixels instead of five.
//
// Filter size FS = 5 (M = 1; the forum page's depthwise layer with a 5x5 kernel): the
// taps pair within a filter row, (dh,0)+(dh,1) and (dh,2)+(dh,3), and down the last
// column, (0,4)+(1,4), (2,4)+(3,4), (4,4) alone: 13 products per 16 channels x 16 pixels.
// The depthwise operands stay in registers in compact form (one 32-bit word each) and
// are expanded where used, and phase A runs block by block, so that only one block's
// operand reads are held at a time.
#include <type_traits>

#include "mm_common.h"

namespace fcm {

// f(std::integral_constant<int, I>) for I = B .. E - 1: loop indices that are constants
// (the scheduling-group builtin takes constant instruction counts)
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

template <typename T, int S, int TH, int TW, int KT, int CC, int NW, int OCC, int M, int FS>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(OCC, 8)))
void dwpw_mm_kernel(KArgs a) {
    constexpr int NT = 64 * NW;
    static_assert(M == 1 || M == 2, "depth multiplier 1 or 2");
    static_assert(FS == 3 || (FS == 5 && M == 1), "3x3 filters, or 5x5 with multiplier 1");
    static_assert(TH == 4 && TW == 16, "4 rows of 16 pixels per tile");
    static_assert(NW == 4 || NW == 8, "4 or 8 waves");
    // wave w works on channel / output group w % 4 and rows RW * (w / 4) .. + RW - 1
    constexpr int RW = TH * 4 / NW;
    constexpr int IH = (TH - 1) * S + FS, IW = (TW - 1) * S + FS, NPIX = IH * IW;
    constexpr int CH = CC / (8 * M);  // 16-byte chunks per pixel (CC / M input channels)
    static_assert(CH == 4 || CH == 8 || CH == 16, "swizzle needs 4, 8 or 16 chunks per pixel");
    constexpr int SLOTS = NPIX * CH;
    constexpr int R = (SLOTS + NT - 1) / NT;  // direct-load rounds per tile
    constexpr int SLOTS_P = R * NT;
    // depthwise operands per channel block: NPR tap pairs per filter row, NQP pairs down
    // the last column (M = 1); one per filter row (M = 2)
    constexpr int NPR = FS / 2, NQP = (FS + 1) / 2;
    constexpr int NCB = CC / 16, NKS = CC / 32, NTP = M == 1 ? FS * NPR + NQP : 3;
    constexpr int CBW = NCB / 4;  // depthwise channel blocks per wave
    // 5x5 phase A: wave w owns channel blocks w, w + NW, ... for all TH rows (fewer
    // filter operands per wave than CBW blocks over RW rows)
    constexpr int CBD = FS == 5 ? NCB / NW : CBW;
    static_assert(FS == 3 || NCB % NW == 0, "5x5: whole channel blocks per wave");
    static_assert(NCB % 4 == 0, "each wave owns whole channel blocks");
    constexpr int KW = KT / 4;    // pointwise output channels per wave
    constexpr int KBW = KW / 16;  // 16-channel output blocks per wave
    static_assert(KT % 128 == 0, "each wave stores 16-byte runs of 8 output channels");
    constexpr int NST = RW * (KBW / 2);  // buffer stores per lane per step
    static_assert(NST < 64, "vmcnt range");
    constexpr uint32_t IROW_BYTES = (uint32_t)IW * CH * 16;  // one input row down
    constexpr uint32_t ROW_BYTES = S * IROW_BYTES;             // one output row down
    constexpr int IHW = (RW - 1) * S + FS;  // input rows under a wave's RW output rows

    // separate arrays per buffer: the compiler then sees that reading one buffer does
    // not depend on the direct loads still in flight into the other
    __shared__ __attribute__((aligned(16))) u32x4 xs0[SLOTS_P];
    __shared__ __attribute__((aligned(16))) u32x4 xs1[SLOTS_P];
    __shared__ __attribute__((aligned(16))) u32x4 tl0[TH * NKS * 64];
    __shared__ __attribute__((aligned(16))) u32x4 tl1[TH * NKS * 64];
    // the lambdas below see the buffers through these pointers
    u32x4* const X0 = xs0;
    u32x4* const X1 = xs1;
    u32x4* const T0 = tl0;
    u32x4* const T1 = tl1;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int og = wave & 3, row0 = RW * (wave >> 2);
    // the depthwise channel block j of this wave
    auto blk = [&](int j) { return FS == 5 ? wave + NW * j : og + 4 * j; };
    const int lr = lane & 15, lg = lane >> 4;
    const Act act1 = act_bounds(a.act1), act2 = act_bounds(a.act2);
    const int G = gridDim.x;
    const int L = xcd_logical_id(blockIdx.x, G);
    const int k0 = (L % a.num_ktiles) * KT;
    const int kw0 = k0 + og * KW;  // this wave's output channels
    const T* __restrict__ wdw = (const T*)a.w1;
    const T* __restrict__ wpw = (const T*)a.w2;
    // one buffer resource per tensor (the host guarantees whole tensors below 2 GiB)
    const int es = (int)sizeof(T);
    const __amdgpu_buffer_rsrc_t rx = mm::rsrc(a.x, (uint32_t)(a.N * a.H * a.W * a.C * es));
    const __amdgpu_buffer_rsrc_t ry = mm::rsrc(a.y, (uint32_t)(a.N * a.Ho * a.Wo * a.K * es));
    const int in_img = a.H * a.W * a.C * es, in_row = a.W * a.C * es;
    const int out_img = a.Ho * a.Wo * a.K * es, out_row = a.Wo * a.K * es;

    // ---- tile walk: tiles pt0, pt0 + pstep, ... as (image, tile row, tile column),
    // advanced by mixed-radix addition (no division inside the loop) -----------------
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

    // ---- direct-load plan (tile invariant) ---------------------------------------------
    // LDS slot s holds chunk q of window pixel p = s / CH with s % CH = q ^ key(column),
    // key = column & (CH - 1): the 16 lanes of an operand read (consecutive columns, same
    // chunk) then fall in distinct bank groups (a pixel is CH 16-byte chunks, so without
    // the swizzle they would all share one), and moving down a row moves every slot by a
    // constant.  With 4 chunks per pixel two neighbouring pixels fill one 128-byte bank
    // line, so the key is (column / 2) & 3: 8 consecutive columns then take 8 distinct
    // 16-byte bank groups.
    // dl_off: byte offset of the slot's source relative to the window origin (kOob for
    // padding slots); dl_pos: the slot's window row and column.
    auto swz = [](int col) { return CH >= 8 ? col & (CH - 1) : (col >> 1) & (CH - 1); };
    uint32_t dl_off[R];
    int dl_pos[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int s = r * NT + tid;
        const int p = s / CH, ihl = p / IW, iwl = p % IW;
        const int q = (s % CH) ^ swz(iwl);
        const bool real = s < SLOTS && q * 8 < a.C;
        dl_off[r] = real ? (uint32_t)((ihl * a.W + iwl) * a.C + q * 8) * (uint32_t)sizeof(T)
                         : mm::kOob;
        dl_pos[r] = real ? (ihl << 16) | iwl : 0;
    }
    // The loads of one tile, always R per lane (a tile past the end loads nothing: every
    // lane gets the out-of-range offset), so the wait counts below are exact.  A window
    // inside the image needs no per-lane test: the window origin is a scalar offset.
    auto issue_tile = [&](const Pos& t, auto buf) {
        u32x4* dst = decltype(buf)::value == 0 ? X0 : X1;
        const bool live = t.n < a.N;
        const bool inside = live && t.ih0 >= 0 && t.iw0 >= 0 && t.ih0 + IH <= a.H &&
                            t.iw0 + IW <= a.W;
        if (inside) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                // (a copy: an element of the captured array passed straight to the
                // builtin makes the host pass drop the kernel's launch stub)
                const uint32_t off = dl_off[r];
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rx, (__attribute__((address_space(3))) void*)(dst + r * NT + wave * 64), 16,
                    off, t.in_base, 0, 0);
            }
        } else {
            // border tile (or past the end): test every lane's pixel
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

    // ---- per-wave constants ----------------------------------------------------------
    // The first tile's input is requested first (it comes from HBM, the constants from
    // L2), then all constants, unconditionally (clamped addresses, absent epilogue
    // arrays read from another valid tensor), then the second tile's input, and only
    // then are the loaded values used: the wait for the constants does not also wait
    // for the second tile (vector-memory operations complete in issue order).
    Pos cur = split(L / a.num_ktiles);
    Pos nxt = advance(cur);
    issue_tile(cur, std::integral_constant<int, 0>{});
    //
    // depthwise: this wave owns channel blocks cb = og + 4j.  The nine taps (dh, dw),
    // numbered 3 dh + dw, are paired as (dh,0)+(dh,1) for dh = 0, 1, 2, then
    // (0,2)+(1,2), then (2,2) with an empty tenth tap (zero weights): with this pairing
    // the matrix operand of every pair depends on one input row only (the dw = 2
    // pairs on two consecutive rows), so one LDS read serves all the output rows that
    // use it.  Matrix operand of block cb and pair tp, lane (l%16, l/16): row = channel
    // 16cb + l%16, reduction index 8(l/16) + e = (tap pair_tap(tp, (l/16)/2), channel
    // 16cb + 8((l/16)&1) + e); non-zero only where that channel is the row's, i.e. one
    // 16-bit element per lane.
    // M = 2: operand tp = dh, lane (l%16, l/16): row = intermediate channel 16cb + l%16,
    // reduction index 8(l/16) + e = (tap (dh, l/16), input channel 8cb + e) for l/16 < 3
    // (the fourth slot has zero weights); non-zero only at e = (l%16)/2, the row's input
    // channel.
    // (general FS: operand tp < FS * NPR pairs the taps (tp / NPR, 2 (tp % NPR) + hh), the
    // others the taps (2 (tp - FS * NPR) + hh, FS - 1); FS * FS marks an absent tap)
    auto pair_tap = [](int tp, int hh) {
        if (tp < FS * NPR) return (tp / NPR) * FS + 2 * (tp % NPR) + hh;
        const int dh = 2 * (tp - FS * NPR) + hh;
        return dh < FS ? dh * FS + FS - 1 : FS * FS;
    };
    auto lane_tap = [&](int tp) { return M == 1 ? pair_tap(tp, lg >> 1) : lg < 3 ? 3 * tp + lg : 0; };
    const bool dw_active = M == 1 ? (lr >> 3) == (lg & 1) : lg < 3;
    const int dw_e = M == 1 ? lr & 7 : lr >> 1;
    const int C1 = a.C * M;  // intermediate channels
    const float* s1p = a.s1 ? a.s1 : (const float*)a.w2;
    const float* b1p = a.b1 ? a.b1 : (const float*)a.w2;
    const float* s2p = a.s2 ? a.s2 : (const float*)a.w2;
    const float* b2p = a.b2 ? a.b2 : (const float*)a.w2;
    uint16_t wdr[CBD][NTP];
    float s1l[CBD][4], b1l[CBD][4];
#pragma unroll
    for (int j = 0; j < CBD; ++j) {
        const int cb = blk(j);
#pragma unroll
        for (int tp = 0; tp < NTP; ++tp) {
            const int t = lane_tap(tp), c = cb * 16 + lr;
            wdr[j][tp] = __builtin_bit_cast(uint16_t,
                                            wdw[(t < FS * FS ? t : 0) * C1 + (c < C1 ? c : 0)]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = cb * 16 + lg * 4 + i, cc = c < C1 ? c : 0;
            s1l[j][i] = s1p[cc];
            b1l[j][i] = b1p[cc];
        }
    }
    // pointwise A operand of this wave's 32-channel slice for reduction step ks, block
    // kb: block (kw0/32, ks, kb) of the blocked copy after the plain [K][C] array (one
    // contiguous kilobyte; row kperm<32>(kb, l%16) of the slice, reduction channels
    // 32ks + 8(l/16) + [0,8), the order the depthwise result is stored in).  Blocks past
    // K or C are clamped to existing ones: their rows are never stored, and the
    // intermediate channels they would multiply are zero.
    static_assert(KW == 32, "one 32-channel block group per wave");
    const u32x4* __restrict__ wpb = reinterpret_cast<const u32x4*>(wpw + (int64_t)a.K * C1);
    u32x4 wa[NKS][KBW];
    {
        const int g = min(kw0 >> 5, (a.K + 31) / 32 - 1), s32 = (C1 + 31) / 32;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int kb = 0; kb < KBW; ++kb)
                wa[ks][kb] = wpb[((g * s32 + min(ks, s32 - 1)) * 2 + kb) * 64 + lane];
    }
    // epilogue-2 constants of the lane's output channels kw0 + (KW/4)(l/16) + [0,KW/4)
    float s2r[KW / 4], b2r[KW / 4];
#pragma unroll
    for (int i = 0; i < KW / 4; ++i) {
        const int k = kw0 + lg * (KW / 4) + i, kk = k < a.K ? k : 0;
        s2r[i] = s2p[kk];
        b2r[i] = b2p[kk];
    }

    // the second tile's input
    issue_tile(nxt, std::integral_constant<int, 1>{});

    // now the loaded values are used
    uint32_t wdc[CBD][NTP];
    float s1r[CBD][4], b1r[CBD][4];
#pragma unroll
    for (int j = 0; j < CBD; ++j) {
        const int cb = blk(j);
#pragma unroll
        for (int tp = 0; tp < NTP; ++tp) {
            const int t = lane_tap(tp), c = cb * 16 + lr;
            const bool ok = dw_active && t < FS * FS && c < C1;
            const uint32_t v = ok ? (uint32_t)wdr[j][tp] : 0u;
            wdc[j][tp] = (dw_e & 1) ? (v << 16) : v;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = cb * 16 + lg * 4 + i < C1;
            s1r[j][i] = (a.s1 && ok) ? s1l[j][i] : 1.0f;
            b1r[j][i] = (a.b1 && ok) ? b1l[j][i] : 0.0f;
        }
    }
    auto dw_operand = [&](uint32_t v) {
        const int w = dw_e >> 1;
        return u32x4{w == 0 ? v : 0u, w == 1 ? v : 0u, w == 2 ? v : 0u, w == 3 ? v : 0u};
    };
    // the expanded operands stay in registers for the whole kernel (3x3; the thirteen of
    // a 5x5 filter are expanded where used)
    u32x4 wdf[CBW][FS == 3 ? NTP : 1];
    if constexpr (FS == 3) {
#pragma unroll
        for (int j = 0; j < CBW; ++j)
#pragma unroll
            for (int tp = 0; tp < NTP; ++tp) wdf[j][tp] = dw_operand(wdc[j][tp]);
    }
#pragma unroll
    for (int i = 0; i < KW / 4; ++i) {
        const bool ok = kw0 + lg * (KW / 4) + i < a.K;
        s2r[i] = (a.s2 && ok) ? s2r[i] : 1.0f;
        b2r[i] = (a.b2 && ok) ? b2r[i] : 0.0f;
    }
    // LDS byte offsets of this lane's depthwise operand reads from input row 0 of the
    // tile, block cb = og + 4j (input row ir adds ir * IROW_BYTES): xo_p for the
    // (dh,0)+(dh,1) pairs (column lr*S + (l/16)/2), xo_q for the dw = 2 pairs (column
    // lr*S + 2, the upper lane half one row down), xo_qc the same without the row step
    // (for the window's last row, where only the (2,2) pair uses the read: the upper
    // half then meets zero weights and must only stay inside the tile).  M = 2: one
    // read per input row, xo_p at column lr*S + l/16 of chunk cb (the zero-weighted
    // fourth slot reads column lr*S).
    const int hh = lg >> 1;
    auto lds_off = [&](int j, int row, int col) {
        const int q = M == 1 ? 2 * blk(j) + (lg & 1) : blk(j);
        return (uint32_t)((row * IW + col) * CH + (q ^ swz(col))) * 16u;
    };
    // (FS = 5: xo_p5[j][i] for the (dh,2i)+(dh,2i+1) pairs, xo_q / xo_qc at column lr*S + 4)
    uint32_t xo_p[CBD], xo_q[CBD], xo_qc[CBD], xo_p5[CBD][NPR];
#pragma unroll
    for (int j = 0; j < CBD; ++j) {
        if constexpr (M == 1) {
            xo_p[j] = lds_off(j, 0, lr * S + hh);
            xo_q[j] = lds_off(j, hh, lr * S + FS - 1);
            xo_qc[j] = lds_off(j, 0, lr * S + FS - 1);
#pragma unroll
            for (int i = 0; i < NPR; ++i) xo_p5[j][i] = lds_off(j, 0, lr * S + 2 * i + hh);
        } else {
            xo_p[j] = lds_off(j, 0, lr * S + (lg < 3 ? lg : 0));
            xo_q[j] = xo_qc[j] = xo_p[j];
        }
    }
    // intermediate: depthwise rows 4(l/16)+i of channel block cb are channels
    // 16(cb%2) + 4(l/16) + i of slice cb/2, i.e. lane group 2(cb%2) + (l/16)/2, bytes
    // 8((l/16)%2)..+7 of its 16-byte operand (cb % 2 == og % 2 for every block)
    const uint32_t tls_w =
        (uint32_t)(((2 * (og & 1) + (lg >> 1)) * 16 + lr) * 16 + (lg & 1) * 8);
    // store offset of the lane's first output channel within a pixel row of the tile
    // (kOob when the channel does not exist); the pixel row enters as a scalar offset
    const int kl = kw0 + lg * (KW / 4);
    const uint32_t st_lane =
        kl < a.K ? (uint32_t)(lr * a.K + kl) * (uint32_t)sizeof(T) : mm::kOob;

    // Two forms of the tile loop, chosen once per launch: the general one, and one for
    // layers whose epilogue 1 is the identity (no scale, no bias, no activation) and
    // whose epilogue 2 has no scale (a CIFAR-style block: bias and activation after the
    // pointwise layer only).  The second skips epilogue 1 and starts the pointwise
    // accumulators at the bias, so that epilogue 2 is the activation alone (a quarter of
    // the vector instructions of a step fewer).  (Instantiating all four combinations made
    // the general form slower.)
    const bool id1 = !a.s1 && !a.b1 && a.act1 == 0;
    const bool bias_init2 = !a.s2;

    // phase A of one tile: depthwise on the matrix cores, this wave's channel blocks
    // for its RW rows; epilogue 1; 8 bytes per lane into the intermediate tile, where
    // they form half of a pointwise B operand
    // operand reads of one input row of the window: the (dh,0)+(dh,1) operand always,
    // the dw = 2 operand when a (0,2)+(1,2) or (2,2) product uses the row (M = 1; with
    // M = 2 the one read of a row holds all three of its taps)
    // (general FS: the last-column operand of a row when any pair (2jq, FS-1)+(2jq+1,
    // FS-1) of an output row starts on it)
    auto q_used = [](int ir) {
        bool u = false;
        for (int jq = 0; jq < NQP; ++jq)
            u = u || (ir >= 2 * jq && (ir - 2 * jq) % S == 0 && (ir - 2 * jq) / S < RW);
        return u;
    };
    constexpr int NQ = [] {
        int n = 0;
        for (int ir = 0; ir < IHW; ++ir) {
            bool u = false;
            for (int jq = 0; jq < NQP; ++jq)
                u = u || (ir >= 2 * jq && (ir - 2 * jq) % S == 0 && (ir - 2 * jq) / S < RW);
            n += u;
        }
        return n;
    }();
    // epilogue 1 of block j's TH rows and their intermediate writes (5x5 phase A; the
    // block's parity picks the lane group and half, as tls_w does for og)
    auto store_block = [&](int j, const f32x4* d, u32x4* dst, auto identity1) {
        const int cb = blk(j);
        const uint32_t tw =
            (uint32_t)(((2 * (cb & 1) + (lg >> 1)) * 16 + lr) * 16 + (lg & 1) * 8);
#pragma unroll
        for (int r = 0; r < TH; ++r) {
            float o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                o[i] = decltype(identity1)::value ? d[r][i]
                                                  : epilogue(d[r][i], s1r[j][i], b1r[j][i], act1);
            st8(reinterpret_cast<char*>(dst) + ((r * NKS + (cb >> 1)) * 64) * 16 + tw,
                pack8<T>(o));
        }
    };
    auto phase_a = [&](const u32x4* src, u32x4* dst, auto identity1) {
        const char* xb = reinterpret_cast<const char*>(src) + row0 * ROW_BYTES;
        if constexpr (FS == 5) {
            // block by block, software-pipelined by input row: row ir + 1's operand reads
            // are issued before row ir's products (the scheduling groups keep that order),
            // so that about two rows of reads are held at a time
            // (all TH output rows of the tile, IH input rows of the window)
            const char* xw = reinterpret_cast<const char*>(src);
            constexpr auto valid = [](int rr) { return rr >= 0 && rr % S == 0 && rr / S < TH; };
            constexpr auto n_reads = [](int ir) {
                bool q = false;
                for (int jq = 0; jq < NQP; ++jq)
                    q = q || (ir >= 2 * jq && (ir - 2 * jq) % S == 0 && (ir - 2 * jq) / S < TH);
                return NPR + (q ? 1 : 0);
            };
            constexpr auto n_products = [](int ir) {
                int n = 0;
                for (int dh = 0; dh < FS; ++dh)
                    n += (ir >= dh && (ir - dh) % S == 0 && (ir - dh) / S < TH) ? NPR : 0;
                for (int jq = 0; jq < NQP; ++jq)
                    n += (ir >= 2 * jq && (ir - 2 * jq) % S == 0 && (ir - 2 * jq) / S < TH) ? 1 : 0;
                return n;
            };
            static_for<0, CBD>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                u32x4 bp[IH][NPR], bq[IH];
                auto rd = [&](auto irc) {
                    constexpr int ir = decltype(irc)::value;
#pragma unroll
                    for (int i = 0; i < NPR; ++i)
                        bp[ir][i] =
                            *reinterpret_cast<const u32x4*>(xw + xo_p5[j][i] + ir * IROW_BYTES);
                    if constexpr (n_reads(ir) > NPR)
                        bq[ir] = *reinterpret_cast<const u32x4*>(
                            xw + (ir + 1 < IH ? xo_q[j] : xo_qc[j]) + ir * IROW_BYTES);
                };
                f32x4 d[TH];
#pragma unroll
                for (int r = 0; r < TH; ++r) d[r] = f32x4{0.f, 0.f, 0.f, 0.f};
                rd(std::integral_constant<int, 0>{});
                __builtin_amdgcn_sched_group_barrier(0x100, n_reads(0), 0);
                static_for<0, IH>([&](auto irc) {
                    constexpr int ir = decltype(irc)::value;
                    if constexpr (ir + 1 < IH) rd(std::integral_constant<int, ir + 1>{});
#pragma unroll
                    for (int dh = 0; dh < FS; ++dh)
                        if (valid(ir - dh))
#pragma unroll
                            for (int i = 0; i < NPR; ++i)
                                d[(ir - dh) / S] = mfma<T>(dw_operand(wdc[j][dh * NPR + i]),
                                                           bp[ir][i], d[(ir - dh) / S]);
#pragma unroll
                    for (int jq = 0; jq < NQP; ++jq)
                        if (valid(ir - 2 * jq))
                            d[(ir - 2 * jq) / S] = mfma<T>(dw_operand(wdc[j][FS * NPR + jq]),
                                                           bq[ir], d[(ir - 2 * jq) / S]);
                    if constexpr (ir + 1 < IH)
                        __builtin_amdgcn_sched_group_barrier(0x100, n_reads(ir + 1), 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, n_products(ir), 0);
                });
                store_block(j, d, dst, identity1);
            });
        } else {
        // every operand of the window is requested first, then the products run (the
        // scheduling groups below keep that order), so the LDS latency is paid once per
        // phase instead of once per product
        u32x4 bp[CBW][IHW], bq[CBW][IHW];
#pragma unroll
        for (int j = 0; j < CBW; ++j)
#pragma unroll
            for (int ir = 0; ir < IHW; ++ir) {
                bp[j][ir] = *reinterpret_cast<const u32x4*>(xb + xo_p[j] + ir * IROW_BYTES);
                if (M == 1 && q_used(ir))
                    bq[j][ir] = *reinterpret_cast<const u32x4*>(
                        xb + (ir + 1 < IHW ? xo_q[j] : xo_qc[j]) + ir * IROW_BYTES);
            }
#pragma unroll
        for (int j = 0; j < CBW; ++j) {
            const u32x4* wf = wdf[j];
            const int cb = og + 4 * j;
            // input rows outer: each operand applied to every output row that uses it
            // (RW independent accumulation chains); wf[dh] holds the taps (dh, 0) and
            // (dh, 1) (M = 1) or the whole filter row dh (M = 2)
            f32x4 d[RW];
#pragma unroll
            for (int r = 0; r < RW; ++r) d[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ir = 0; ir < IHW; ++ir) {
#pragma unroll
                for (int dh = 0; dh < 3; ++dh)
                    if (ir >= dh && (ir - dh) % S == 0 && (ir - dh) / S < RW)
                        d[(ir - dh) / S] = mfma<T>(wf[dh], bp[j][ir], d[(ir - dh) / S]);
                if constexpr (M == 1) {
                    if (ir % S == 0 && ir / S < RW)
                        d[ir / S] = mfma<T>(wf[3], bq[j][ir], d[ir / S]);
                    if (ir >= 2 && (ir - 2) % S == 0 && (ir - 2) / S < RW)
                        d[(ir - 2) / S] = mfma<T>(wf[4], bq[j][ir], d[(ir - 2) / S]);
                }
            }
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                float o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    o[i] = decltype(identity1)::value
                               ? d[r][i]
                               : epilogue(d[r][i], s1r[j][i], b1r[j][i], act1);
                st8(reinterpret_cast<char*>(dst) + (((row0 + r) * NKS + (cb >> 1)) * 64) * 16 +
                        tls_w,
                    pack8<T>(o));
            }
        }
        __builtin_amdgcn_sched_group_barrier(0x100, CBW * (IHW + (M == 1 ? NQ : 0)), 0);  // reads
        __builtin_amdgcn_sched_group_barrier(0x008, CBW * RW * NTP, 0);  // products
        }
    };
    // phase B of one tile: pointwise on the matrix cores, this wave's KW output
    // channels for its RW rows, epilogue 2, 16-byte stores; always NST stores per lane
    // (rows or lanes outside the output get the out-of-range offset)
    auto phase_b = [&](const u32x4* src, const Pos& t, auto from_bias) {
        constexpr bool FB = decltype(from_bias)::value;
        u32x4 bfr[RW][NKS];
#pragma unroll
        for (int mb = 0; mb < RW; ++mb)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                bfr[mb][ks] = src[((row0 + mb) * NKS + ks) * 64 + lane];
        // reduction step outermost, so that each accumulator is updated in place
        f32x4 acc[RW][KBW];
#pragma unroll
        for (int mb = 0; mb < RW; ++mb)
#pragma unroll
            for (int kb = 0; kb < KBW; ++kb)
                acc[mb][kb] = FB ? f32x4{b2r[kb * 4], b2r[kb * 4 + 1], b2r[kb * 4 + 2],
                                         b2r[kb * 4 + 3]}
                                 : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int mb = 0; mb < RW; ++mb)
#pragma unroll
                for (int kb = 0; kb < KBW; ++kb)
                    acc[mb][kb] = mfma<T>(wa[ks][kb], bfr[mb][ks], acc[mb][kb]);
        // all intermediate reads first, then the products
        __builtin_amdgcn_sched_group_barrier(0x100, RW * NKS, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, RW * NKS * KBW, 0);
        const uint32_t voff = t.ow0 + lr < a.Wo ? st_lane : mm::kOob;
#pragma unroll
        for (int mb = 0; mb < RW; ++mb) {
            const bool row_ok = t.oh0 + row0 + mb < a.Ho;
            const uint32_t v = row_ok ? voff : mm::kOob;
            const int srow = row_ok ? t.out_base + (row0 + mb) * out_row : 0;
#pragma unroll
            for (int kb = 0; kb < KBW; kb += 2) {
                float o[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if constexpr (FB) {
                        o[i] = __builtin_amdgcn_fmed3f(acc[mb][kb][i], act2.lo, act2.hi);
                        o[4 + i] = __builtin_amdgcn_fmed3f(acc[mb][kb + 1][i], act2.lo, act2.hi);
                    } else {
                        o[i] = epilogue(acc[mb][kb][i], s2r[kb * 4 + i], b2r[kb * 4 + i], act2);
                        o[4 + i] = epilogue(acc[mb][kb + 1][i], s2r[kb * 4 + 4 + i],
                                            b2r[kb * 4 + 4 + i], act2);
                    }
                }
                // the whole offset goes in the vector operand (scalar offset 0): with a
                // register scalar offset the compiler omits the wait state that a store
                // of more than 64 bits needs before its data registers are rewritten
                __builtin_amdgcn_raw_buffer_store_b128(
                    pack16<T>(o), ry,
                    v == mm::kOob ? mm::kOob : (uint32_t)srow + v + kb * 4 * (uint32_t)sizeof(T),
                    0, mm::kStoreStream);
            }
        }
    };

    // ---- software-pipelined tile loop -----------------------------------------------
    // Step i (buffers P = i % 2): wait for tile i+1's input; barrier (all of phase A of
    // tile i is in tls[P], nobody reads xs[P] or tls[1-P] any more); request tile i+2
    // into xs[P]; phase A of tile i+1 (xs[1-P] -> tls[1-P]); phase B of tile i (tls[P]).
    // Vector-memory operations issued after tile i+1's loads: none before step 0, the
    // NST stores of step i-1 before step i.
    mm::wait_vmcnt<R>();
    __builtin_amdgcn_s_barrier();
    auto run = [&](auto identity1, auto from_bias) {
        if (cur.n < a.N) phase_a(X0, T0, identity1);
        auto step_fn = [&](auto par, bool first) {
            constexpr int P = decltype(par)::value;
            if (first) mm::wait_vmcnt<0>(); else mm::wait_vmcnt<NST>();
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): own intermediate writes done
            __builtin_amdgcn_s_barrier();
            const Pos nn = advance(nxt);
            issue_tile(nn, std::integral_constant<int, P>{});
            if (nxt.n < a.N) phase_a(P == 0 ? X1 : X0, P == 0 ? T1 : T0, identity1);
            phase_b(P == 0 ? T0 : T1, cur, from_bias);
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
    };
    if (id1 && bias_init2) run(std::true_type{}, std::true_type{});
    else run(std::false_type{}, std::false_type{});
    // loads of tiles past the end may still be in flight into LDS: drain them before
    // the workgroup's LDS can be handed to another workgroup
    mm::wait_vmcnt<0>();
}

template <typename T, int S, int TH, int TW, int KT, int CC, int NW, int OCC, int M, int FS>
int launch_dwpw_mm(const KArgs& a, int grid, void* stream) {
    (void)hipGetLastError();
    hipLaunchKernelGGL((dwpw_mm_kernel<T, S, TH, TW, KT, CC, NW, OCC, M, FS>), dim3(grid),
                       dim3(64 * NW), 0, (hipStream_t)stream, a);
    return (int)hipGetLastError();
}
template <typename T, int S, int TH, int TW, int KT, int CC, int NW, int OCC, int M, int FS>
int occ_dwpw_mm() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, dwpw_mm_kernel<T, S, TH, TW, KT, CC, NW, OCC, M, FS>, 64 * NW, 0) != hipSuccess)
        return 0;
    return n;
}

#define FCM_V_DWPW(...)
#define FCM_V_DWPW32(...)
#define FCM_V_B2B(...)
#define FCM_V_B2B_MM(...)
#define FCM_V_DWPW_MM(name, dt, CT, S, TH, TW, KT, CC, NW, OCC)                                    \
    template int launch_dwpw_mm<CT, S, TH, TW, KT, CC, NW, OCC, 1, 3>(const KArgs&, int, void*); \
    template int occ_dwpw_mm<CT, S, TH, TW, KT, CC, NW, OCC, 1, 3>();
#define FCM_V_DWPW_MMM(name, dt, CT, S, M, TH, TW, KT, CC, NW, OCC)                               \
    template int launch_dwpw_mm<CT, S, TH, TW, KT, CC, NW, OCC, M, 3>(const KArgs&, int, void*); \
    template int occ_dwpw_mm<CT, S, TH, TW, KT, CC, NW, OCC, M, 3>();
#define FCM_V_DWPW_MMF(name, dt, CT, S, FS, TH, TW, KT, CC, NW, OCC)                               \
    template int launch_dwpw_mm<CT, S, TH, TW, KT, CC, NW, OCC, 1, FS>(const KArgs&, int, void*); \
    template int occ_dwpw_mm<CT, S, TH, TW, KT, CC, NW, OCC, 1, FS>();
#define FCM_V_DWPW_MMW(...)
#include "../variants.def"
#undef FCM_V_DWPW
#undef FCM_V_DWPW32
#undef FCM_V_B2B
#undef FCM_V_DWPW_MM
#undef FCM_V_DWPW_MMM
#undef FCM_V_DWPW_MMF
#undef FCM_V_B2B_MM
#undef FCM_V_DWPW_MMW

}  // namespace fcm
