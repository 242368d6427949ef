// dwpw_i8.hip -- INT8 fused depthwise 3x3 -> pointwise 1x1 (the FCM DWPW module in INT8)
// on the gfx950 matrix cores, the INT8 layer-by-layer baselines, and INT8 weight packing.
//
// INT8 in the FCM paper ("Fusing Depthwise and Pointwise Convolutions for Efficient
// Inference on GPUs", Sec. III-B): int8 operands, four-way int8 dot products with 32-bit
// accumulation, the convolution-normalisation-activation result packed to 8 bits before
// it is written to any buffer (the intermediate included), weights packed offline.  Here
// each storage point requantizes in binary32: v = fma(scale, acc, bias), clamp to the
// activation's range and to [-128, 127], nearest integer with ties to even.
//
// Single-pass fused kernel, one workgroup of four waves per 4x16 tile of outputs and 64
// output channels (C <= 64 input channels, C and K multiples of 16; the chunked kernel
// further down takes wider layers):
//   phase A  wave w: depthwise layer of channels 16w .. 16w+15 for the 4 output rows, on
//            the matrix cores in block-diagonal form: v_mfma_i32_16x16x64_i8 takes four
//            taps x 16 channels per instruction, so one instruction per filter row
//            (three taps and an empty fourth) -- 3 products per 16 channels x 16 pixels.
//            The B operand of filter row dh is 16 bytes per lane (16 channels of one
//            pixel) from one input row, so each input row is read once for the output
//            rows that use it.  The result, 4 channels of one pixel per lane, is
//            requantized and written as 4 bytes to the LDS intermediate, where the
//            outputs of the four waves interleave into ready-made pointwise operands.
//   phase B  wave w: pointwise layer of output row w, all 64 output channels: one
//            product per 16 output channels (the reduction over 64 channels is one
//            instruction); output rows are permuted so that each lane ends with 16
//            consecutive channels of its pixel, stored as one 16-byte store.
// The phases are software-pipelined over the workgroup's tiles exactly as in the 16-bit
// matrix-core kernel: step i runs phase A of tile i+1 and phase B of tile i, one barrier
// per step, two input and two intermediate buffers, input tiles by direct global->LDS
// loads with exact vector-memory waits (one store per lane per step).
#include <type_traits>

#include "mm_common.h"

namespace fcm {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

namespace q8 {

// binary32 requantization of one accumulator: fma, clamp to [lo, hi] (the activation's
// range already narrowed to [-128, 127]); adding 1.5 * 2^23 then rounds to an integer in
// the default round-to-nearest-even mode, and the low byte of the sum's bit pattern is
// the two's-complement code
__device__ __forceinline__ uint32_t requant(int32_t acc, float s, float b, float lo, float hi) {
    const float v = __builtin_amdgcn_fmed3f(__builtin_fmaf(s, (float)acc, b), lo, hi);
    return __builtin_bit_cast(uint32_t, v + 12582912.0f);
}

// the low bytes of four words, packed (byte i from word i)
__device__ __forceinline__ uint32_t pack4(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
    const uint32_t lo = __builtin_amdgcn_perm(w1, w0, 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(w3, w2, 0x04000c0cu);
    return lo | hi;
}

__device__ __forceinline__ int32_t sbyte(uint32_t w, int i) {
    return (int32_t)(int8_t)(w >> (8 * i));
}

struct Bounds {
    float lo, hi;
};
__device__ __forceinline__ Bounds bounds(int act) {
    const Act a = act_bounds(act);
    return Bounds{a.lo > -128.0f ? a.lo : -128.0f, a.hi < 127.0f ? a.hi : 127.0f};
}

__device__ __forceinline__ i32x4 mfma(u32x4 a, u32x4 b, i32x4 c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a),
                                                 __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

}  // namespace q8

template <int S, int OCC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC, 8)))
void dwpw_i8_kernel(KArgs a) {
    constexpr int TH = 4, TW = 16, NT = 256, KT = 64;
    constexpr int IH = (TH - 1) * S + 3, IW = (TW - 1) * S + 3, NPIX = IH * IW;
    constexpr int CH = 4;  // 16-byte chunks (16 channels) per pixel in LDS
    constexpr int SLOTS = NPIX * CH;
    constexpr int R = (SLOTS + NT - 1) / NT;  // direct-load rounds per tile
    constexpr int SLOTS_P = R * NT;
    constexpr int NST = 1;                    // stores per lane per step
    constexpr uint32_t IROW_BYTES = (uint32_t)IW * CH * 16;
    constexpr int IHW = IH;                   // input rows under the tile's 4 output rows

    __shared__ __attribute__((aligned(16))) u32x4 xs0[SLOTS_P];
    __shared__ __attribute__((aligned(16))) u32x4 xs1[SLOTS_P];
    // intermediate, [row][pixel][lane group] x 16 bytes (bytes 4b .. 4b+3 from wave b)
    __shared__ __attribute__((aligned(16))) u32x4 tl0[TH * 64];
    __shared__ __attribute__((aligned(16))) u32x4 tl1[TH * 64];
    u32x4* const X0 = xs0;
    u32x4* const X1 = xs1;
    u32x4* const T0 = tl0;
    u32x4* const T1 = tl1;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const q8::Bounds bd1 = q8::bounds(a.act1), bd2 = q8::bounds(a.act2);
    const int G = gridDim.x;
    const int L = xcd_logical_id(blockIdx.x, G);
    const int k0 = (L % a.num_ktiles) * KT;
    const int8_t* __restrict__ wdw = (const int8_t*)a.w1;  // [9][C]
    const __amdgpu_buffer_rsrc_t rx = mm::rsrc(a.x, (uint32_t)(a.N * a.H * a.W * a.C));
    const __amdgpu_buffer_rsrc_t ry = mm::rsrc(a.y, (uint32_t)(a.N * a.Ho * a.Wo * a.K));
    const int in_img = a.H * a.W * a.C, in_row = a.W * a.C;
    const int out_img = a.Ho * a.Wo * a.K, out_row = a.Wo * a.K;

    // ---- tile walk (image, tile row, tile column), mixed-radix advance ----------------
    const int pstep = G / a.num_ktiles;
    using Pos = mm::TilePos;
    auto derive = [&](Pos& p) {
        p.oh0 = p.th * TH;
        p.ow0 = p.tw * TW;
        p.ih0 = p.oh0 * S - a.pad_h;
        p.iw0 = p.ow0 * S - a.pad_w;
        p.in_base = p.n * in_img + p.ih0 * in_row + p.iw0 * a.C;
        p.out_base = p.n * out_img + p.oh0 * out_row + p.ow0 * a.K;
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

    // ---- direct-load plan (tile invariant) ------------------------------------------
    // LDS slot s holds chunk position s % 4 of window pixel p = s / 4, i.e. input chunk
    // q = (s % 4) ^ ((column >> 2) & 3): the 16 lanes of an operand read (16
    // consecutive columns, one chunk) then hit distinct bank groups, and the swizzle does
    // not depend on the row, so a row down is a constant offset.
    uint32_t dl_off[R];
    int dl_pos[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int s = r * NT + tid;
        const int p = s / CH, wr = p / IW, wc = p % IW;
        const int q = (s % CH) ^ ((wc >> 2) & 3);
        const bool real = p < NPIX && q * 16 < a.C;
        dl_off[r] = real ? (uint32_t)((wr * a.W + wc) * a.C + q * 16) : mm::kOob;
        dl_pos[r] = real ? (wr << 16) | wc : 0;
    }
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

    Pos cur = split(L / a.num_ktiles);
    Pos nxt = advance(cur);
    issue_tile(cur, std::integral_constant<int, 0>{});

    // ---- constants (requested after the first tile, before the second) --------------
    // depthwise A operand of filter row dh, lane (l%16, l/16): byte e of the lane's 16
    // bytes multiplies channel 16w + e of the pixel at tap (dh, l/16) (l/16 = 3: empty
    // tap); the diagonal keeps byte e = l%16 only
    const int cdw = 16 * wave + lr;
    uint32_t wdr[3];
#pragma unroll
    for (int dh = 0; dh < 3; ++dh) {
        const int t = 3 * dh + (lg < 3 ? lg : 0);
        wdr[dh] = (uint32_t)(uint8_t)wdw[t * a.C + (cdw < a.C ? cdw : 0)];
    }
    const float* s1p = a.s1 ? a.s1 : (const float*)a.w2;
    const float* b1p = a.b1 ? a.b1 : (const float*)a.w2;
    const float* s2p = a.s2 ? a.s2 : (const float*)a.w2;
    const float* b2p = a.b2 ? a.b2 : (const float*)a.w2;
    float s1r[4], b1r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = 16 * wave + 4 * lg + i, cc = c < a.C ? c : 0;
        s1r[i] = s1p[cc];
        b1r[i] = b1p[cc];
    }
    // pointwise A operands: blocked copy after the plain [K][C] filters, block (k tile,
    // kb) of 64 lanes x 16 bytes (output channel k0 + 16((l%16)/4) + 4kb + (l%16)%4,
    // input channel 16(e/4) + 4(l/16) + e%4 for byte e), one 16-byte load per lane
    const int nkt = (a.K + KT - 1) / KT;
    const u32x4* __restrict__ wpb =
        reinterpret_cast<const u32x4*>((const int8_t*)a.w2 + (int64_t)a.K * a.C);
    u32x4 wa[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
        wa[kb] = wpb[((k0 / KT < nkt ? k0 / KT : 0) * 4 + kb) * 64 + lane];
    // epilogue-2 constants of the lane's output channels k0 + 16(l/16) + j
    float s2r[16], b2r[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int k = k0 + 16 * lg + j, kk = k < a.K ? k : 0;
        s2r[j] = s2p[kk];
        b2r[j] = b2p[kk];
    }
    issue_tile(nxt, std::integral_constant<int, 1>{});

    // now the loaded values are used
    u32x4 adw[3];
#pragma unroll
    for (int dh = 0; dh < 3; ++dh) {
        const bool ok = lg < 3 && cdw < a.C;
        const uint32_t v = ok ? (wdr[dh] << (8 * (lr & 3))) : 0u;
        const int w4 = lr >> 2;
        adw[dh] = u32x4{w4 == 0 ? v : 0u, w4 == 1 ? v : 0u, w4 == 2 ? v : 0u, w4 == 3 ? v : 0u};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool ok = 16 * wave + 4 * lg + i < a.C;
        s1r[i] = (a.s1 && ok) ? s1r[i] : 1.0f;
        b1r[i] = (a.b1 && ok) ? b1r[i] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const bool ok = k0 + 16 * lg + j < a.K;
        s2r[j] = (a.s2 && ok) ? s2r[j] : 1.0f;
        b2r[j] = (a.b2 && ok) ? b2r[j] : 0.0f;
    }
    // phase A operand read of input row 0: column l%16 * S + (l/16 < 3 ? l/16 : 0),
    // chunk w (input row ir adds ir * IROW_BYTES)
    const int ccol = lr * S + (lg < 3 ? lg : 0);
    const uint32_t xo = (uint32_t)((ccol * CH + (wave ^ ((ccol >> 2) & 3))) * 16);
    // intermediate write of row r: pixel l%16, lane group l/16, bytes 4w .. 4w+3
    const uint32_t tw_off = (uint32_t)((lr * 4 + lg) * 16 + wave * 4);
    // output store: the lane's 16 channels of pixel (row w, column l%16); lane part
    // (column and channel; out of range when either does not exist) and row part
    constexpr uint32_t kLaneOob = 0x40000000u, kRowOob = 0x80000000u;
    const uint32_t st_lane = (k0 + 16 * lg < a.K) ? (uint32_t)(lr * a.K + k0 + 16 * lg) : kLaneOob;

    // phase A: depthwise of this wave's 16 channels for the 4 rows of tile src -> dst
    auto phase_a = [&](const u32x4* src, u32x4* dst) __attribute__((always_inline)) {
        const char* xb = reinterpret_cast<const char*>(src);
        u32x4 b[IHW];
#pragma unroll
        for (int ir = 0; ir < IHW; ++ir)
            b[ir] = *reinterpret_cast<const u32x4*>(xb + ir * IROW_BYTES + xo);
        i32x4 d[TH];
#pragma unroll
        for (int r = 0; r < TH; ++r) d[r] = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int ir = 0; ir < IHW; ++ir)
#pragma unroll
            for (int dh = 0; dh < 3; ++dh)
                if (ir >= dh && (ir - dh) % S == 0 && (ir - dh) / S < TH)
                    d[(ir - dh) / S] = q8::mfma(adw[dh], b[ir], d[(ir - dh) / S]);
        __builtin_amdgcn_sched_group_barrier(0x100, IHW, 0);     // operand reads
        __builtin_amdgcn_sched_group_barrier(0x008, 3 * TH, 0);  // products
#pragma unroll
        for (int r = 0; r < TH; ++r) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = q8::requant(d[r][i], s1r[i], b1r[i], bd1.lo, bd1.hi);
            *reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(dst) + r * 1024 + tw_off) =
                q8::pack4(w[0], w[1], w[2], w[3]);
        }
    };
    // phase B: pointwise of output row w of tile t from src; one 16-byte store per lane
    auto phase_b = [&](const u32x4* src, const Pos& t) __attribute__((always_inline)) {
        const u32x4 bf = src[(wave * 16 + lr) * 4 + lg];
        i32x4 acc[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc[kb] = q8::mfma(wa[kb], bf, i32x4{0, 0, 0, 0});
        uint32_t o[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                w[i] = q8::requant(acc[kb][i], s2r[4 * kb + i], b2r[4 * kb + i], bd2.lo, bd2.hi);
            o[kb] = q8::pack4(w[0], w[1], w[2], w[3]);
        }
        const uint32_t lanev = t.ow0 + lr < a.Wo ? st_lane : kLaneOob;
        const uint32_t row = t.oh0 + wave < a.Ho ? (uint32_t)(t.out_base + wave * out_row) : kRowOob;
        // the whole offset in the vector operand, scalar offset 0
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{o[0], o[1], o[2], o[3]}, ry, lanev + row, 0,
                                               mm::kStoreStream);
    };

    // ---- software-pipelined tile loop (as in the 16-bit matrix-core kernel) ---------
    // Step (buffers P): wait for the next tile's input (ops issued after its loads: the
    // NST stores of the previous step, none before the first step); barrier; request the
    // tile after into X[P]; phase A of the next tile (X[1-P] -> T[1-P]); phase B of the
    // current tile (T[P]).
    mm::wait_vmcnt<R>();
    __builtin_amdgcn_s_barrier();
    if (cur.n < a.N) phase_a(X0, T0);
    auto step_fn = [&](auto par, bool first) __attribute__((always_inline)) {
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
    // loads of tiles past the end may still be in flight into LDS
    mm::wait_vmcnt<0>();
}

// Chunked INT8 kernel for C up to CMAX (wider layers: the depthwise and pointwise layers of
// MobileNetV2-style bottlenecks run 96 to 960 channels).  The same 4x16 tiles, four waves
// and 64 output channels per workgroup; a step is one (tile, 64-channel slice) pair:
//   phase A  the slice's depthwise layer exactly as in the single-pass kernel (wave w:
//            channels 64c + 16w .. +15), with the depthwise filters and epilogue-1
//            constants of every channel read from LDS (copied there once);
//   phase B  the pointwise product of the slice, accumulated in int32 registers across
//            the tile's slices (output stationary); the slice's operands come from the
//            blocked copy (block (k tile, slice, kb)) one step ahead, in one of two
//            register sets named by the step's parity.
// After a tile's last slice, epilogue 2 and the 16-byte store; every other step issues
// the same store with an out-of-range offset, so each step ends with the same number of
// vector-memory operations and its wait counts them exactly.  Channels past C (a
// partial last slice) load as zeros, have zero depthwise filters and zero pointwise
// filters.
template <int S, int OCC, int CMAX>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC, 8)))
void dwpw_i8c_kernel(KArgs a) {
    constexpr int TH = 4, TW = 16, NT = 256, KT = 64, CC = 64;
    constexpr int IH = (TH - 1) * S + 3, IW = (TW - 1) * S + 3, NPIX = IH * IW;
    constexpr int CH = 4;  // 16-byte chunks (16 channels) per pixel of a slice in LDS
    constexpr int SLOTS = NPIX * CH;
    constexpr int R = (SLOTS + NT - 1) / NT;  // direct-load rounds per slice
    constexpr int SLOTS_P = R * NT;
    constexpr uint32_t IROW_BYTES = (uint32_t)IW * CH * 16;
    constexpr int IHW = IH;
    static_assert(CMAX % CC == 0, "whole slices");

    __shared__ __attribute__((aligned(16))) u32x4 xs0[SLOTS_P];
    __shared__ __attribute__((aligned(16))) u32x4 xs1[SLOTS_P];
    __shared__ __attribute__((aligned(16))) u32x4 tl0[TH * 64];
    __shared__ __attribute__((aligned(16))) u32x4 tl1[TH * 64];
    __shared__ __attribute__((aligned(16))) uint32_t wd4[9 * CMAX / 4];  // depthwise [9][CMAX]
    __shared__ __attribute__((aligned(16))) float s1s[CMAX];
    __shared__ __attribute__((aligned(16))) float b1s[CMAX];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const q8::Bounds bd1 = q8::bounds(a.act1), bd2 = q8::bounds(a.act2);
    const int G = gridDim.x;
    const int L = xcd_logical_id(blockIdx.x, G);
    const int k0 = (L % a.num_ktiles) * KT;
    const int nch = (a.C + CC - 1) / CC;
    const __amdgpu_buffer_rsrc_t rx = mm::rsrc(a.x, (uint32_t)(a.N * a.H * a.W * a.C));
    const __amdgpu_buffer_rsrc_t ry = mm::rsrc(a.y, (uint32_t)(a.N * a.Ho * a.Wo * a.K));
    const int in_img = a.H * a.W * a.C, in_row = a.W * a.C;
    const int out_img = a.Ho * a.Wo * a.K, out_row = a.Wo * a.K;

    // ---- (tile, slice) walk --------------------------------------------------------
    const int pstep = G / a.num_ktiles;
    using Pos = mm::TilePos;
    auto derive = [&](Pos& p) {
        p.oh0 = p.th * TH;
        p.ow0 = p.tw * TW;
        p.ih0 = p.oh0 * S - a.pad_h;
        p.iw0 = p.ow0 * S - a.pad_w;
        p.in_base = p.n * in_img + p.ih0 * in_row + p.iw0 * a.C;
        p.out_base = p.n * out_img + p.oh0 * out_row + p.ow0 * a.K;
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
    auto next = [&](const Step& st) {
        Step n;
        if (st.c + 1 < nch) {
            n.t = st.t;
            n.c = st.c + 1;
        } else {
            n.t = advance(st.t);
            n.c = 0;
        }
        return n;
    };

    // ---- direct-load plan of one slice (as in the single-pass kernel; the channel
    // group of each slot is kept to drop groups past C in a partial last slice) --------
    uint32_t dl_off[R];
    int dl_pos[R], dl_q[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int s = r * NT + tid;
        const int p = s / CH, wr = p / IW, wc = p % IW;
        const int q = (s % CH) ^ ((wc >> 2) & 3);
        const bool real = p < NPIX;
        dl_off[r] = real ? (uint32_t)((wr * a.W + wc) * a.C + q * 16) : mm::kOob;
        dl_pos[r] = real ? (wr << 16) | wc : 0;
        dl_q[r] = q;
    }
    auto issue_slice = [&](const Step& st, u32x4* dst) __attribute__((always_inline)) {
        const Pos& t = st.t;
        const bool live = t.n < a.N;
        const int cb = st.c * CC, cl = a.C - cb;  // channels of the slice present
        const bool inside = live && t.ih0 >= 0 && t.iw0 >= 0 && t.ih0 + IH <= a.H &&
                            t.iw0 + IW <= a.W;
        if (inside) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t off = dl_q[r] * 16 < cl ? dl_off[r] : mm::kOob;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rx, (__attribute__((address_space(3))) void*)(dst + r * NT + wave * 64), 16,
                    off, t.in_base + cb, 0, 0);
            }
        } else {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int ih = t.ih0 + (dl_pos[r] >> 16), iw = t.iw0 + (dl_pos[r] & 0xffff);
                const bool ok = live && dl_off[r] != mm::kOob && dl_q[r] * 16 < cl &&
                                (unsigned)ih < (unsigned)a.H && (unsigned)iw < (unsigned)a.W;
                const uint32_t off = ok ? (uint32_t)(t.in_base + cb + (int)dl_off[r]) : mm::kOob;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rx, (__attribute__((address_space(3))) void*)(dst + r * NT + wave * 64), 16,
                    off, 0, 0, 0);
            }
        }
    };

    // ---- constants: depthwise filters and epilogue-1 constants of every channel to LDS,
    // epilogue-2 constants of the lane's output channels in registers ------------------
    constexpr int IWD = (9 * CMAX / 4 + NT - 1) / NT, I1 = (CMAX + NT - 1) / NT;
    const int nwd = 9 * a.C / 4;  // (C a multiple of 16)
    uint32_t wdv[IWD];
    float s1v[I1], b1v[I1];
#pragma unroll
    for (int r = 0; r < IWD; ++r) {
        const int i = tid + r * NT;
        wdv[r] = i < nwd ? reinterpret_cast<const uint32_t*>(a.w1)[i] : 0u;
    }
#pragma unroll
    for (int r = 0; r < I1; ++r) {
        const int i = tid + r * NT;
        s1v[r] = (a.s1 && i < a.C) ? a.s1[i] : 1.0f;
        b1v[r] = (a.b1 && i < a.C) ? a.b1[i] : 0.0f;
    }
    float s2r[16], b2r[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int k = k0 + 16 * lg + j;
        const bool ok = k < a.K;
        s2r[j] = (a.s2 && ok) ? a.s2[k] : 1.0f;
        b2r[j] = (a.b2 && ok) ? a.b2[k] : 0.0f;
    }
    // pointwise operands of slice c: blocked copy after the plain [K][C] filters, block
    // ((k tile) * nch + c) * 4 + kb of 64 lanes x 16 bytes
    const int nkt = (a.K + KT - 1) / KT;
    const u32x4* __restrict__ wpb =
        reinterpret_cast<const u32x4*>((const int8_t*)a.w2 + (int64_t)a.K * a.C);
    const int kt_blk = (k0 / KT < nkt ? k0 / KT : 0) * nch;
    auto load_pw = [&](const Step& st, u32x4 (&w)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) w[kb] = wpb[((kt_blk + st.c) * 4 + kb) * 64 + lane];
    };

    // phase A operand read of input row 0 (input row ir adds ir * IROW_BYTES); the
    // intermediate write of row r; the output store's lane part
    const int ccol = lr * S + (lg < 3 ? lg : 0);
    const uint32_t xo = (uint32_t)((ccol * CH + (wave ^ ((ccol >> 2) & 3))) * 16);
    const uint32_t tw_off = (uint32_t)((lr * 4 + lg) * 16 + wave * 4);
    constexpr uint32_t kLaneOob = 0x40000000u, kRowOob = 0x80000000u;
    const uint32_t st_lane = (k0 + 16 * lg < a.K) ? (uint32_t)(lr * a.K + k0 + 16 * lg) : kLaneOob;
    const uint8_t* wd8 = reinterpret_cast<const uint8_t*>(wd4);

    // phase A: depthwise of this wave's 16 channels of slice c for the 4 rows of the tile
    auto phase_a = [&](const u32x4* src, u32x4* dst, int c) __attribute__((always_inline)) {
        const int cdw = c * CC + 16 * wave + lr;
        u32x4 adw[3];
#pragma unroll
        for (int dh = 0; dh < 3; ++dh) {
            const bool ok = lg < 3 && cdw < a.C;
            const uint32_t wv = (uint32_t)wd8[(3 * dh + (lg < 3 ? lg : 0)) * CMAX + (ok ? cdw : 0)];
            const uint32_t v = ok ? (wv << (8 * (lr & 3))) : 0u;
            const int w4 = lr >> 2;
            adw[dh] = u32x4{w4 == 0 ? v : 0u, w4 == 1 ? v : 0u, w4 == 2 ? v : 0u, w4 == 3 ? v : 0u};
        }
        const f32x4 sc = *reinterpret_cast<const f32x4*>(s1s + c * CC + 16 * wave + 4 * lg);
        const f32x4 bi = *reinterpret_cast<const f32x4*>(b1s + c * CC + 16 * wave + 4 * lg);
        const char* xb = reinterpret_cast<const char*>(src);
        u32x4 b[IHW];
#pragma unroll
        for (int ir = 0; ir < IHW; ++ir)
            b[ir] = *reinterpret_cast<const u32x4*>(xb + ir * IROW_BYTES + xo);
        i32x4 d[TH];
#pragma unroll
        for (int r = 0; r < TH; ++r) d[r] = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int ir = 0; ir < IHW; ++ir)
#pragma unroll
            for (int dh = 0; dh < 3; ++dh)
                if (ir >= dh && (ir - dh) % S == 0 && (ir - dh) / S < TH)
                    d[(ir - dh) / S] = q8::mfma(adw[dh], b[ir], d[(ir - dh) / S]);
#pragma unroll
        for (int r = 0; r < TH; ++r) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = q8::requant(d[r][i], sc[i], bi[i], bd1.lo, bd1.hi);
            *reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(dst) + r * 1024 + tw_off) =
                q8::pack4(w[0], w[1], w[2], w[3]);
        }
    };
    i32x4 acc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) acc[kb] = i32x4{0, 0, 0, 0};

    // ---- prologue: slice 0's window and operands, constants to LDS, phase A of step 0
    Step cur;
    cur.t = split(L / a.num_ktiles);
    cur.c = 0;
    Step nx = next(cur);
    u32x4 wa0[4], wa1[4];
    load_pw(cur, wa0);
    issue_slice(cur, xs0);
#pragma unroll
    for (int r = 0; r < IWD; ++r) {
        const int i = tid + r * NT;
        if (i < nwd) {
            const int t = i / (a.C / 4), c4 = i - t * (a.C / 4);
            wd4[t * (CMAX / 4) + c4] = wdv[r];
        }
    }
#pragma unroll
    for (int r = 0; r < I1; ++r) {
        const int i = tid + r * NT;
        if (i < CMAX) {
            s1s[i] = s1v[r];
            b1s[i] = b1v[r];
        }
    }
    mm::wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): constants written
    __builtin_amdgcn_s_barrier();
    phase_a(xs0, tl0, cur.c);

    // ---- steps: the workgroup's step count is known up front, so the loop runs two
    // steps per round (parity P names the buffers and the operand set) and at most one
    // more ----------------------------------------------------------------------------
    // step (parity P): barrier; next step's operands into the other set; window of step
    // s+2 into X[P]; phase A of step s+1 (X[1-P] -> T[1-P]); phase B of step s (T[P]);
    // the tile's store (or its out-of-range twin); wait for all but that store
    auto step = [&](auto par, const u32x4 (&use)[4], u32x4 (&fill)[4])
                    __attribute__((always_inline)) {
        constexpr int P = decltype(par)::value;
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): own intermediate writes done
        __builtin_amdgcn_s_barrier();
        const Step n2 = next(nx);
        load_pw(nx, fill);
        issue_slice(n2, P == 0 ? xs0 : xs1);
        phase_a(P == 0 ? xs1 : xs0, P == 0 ? tl1 : tl0, nx.c);
        const u32x4 bf = (P == 0 ? tl0 : tl1)[(wave * 16 + lr) * 4 + lg];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc[kb] = q8::mfma(use[kb], bf, acc[kb]);
        const bool done = cur.c == nch - 1;
        uint32_t o[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                w[i] = q8::requant(acc[kb][i], s2r[4 * kb + i], b2r[4 * kb + i], bd2.lo, bd2.hi);
            o[kb] = q8::pack4(w[0], w[1], w[2], w[3]);
        }
        const Pos& t = cur.t;
        const uint32_t lanev = (done && t.ow0 + lr < a.Wo) ? st_lane : kLaneOob;
        const uint32_t row =
            t.oh0 + wave < a.Ho ? (uint32_t)(t.out_base + wave * out_row) : kRowOob;
        // the whole offset in the vector operand, scalar offset 0
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{o[0], o[1], o[2], o[3]}, ry, lanev + row,
                                               0, mm::kStoreStream);
        if (done) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) acc[kb] = i32x4{0, 0, 0, 0};
        }
        mm::wait_vmcnt<1>();  // this step's operands and window; the store may still run
        cur = nx;
        nx = n2;
    };
    const int t_first = L / a.num_ktiles;
    const int n_tiles = t_first < a.num_ptiles ? (a.num_ptiles - 1 - t_first) / pstep + 1 : 0;
    const int n_steps = n_tiles * nch;
    // (phase A above ran on step 0's window: the first step needs step 1's window and
    // operands, issued here)
    issue_slice(nx, xs1);
    mm::wait_vmcnt<0>();
    int si = 0;
    for (; si + 2 <= n_steps; si += 2) {
        step(std::integral_constant<int, 0>{}, wa0, wa1);
        step(std::integral_constant<int, 1>{}, wa1, wa0);
    }
    if (si < n_steps) step(std::integral_constant<int, 0>{}, wa0, wa1);
    // windows of steps past the end may still be in flight into LDS
    mm::wait_vmcnt<0>();
}

template <int S, int OCC, int CMAX>
int launch_dwpw_i8(const KArgs& a, int grid, void* stream) {
    (void)hipGetLastError();
    if constexpr (CMAX == 64)
        hipLaunchKernelGGL((dwpw_i8_kernel<S, OCC>), dim3(grid), dim3(256), 0,
                           (hipStream_t)stream, a);
    else
        hipLaunchKernelGGL((dwpw_i8c_kernel<S, OCC, CMAX>), dim3(grid), dim3(256), 0,
                           (hipStream_t)stream, a);
    return (int)hipGetLastError();
}
template <int S, int OCC, int CMAX>
int occ_dwpw_i8() {
    int n = 0;
    hipError_t e;
    if constexpr (CMAX == 64)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, dwpw_i8_kernel<S, OCC>, 256, 0);
    else
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, dwpw_i8c_kernel<S, OCC, CMAX>, 256, 0);
    return e == hipSuccess ? n : 0;
}

// ---- INT8 layer-by-layer baselines -------------------------------------------------
// Depthwise: one thread per (output pixel, 4 channels); 9 taps x 4 channels of exact
// int32 sums; requantized; 4 bytes stored.  x: [N][H][W][C], w: [9][C], t: [N][Ho][Wo][C].
template <int S>
__global__ __launch_bounds__(256) void dw_lbl_i8_kernel(KArgs a) {
    const int C4 = a.C / 4;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)a.N * a.Ho * a.Wo * C4;
    if (idx >= total) return;
    const int c4 = (int)(idx % C4);
    const int64_t pix = idx / C4;
    const int ow = (int)(pix % a.Wo), oh = (int)((pix / a.Wo) % a.Ho), n = (int)(pix / ((int64_t)a.Wo * a.Ho));
    const uint32_t* __restrict__ x = (const uint32_t*)a.x;
    const uint32_t* __restrict__ w = (const uint32_t*)a.w1;
    int32_t acc[4] = {0, 0, 0, 0};
    for (int r = 0; r < 3; ++r)
        for (int s = 0; s < 3; ++s) {
            const int ih = oh * S - a.pad_h + r, iw = ow * S - a.pad_w + s;
            if ((unsigned)ih >= (unsigned)a.H || (unsigned)iw >= (unsigned)a.W) continue;
            const uint32_t xv = x[(((int64_t)n * a.H + ih) * a.W + iw) * C4 + c4];
            const uint32_t wv = w[(3 * r + s) * C4 + c4];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += q8::sbyte(xv, i) * q8::sbyte(wv, i);
        }
    const q8::Bounds bd = q8::bounds(a.act1);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = 4 * c4 + i;
        o[i] = q8::requant(acc[i], a.s1 ? a.s1[c] : 1.0f, a.b1 ? a.b1[c] : 0.0f, bd.lo, bd.hi);
    }
    ((uint32_t*)a.y)[pix * C4 + c4] = q8::pack4(o[0], o[1], o[2], o[3]);
}

// Pointwise: one thread per (pixel, 16 output channels); the workgroup's 16 filters are
// staged in LDS (every lane reads the same word: a broadcast); four-way int8 dot
// products with 32-bit accumulation over C (the pages' dp4a), the pixel's channels read
// 16 bytes at a time; requantized; one 16-byte store.  t: [M][C], w: [K][C] (plain),
// y: [M][K], M = N * Ho * Wo; blockIdx.y = group of 16 output channels; C <= 1024.
__global__ __launch_bounds__(256) void pw_lbl_i8_kernel(KArgs a) {
    __shared__ uint32_t ws[16 * 256];
    const int C4 = a.C / 4, kg = blockIdx.y;
    const int64_t M = (int64_t)a.N * a.Ho * a.Wo;
    const uint32_t* __restrict__ w = (const uint32_t*)a.w2 + (int64_t)16 * kg * C4;
    for (int i = threadIdx.x; i < 16 * C4; i += 256) ws[i] = w[i];
    __syncthreads();
    const int64_t m = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (m >= M) return;
    const u32x4* __restrict__ t = (const u32x4*)((const uint32_t*)a.x + m * C4);
    int32_t acc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = 0;
    for (int c16 = 0; c16 < C4 / 4; ++c16) {
        const u32x4 tv = t[c16];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int k = 0; k < 16; ++k)
                acc[k] = __builtin_amdgcn_sdot4((int)tv[j], (int)ws[k * C4 + 4 * c16 + j], acc[k],
                                                false);
    }
    const q8::Bounds bd = q8::bounds(a.act2);
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = 16 * kg + 4 * q + i;
            v[i] = q8::requant(acc[4 * q + i], a.s2 ? a.s2[k] : 1.0f, a.b2 ? a.b2[k] : 0.0f,
                               bd.lo, bd.hi);
        }
        o[q] = q8::pack4(v[0], v[1], v[2], v[3]);
    }
    *reinterpret_cast<u32x4*>((int8_t*)a.y + m * a.K + 16 * kg) = u32x4{o[0], o[1], o[2], o[3]};
}

int launch_dw_lbl_i8(int stride, const KArgs& a, void* stream) {
    const int64_t total = (int64_t)a.N * a.Ho * a.Wo * (a.C / 4);
    const dim3 g((unsigned)((total + 255) / 256));
    (void)hipGetLastError();
    if (stride == 2)
        hipLaunchKernelGGL(dw_lbl_i8_kernel<2>, g, dim3(256), 0, (hipStream_t)stream, a);
    else
        hipLaunchKernelGGL(dw_lbl_i8_kernel<1>, g, dim3(256), 0, (hipStream_t)stream, a);
    return (int)hipGetLastError();
}

int launch_pw_lbl_i8(const KArgs& a, void* stream) {
    if (a.C > 1024) return (int)hipErrorInvalidValue;
    const int64_t M = (int64_t)a.N * a.Ho * a.Wo;
    (void)hipGetLastError();
    hipLaunchKernelGGL(pw_lbl_i8_kernel, dim3((unsigned)((M + 255) / 256), (unsigned)(a.K / 16)),
                       dim3(256), 0, (hipStream_t)stream, a);
    return (int)hipGetLastError();
}

// ---- INT8 weight packing -----------------------------------------------------------
// depthwise [C][9] -> [9][C]
__global__ void pack_dw_i8_kernel(const int8_t* __restrict__ src, int8_t* __restrict__ dst, int C) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= 9 * C) return;
    const int t = i / C, c = i % C;
    dst[i] = src[c * 9 + t];
}
// pointwise [K][C] -> blocks (k tile of 64, 64-channel slice sc, kb) of 64 lanes x 16
// bytes: lane l = 16 g + r, byte e holds filter [64 kt + 16 (r / 4) + 4 kb + r % 4]
// [64 sc + 16 (e / 4) + 4 g + e % 4] (zero outside K x C); block index (kt * nch + sc) * 4
// + kb, nch = ceil(C / 64)
__global__ void pack_pw_i8_kernel(const int8_t* __restrict__ src, int8_t* __restrict__ dst,
                                  int K, int C, int nkt, int nch) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= nkt * nch * 4 * 64 * 16) return;
    const int e = i % 16, l = (i / 16) % 64, kb = (i / 1024) % 4, blk = i / 4096;
    const int sc = blk % nch, kt = blk / nch;
    const int r = l % 16, g = l / 16;
    const int k = 64 * kt + 16 * (r / 4) + 4 * kb + r % 4;
    const int c = 64 * sc + 16 * (e / 4) + 4 * g + e % 4;
    dst[i] = (k < K && c < C) ? src[(int64_t)k * C + c] : (int8_t)0;
}

int launch_pack_i8(const void* w_dw, void* dw_dst, const void* w_pw, void* pw_dst, int C, int K,
                   void* stream) {
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    if (w_dw)
        hipLaunchKernelGGL(pack_dw_i8_kernel, dim3((9 * C + 255) / 256), dim3(256), 0, s,
                           (const int8_t*)w_dw, (int8_t*)dw_dst, C);
    if (w_pw) {
        const int nkt = (K + 63) / 64, nch = (C + 63) / 64;
        if (hipMemcpyAsync(pw_dst, w_pw, (size_t)K * C, hipMemcpyDeviceToDevice, s) != hipSuccess)
            return (int)hipErrorUnknown;
        hipLaunchKernelGGL(pack_pw_i8_kernel, dim3((nkt * nch * 4096 + 255) / 256), dim3(256), 0,
                           s, (const int8_t*)w_pw, (int8_t*)pw_dst + (int64_t)K * C, K, C, nkt,
                           nch);
    }
    return (int)hipGetLastError();
}

#define FCM_V_DWPW(...)
#define FCM_V_DWPW32(...)
#define FCM_V_B2B(...)
#define FCM_V_B2B_MM(...)
#define FCM_V_DWPW_MM(...)
#define FCM_V_DWPW_MMW(...)
#define FCM_V_PWDW_MM(...)
#define FCM_V_DWPW_I8(name, S, OCC, CMAX)                                   \
    template int launch_dwpw_i8<S, OCC, CMAX>(const KArgs&, int, void*); \
    template int occ_dwpw_i8<S, OCC, CMAX>();
#include "../variants.def"
#undef FCM_V_DWPW
#undef FCM_V_DWPW32
#undef FCM_V_B2B
#undef FCM_V_DWPW_MM
#undef FCM_V_B2B_MM
#undef FCM_V_DWPW_MMW
#undef FCM_V_PWDW_MM
#undef FCM_V_DWPW_I8

}  // namespace fcm
