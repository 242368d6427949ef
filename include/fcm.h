/*
 * fcm.h -- C ABI of the MI355X (gfx950) fused convolution module library (libfcm.so).
 *
 * The library runs a depthwise 3x3 convolution and the 1x1 (pointwise) convolution
 * that follows it in ONE kernel, keeping the intermediate feature-map tile on chip
 * (LDS / registers) instead of writing it to HBM: the "Fused Convolutional Module"
 * (FCM) of "Fusing Depthwise and Pointwise Convolutions for Efficient Inference on
 * GPUs" (Sec. III, DWPW case, Fig. 3(b)).  The same family covers the back-to-back
 * pair of a standard 3x3 convolution followed by a 1x1 convolution ("Fusing two
 * back-to-back convolutions", the CONV1/CONV2 example); the second convolution must
 * be 1x1 so that every workgroup's input to it is produced by that workgroup alone
 * (same discussion).  The PW->DW module (the PWDW / PWDW_R fusion case, FCM paper
 * Sec. II-D, Fig. 3(b), and Sec. III) runs the other order: a pointwise layer expands
 * the channels and a depthwise 3x3 layer filters its output, the intermediate again
 * kept on chip; a tile of outputs recomputes the intermediate over its whole input
 * window, the overlap with neighbouring tiles included.  The PW->PW module (the PWPW
 * fusion case, FCM paper Sec. III, Table II) chains two 1x1 layers per pixel.  Each
 * convolution is followed
 * by a per-channel scale, bias and ReLU/ReLU6 epilogue (conv -> normalisation ->
 * activation, FCM paper Sec. III-A).
 * Unfused layer-by-layer entry points, with the same stage code, serve as the
 * baseline the FCM paper compares against (Sec. V-C) and as the fallback when a plan
 * says not to fuse (Sec. IV).
 *
 * Conventions for every entry point:
 *  - Activations are NHWC and densely packed: x[N][H][W][C], y[N][Ho][Wo][K] with
 *    Ho = (H + 2*pad_h - R)/stride_h + 1 (floor), likewise Wo.
 *  - Convolution is cross-correlation (no filter flip) with zero padding.
 *  - Activations and weights share one storage type (fcm_dtype); accumulation and
 *    the epilogue are fp32; each layer's output is rounded to the storage type with
 *    round-to-nearest-even.  FCM_I8 (DWPW only; FCM paper Sec. III-B: int8 operands,
 *    32-bit accumulation, results packed to 8 bits before they are written): exact
 *    int32 sums; each layer's output is v = fmaf(scale, acc, bias) in fp32, clamped to
 *    the activation's range, rounded to the nearest integer (ties to even) and
 *    saturated to [-128, 127].
 *  - Epilogue of a layer with n output channels: out[c] = act(scale[c]*acc[c] +
 *    bias[c]) with fp32 arrays scale[n], bias[n] in device memory; a NULL scale means
 *    1 and a NULL bias means 0.
 *  - All tensor pointers are device pointers owned by the caller; the library never
 *    allocates, frees or retains device memory.  Every device pointer must be 16-byte
 *    aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  *_fwd and
 *    fcm_pack_weights are asynchronous on that stream; they validate every argument
 *    on the host before enqueueing anything, and return a status.
 *  - No function throws or aborts.  On error nothing is enqueued and a description
 *    is available from fcm_last_error() on the calling thread.
 *  - The library is stateless apart from a per-thread error string and a per-process
 *    cache of device properties; concurrent calls from several threads are safe.
 */
#ifndef FCM_H
#define FCM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FCM_PLAN_VERSION 4

typedef enum {
    FCM_OK = 0,
    FCM_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, plan mismatch */
    FCM_ERR_UNSUPPORTED = 2, /* valid problem this library has no kernel for */
    FCM_ERR_HIP = 3          /* a HIP runtime call or kernel launch failed */
} fcm_status;

typedef enum { FCM_F32 = 0, FCM_F16 = 1, FCM_BF16 = 2, FCM_I8 = 3 } fcm_dtype;

typedef enum { FCM_ACT_NONE = 0, FCM_ACT_RELU = 1, FCM_ACT_RELU6 = 2 } fcm_act;

typedef enum {
    FCM_KIND_DWPW = 0, /* depthwise RxS conv (C -> C) then pointwise 1x1 (C -> K) */
    FCM_KIND_B2B = 1,  /* standard RxS conv (C -> K1) then 1x1 conv (K1 -> K) */
    FCM_KIND_PWDW = 2, /* pointwise 1x1 (C -> K1) then depthwise RxS conv (K1 -> K1) */
    FCM_KIND_PWPW = 3, /* pointwise 1x1 (C -> K1) then pointwise 1x1 (K1 -> K); R = S = 1,
                          stride 1, no padding */
    FCM_KIND_PWDWPW = 4 /* the three layers of an inverted-residual block (FCM paper
                          Sec. II-B: PW-DW-PW; Fig. 4): pointwise 1x1 expansion (C -> K1),
                          depthwise RxS conv (K1 -> K1, the stride and padding below),
                          pointwise 1x1 projection (K1 -> K), each with its epilogue, and
                          optionally the block's identity shortcut (`residual`) */
} fcm_kind;

/* The problem, in the pages' terms: NHWC input feature maps, per-channel depthwise
 * filters or a [CRSK]-style standard filter bank, a CxK pointwise filter matrix,
 * stride/padding, and one epilogue per convolution. */
typedef struct {
    int32_t kind;     /* fcm_kind */
    int32_t dtype;    /* fcm_dtype of activations and weights */
    int32_t N, H, W;  /* input batch and spatial extent */
    int32_t C;        /* input channels */
    int32_t K1;       /* B2B: output channels of the first conv.  DWPW: must equal
                         C * mult (the depthwise layer's outputs).  PWDW: output
                         channels of the pointwise layer */
    int32_t K;        /* output channels of the module (PWDW: must equal K1) */
    int32_t R, S;     /* the RxS conv's filter height/width: 3x3 for every module;
                         the DWPW module also takes 5x5 and 7x7 depthwise filters
                         (the combinations compiled into the library; any other is
                         FCM_ERR_UNSUPPORTED) */
    int32_t stride_h, stride_w, pad_h, pad_w; /* of the RxS conv (the first layer for
                         DWPW and B2B, the second for PWDW); the 1x1 is stride 1 */
    int32_t act1, act2; /* fcm_act after the first / second conv */
    /* Generalised depthwise layer of a DWPW module (PyTorch forum "Using optimised
     * depthwise convolutions": a grouped convolution with one group per input
     * channel and k outputs per group, any filter size, and the dilation the
     * thread's separable module gives it).  0 means 1, so a zero-initialised
     * problem is the plain module.
     *  - dil_h, dil_w: spacing of the filter taps; the window of one output spans
     *    (R-1)*dil_h + 1 rows and (S-1)*dil_w + 1 columns, and Ho, Wo follow from
     *    that extent;
     *  - mult: depth multiplier m; the depthwise layer has C*m outputs (K1 must equal
     *    C*m), output channel j reads input channel j / m, depthwise filters are
     *    [C*m][R][S] and pointwise filters [K][C*m].
     * Kernels exist for square R = S in {3, 5, 7}, dil_h = dil_w, 16-bit storage, and
     * the compiled (stride, filter, dilation, multiplier) combinations; other values
     * are FCM_ERR_UNSUPPORTED (plain 3x3 problems keep every kernel listed above).
     * Other kinds require 0 or 1 here (FCM_ERR_INVALID_ARG otherwise). */
    int32_t dil_h, dil_w;
    int32_t mult;
    /* PW->DW->PW module only (other kinds require 0 here, FCM_ERR_INVALID_ARG otherwise):
     *  - act3: fcm_act after the projection's scale/bias (an inverted residual's linear
     *    bottleneck is FCM_ACT_NONE);
     *  - residual: 1 adds the module's input pixel to its output after act3, before the
     *    single rounding to the storage type (the block's identity shortcut); needs
     *    stride 1, K == C and an output extent equal to the input's. */
    int32_t act3;
    int32_t residual;
} fcm_problem;

/* What the planner needs to know about the GPU (FusePlanner's inputs: number of
 * compute units, on-chip memory sizes; FCM paper Sec. IV). */
typedef struct {
    int32_t num_cus;             /* 256 on MI355X */
    int32_t num_xcds;            /* 8 */
    int32_t simds_per_cu;        /* 4 */
    int32_t wave_size;           /* 64 */
    int32_t max_waves_per_simd;  /* 8 */
    int32_t vgprs_per_simd_lane; /* 512 (architectural + accumulation) */
    int32_t lds_bytes_per_cu;    /* 163840 */
    int32_t lds_bytes_per_wg;    /* largest LDS allocation of one workgroup */
    int64_t l2_bytes_per_xcd;    /* 4 MiB */
    double hbm_bytes_per_s;      /* 8.0e12 */
    double mfma_f16_flops;       /* dense fp16/bf16 matrix peak, 2.5e15 */
    double mfma_f32_flops;       /* dense fp32 matrix peak, 157.3e12 */
    double valu_f32_flops;       /* fp32 vector FMA peak without packed math */
} fcm_device_spec;

/* A plan: the problem plus the tiling and launch shape chosen for it.  POD; the
 * caller owns it.  Produced by fcm_plan / fcm_plan_variant, consumed by *_fwd. */
typedef struct {
    int32_t version;        /* FCM_PLAN_VERSION */
    fcm_problem prob;
    int32_t Ho, Wo;
    int32_t variant;        /* index of the fused kernel variant chosen */
    int32_t tile_h, tile_w; /* output pixels of one workgroup tile */
    int32_t k_tile;         /* output channels of one workgroup tile */
    int32_t c_chunk;        /* input channels staged in LDS per pass */
    int32_t waves_per_wg;
    int32_t wgs_per_cu;     /* occupancy the LDS/VGPR budgets allow */
    int32_t num_tiles;      /* pixel tiles x K tiles */
    int32_t grid;           /* workgroups launched (persistent kernels loop) */
    int32_t lds_bytes;      /* LDS of one workgroup */
    int32_t fuse;           /* 1: the fused module's modelled HBM bytes (compulsory
                               bytes, filters once per XCD) are below the layer-by-layer
                               kernels'; the Eq. 1-4 figures are gma_paper_* */
    int64_t w1_packed_bytes, w2_packed_bytes; /* sizes fcm_pack_weights writes */
    int64_t workspace_bytes;  /* intermediate tensor of the unfused path */
    int64_t alg_bytes_fused;  /* compulsory HBM bytes: X + Y + weights + epilogue */
    int64_t alg_bytes_unfused;/* ... + intermediate written and read back */
    int64_t pred_bytes_fused;   /* bytes the chosen tiling requests from L2 */
    int64_t pred_bytes_unfused; /* same for the layer-by-layer kernels */
    double gma_paper_fused;   /* FusePlanner estimate (Eq. 1-4 style), bytes */
    double gma_paper_unfused; /* Eq. 2 + Eq. 3, bytes */
    double flops;             /* 2 * multiply-adds of both convolutions */
    double pred_us_fused;     /* time model of the chosen variant, us: a fixed launch
                                 cost plus its slowest roofline term at the fraction of
                                 peak the kernels reach (calibrated on MI355X) */
    double tuned_us;          /* fcm_tune: measured time of this plan, us (0 otherwise) */
} fcm_plan_t;

/* MI355X published figures; no HIP call (usable without a GPU). */
fcm_status fcm_default_device_spec(fcm_device_spec* out);

/* Properties of HIP device `device` (CU count, LDS sizes) over the MI355X defaults.
 * Returns FCM_ERR_HIP if the device cannot be queried. */
fcm_status fcm_query_device_spec(int device, fcm_device_spec* out);

/* FusePlanner for gfx950 (FCM paper Sec. IV): validates the problem, enumerates the
 * compiled kernel variants whose tiles fit the LDS and register budgets, estimates
 * each one's memory traffic and, since a gfx950 workgroup can also be bound by its
 * matrix or vector units, a roofline time (the slowest of HBM, on-chip traffic,
 * matrix and vector work including recomputation); keeps the fastest; and decides
 * with the pages' rule (fewer estimated global memory accesses) whether fusing
 * beats the layer-by-layer kernels.  spec == NULL uses the MI355X defaults.
 * Host only; makes no HIP call.  Errors: INVALID_ARG (null pointer, non-positive
 * size, K1 != C for DWPW, K != K1 for PWDW, padding >= filter, act3 or residual set for
 * a kind other than PWDWPW, a shortcut whose shapes do not match), UNSUPPORTED (filter
 * not 3x3, stride not 1 or 2, padding not 0 or 1, a channel count not a multiple of 8,
 * fp32 storage for B2B, PWDW or PWDWPW, int8 storage other than DWPW or with C or K
 * not a multiple of 16, or no variant fits). */
fcm_status fcm_plan(const fcm_problem* prob, const fcm_device_spec* spec, fcm_plan_t* out);

/* Same, but with the fused kernel variant forced (for tests and on-device tuning).
 * UNSUPPORTED if that variant cannot run the problem. */
fcm_status fcm_plan_variant(const fcm_problem* prob, const fcm_device_spec* spec,
                            int32_t variant, fcm_plan_t* out);

/* Measured selection (the profiling step of the TVM conv2d profiler page: every
 * candidate kernel is compiled once, run on the device, and the fastest is kept).
 * Runs every fused variant able to take `prob`, at persistent grids of 1, 2, 3 and 4
 * workgroups per CU (as far as its occupancy allows), `iters` times each on `stream`,
 * rotating over `nsets` input/output pairs x[i], y[i] (laid out as for fcm_dwpw_fwd /
 * fcm_b2b_conv_fwd / fcm_pwdw_fwd, with w1, w2 the first and second layer's packed
 * filters and scale1/bias1, scale2/bias2 their epilogues; several pairs whose total exceeds the 256 MB Infinity Cache make
 * the candidates stream from HBM as in a real network) with the shared filters and
 * epilogue arrays (weights packed by fcm_pack_weights); every y[i] is overwritten.
 * Writes the plan of the fastest to *out, with out->grid the chosen grid and
 * out->tuned_us its mean time per call.  Synchronises `stream`.  Allocates no device
 * memory.  Errors: FCM_ERR_INVALID_ARG / FCM_ERR_UNSUPPORTED as fcm_plan and the *_fwd
 * calls (also for nsets < 1 or NULL arrays); FCM_ERR_HIP if a launch or an event fails. */
fcm_status fcm_tune(const fcm_problem* prob, const fcm_device_spec* spec, int32_t nsets,
                    const void* const* x, const void* w1, const float* scale1,
                    const float* bias1, const void* w2, const float* scale2,
                    const float* bias2, void* const* y, void* stream, int32_t iters,
                    fcm_plan_t* out);

/* A layer of a chain (a linear network of depthwise and pointwise layers, MobileNet-style;
 * FCM paper Sec. IV, Fig. 4): shapes only. */
typedef enum { FCM_LAYER_DW = 0, FCM_LAYER_PW = 1 } fcm_layer_type;
typedef struct {
    int32_t type;   /* fcm_layer_type: depthwise 3x3 (padding 1) or pointwise 1x1 */
    int32_t C, K;   /* input / output channels (depthwise: K == C) */
    int32_t stride; /* depthwise: 1 or 2; pointwise: 1 */
    int32_t act;    /* fcm_act after the layer's scale/bias */
} fcm_layer;

/* One group of the chain's schedule: a single layer run by itself, or two consecutive
 * layers run as one fused module. */
typedef struct {
    int32_t first;   /* index of the group's first layer */
    int32_t count;   /* 1 (layer by layer) or 2 (a fused module) */
    int32_t kind;    /* fcm_kind of the module; -1 for a single layer */
    int32_t variant; /* the module's planned kernel variant; -1 for a single layer */
    double gma;      /* estimated global memory accesses of the group, bytes */
} fcm_chain_group;

/* FusePlanner over a chain (FCM paper Sec. IV): for each pair of consecutive layers that
 * forms a module with a kernel here (DW->PW, PW->DW, PW->PW; the pair's plan must be
 * feasible), the fused estimate of fcm_plan (Eq. 4 style) competes with the two layers'
 * layer-by-layer estimates (Eq. 3 for a depthwise layer, Eq. 2 for a pointwise layer, with
 * the baseline kernels' tilings); a dynamic program over the chain picks the partition into
 * single layers and fused pairs with the fewest estimated accesses (ties: fewer groups).
 * The chain's input is N x H x W with layers[0].C channels; a layer's output extent is the
 * next layer's input.  groups (capacity n) receives the schedule in order, *ngroups its
 * length, *gma_chain its total and *gma_layer_by_layer the total with every layer alone.
 * spec == NULL uses the MI355X defaults.  Host only.  Errors: INVALID_ARG (NULL outputs,
 * n < 1, consecutive layers whose channel counts do not chain, a depthwise layer with
 * K != C), UNSUPPORTED (a layer the library could not run alone: see fcm_plan). */
fcm_status fcm_plan_chain(const fcm_layer* layers, int32_t n, int32_t N, int32_t H, int32_t W,
                          int32_t dtype, const fcm_device_spec* spec, fcm_chain_group* groups,
                          int32_t* ngroups, double* gma_chain, double* gma_layer_by_layer);

/* Number of fused kernel variants compiled into the library, and a short name for
 * one of them ("" if out of range). */
int32_t fcm_num_variants(void);
const char* fcm_variant_name(int32_t variant);

/* Offline weight packing ("weights are packed offline since they do not change in
 * inference", FCM paper Sec. III-B): converts PyTorch-layout filters into the
 * layouts the kernels read.
 *   DWPW: w1_src depthwise [C][R][S]      -> w1_dst [R*S][C]      (channel fastest)
 *         w2_src pointwise [K][C]         -> w2_dst [K][C]        (copied as is), and for
 *                                            fp16/bf16 followed by the same filters in
 *                                            32x32 blocks in matrix-operand order (K and C
 *                                            rounded up to multiples of 32, zero filled)
 *   B2B:  w1_src standard  [K1][C][R][S]  -> w1_dst [K1][R*S][C]  (channel fastest), and
 *                                            for fp16/bf16 followed by the same filters in
 *                                            16x32 blocks in matrix-operand order (K1
 *                                            rounded up to 16, C to 64, zero filled)
 *         w2_src 1x1       [K][K1]        -> w2_dst [K][K1], and for fp16/bf16 followed by
 *                                            32x32 blocks as for DWPW
 *   DWPW in FCM_I8: w1 as above; w2 [K][C] copied, then 64 x 64 blocks (K tile of 64
 *         output channels, four 16-row operands) in the int8 matrix-operand order
 *         (K rounded up to 64, C <= 64, zero filled)
 *   PWPW: w1_src [K1][C] copied as is; w2_src [K][K1] copied, then blocked as for DWPW
 *   PWDW: w1_src pointwise [K1][C]        -> w1_dst [K1][C]       (copied as is)
 *         w2_src depthwise [K1][R][S]     -> w2_dst [R*S][K1]     (channel fastest)
 *   PWDWPW: w1 and w2 as for PWDW; the projection's [K][K1] filters are read as
 *         PyTorch stores them ([K][K1][1][1]), with no packing
 * Sizes in bytes are plan->w1_packed_bytes / w2_packed_bytes.  Either pair may be
 * NULL to skip it.  Source and destination must not overlap. */
fcm_status fcm_pack_weights(const fcm_plan_t* plan, const void* w1_src, void* w1_dst,
                            const void* w2_src, void* w2_dst, void* stream);

/* Fused DW -> PW module (FCM DWPW).  x: [N][H][W][C]; w_dw: packed [R*S][C];
 * w_pw: as fcm_pack_weights writes it (plan->w2_packed_bytes: [K][C], then for fp16/bf16
 * the blocked copy); scale1/bias1: [C] or NULL; scale2/bias2: [K] or NULL;
 * y: [N][Ho][Wo][K].  plan->prob.kind must be FCM_KIND_DWPW. */
fcm_status fcm_dwpw_fwd(const fcm_plan_t* plan, const void* x, const void* w_dw,
                        const float* scale1, const float* bias1, const void* w_pw,
                        const float* scale2, const float* bias2, void* y, void* stream);

/* Fused standard 3x3 conv -> 1x1 conv (back-to-back).  x: [N][H][W][C];
 * w1, w2: as fcm_pack_weights writes them (plan->w1_packed_bytes / w2_packed_bytes: the
 * plain [K1][R*S][C] and [K][K1] arrays, then for fp16/bf16 their blocked copies);
 * scale1/bias1: [K1] or NULL;
 * scale2/bias2: [K] or NULL; y: [N][Ho][Wo][K].  plan->prob.kind must be
 * FCM_KIND_B2B. */
fcm_status fcm_b2b_conv_fwd(const fcm_plan_t* plan, const void* x, const void* w1,
                            const float* scale1, const float* bias1, const void* w2,
                            const float* scale2, const float* bias2, void* y,
                            void* stream);

/* Fused PW -> DW module (FCM PWDW_R; PWDW when one tile covers the plane).
 * x: [N][H][W][C]; w_pw: packed [K1][C]; scale1/bias1: [K1] or NULL (epilogue of the
 * pointwise layer); w_dw: packed [R*S][K1]; scale2/bias2: [K1] or NULL (epilogue of the
 * depthwise layer); y: [N][Ho][Wo][K1].  The depthwise layer's zero padding surrounds
 * the intermediate.  plan->prob.kind must be FCM_KIND_PWDW. */
fcm_status fcm_pwdw_fwd(const fcm_plan_t* plan, const void* x, const void* w_pw,
                        const float* scale1, const float* bias1, const void* w_dw,
                        const float* scale2, const float* bias2, void* y, void* stream);

/* Fused PW -> PW module (FCM PWPW).  x: [N][H][W][C]; w1: packed [K1][C] (copied as
 * is); scale1/bias1: [K1] or NULL; w2: packed [K][K1], then for fp16/bf16 its blocked
 * copy (as for DWPW's pointwise filters); scale2/bias2: [K] or NULL; y: [N][H][W][K].
 * plan->prob.kind must be FCM_KIND_PWPW. */
fcm_status fcm_pwpw_fwd(const fcm_plan_t* plan, const void* x, const void* w1,
                        const float* scale1, const float* bias1, const void* w2,
                        const float* scale2, const float* bias2, void* y, void* stream);

/* Fused PW -> DW -> PW module (the inverted-residual block).  x: [N][H][W][C];
 * w1: packed [K1][C] expansion filters; scale1/bias1: [K1] or NULL; w2: packed
 * [R*S][K1] depthwise filters; scale2/bias2: [K1] or NULL; w3: [K][K1] projection
 * filters (PyTorch layout, not packed); scale3/bias3: [K] or NULL; y: [N][Ho][Wo][K].
 * With plan->prob.residual the input pixel is added after epilogue 3 (x must then also
 * be the shortcut: stride 1, K == C).  The two intermediates stay on chip.  All tensor
 * pointers 16-byte aligned, epilogue arrays 4-byte aligned; y must not overlap x.
 * plan->prob.kind must be FCM_KIND_PWDWPW.  Errors: INVALID_ARG (plan/pointer checks),
 * HIP (launch failure). */
fcm_status fcm_pwdwpw_fwd(const fcm_plan_t* plan, const void* x, const void* w1,
                          const float* scale1, const float* bias1, const void* w2,
                          const float* scale2, const float* bias2, const void* w3,
                          const float* scale3, const float* bias3, void* y, void* stream);

/* Layer-by-layer baseline of the PW -> DW -> PW module: the pointwise kernel writes the
 * expansion t1: [N][H][W][K1], the depthwise kernel reads it and writes t2:
 * [N][Ho][Wo][K1], the pointwise kernel reads t2 and writes y (adding x for the
 * shortcut).  t1 and t2 are caller buffers (plan->workspace_bytes in total: t1's bytes
 * then t2's).  Same arguments and errors as fcm_pwdwpw_fwd otherwise. */
fcm_status fcm_pwdwpw_lbl(const fcm_plan_t* plan, const void* x, const void* w1,
                          const float* scale1, const float* bias1, const void* w2,
                          const float* scale2, const float* bias2, const void* w3,
                          const float* scale3, const float* bias3, void* t1, void* t2, void* y,
                          void* stream);

/* Largest workspace (plan->workspace_bytes) fcm_pwdwpw_lbl_noalloc takes: 32 MiB. */
#define FCM_NOALLOC_SCRATCH_BYTES (32ll << 20)

/* fcm_pwdwpw_lbl for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same three kernels,
 * with t1 and t2 placed in a static device array of FCM_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends (t1's bytes, then t2's).
 * Allocates nothing.  Every call on one GPU shares that array, so calls that overlap on
 * one GPU (two streams, or two host threads) race; calls in one stream are ordered.
 * Nothing in the array needs clearing: each call writes t1 and t2 whole before reading
 * them.  Same arguments as fcm_pwdwpw_lbl without t1 and t2.  Errors: INVALID_ARG
 * (plan/pointer checks), UNSUPPORTED (plan->workspace_bytes above
 * FCM_NOALLOC_SCRATCH_BYTES), HIP (device query, symbol address or launch failure). */
fcm_status fcm_pwdwpw_lbl_noalloc(const fcm_plan_t* plan, const void* x, const void* w1,
                                  const float* scale1, const float* bias1, const void* w2,
                                  const float* scale2, const float* bias2, const void* w3,
                                  const float* scale3, const float* bias3, void* y,
                                  void* stream);

/* fcm_tune for the PW -> DW -> PW module: every fused variant able to take `prob`
 * (kind FCM_KIND_PWDWPW) at each persistent grid, timed over the nsets pairs x[i], y[i]
 * with the three layers' filters and epilogues as fcm_pwdwpw_fwd takes them.  Writes
 * the fastest plan to *out (out->tuned_us its mean time per call); synchronises
 * `stream`; allocates no device memory.  Errors as fcm_tune. */
fcm_status fcm_tune_pwdwpw(const fcm_problem* prob, const fcm_device_spec* spec, int32_t nsets,
                           const void* const* x, const void* w1, const float* scale1,
                           const float* bias1, const void* w2, const float* scale2,
                           const float* bias2, const void* w3, const float* scale3,
                           const float* bias3, void* const* y, void* stream, int32_t iters,
                           fcm_plan_t* out);

/* Layer-by-layer baseline, first layer of a DWPW plan: depthwise conv + epilogue 1,
 * writing the intermediate t: [N][Ho][Wo][C] (plan->workspace_bytes bytes).
 * For a PWDW plan: the second layer, depthwise conv + epilogue (scale/bias [K1]) over
 * the intermediate x = t: [N][H][W][K1], writing y: [N][Ho][Wo][K1]. */
fcm_status fcm_dw_fwd(const fcm_plan_t* plan, const void* x, const void* w_dw,
                      const float* scale1, const float* bias1, void* t, void* stream);

/* Layer-by-layer baseline, second layer of a DWPW or B2B plan: 1x1 conv + epilogue 2
 * reading the intermediate t: [N][Ho][Wo][C or K1], writing y: [N][Ho][Wo][K].
 * For a PWDW plan: the first layer, 1x1 conv + epilogue (scale/bias [K1]) over the
 * input t = x: [N][H][W][C] with the packed [K1][C] filters, writing the intermediate
 * y: [N][H][W][K1] (plan->workspace_bytes bytes). */
fcm_status fcm_pw_fwd(const fcm_plan_t* plan, const void* t, const void* w_pw,
                      const float* scale2, const float* bias2, void* y, void* stream);

/* Layer-by-layer baseline, first layer of a B2B plan: standard conv + epilogue 1,
 * writing t: [N][Ho][Wo][K1].  For a PWPW plan: the first 1x1 layer + epilogue 1 with the
 * packed [K1][C] filters, writing t: [N][H][W][K1] (the second layer is fcm_pw_fwd). */
fcm_status fcm_conv_fwd(const fcm_plan_t* plan, const void* x, const void* w1,
                        const float* scale1, const float* bias1, void* t, void* stream);

/* Static description of a status code, and the calling thread's last error detail
 * (empty after a successful call). */
const char* fcm_status_str(fcm_status s);
const char* fcm_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FCM_H */
