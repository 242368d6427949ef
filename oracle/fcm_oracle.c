/*
 * fcm_oracle.c -- CPU oracle for the fused depthwise->pointwise convolution module
 * (FCM) and the back-to-back 3x3 -> 1x1 convolution pair.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this
 * file: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use it.
 * It shares no code, header, table or helper with the HIP library.
 *
 * What it computes is the plain, unfused definition, evaluated in double precision
 * with direct loops in a fixed order:
 *
 *   depthwise conv   -- one filter per channel slid over height and width
 *                       ("Fusing Depthwise and Pointwise Convolutions for Efficient
 *                       Inference on GPUs", Sec. II-B, Fig. 2);
 *   pointwise conv   -- a 1x1 filter spanning all channels (same section);
 *   PW -> DW module  -- the pointwise layer first, then the depthwise layer over its
 *                       output (the PWDW / PWDW_R fusion cases, FCM paper Sec. II-D,
 *                       Fig. 3(b), and Sec. III); the depthwise layer's zero padding
 *                       pads the intermediate, not the module's input;
 *   PW -> PW module  -- two pointwise layers (the PWPW fusion case, FCM paper Sec. III,
 *                       Table II): pixel by pixel, so a tile needs no halo;
 *   PW -> DW -> PW   -- the three convolutional layers of an inverted-residual block
 *                       (FCM paper Sec. II-B, Fig. 4): the PW -> DW module followed by
 *                       a third, pointwise layer; with the block's identity shortcut
 *                       the input pixel is added after the third layer's activation,
 *                       before its one rounding;
 *   generalised DW   -- any R x S filter, a dilation and a depth multiplier m (PyTorch
 *                       forum "Using optimised depthwise convolutions": a grouped
 *                       convolution with one group per input channel and k outputs per
 *                       group, dilated in the thread's separable module); output
 *                       channel j reads input channel j / m;
 *   standard conv    -- the first layer of the back-to-back pair, [N,H,W,C] x
 *                       [K,C,R,S] ("Fusing two back-to-back convolutions", the
 *                       CONV1/CONV2 example);
 *   epilogue         -- conv -> normalisation -> activation, i.e. a per-channel
 *                       scale and bias followed by ReLU or ReLU6 (FCM paper Sec. III-A
 *                       "up to 6 layers"; the CUTLASS discussion's scale_bias_relu);
 *   storage rounding -- each layer's output is rounded to the storage type before the
 *                       next layer reads it, exactly as a layer-by-layer execution
 *                       that writes its output feature maps to memory would do (FCM
 *                       paper Sec. II-D, Fig. 3(a)).  Fusion changes where the
 *                       intermediate lives, not its value.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - cross-correlation (no filter flip), as PyTorch's nn.Conv2d used on the forum
 *     page ("Using optimised depthwise convolutions", SeparableConv2d listing);
 *   - zero padding; output size floor((H + 2p - R)/s) + 1;
 *   - epilogue y = act(scale[c]*acc + bias[c]); a NULL scale means 1, a NULL bias 0;
 *   - rounding to binary16 / bfloat16 / binary32 is IEEE round-to-nearest-even,
 *     implemented below from the format definitions (not with a library cast);
 *   - INT8 storage (FCM paper Sec. III-B: int8 operands, four-way int8 dot products
 *     with 32-bit accumulation, results packed to 8 bits before they are written):
 *     the sums are exact integers; the epilogue is evaluated in binary32 -- one fused
 *     multiply-add v = fmaf(scale, acc, bias), the activation's clamp -- and v is
 *     rounded to the nearest integer (ties to even) and saturated to [-128, 127].
 *     Because a floating-point step decides an integer code here, the oracle takes it
 *     in the same precision as the kernels (binary32 FMA, then round-to-nearest-even).
 *
 * Layouts (PyTorch's, independent of the GPU library's packed layouts):
 *   activations NHWC [N][H][W][C]; depthwise weights [C][R][S]; pointwise weights
 *   [K][C]; standard conv weights [K][C][R][S].
 *
 * Parallelism: an OpenMP loop over output rows; every output element is still a
 * sequential sum in a fixed order, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the OpenMP loops below use (1 without OpenMP). */
int fcm_oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the threads later OpenMP loops use (for timing the checker on one core). */
void fcm_oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

#define ORACLE_F32 0
#define ORACLE_F16 1
#define ORACLE_BF16 2
#define ORACLE_I8 3

#define ACT_NONE 0
#define ACT_RELU 1
#define ACT_RELU6 2

/* ------------------------------------------------------------------------------ */
/* IEEE-754 round-to-nearest-even into a binary format with `mant` explicit       */
/* fraction bits and exponent range [emin, emax].  binary16: (10, -14, 15);       */
/* bfloat16: (7, -126, 127); binary32: (23, -126, 127).  Works on the value: the  */
/* representable numbers near |v| are integer multiples of the quantum            */
/* 2^(max(e, emin) - mant) where 2^e <= |v| < 2^(e+1); subnormals share the       */
/* quantum of the smallest normal binade.                                           */
/* ------------------------------------------------------------------------------ */
static double round_binary(double v, int mant, int emin, int emax) {
    if (v != v || v == 0.0 || isinf(v)) return v;
    double a = fabs(v);
    int e2;
    frexp(a, &e2);          /* a = f * 2^e2 with f in [0.5, 1)  =>  2^(e2-1) <= a */
    int e = e2 - 1;
    if (e < emin) e = emin;
    double quantum = ldexp(1.0, e - mant);
    double n = a / quantum; /* exact: scaling by a power of two */
    double fl = floor(n);
    double rem = n - fl;    /* exact */
    if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    double r = fl * quantum;
    double max_finite = ldexp(2.0 - ldexp(1.0, -mant), emax);
    if (r > max_finite) r = INFINITY;
    return copysign(r, v);
}

/* Nearest int8 code: round to the nearest integer, ties to even, then saturate. */
static double round_i8(double v) {
    double r = rint(v); /* default rounding mode: to nearest, ties to even */
    if (r < -128.0) r = -128.0;
    if (r > 127.0) r = 127.0;
    return r;
}

double fcm_oracle_round(double v, int dtype) {
    switch (dtype) {
    case ORACLE_F16: return round_binary(v, 10, -14, 15);
    case ORACLE_BF16: return round_binary(v, 7, -126, 127);
    case ORACLE_I8: return round_i8(v);
    default: return round_binary(v, 23, -126, 127);
    }
}

void fcm_oracle_round_array(double* a, int64_t n, int dtype) {
    for (int64_t i = 0; i < n; ++i) a[i] = fcm_oracle_round(a[i], dtype);
}

/* Bit pattern of the binary16 / bfloat16 value nearest to v (RNE).  Built from the
 * rounded value: sign, biased exponent, fraction. */
static uint16_t encode16(double v, int mant, int emin, int bias) {
    double r = (mant == 10) ? round_binary(v, 10, -14, 15) : round_binary(v, 7, -126, 127);
    uint16_t sign = (uint16_t)(signbit(r) ? 0x8000u : 0u);
    int ebits = 15 - mant;
    uint16_t exp_all = (uint16_t)(((1u << ebits) - 1u) << mant);
    if (r != r) return (uint16_t)(exp_all | (1u << (mant - 1)));
    double a = fabs(r);
    if (isinf(a)) return (uint16_t)(sign | exp_all);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);
    int e = e2 - 1;
    if (e < emin) { /* subnormal: a = frac * 2^(emin - mant) */
        uint16_t frac = (uint16_t)ldexp(a, mant - emin);
        return (uint16_t)(sign | frac);
    }
    uint16_t frac = (uint16_t)(ldexp(a, mant - e) - ldexp(1.0, mant));
    return (uint16_t)(sign | ((uint16_t)(e + bias) << mant) | frac);
}

uint16_t fcm_oracle_f16_bits(double v) { return encode16(v, 10, -14, 15); }
uint16_t fcm_oracle_bf16_bits(double v) { return encode16(v, 7, -126, 127); }

/* ------------------------------------------------------------------------------ */
/* Layers                                                                           */
/* ------------------------------------------------------------------------------ */
static int out_size(int in, int pad, int filt, int stride) {
    return (in + 2 * pad - filt) / stride + 1;
}

/* Depthwise convolution: t[n][oh][ow][c] = sum_{r,s} x[n][ih][iw][c] * w[c][r][s],
 * ih = oh*sh - ph + r, iw = ow*sw - pw + s, x = 0 outside the image. */
void fcm_oracle_dw(const double* x, int N, int H, int W, int C, const double* w, int R,
                   int S, int sh, int sw, int ph, int pw, double* t) {
    int Ho = out_size(H, ph, R, sh), Wo = out_size(W, pw, S, sw);
#pragma omp parallel for collapse(2) schedule(static)
    for (int n = 0; n < N; ++n)
        for (int oh = 0; oh < Ho; ++oh)
            for (int ow = 0; ow < Wo; ++ow)
                for (int c = 0; c < C; ++c) {
                    double acc = 0.0;
                    for (int r = 0; r < R; ++r)
                        for (int s = 0; s < S; ++s) {
                            int ih = oh * sh - ph + r, iw = ow * sw - pw + s;
                            if (ih < 0 || ih >= H || iw < 0 || iw >= W) continue;
                            acc += x[(((int64_t)n * H + ih) * W + iw) * C + c] *
                                   w[((int64_t)c * R + r) * S + s];
                        }
                    t[(((int64_t)n * Ho + oh) * Wo + ow) * C + c] = acc;
                }
}

/* Pointwise (1x1) convolution over M = N*H*W pixels: y[m][k] = sum_c t[m][c]*w[k][c]. */
static void pw_row(const double* t, int C, const double* w, int K, double* y);
void fcm_oracle_pw(const double* t, int64_t M, int C, const double* w, int K, double* y) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) pw_row(t + m * C, C, w, K, y + m * K);
}

/* Standard convolution: y[n][oh][ow][k] = sum_{c,r,s} x[n][ih][iw][c] * w[k][c][r][s]. */
void fcm_oracle_conv(const double* x, int N, int H, int W, int C, const double* w, int K,
                     int R, int S, int sh, int sw, int ph, int pw, double* y) {
    int Ho = out_size(H, ph, R, sh), Wo = out_size(W, pw, S, sw);
#pragma omp parallel for collapse(2) schedule(static)
    for (int n = 0; n < N; ++n)
        for (int oh = 0; oh < Ho; ++oh)
            for (int ow = 0; ow < Wo; ++ow)
                for (int k = 0; k < K; ++k) {
                    double acc = 0.0;
                    for (int c = 0; c < C; ++c)
                        for (int r = 0; r < R; ++r)
                            for (int s = 0; s < S; ++s) {
                                int ih = oh * sh - ph + r, iw = ow * sw - pw + s;
                                if (ih < 0 || ih >= H || iw < 0 || iw >= W) continue;
                                acc += x[(((int64_t)n * H + ih) * W + iw) * C + c] *
                                       w[(((int64_t)k * C + c) * R + r) * S + s];
                            }
                    y[(((int64_t)n * Ho + oh) * Wo + ow) * K + k] = acc;
                }
}

/* Per-channel normalisation + activation of one pixel's C values, in place. */
static void epilogue_row(double* a, int C, const double* scale, const double* bias, int act) {
    for (int c = 0; c < C; ++c) {
        double v = a[c];
        if (scale) v = scale[c] * v;
        if (bias) v = v + bias[c];
        if (act == ACT_RELU || act == ACT_RELU6) v = v > 0.0 ? v : 0.0;
        if (act == ACT_RELU6) v = v < 6.0 ? v : 6.0;
        a[c] = v;
    }
}

/* One pixel of the pointwise conv: y[k] = sum_c t[c] * w[k][c]. */
static void pw_row(const double* t, int C, const double* w, int K, double* y) {
    for (int k = 0; k < K; ++k) {
        double acc = 0.0;
        for (int c = 0; c < C; ++c) acc += t[c] * w[(int64_t)k * C + c];
        y[k] = acc;
    }
}

/* One pixel's C values leave a layer: normalisation + activation, then rounding to the
 * storage type.  Floating-point storage: the epilogue in double precision, one rounding.
 * INT8: the epilogue in binary32 (fmaf, clamp), then the nearest int8 code. */
static void store_row(double* a, int C, const double* scale, const double* bias, int act,
                      int dtype) {
    if (dtype != ORACLE_I8) {
        epilogue_row(a, C, scale, bias, act);
        fcm_oracle_round_array(a, C, dtype);
        return;
    }
    for (int c = 0; c < C; ++c) {
        float acc = (float)a[c]; /* exact: |acc| < 2^24 for int8 operands */
        float sc = scale ? (float)scale[c] : 1.0f;
        float bi = bias ? (float)bias[c] : 0.0f;
        float v = fmaf(sc, acc, bi);
        if (act == ACT_RELU || act == ACT_RELU6) v = v > 0.0f ? v : 0.0f;
        if (act == ACT_RELU6) v = v < 6.0f ? v : 6.0f;
        a[c] = round_i8((double)v);
    }
}

static void store_rows(double* a, int64_t M, int C, const double* scale, const double* bias,
                       int act, int dtype) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) store_row(a + m * C, C, scale, bias, act, dtype);
}

/* Per-channel normalisation + activation in place over a [M][C] array. */
void fcm_oracle_epilogue(double* a, int64_t M, int C, const double* scale,
                         const double* bias, int act) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) epilogue_row(a + m * C, C, scale, bias, act);
}

/* ------------------------------------------------------------------------------ */
/* The two modules, layer by layer.  t_out (optional) receives the rounded          */
/* intermediate that a layer-by-layer execution would store.  Returns 0, or -1 if   */
/* memory for the intermediate could not be obtained.                               */
/* ------------------------------------------------------------------------------ */
int fcm_oracle_dwpw(const double* x, int N, int H, int W, int C, const double* w_dw,
                    int R, int S, int sh, int sw, int ph, int pw, const double* scale1,
                    const double* bias1, int act1, const double* w_pw, int K,
                    const double* scale2, const double* bias2, int act2, int dtype,
                    double* t_out, double* y) {
    int Ho = out_size(H, ph, R, sh), Wo = out_size(W, pw, S, sw);
    int64_t M = (int64_t)N * Ho * Wo;
    double* t = t_out ? t_out : (double*)malloc(sizeof(double) * (size_t)(M * C));
    if (!t) return -1;
    fcm_oracle_dw(x, N, H, W, C, w_dw, R, S, sh, sw, ph, pw, t);
    store_rows(t, M, C, scale1, bias1, act1, dtype);
    fcm_oracle_pw(t, M, C, w_pw, K, y);
    store_rows(y, M, K, scale2, bias2, act2, dtype);
    if (!t_out) free(t);
    return 0;
}

int fcm_oracle_b2b(const double* x, int N, int H, int W, int C, const double* w1, int K1,
                   int R, int S, int sh, int sw, int ph, int pw, const double* scale1,
                   const double* bias1, int act1, const double* w2, int K,
                   const double* scale2, const double* bias2, int act2, int dtype,
                   double* t_out, double* y) {
    int Ho = out_size(H, ph, R, sh), Wo = out_size(W, pw, S, sw);
    int64_t M = (int64_t)N * Ho * Wo;
    double* t = t_out ? t_out : (double*)malloc(sizeof(double) * (size_t)(M * K1));
    if (!t) return -1;
    fcm_oracle_conv(x, N, H, W, C, w1, K1, R, S, sh, sw, ph, pw, t);
    fcm_oracle_epilogue(t, M, K1, scale1, bias1, act1);
    fcm_oracle_round_array(t, M * K1, dtype);
    fcm_oracle_pw(t, M, K1, w2, K, y);
    store_rows(y, M, K, scale2, bias2, act2, dtype);
    if (!t_out) free(t);
    return 0;
}

/* Same modules evaluated only at a list of output pixels (n, oh, ow), for checks at
 * full size where the whole output is not needed: y_rows[i][k] for pixel i.  The
 * intermediate at one pixel depends only on that pixel's input window, so each
 * sampled row is computed from scratch by the definitions above. */
int fcm_oracle_dwpw_at(const double* x, int N, int H, int W, int C, const double* w_dw,
                       int R, int S, int sh, int sw, int ph, int pw, const double* scale1,
                       const double* bias1, int act1, const double* w_pw, int K,
                       const double* scale2, const double* bias2, int act2, int dtype,
                       const int32_t* pix /* [P][3] */, int64_t P, double* y_rows) {
    (void)N;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < P; ++i) {
        int n = pix[3 * i], oh = pix[3 * i + 1], ow = pix[3 * i + 2];
        double* t = (double*)malloc(sizeof(double) * (size_t)C);
        if (!t) continue;
        for (int c = 0; c < C; ++c) {
            double acc = 0.0;
            for (int r = 0; r < R; ++r)
                for (int s = 0; s < S; ++s) {
                    int ih = oh * sh - ph + r, iw = ow * sw - pw + s;
                    if (ih < 0 || ih >= H || iw < 0 || iw >= W) continue;
                    acc += x[(((int64_t)n * H + ih) * W + iw) * C + c] *
                           w_dw[((int64_t)c * R + r) * S + s];
                }
            t[c] = acc;
        }
        store_row(t, C, scale1, bias1, act1, dtype);
        double* yr = y_rows + i * K;
        pw_row(t, C, w_pw, K, yr);
        store_row(yr, K, scale2, bias2, act2, dtype);
        free(t);
    }
    return 0;
}

int fcm_oracle_b2b_at(const double* x, int N, int H, int W, int C, const double* w1,
                      int K1, int R, int S, int sh, int sw, int ph, int pw,
                      const double* scale1, const double* bias1, int act1, const double* w2,
                      int K, const double* scale2, const double* bias2, int act2, int dtype,
                      const int32_t* pix, int64_t P, double* y_rows) {
    (void)N;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < P; ++i) {
        int n = pix[3 * i], oh = pix[3 * i + 1], ow = pix[3 * i + 2];
        double* t = (double*)malloc(sizeof(double) * (size_t)K1);
        if (!t) continue;
        for (int k1 = 0; k1 < K1; ++k1) {
            double acc = 0.0;
            for (int c = 0; c < C; ++c)
                for (int r = 0; r < R; ++r)
                    for (int s = 0; s < S; ++s) {
                        int ih = oh * sh - ph + r, iw = ow * sw - pw + s;
                        if (ih < 0 || ih >= H || iw < 0 || iw >= W) continue;
                        acc += x[(((int64_t)n * H + ih) * W + iw) * C + c] *
                               w1[(((int64_t)k1 * C + c) * R + r) * S + s];
                    }
            t[k1] = acc;
        }
        epilogue_row(t, K1, scale1, bias1, act1);
        fcm_oracle_round_array(t, K1, dtype);
        double* yr = y_rows + i * K;
        pw_row(t, K1, w2, K, yr);
        store_row(yr, K, scale2, bias2, act2, dtype);
        free(t);
    }
    return 0;
}


/* PW -> DW module, layer by layer (FCM paper Sec. II-D, Fig. 3(b), PWDW_R):
 *   t = round(act1(scale1 * (x . w_pw^T) + bias1))   over every input pixel,
 *   y = round(act2(scale2 * dw(t, w_dw) + bias2)),
 * w_pw [K1][C], w_dw [K1][R][S]; the depthwise layer's padding is zeros around t. */
int fcm_oracle_pwdw(const double* x, int N, int H, int W, int C, const double* w_pw, int K1,
                    const double* scale1, const double* bias1, int act1, const double* w_dw,
                    int R, int S, int sh, int sw, int ph, int pw, const double* scale2,
                    const double* bias2, int act2, int dtype, double* t_out, double* y) {
    int Ho = out_size(H, ph, R, sh), Wo = out_size(W, pw, S, sw);
    int64_t M = (int64_t)N * H * W;
    double* t = t_out ? t_out : (double*)malloc(sizeof(double) * (size_t)(M * K1));
    if (!t) return -1;
    fcm_oracle_pw(x, M, C, w_pw, K1, t);
    fcm_oracle_epilogue(t, M, K1, scale1, bias1, act1);
    fcm_oracle_round_array(t, M * K1, dtype);
    fcm_oracle_dw(t, N, H, W, K1, w_dw, R, S, sh, sw, ph, pw, y);
    int64_t Mo = (int64_t)N * Ho * Wo;
    fcm_oracle_epilogue(y, Mo, K1, scale2, bias2, act2);
    fcm_oracle_round_array(y, Mo * K1, dtype);
    if (!t_out) free(t);
    return 0;
}

/* The PW -> DW module at listed output pixels only: every intermediate value the
 * pixel's window reads is recomputed from the input (exactly the redundant
 * computation of the PWDW_R case), window positions outside the image contribute
 * nothing. */
int fcm_oracle_pwdw_at(const double* x, int N, int H, int W, int C, const double* w_pw,
                       int K1, const double* scale1, const double* bias1, int act1,
                       const double* w_dw, int R, int S, int sh, int sw, int ph, int pw,
                       const double* scale2, const double* bias2, int act2, int dtype,
                       const int32_t* pix /* [P][3] */, int64_t P, double* y_rows) {
    (void)N;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < P; ++i) {
        int n = pix[3 * i], oh = pix[3 * i + 1], ow = pix[3 * i + 2];
        double* t = (double*)malloc(sizeof(double) * (size_t)K1);
        if (!t) continue;
        double* yr = y_rows + i * K1;
        for (int k = 0; k < K1; ++k) yr[k] = 0.0;
        for (int r = 0; r < R; ++r)
            for (int s = 0; s < S; ++s) {
                int ih = oh * sh - ph + r, iw = ow * sw - pw + s;
                if (ih < 0 || ih >= H || iw < 0 || iw >= W) continue;
                pw_row(x + (((int64_t)n * H + ih) * W + iw) * C, C, w_pw, K1, t);
                epilogue_row(t, K1, scale1, bias1, act1);
                fcm_oracle_round_array(t, K1, dtype);
                for (int k = 0; k < K1; ++k) yr[k] += t[k] * w_dw[((int64_t)k * R + r) * S + s];
            }
        epilogue_row(yr, K1, scale2, bias2, act2);
        fcm_oracle_round_array(yr, K1, dtype);
        free(t);
    }
    return 0;
}


/* PW -> PW module, layer by layer, over M pixels: t = store(x . w1^T), y = store(t . w2^T),
 * w1 [K1][C], w2 [K][K1]; store = epilogue + rounding to the storage type. */
int fcm_oracle_pwpw(const double* x, int64_t M, int C, const double* w1, int K1,
                    const double* scale1, const double* bias1, int act1, const double* w2,
                    int K, const double* scale2, const double* bias2, int act2, int dtype,
                    double* t_out, double* y) {
    double* t = t_out ? t_out : (double*)malloc(sizeof(double) * (size_t)(M * K1));
    if (!t) return -1;
    fcm_oracle_pw(x, M, C, w1, K1, t);
    store_rows(t, M, K1, scale1, bias1, act1, dtype);
    fcm_oracle_pw(t, M, K1, w2, K, y);
    store_rows(y, M, K, scale2, bias2, act2, dtype);
    if (!t_out) free(t);
    return 0;
}

/* ------------------------------------------------------------------------------ */
/* PW -> DW -> PW: the three convolutional layers of an inverted-residual block     */
/* (FCM paper Sec. II-B; Fig. 4 shows two such blocks in sequence).                 */
/* ------------------------------------------------------------------------------ */

/* Third layer of one output pixel, in place of its K1 depthwise outputs t2 (already
 * rounded): y[k] = round(act3(scale3[k] * sum_c t2[c] * w3[k][c] + bias3[k]) + xs[k]),
 * xs the shortcut row (the module's input at the same pixel) or NULL.  The shortcut
 * joins after the activation and before the single rounding. */
static void pw3_row(const double* t2, int K1, const double* w3, int K, const double* scale3,
                    const double* bias3, int act3, const double* xs, int dtype, double* y) {
    pw_row(t2, K1, w3, K, y);
    epilogue_row(y, K, scale3, bias3, act3);
    if (xs)
        for (int k = 0; k < K; ++k) y[k] += xs[k];
    fcm_oracle_round_array(y, K, dtype);
}

/* The module layer by layer:
 *   t1 = round(act1(scale1 * (x . w1^T) + bias1))          [N][H][W][K1]
 *   t2 = round(act2(scale2 * dw(t1, w2) + bias2))          [N][Ho][Wo][K1]
 *   y  = round(act3(scale3 * (t2 . w3^T) + bias3) [+ x])   [N][Ho][Wo][K]
 * w1 [K1][C], w2 [K1][R][S], w3 [K][K1].  residual != 0 adds the input pixel (the
 * block's identity shortcut); it needs Ho == H, Wo == W and K == C (else -2).
 * Floating-point storage only (-2 for int8). */
int fcm_oracle_pwdwpw(const double* x, int N, int H, int W, int C, const double* w1, int K1,
                      const double* scale1, const double* bias1, int act1, const double* w2,
                      int R, int S, int sh, int sw, int ph, int pw, const double* scale2,
                      const double* bias2, int act2, const double* w3, int K,
                      const double* scale3, const double* bias3, int act3, int residual,
                      int dtype, double* t1_out, double* t2_out, double* y) {
    int Ho = out_size(H, ph, R, sh), Wo = out_size(W, pw, S, sw);
    if (dtype == ORACLE_I8) return -2;
    if (residual && (Ho != H || Wo != W || K != C)) return -2;
    int64_t Mo = (int64_t)N * Ho * Wo;
    double* t2 = t2_out ? t2_out : (double*)malloc(sizeof(double) * (size_t)(Mo * K1));
    if (!t2) return -1;
    int rc = fcm_oracle_pwdw(x, N, H, W, C, w1, K1, scale1, bias1, act1, w2, R, S, sh, sw, ph,
                             pw, scale2, bias2, act2, dtype, t1_out, t2);
    if (rc == 0) {
#pragma omp parallel for schedule(static)
        for (int64_t m = 0; m < Mo; ++m)
            pw3_row(t2 + m * K1, K1, w3, K, scale3, bias3, act3, residual ? x + m * C : NULL,
                    dtype, y + m * K);
    }
    if (!t2_out) free(t2);
    return rc;
}

/* The module at listed output pixels only: the first two layers as fcm_oracle_pwdw_at
 * (every intermediate value the pixel's window reads recomputed from the input), then
 * the third layer and the shortcut of that pixel. */
int fcm_oracle_pwdwpw_at(const double* x, int N, int H, int W, int C, const double* w1,
                         int K1, const double* scale1, const double* bias1, int act1,
                         const double* w2, int R, int S, int sh, int sw, int ph, int pw,
                         const double* scale2, const double* bias2, int act2,
                         const double* w3, int K, const double* scale3, const double* bias3,
                         int act3, int residual, int dtype, const int32_t* pix /* [P][3] */,
                         int64_t P, double* y_rows) {
    int Ho = out_size(H, ph, R, sh), Wo = out_size(W, pw, S, sw);
    if (dtype == ORACLE_I8) return -2;
    if (residual && (Ho != H || Wo != W || K != C)) return -2;
    double* t2 = (double*)malloc(sizeof(double) * (size_t)(P * K1 + 1));
    if (!t2) return -1;
    fcm_oracle_pwdw_at(x, N, H, W, C, w1, K1, scale1, bias1, act1, w2, R, S, sh, sw, ph, pw,
                       scale2, bias2, act2, dtype, pix, P, t2);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < P; ++i) {
        int n = pix[3 * i], oh = pix[3 * i + 1], ow = pix[3 * i + 2];
        const double* xs =
            residual ? x + (((int64_t)n * H + oh) * W + ow) * C : NULL;
        pw3_row(t2 + i * K1, K1, w3, K, scale3, bias3, act3, xs, dtype, y_rows + i * K);
    }
    free(t2);
    return 0;
}

/* ------------------------------------------------------------------------------ */
/* Generalised depthwise layer: any R x S filter, dilation and depth multiplier.    */
/* The PyTorch forum thread "Using optimised depthwise convolutions" describes the   */
/* depthwise layer as a grouped convolution with one group per input channel and k  */
/* filters per group, any filter size; its separable module also gives that layer a */
/* dilation.  With one group per channel (C groups), output                        */
/* channel j belongs to group j / k, i.e. reads input channel j / k; a dilation d     */
/* spaces the filter taps d pixels apart.                                            */
/* ------------------------------------------------------------------------------ */

/* t[n][oh][ow][c*M + i] = sum_{r,s} x[n][oh*sh - ph + r*dh][ow*sw - pw + s*dw][c] *
 * w[c*M + i][r][s], x = 0 outside the image; w is [C*M][R][S], t has C*M channels. */
void fcm_oracle_dw_gen(const double* x, int N, int H, int W, int C, const double* w, int R,
                       int S, int sh, int sw, int ph, int pw, int dh, int dw, int M,
                       double* t) {
    int Ho = out_size(H, ph, (R - 1) * dh + 1, sh), Wo = out_size(W, pw, (S - 1) * dw + 1, sw);
    int CM = C * M;
#pragma omp parallel for collapse(2) schedule(static)
    for (int n = 0; n < N; ++n)
        for (int oh = 0; oh < Ho; ++oh)
            for (int ow = 0; ow < Wo; ++ow)
                for (int j = 0; j < CM; ++j) {
                    int c = j / M;
                    double acc = 0.0;
                    for (int r = 0; r < R; ++r)
                        for (int s = 0; s < S; ++s) {
                            int ih = oh * sh - ph + r * dh, iw = ow * sw - pw + s * dw;
                            if (ih < 0 || ih >= H || iw < 0 || iw >= W) continue;
                            acc += x[(((int64_t)n * H + ih) * W + iw) * C + c] *
                                   w[((int64_t)j * R + r) * S + s];
                        }
                    t[(((int64_t)n * Ho + oh) * Wo + ow) * CM + j] = acc;
                }
}

/* DW -> PW module with the generalised depthwise layer, layer by layer: the C*M
 * depthwise outputs are stored (epilogue 1, rounding), then the pointwise layer
 * w_pw [K][C*M] and epilogue 2. */
int fcm_oracle_dwpw_gen(const double* x, int N, int H, int W, int C, const double* w_dw,
                        int R, int S, int sh, int sw, int ph, int pw, int dh, int dw, int M,
                        const double* scale1, const double* bias1, int act1,
                        const double* w_pw, int K, const double* scale2, const double* bias2,
                        int act2, int dtype, double* t_out, double* y) {
    int Ho = out_size(H, ph, (R - 1) * dh + 1, sh), Wo = out_size(W, pw, (S - 1) * dw + 1, sw);
    int64_t P = (int64_t)N * Ho * Wo;
    int CM = C * M;
    double* t = t_out ? t_out : (double*)malloc(sizeof(double) * (size_t)(P * CM));
    if (!t) return -1;
    fcm_oracle_dw_gen(x, N, H, W, C, w_dw, R, S, sh, sw, ph, pw, dh, dw, M, t);
    store_rows(t, P, CM, scale1, bias1, act1, dtype);
    fcm_oracle_pw(t, P, CM, w_pw, K, y);
    store_rows(y, P, K, scale2, bias2, act2, dtype);
    if (!t_out) free(t);
    return 0;
}
