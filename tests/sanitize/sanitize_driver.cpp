// sanitize_driver.cpp -- host-only driver for an AddressSanitizer + UndefinedBehaviorSanitizer
// build (g++ -fsanitize=address,undefined) of the planner (csrc/plan.cpp: problem
// validation, variant tables, the FusePlanner cost models, the chain planner) and of the
// CPU oracle (oracle/fcm_oracle.c).  It drives both over the benchmark shapes, thousands of
// random valid and invalid problems and device specs, random chains, and small random
// oracle evaluations; any out-of-bounds access, leak, overflow or other undefined
// behaviour aborts the process with the sanitizer's report.  Test infrastructure: built and
// run by tests/test_sanitize.py on the CPU.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <random>
#include <string>
#include <vector>

#include "plan.h"

extern "C" {
int fcm_oracle_dwpw(const double* x, int N, int H, int W, int C, const double* w_dw, int R,
                    int S, int sh, int sw, int ph, int pw, const double* scale1,
                    const double* bias1, int act1, const double* w_pw, int K,
                    const double* scale2, const double* bias2, int act2, int dtype,
                    double* t_out, double* y);
int fcm_oracle_dwpw_at(const double* x, int N, int H, int W, int C, const double* w_dw, int R,
                       int S, int sh, int sw, int ph, int pw, const double* scale1,
                       const double* bias1, int act1, const double* w_pw, int K,
                       const double* scale2, const double* bias2, int act2, int dtype,
                       const int32_t* pix, int64_t P, double* y_rows);
int fcm_oracle_b2b(const double* x, int N, int H, int W, int C, const double* w1, int K1, int R,
                   int S, int sh, int sw, int ph, int pw, const double* scale1,
                   const double* bias1, int act1, const double* w2, int K, const double* scale2,
                   const double* bias2, int act2, int dtype, double* t_out, double* y);
int fcm_oracle_b2b_at(const double* x, int N, int H, int W, int C, const double* w1, int K1,
                      int R, int S, int sh, int sw, int ph, int pw, const double* scale1,
                      const double* bias1, int act1, const double* w2, int K,
                      const double* scale2, const double* bias2, int act2, int dtype,
                      const int32_t* pix, int64_t P, double* y_rows);
int fcm_oracle_pwdw(const double* x, int N, int H, int W, int C, const double* w_pw, int K1,
                    const double* scale1, const double* bias1, int act1, const double* w_dw,
                    int R, int S, int sh, int sw, int ph, int pw, const double* scale2,
                    const double* bias2, int act2, int dtype, double* t_out, double* y);
int fcm_oracle_pwdw_at(const double* x, int N, int H, int W, int C, const double* w_pw, int K1,
                       const double* scale1, const double* bias1, int act1,
                       const double* w_dw, int R, int S, int sh, int sw, int ph, int pw,
                       const double* scale2, const double* bias2, int act2, int dtype,
                       const int32_t* pix, int64_t P, double* y_rows);
int fcm_oracle_pwpw(const double* x, int64_t M, int C, const double* w1, int K1,
                    const double* scale1, const double* bias1, int act1, const double* w2,
                    int K, const double* scale2, const double* bias2, int act2, int dtype,
                    double* t_out, double* y);
int fcm_oracle_pwdwpw(const double* x, int N, int H, int W, int C, const double* w1, int K1,
                      const double* scale1, const double* bias1, int act1, const double* w2,
                      int R, int S, int sh, int sw, int ph, int pw, const double* scale2,
                      const double* bias2, int act2, const double* w3, int K,
                      const double* scale3, const double* bias3, int act3, int residual,
                      int dtype, double* t1_out, double* t2_out, double* y);
int fcm_oracle_pwdwpw_at(const double* x, int N, int H, int W, int C, const double* w1, int K1,
                         const double* scale1, const double* bias1, int act1,
                         const double* w2, int R, int S, int sh, int sw, int ph, int pw,
                         const double* scale2, const double* bias2, int act2,
                         const double* w3, int K, const double* scale3, const double* bias3,
                         int act3, int residual, int dtype, const int32_t* pix, int64_t P,
                         double* y_rows);
int fcm_oracle_dwpw_gen(const double* x, int N, int H, int W, int C, const double* w_dw, int R,
                        int S, int sh, int sw, int ph, int pw, int dh, int dw, int M,
                        const double* scale1, const double* bias1, int act1,
                        const double* w_pw, int K, const double* scale2, const double* bias2,
                        int act2, int dtype, double* t_out, double* y);
}

namespace {

std::mt19937_64 rng(12345);

int pick(int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); }

std::vector<double> rnd(size_t n) {
    std::normal_distribution<double> d(0.0, 1.0);
    std::vector<double> v(n);
    for (auto& x : v) x = d(rng);
    return v;
}

int out_extent(int in, int pad, int ext, int s) { return (in + 2 * pad - ext) / s + 1; }

// A problem drawn from everything the boundary might be handed: mostly plausible values,
// sometimes zero, negative or huge ones.
fcm_problem random_problem() {
    fcm_problem p;
    memset(&p, 0, sizeof(p));
    auto v = [](int lo, int hi) {
        const int r = pick(0, 19);
        if (r == 0) return 0;
        if (r == 1) return -pick(1, 5);
        if (r == 2) return pick(1 << 20, 1 << 30);
        return pick(lo, hi);
    };
    p.kind = pick(-1, 5);
    p.dtype = pick(-1, 4);
    p.N = v(1, 4);
    p.H = v(1, 40);
    p.W = v(1, 40);
    const int c8[] = {8, 16, 24, 32, 40, 64, 96, 128, 144, 256, 1024};
    p.C = pick(0, 9) ? c8[pick(0, 10)] : v(1, 300);
    p.K1 = pick(0, 9) ? c8[pick(0, 10)] : v(1, 300);
    p.K = pick(0, 9) ? c8[pick(0, 10)] : v(1, 300);
    p.R = pick(0, 5) ? 3 : v(1, 8);
    p.S = pick(0, 5) ? p.R : v(1, 8);
    p.stride_h = p.stride_w = pick(0, 7) ? pick(1, 2) : v(1, 4);
    p.pad_h = p.pad_w = pick(0, 7) ? pick(0, 1) : v(0, 4);
    p.act1 = pick(-1, 3);
    p.act2 = pick(-1, 3);
    p.dil_h = p.dil_w = pick(0, 5) ? 0 : pick(-1, 3);
    p.mult = pick(0, 5) ? 0 : pick(-1, 3);
    if (p.kind == FCM_KIND_DWPW && pick(0, 3))  // (saturated: C may be drawn huge)
        p.K1 = (int)std::min<int64_t>((int64_t)p.C * (p.mult > 0 ? p.mult : 1), INT32_MAX);
    if (p.kind == FCM_KIND_PWDW && pick(0, 3)) p.K = p.K1;
    if (p.kind == FCM_KIND_PWPW && pick(0, 3)) {
        p.R = p.S = 1;
        p.pad_h = p.pad_w = 0;
        p.stride_h = p.stride_w = 1;
    }
    p.act3 = pick(0, 5) ? 0 : pick(-1, 3);
    p.residual = pick(0, 5) ? 0 : pick(-1, 2);
    if (p.kind == FCM_KIND_PWDWPW && pick(0, 2)) {
        p.act3 = pick(0, 2);
        p.residual = pick(0, 1);
        if (p.residual) p.K = p.C;
    }
    return p;
}

// A problem of a kind the library has kernels for, with sizes in the ranges they take.
fcm_problem plausible_problem() {
    fcm_problem p;
    memset(&p, 0, sizeof(p));
    p.kind = pick(0, 4);
    p.dtype = pick(0, 2);
    p.N = pick(1, 8);
    p.H = pick(1, 60);
    p.W = pick(1, 60);
    p.C = 8 * pick(1, p.kind == FCM_KIND_DWPW ? 128 : 8);
    p.K = 8 * pick(1, 64);
    p.K1 = 8 * pick(1, 24);
    p.R = p.S = 3;
    p.stride_h = p.stride_w = pick(1, 2);
    p.pad_h = p.pad_w = pick(0, 1);
    p.act1 = pick(0, 2);
    p.act2 = pick(0, 2);
    switch (p.kind) {
    case FCM_KIND_DWPW:
        if (pick(0, 3) == 0) {  // generalised depthwise layer
            p.R = p.S = 3 + 2 * pick(0, 2);
            p.dil_h = p.dil_w = pick(1, 2);
            p.mult = pick(1, 2);
            p.pad_h = p.pad_w = (p.R - 1) * p.dil_h / 2;
        }
        p.K1 = p.C * (p.mult > 0 ? p.mult : 1);
        if (pick(0, 4) == 0) p.dtype = FCM_I8;
        break;
    case FCM_KIND_PWDW: p.K = p.K1; break;
    case FCM_KIND_PWPW:
        p.R = p.S = 1;
        p.pad_h = p.pad_w = 0;
        p.stride_h = p.stride_w = 1;
        break;
    case FCM_KIND_PWDWPW:
        p.C = 8 * pick(1, 4);
        p.K1 = 8 * pick(1, 20);
        p.K = 8 * pick(1, 4);
        p.act3 = pick(0, 2);
        if (p.stride_h == 1 && p.pad_h == 1 && pick(0, 1)) {
            p.residual = 1;
            p.K = p.C;
        }
        break;
    default: break;
    }
    return p;
}

fcm_device_spec random_spec() {
    fcm_device_spec d;
    fcm::default_spec(&d);
    switch (pick(0, 6)) {
    case 0: d.num_cus = pick(-1, 1024); break;
    case 1: d.lds_bytes_per_wg = pick(0, 200000); break;
    case 2: d.vgprs_per_simd_lane = pick(0, 1024); break;
    case 3: d.max_waves_per_simd = pick(0, 16); break;
    case 4: d.lds_bytes_per_cu = pick(0, 200000); break;
    default: break;
    }
    return d;
}

int run_planner(int iters) {
    int planned = 0;
    std::string err;
    for (int i = 0; i < fcm::kNumVariants; ++i) {
        const fcm::VariantDesc& v = fcm::kVariants[i];
        if (fcm::variant_lds_bytes(v) <= 0 || fcm::variant_vgpr_estimate(v) <= 0) {
            fprintf(stderr, "variant %s: non-positive LDS or register estimate\n", v.name);
            return -1;
        }
    }
    for (int it = 0; it < iters; ++it) {
        fcm_problem p = (it & 1) ? random_problem() : plausible_problem();
        const bool with_spec = pick(0, 2) == 0;
        fcm_device_spec d = random_spec();
        const int forced = pick(0, 3) == 0 ? pick(-2, fcm::kNumVariants + 2) : -1;
        fcm_plan_t out;
        err.clear();
        const fcm_status st = fcm::plan_problem(&p, with_spec ? &d : nullptr, forced, &out, &err);
        if (st == FCM_OK) {
            ++planned;
            if (out.grid <= 0 || out.variant < 0 || out.variant >= fcm::kNumVariants) {
                fprintf(stderr, "plan %d: bad grid %d / variant %d\n", it, out.grid, out.variant);
                return -1;
            }
        } else if (err.empty()) {
            fprintf(stderr, "plan %d: status %d without a message\n", it, (int)st);
            return -1;
        }
        // every variant against the problem, with and without a reason string
        for (int i = 0; i < fcm::kNumVariants; i += pick(1, 5)) {
            std::string why;
            (void)fcm::variant_runs(fcm::kVariants[i], p, pick(0, 1) ? &why : nullptr);
        }
        (void)fcm::persistent_grid(pick(0, 100000), pick(1, 64), pick(0, 4096));
    }
    return planned;
}

int run_chains(int iters) {
    int ok = 0;
    for (int it = 0; it < iters; ++it) {
        const int n = pick(1, 12);
        std::vector<fcm_layer> layers(n);
        int c = 8 * pick(1, 16);
        for (int i = 0; i < n; ++i) {
            fcm_layer& l = layers[i];
            l.type = pick(0, 9) ? pick(0, 1) : pick(-1, 3);
            l.C = pick(0, 15) ? c : pick(-1, 64);
            l.K = l.type == FCM_LAYER_DW ? l.C : 8 * pick(1, 32);
            l.stride = l.type == FCM_LAYER_DW ? pick(1, 2) : 1;
            l.act = pick(0, 2);
            c = l.K;
        }
        std::vector<fcm_chain_group> groups(n);
        int ng = 0;
        double gc = 0, gl = 0;
        std::string err;
        fcm_device_spec d = random_spec();
        const fcm_status st =
            fcm::plan_chain(layers.data(), n, pick(1, 8), pick(1, 112), pick(1, 112),
                            pick(0, 2), pick(0, 1) ? &d : nullptr, groups.data(), &ng, &gc, &gl,
                            &err);
        if (st == FCM_OK) {
            ++ok;
            if (ng < 1 || ng > n) {
                fprintf(stderr, "chain %d: %d groups for %d layers\n", it, ng, n);
                return -1;
            }
        }
    }
    return ok;
}

int run_oracle(int iters) {
    for (int it = 0; it < iters; ++it) {
        const int N = pick(1, 2), H = pick(1, 9), W = pick(1, 9), C = pick(1, 12);
        const int K1 = pick(1, 12), K = pick(1, 12), s = pick(1, 2), pad = pick(0, 1);
        const int dtype = pick(0, 2), a1 = pick(0, 2), a2 = pick(0, 2);
        if (H + 2 * pad < 3 || W + 2 * pad < 3) continue;
        const int Ho = out_extent(H, pad, 3, s), Wo = out_extent(W, pad, 3, s);
        std::vector<double> x = rnd((size_t)N * H * W * C), s1 = rnd(64), b1 = rnd(64),
                            s2 = rnd(64), b2 = rnd(64), s3 = rnd(64), b3 = rnd(64);
        std::vector<int32_t> pix;
        for (int i = 0; i < 5; ++i) {
            pix.push_back(pick(0, N - 1));
            pix.push_back(pick(0, Ho - 1));
            pix.push_back(pick(0, Wo - 1));
        }
        const int64_t P = 5;
        const double* sc1 = pick(0, 1) ? s1.data() : nullptr;
        const double* bi2 = pick(0, 1) ? b2.data() : nullptr;
        {  // DW -> PW (K1 = C), sampled rows
            std::vector<double> wd = rnd((size_t)C * 9), wp = rnd((size_t)K * C);
            std::vector<double> y((size_t)N * Ho * Wo * K), rows((size_t)P * K);
            if (fcm_oracle_dwpw(x.data(), N, H, W, C, wd.data(), 3, 3, s, s, pad, pad, sc1,
                                b1.data(), a1, wp.data(), K, s2.data(), bi2, a2, dtype, nullptr,
                                y.data()) != 0)
                return -1;
            fcm_oracle_dwpw_at(x.data(), N, H, W, C, wd.data(), 3, 3, s, s, pad, pad, sc1,
                               b1.data(), a1, wp.data(), K, s2.data(), bi2, a2, dtype, pix.data(),
                               P, rows.data());
        }
        {  // 3x3 conv -> 1x1 conv
            std::vector<double> w1 = rnd((size_t)K1 * C * 9), w2 = rnd((size_t)K * K1);
            std::vector<double> t((size_t)N * Ho * Wo * K1), y((size_t)N * Ho * Wo * K),
                rows((size_t)P * K);
            if (fcm_oracle_b2b(x.data(), N, H, W, C, w1.data(), K1, 3, 3, s, s, pad, pad, sc1,
                               b1.data(), a1, w2.data(), K, s2.data(), bi2, a2, dtype, t.data(),
                               y.data()) != 0)
                return -1;
            fcm_oracle_b2b_at(x.data(), N, H, W, C, w1.data(), K1, 3, 3, s, s, pad, pad, sc1,
                              b1.data(), a1, w2.data(), K, s2.data(), bi2, a2, dtype, pix.data(),
                              P, rows.data());
        }
        {  // PW -> DW, PW -> DW -> PW (with the shortcut when the shapes allow it)
            std::vector<double> wp = rnd((size_t)K1 * C), wd = rnd((size_t)K1 * 9),
                                w3 = rnd((size_t)K * K1);
            std::vector<double> t((size_t)N * H * W * K1), y((size_t)N * Ho * Wo * K1),
                rows((size_t)P * K1);
            if (fcm_oracle_pwdw(x.data(), N, H, W, C, wp.data(), K1, sc1, b1.data(), a1,
                                wd.data(), 3, 3, s, s, pad, pad, s2.data(), bi2, a2, dtype,
                                t.data(), y.data()) != 0)
                return -1;
            fcm_oracle_pwdw_at(x.data(), N, H, W, C, wp.data(), K1, sc1, b1.data(), a1,
                               wd.data(), 3, 3, s, s, pad, pad, s2.data(), bi2, a2, dtype,
                               pix.data(), P, rows.data());
            const int res = (s == 1 && pad == 1 && pick(0, 1)) ? 1 : 0;
            const int K3 = res ? C : K;
            std::vector<double> w3r = rnd((size_t)K3 * K1), y3((size_t)N * Ho * Wo * K3),
                                rows3((size_t)P * K3);
            if (fcm_oracle_pwdwpw(x.data(), N, H, W, C, wp.data(), K1, sc1, b1.data(), a1,
                                  wd.data(), 3, 3, s, s, pad, pad, s2.data(), bi2, a2,
                                  w3r.data(), K3, s3.data(), b3.data(), pick(0, 2), res,
                                  pick(0, 2), nullptr, nullptr, y3.data()) != 0)
                return -1;
            fcm_oracle_pwdwpw_at(x.data(), N, H, W, C, wp.data(), K1, sc1, b1.data(), a1,
                                 wd.data(), 3, 3, s, s, pad, pad, s2.data(), bi2, a2,
                                 w3r.data(), K3, s3.data(), b3.data(), 0, res, 1, pix.data(), P,
                                 rows3.data());
        }
        {  // PW -> PW over every pixel
            const int64_t M = (int64_t)N * H * W;
            std::vector<double> w1 = rnd((size_t)K1 * C), w2 = rnd((size_t)K * K1);
            std::vector<double> y((size_t)M * K);
            if (fcm_oracle_pwpw(x.data(), M, C, w1.data(), K1, sc1, b1.data(), a1, w2.data(), K,
                                s2.data(), bi2, a2, dtype, nullptr, y.data()) != 0)
                return -1;
        }
        {  // generalised depthwise layer: 5x5 or dilated 3x3, multiplier 1 or 2
            const int f = pick(0, 1) ? 5 : 3, dil = f == 3 ? pick(1, 2) : 1, m = pick(1, 2);
            const int ext = (f - 1) * dil + 1, gp = ext / 2;
            if (H + 2 * gp < ext || W + 2 * gp < ext) continue;
            const int Hg = out_extent(H, gp, ext, s), Wg = out_extent(W, gp, ext, s);
            std::vector<double> wd = rnd((size_t)C * m * f * f), wp = rnd((size_t)K * C * m);
            std::vector<double> y((size_t)N * Hg * Wg * K);
            if (fcm_oracle_dwpw_gen(x.data(), N, H, W, C, wd.data(), f, f, s, s, gp, gp, dil,
                                    dil, m, sc1, b1.data(), a1, wp.data(), K, s2.data(), bi2,
                                    a2, dtype, nullptr, y.data()) != 0)
                return -1;
        }
    }
    return 0;
}

}  // namespace

int main() {
    const int planned = run_planner(20000);
    if (planned < 0) return 1;
    const int chains = run_chains(2000);
    if (chains < 0) return 1;
    if (run_oracle(300) != 0) return 1;
    printf("sanitized run done: %d of 20000 random problems planned, %d of 2000 chains, "
           "300 oracle rounds\n", planned, chains);
    return 0;
}
