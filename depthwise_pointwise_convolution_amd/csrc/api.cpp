// api.cpp -- the C ABI of libfcm.so: argument validation, plan checks, dispatch to the
// kernel variants and the layer-by-layer baselines.  Every check happens on the host
// before anything is enqueued; errors come back as status codes with a per-thread
// message (fcm_last_error).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "../../include/fcm.h"
#include "kargs.h"
#include "launchers.h"
#include "lbl_tiles.h"
#include "plan.h"

namespace fcm {
namespace {

thread_local std::string g_last_error;

fcm_status fail(fcm_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}
fcm_status ok() {
    g_last_error.clear();
    return FCM_OK;
}

struct VariantImpl {
    launch_fn launch;
    occupancy_fn occupancy;
    launch_fn lbl_first;  // generalised DW->PW: its layer-by-layer depthwise kernel
};

const VariantImpl kImpls[] = {
#define FCM_V_DWPW(name, dt, CT, S, TH, TW, KT, CC, WRES, OCC)  \
    {launch_dwpw_mfma<CT, S, TH, TW, KT, CC, WRES, OCC>,          \
     occ_dwpw_mfma<CT, S, TH, TW, KT, CC, WRES, OCC>},
#define FCM_V_DWPW32(name, S, TH, TW, KT, CC) \
    {launch_dwpw_f32<S, TH, TW, KT, CC>, occ_dwpw_f32<S, TH, TW, KT, CC>},
#define FCM_V_B2B(name, dt, CT, S, TH, TW, K1, KT, CC) \
    {launch_b2b_mfma<CT, S, TH, TW, K1, KT, CC>, occ_b2b_mfma<CT, S, TH, TW, K1, KT, CC>},
#define FCM_V_DWPW_MM(name, dt, CT, S, TH, TW, KT, CC, NW, OCC) \
    {launch_dwpw_mm<CT, S, TH, TW, KT, CC, NW, OCC, 1, 3>,      \
     occ_dwpw_mm<CT, S, TH, TW, KT, CC, NW, OCC, 1, 3>},
#define FCM_V_DWPW_MMM(name, dt, CT, S, M, TH, TW, KT, CC, NW, OCC) \
    {launch_dwpw_mm<CT, S, TH, TW, KT, CC, NW, OCC, M, 3>,          \
     occ_dwpw_mm<CT, S, TH, TW, KT, CC, NW, OCC, M, 3>},
#define FCM_V_DWPW_MMF(name, dt, CT, S, FS, TH, TW, KT, CC, NW, OCC) \
    {launch_dwpw_mm<CT, S, TH, TW, KT, CC, NW, OCC, 1, FS>,          \
     occ_dwpw_mm<CT, S, TH, TW, KT, CC, NW, OCC, 1, FS>},
#define FCM_V_B2B_MM(name, dt, CT, S, OCC) {launch_b2b_mm<CT, S, OCC>, occ_b2b_mm<CT, S, OCC>},
#define FCM_V_DWPW_MMW(name, dt, CT, S, TH, TW, KT, CMAX, NW, OCC) \
    {launch_dwpw_mmw<CT, S, TH, TW, KT, CMAX, NW, OCC, 1>,        \
     occ_dwpw_mmw<CT, S, TH, TW, KT, CMAX, NW, OCC, 1>},
#define FCM_V_DWPW_MMWD(name, dt, CT, S, D, TH, TW, KT, CMAX, NW, OCC) \
    {launch_dwpw_mmw<CT, S, TH, TW, KT, CMAX, NW, OCC, D>,             \
     occ_dwpw_mmw<CT, S, TH, TW, KT, CMAX, NW, OCC, D>},
#define FCM_V_DWPW_WS(name, dt, CTy, S, TH, TW, CT, KT, NW) \
    {launch_dwpw_ws<CTy, S, TH, TW, CT, KT, NW>, occ_dwpw_ws<CTy, S, TH, TW, CT, KT, NW>},
#define FCM_V_DWPW_WSL(name, dt, CT, S, TH, TW, KT, CMAX, NW) \
    {launch_dwpw_wsl<CT, S, TH, TW, KT, CMAX, NW>, occ_dwpw_wsl<CT, S, TH, TW, KT, CMAX, NW>},
#define FCM_V_PWDW_MM(name, dt, CT, S, TH, CMAX, NW, BPW, OCC) \
    {launch_pwdw_mm<CT, S, TH, CMAX, NW, BPW, OCC>, occ_pwdw_mm<CT, S, TH, CMAX, NW, BPW, OCC>},
#define FCM_V_PWDWPW_MM(name, dt, CT, S, TH, CMAX, NW, BPW, KB, OCC)   \
    {launch_pwdwpw_mm<CT, S, TH, CMAX, NW, BPW, KB, OCC>,                \
     occ_pwdwpw_mm<CT, S, TH, CMAX, NW, BPW, KB, OCC>},
#define FCM_V_DWPW_I8(name, S, OCC, CMAX) \
    {launch_dwpw_i8<S, OCC, CMAX>, occ_dwpw_i8<S, OCC, CMAX>},
#define FCM_V_PWPW_MM(name, dt, CT, PB, OCC, CMAX, KT) \
    {launch_pwpw_mm<CT, PB, OCC, CMAX, KT>, occ_pwpw_mm<CT, PB, OCC, CMAX, KT>},
#define FCM_V_DWPW_GEN(name, dt, CT, S, FS, D, M, TH, TW, KT, CC, NG) \
    {launch_dwpw_gen<CT, S, FS, D, M, TH, TW, KT, CC, NG>,                \
     occ_dwpw_gen<CT, S, FS, D, M, TH, TW, KT, CC, NG>,                   \
     launch_dw_gen_lbl<CT, S, FS, D, M, TH, TW, KT, CC, NG>},
#include "variants.def"
#undef FCM_V_DWPW
#undef FCM_V_DWPW32
#undef FCM_V_B2B
#undef FCM_V_DWPW_MM
#undef FCM_V_B2B_MM
#undef FCM_V_DWPW_MMW
#undef FCM_V_DWPW_MMWD
#undef FCM_V_DWPW_MMM
#undef FCM_V_DWPW_MMF
#undef FCM_V_PWDW_MM
#undef FCM_V_PWDWPW_MM
#undef FCM_V_DWPW_WS
#undef FCM_V_DWPW_WSL
#undef FCM_V_DWPW_I8
#undef FCM_V_PWPW_MM
#undef FCM_V_DWPW_GEN
};
static_assert(sizeof(kImpls) / sizeof(kImpls[0]) > 0, "variants");

// (device, variant) -> (CUs, workgroups per CU), filled on first use.
std::mutex g_occ_mu;
std::map<std::pair<int, int>, std::pair<int, int>> g_occ;

fcm_status device_capacity(int variant, int* cus, int* per_cu) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(FCM_ERR_HIP, "hipGetDevice failed");
    std::lock_guard<std::mutex> lk(g_occ_mu);
    auto it = g_occ.find({dev, variant});
    if (it == g_occ.end()) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return fail(FCM_ERR_HIP, "hipDeviceGetAttribute(MultiprocessorCount) failed");
        const int occ = kImpls[variant].occupancy();
        if (occ <= 0) return fail(FCM_ERR_HIP, "occupancy query failed for the kernel variant");
        it = g_occ.emplace(std::make_pair(dev, variant), std::make_pair(n, occ)).first;
    }
    *cus = it->second.first;
    *per_cu = it->second.second;
    return FCM_OK;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Re-derive what a plan must contain from its problem and compare: a plan that was
// edited, truncated or made for another problem is rejected.
fcm_status check_plan(const fcm_plan_t* plan, int kind) {
    if (!plan) return fail(FCM_ERR_INVALID_ARG, "plan is NULL");
    if (plan->version != FCM_PLAN_VERSION)
        return fail(FCM_ERR_INVALID_ARG, "plan version mismatch");
    std::string err;
    fcm_status st = validate_problem(&plan->prob, &err);
    if (st != FCM_OK) return fail(st, "plan holds an invalid problem: " + err);
    if (plan->prob.kind != kind)
        return fail(FCM_ERR_INVALID_ARG, "plan is for the other module kind");
    if (plan->Ho != conv_out(plan->prob.H, plan->prob.pad_h, prob_ext_h(plan->prob),
                             plan->prob.stride_h) ||
        plan->Wo != conv_out(plan->prob.W, plan->prob.pad_w, prob_ext_w(plan->prob),
                             plan->prob.stride_w))
        return fail(FCM_ERR_INVALID_ARG, "plan output extent does not match its problem");
    return FCM_OK;
}

fcm_status check_variant(const fcm_plan_t* plan) {
    if (plan->variant < 0 || plan->variant >= kNumVariants)
        return fail(FCM_ERR_INVALID_ARG, "plan names no compiled variant");
    const VariantDesc& v = kVariants[plan->variant];
    std::string why;
    if (!variant_runs(v, plan->prob, &why)) return fail(FCM_ERR_INVALID_ARG, "plan variant: " + why);
    if (plan->tile_h != v.th || plan->tile_w != v.tw || plan->k_tile != v.kt ||
        plan->c_chunk != v.cc)
        return fail(FCM_ERR_INVALID_ARG, "plan tiling does not match its variant");
    if (plan->grid <= 0) return fail(FCM_ERR_INVALID_ARG, "plan grid must be positive");
    return FCM_OK;
}

fcm_status need(const void* p, const char* what, uintptr_t align) {
    if (!p) return fail(FCM_ERR_INVALID_ARG, std::string(what) + " is NULL");
    if (!aligned(p, align))
        return fail(FCM_ERR_INVALID_ARG,
                    std::string(what) + " is not " + std::to_string(align) + "-byte aligned");
    return FCM_OK;
}
fcm_status optional(const void* p, const char* what) {
    if (p && !aligned(p, 4))
        return fail(FCM_ERR_INVALID_ARG, std::string(what) + " is not 4-byte aligned");
    return FCM_OK;
}

#define FCM_TRY(expr)                      \
    do {                                   \
        fcm_status _s = (expr);            \
        if (_s != FCM_OK) return _s;       \
    } while (0)

KArgs base_args(const fcm_plan_t* plan) {
    KArgs a;
    memset(&a, 0, sizeof(a));
    const fcm_problem& p = plan->prob;
    a.N = p.N;
    a.H = p.H;
    a.W = p.W;
    a.C = p.C;
    a.K1 = p.K1;
    a.K = p.K;
    a.Ho = plan->Ho;
    a.Wo = plan->Wo;
    a.pad_h = p.pad_h;
    a.pad_w = p.pad_w;
    a.act1 = p.act1;
    a.act2 = p.act2;
    a.act3 = p.act3;
    a.residual = p.residual;
    return a;
}

void set_tiles(KArgs* a, int th, int tw, int kt, int kdim) {
    a->tiles_h = (a->Ho + th - 1) / th;
    a->tiles_w = (a->Wo + tw - 1) / tw;
    a->num_ptiles = a->N * a->tiles_h * a->tiles_w;
    a->num_ktiles = (kdim + kt - 1) / kt;
}

fcm_status launch_fused(const fcm_plan_t* plan, KArgs& a, void* stream) {
    const VariantDesc& v = kVariants[plan->variant];
    set_tiles(&a, v.th, v.tw, v.kt, plan->prob.K);  // (PWDW: K == K1)
    if (plan->prob.kind == FCM_KIND_PWPW) {
        // tiles of th x tw consecutive pixels of the flattened N x H x W extent
        const int64_t M = (int64_t)plan->prob.N * plan->prob.H * plan->prob.W;
        a.num_ptiles = (int)((M + v.th * v.tw - 1) / (v.th * v.tw));
    }
    int cus = 0, per_cu = 0;
    FCM_TRY(device_capacity(plan->variant, &cus, &per_cu));
    // persistent grid within what the GPU holds at once (measured occupancy) and the
    // plan's own grid
    const int64_t cap = std::min<int64_t>(plan->grid, (int64_t)cus * per_cu);
    const int64_t grid = persistent_grid(a.num_ptiles, a.num_ktiles, cap);
    const int rc = kImpls[plan->variant].launch(a, (int)grid, stream);
    if (rc != 0)
        return fail(FCM_ERR_HIP, std::string("kernel launch failed: ") +
                                     hipGetErrorString((hipError_t)rc));
    return ok();
}

}  // namespace
}  // namespace fcm

namespace fcm {
namespace {
// Measured selection shared by fcm_tune and fcm_tune_pwdwpw: `run` launches the module
// with a candidate plan on the next input/output pair.
template <typename Run>
fcm_status tune_impl(const fcm_problem* prob, const fcm_device_spec* spec, int32_t iters,
                     void* stream, fcm_plan_t* out, Run&& run) {
    fcm_plan_t first;
    FCM_TRY(fcm_plan(prob, spec, &first));  // validates the problem
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
        if (e0) (void)hipEventDestroy(e0);
        return fail(FCM_ERR_HIP, "hipEventCreate failed");
    }
    fcm_status st = FCM_OK;
    fcm_plan_t best = first;
    double best_us = 0.0;
    for (int v = 0; v < kNumVariants && st == FCM_OK; ++v) {
        fcm_plan_t pv;
        std::string err;
        if (plan_problem(prob, spec, v, &pv, &err) != FCM_OK) continue;
        const VariantDesc& vd = kVariants[v];
        std::string why;
        if (!variant_runs(vd, pv.prob, &why)) continue;
        int cus = 0, per_cu = 0;
        st = device_capacity(v, &cus, &per_cu);
        if (st != FCM_OK) break;
        const int64_t ptiles =
            prob->kind == FCM_KIND_PWPW
                ? ((int64_t)prob->N * prob->H * prob->W + vd.th * vd.tw - 1) / (vd.th * vd.tw)
                : (int64_t)prob->N * ((pv.Ho + vd.th - 1) / vd.th) * ((pv.Wo + vd.tw - 1) / vd.tw);
        const int ktiles = (prob->K + vd.kt - 1) / vd.kt;  // (PWDW: K == K1)
        int64_t last_grid = -1;
        for (int w = 1; w <= std::min(4, per_cu) && st == FCM_OK; ++w) {
            const int64_t g = persistent_grid(ptiles, ktiles, (int64_t)cus * w);
            if (g == last_grid) continue;
            last_grid = g;
            fcm_plan_t cand = pv;
            cand.grid = (int32_t)g;
            cand.wgs_per_cu = w;
            for (int i = 0; i < 2 && st == FCM_OK; ++i) st = run(&cand);  // warm-up
            if (st != FCM_OK) break;
            if (hipEventRecord(e0, (hipStream_t)stream) != hipSuccess) {
                st = fail(FCM_ERR_HIP, "hipEventRecord failed");
                break;
            }
            for (int i = 0; i < iters && st == FCM_OK; ++i) st = run(&cand);
            if (st != FCM_OK) break;
            float ms = 0.f;
            if (hipEventRecord(e1, (hipStream_t)stream) != hipSuccess ||
                hipEventSynchronize(e1) != hipSuccess ||
                hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
                st = fail(FCM_ERR_HIP, "timing events failed");
                break;
            }
            const double us = 1e3 * ms / iters;
            if (best_us == 0.0 || us < best_us) {
                best_us = us;
                best = cand;
            }
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (st != FCM_OK) return st;
    best.tuned_us = best_us;
    *out = best;
    return ok();
}
}  // namespace
}  // namespace fcm

using namespace fcm;

extern "C" {

const char* fcm_status_str(fcm_status s) {
    switch (s) {
    case FCM_OK: return "FCM_OK";
    case FCM_ERR_INVALID_ARG: return "FCM_ERR_INVALID_ARG";
    case FCM_ERR_UNSUPPORTED: return "FCM_ERR_UNSUPPORTED";
    case FCM_ERR_HIP: return "FCM_ERR_HIP";
    }
    return "FCM_ERR_UNKNOWN";
}

const char* fcm_last_error(void) { return g_last_error.c_str(); }

fcm_status fcm_default_device_spec(fcm_device_spec* out) {
    if (!out) return fail(FCM_ERR_INVALID_ARG, "spec output pointer is NULL");
    default_spec(out);
    return ok();
}

fcm_status fcm_query_device_spec(int device, fcm_device_spec* out) {
    FCM_TRY(fcm_default_device_spec(out));
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
        return fail(FCM_ERR_HIP, "cannot query the device's compute-unit count");
    out->num_cus = n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, device) ==
            hipSuccess &&
        n > 0)
        out->lds_bytes_per_cu = n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerBlock, device) ==
            hipSuccess &&
        n > 0)
        out->lds_bytes_per_wg = n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeL2CacheSize, device) == hipSuccess && n > 0)
        out->l2_bytes_per_xcd = n;
    return ok();
}

fcm_status fcm_plan(const fcm_problem* prob, const fcm_device_spec* spec, fcm_plan_t* out) {
    std::string err;
    fcm_status s = plan_problem(prob, spec, -1, out, &err);
    return s == FCM_OK ? ok() : fail(s, err);
}

fcm_status fcm_plan_variant(const fcm_problem* prob, const fcm_device_spec* spec,
                            int32_t variant, fcm_plan_t* out) {
    if (variant < 0 || variant >= kNumVariants)
        return fail(FCM_ERR_INVALID_ARG, "variant index out of range");
    std::string err;
    fcm_status s = plan_problem(prob, spec, variant, out, &err);
    return s == FCM_OK ? ok() : fail(s, err);
}

fcm_status fcm_plan_chain(const fcm_layer* layers, int32_t n, int32_t N, int32_t H, int32_t W,
                          int32_t dtype, const fcm_device_spec* spec, fcm_chain_group* groups,
                          int32_t* ngroups, double* gma_chain, double* gma_layer_by_layer) {
    std::string err;
    int ng = 0;
    const fcm_status s = plan_chain(layers, n, N, H, W, dtype, spec, groups, &ng, gma_chain,
                                    gma_layer_by_layer, &err);
    if (s != FCM_OK) return fail(s, err);
    *ngroups = ng;
    return ok();
}

int32_t fcm_num_variants(void) { return kNumVariants; }

const char* fcm_variant_name(int32_t variant) {
    if (variant < 0 || variant >= kNumVariants) return "";
    return kVariants[variant].name;
}

fcm_status fcm_pack_weights(const fcm_plan_t* plan, const void* w1_src, void* w1_dst,
                            const void* w2_src, void* w2_dst, void* stream) {
    if (!plan) return fail(FCM_ERR_INVALID_ARG, "plan is NULL");
    FCM_TRY(check_plan(plan, plan->prob.kind));
    const fcm_problem& p = plan->prob;
    const int e = p.dtype == FCM_F32 ? 4 : p.dtype == FCM_I8 ? 1 : 2;
    if ((w1_src == nullptr) != (w1_dst == nullptr))
        return fail(FCM_ERR_INVALID_ARG, "w1_src and w1_dst must both be given or both NULL");
    if ((w2_src == nullptr) != (w2_dst == nullptr))
        return fail(FCM_ERR_INVALID_ARG, "w2_src and w2_dst must both be given or both NULL");
    if (w1_src) {
        if (!aligned(w1_src, e) || !aligned(w1_dst, 16))
            return fail(FCM_ERR_INVALID_ARG, "w1 source must be element-aligned, w1 destination "
                                             "16-byte aligned");
        const char* s = (const char*)w1_src;
        const char* d = (const char*)w1_dst;
        const int64_t ns = prob_has_expansion(p)
                               ? (int64_t)p.K1 * p.C * e
                               : p.kind == FCM_KIND_B2B ? (int64_t)p.K1 * p.R * p.S * p.C * e
                                                        : (int64_t)p.R * p.S * p.K1 * e;
        const int64_t nd = plan->w1_packed_bytes;
        if (s < d + nd && d < s + ns) return fail(FCM_ERR_INVALID_ARG, "w1 buffers overlap");
    }
    if (w2_src) {
        if (!aligned(w2_src, e) || !aligned(w2_dst, 16))
            return fail(FCM_ERR_INVALID_ARG, "w2 source must be element-aligned, w2 destination "
                                             "16-byte aligned");
        const char* s = (const char*)w2_src;
        const char* d = (const char*)w2_dst;
        const int64_t ns = prob_has_expansion(p)
                               ? (int64_t)p.K1 * p.R * p.S * e
                               : (int64_t)p.K * p.K1 * e;  // (DW->PW: K1 = C * mult)
        const int64_t nd = plan->w2_packed_bytes;
        if (s < d + nd && d < s + ns) return fail(FCM_ERR_INVALID_ARG, "w2 buffers overlap");
    }
    if (p.kind == FCM_KIND_PWPW) {
        int rc = 0;
        if (w1_src) rc = launch_copy(w1_src, w1_dst, (int64_t)p.K1 * p.C * e, stream);
        if (rc == 0 && w2_src) {
            const int64_t plain = (int64_t)p.K * p.K1 * e;
            rc = launch_copy(w2_src, w2_dst, plain, stream);
            if (rc == 0) rc = launch_pack_pw_blocked(w2_src, (char*)w2_dst + plain, p.K, p.K1, stream);
        }
        if (rc != 0)
            return fail(FCM_ERR_HIP, std::string("weight packing failed: ") +
                                         hipGetErrorString((hipError_t)rc));
        return ok();
    }
    if (p.dtype == FCM_I8) {
        // int8 DW->PW: depthwise [C][R*S] -> [R*S][C]; pointwise [K][C] copied, then the
        // blocked copy in the int8 matrix-operand order
        const int rc = launch_pack_i8(w1_src, w1_dst, w2_src, w2_dst, p.C, p.K, stream);
        if (rc != 0)
            return fail(FCM_ERR_HIP, std::string("weight packing failed: ") +
                                         hipGetErrorString((hipError_t)rc));
        return ok();
    }
    if (prob_has_expansion(p)) {
        // first layer: pointwise [K1][C] copied as is; second: depthwise [K1][R*S] ->
        // [R*S][K1] (PW->DW->PW: the projection's filters are not packed)
        int rc = 0;
        if (w1_src) rc = launch_copy(w1_src, w1_dst, (int64_t)p.K1 * p.C * e, stream);
        if (rc == 0 && w2_src) rc = launch_pack_dw(e, w2_src, w2_dst, p.K1, p.R * p.S, stream);
        if (rc != 0)
            return fail(FCM_ERR_HIP, std::string("weight packing failed: ") +
                                         hipGetErrorString((hipError_t)rc));
        return ok();
    }
    if (w1_src) {
        int rc;
        if (p.kind == FCM_KIND_DWPW) {
            // [C*mult][R*S] -> [R*S][C*mult] (K1 = C * mult)
            rc = launch_pack_dw(e, w1_src, w1_dst, p.K1, p.R * p.S, stream);
        } else {
            rc = launch_pack_conv(e, w1_src, w1_dst, p.K1, p.C, p.R * p.S, stream);
            const int64_t plain = (int64_t)p.K1 * p.R * p.S * p.C * e;
            if (rc == 0 && plan->w1_packed_bytes > plain)
                rc = launch_pack_conv_blocked(w1_src, (char*)w1_dst + plain, p.K1, p.C, stream);
        }
        if (rc != 0)
            return fail(FCM_ERR_HIP, std::string("weight packing failed: ") +
                                         hipGetErrorString((hipError_t)rc));
    }
    if (w2_src) {
        const int64_t plain = (int64_t)p.K * p.K1 * e;
        int rc = launch_copy(w2_src, w2_dst, plain, stream);
        if (rc == 0 && plan->w2_packed_bytes > plain)
            rc = launch_pack_pw_blocked(w2_src, (char*)w2_dst + plain, p.K, p.K1, stream);
        if (rc != 0)
            return fail(FCM_ERR_HIP, std::string("weight copy failed: ") +
                                         hipGetErrorString((hipError_t)rc));
    }
    return ok();
}

fcm_status fcm_dwpw_fwd(const fcm_plan_t* plan, const void* x, const void* w_dw,
                        const float* scale1, const float* bias1, const void* w_pw,
                        const float* scale2, const float* bias2, void* y, void* stream) {
    FCM_TRY(check_plan(plan, FCM_KIND_DWPW));
    FCM_TRY(check_variant(plan));
    FCM_TRY(need(x, "x", 16));
    FCM_TRY(need(w_dw, "w_dw", 16));
    FCM_TRY(need(w_pw, "w_pw", 16));
    FCM_TRY(need(y, "y", 16));
    FCM_TRY(optional(scale1, "scale1"));
    FCM_TRY(optional(bias1, "bias1"));
    FCM_TRY(optional(scale2, "scale2"));
    FCM_TRY(optional(bias2, "bias2"));
    KArgs a = base_args(plan);
    a.x = x;
    a.w1 = w_dw;
    a.s1 = scale1;
    a.b1 = bias1;
    a.w2 = w_pw;
    a.s2 = scale2;
    a.b2 = bias2;
    a.y = y;
    return launch_fused(plan, a, stream);
}

fcm_status fcm_b2b_conv_fwd(const fcm_plan_t* plan, const void* x, const void* w1,
                            const float* scale1, const float* bias1, const void* w2,
                            const float* scale2, const float* bias2, void* y, void* stream) {
    FCM_TRY(check_plan(plan, FCM_KIND_B2B));
    FCM_TRY(check_variant(plan));
    FCM_TRY(need(x, "x", 16));
    FCM_TRY(need(w1, "w1", 16));
    FCM_TRY(need(w2, "w2", 16));
    FCM_TRY(need(y, "y", 16));
    FCM_TRY(optional(scale1, "scale1"));
    FCM_TRY(optional(bias1, "bias1"));
    FCM_TRY(optional(scale2, "scale2"));
    FCM_TRY(optional(bias2, "bias2"));
    KArgs a = base_args(plan);
    a.x = x;
    a.w1 = w1;
    a.s1 = scale1;
    a.b1 = bias1;
    a.w2 = w2;
    a.s2 = scale2;
    a.b2 = bias2;
    a.y = y;
    return launch_fused(plan, a, stream);
}

fcm_status fcm_pwdw_fwd(const fcm_plan_t* plan, const void* x, const void* w_pw,
                        const float* scale1, const float* bias1, const void* w_dw,
                        const float* scale2, const float* bias2, void* y, void* stream) {
    FCM_TRY(check_plan(plan, FCM_KIND_PWDW));
    FCM_TRY(check_variant(plan));
    FCM_TRY(need(x, "x", 16));
    FCM_TRY(need(w_pw, "w_pw", 16));
    FCM_TRY(need(w_dw, "w_dw", 16));
    FCM_TRY(need(y, "y", 16));
    FCM_TRY(optional(scale1, "scale1"));
    FCM_TRY(optional(bias1, "bias1"));
    FCM_TRY(optional(scale2, "scale2"));
    FCM_TRY(optional(bias2, "bias2"));
    KArgs a = base_args(plan);
    a.x = x;
    a.w1 = w_pw;
    a.s1 = scale1;
    a.b1 = bias1;
    a.w2 = w_dw;
    a.s2 = scale2;
    a.b2 = bias2;
    a.y = y;
    return launch_fused(plan, a, stream);
}

fcm_status fcm_pwpw_fwd(const fcm_plan_t* plan, const void* x, const void* w1,
                        const float* scale1, const float* bias1, const void* w2,
                        const float* scale2, const float* bias2, void* y, void* stream) {
    FCM_TRY(check_plan(plan, FCM_KIND_PWPW));
    FCM_TRY(check_variant(plan));
    FCM_TRY(need(x, "x", 16));
    FCM_TRY(need(w1, "w1", 16));
    FCM_TRY(need(w2, "w2", 16));
    FCM_TRY(need(y, "y", 16));
    FCM_TRY(optional(scale1, "scale1"));
    FCM_TRY(optional(bias1, "bias1"));
    FCM_TRY(optional(scale2, "scale2"));
    FCM_TRY(optional(bias2, "bias2"));
    KArgs a = base_args(plan);
    a.x = x;
    a.w1 = w1;
    a.s1 = scale1;
    a.b1 = bias1;
    a.w2 = w2;
    a.s2 = scale2;
    a.b2 = bias2;
    a.y = y;
    return launch_fused(plan, a, stream);
}

fcm_status fcm_pwdwpw_fwd(const fcm_plan_t* plan, const void* x, const void* w1,
                          const float* scale1, const float* bias1, const void* w2,
                          const float* scale2, const float* bias2, const void* w3,
                          const float* scale3, const float* bias3, void* y, void* stream) {
    FCM_TRY(check_plan(plan, FCM_KIND_PWDWPW));
    FCM_TRY(check_variant(plan));
    FCM_TRY(need(x, "x", 16));
    FCM_TRY(need(w1, "w1", 16));
    FCM_TRY(need(w2, "w2", 16));
    FCM_TRY(need(w3, "w3", 16));
    FCM_TRY(need(y, "y", 16));
    FCM_TRY(optional(scale1, "scale1"));
    FCM_TRY(optional(bias1, "bias1"));
    FCM_TRY(optional(scale2, "scale2"));
    FCM_TRY(optional(bias2, "bias2"));
    FCM_TRY(optional(scale3, "scale3"));
    FCM_TRY(optional(bias3, "bias3"));
    KArgs a = base_args(plan);
    a.x = x;
    a.w1 = w1;
    a.s1 = scale1;
    a.b1 = bias1;
    a.w2 = w2;
    a.s2 = scale2;
    a.b2 = bias2;
    a.w3 = w3;
    a.s3 = scale3;
    a.b3 = bias3;
    a.y = y;
    return launch_fused(plan, a, stream);
}

fcm_status fcm_pwdwpw_lbl(const fcm_plan_t* plan, const void* x, const void* w1,
                          const float* scale1, const float* bias1, const void* w2,
                          const float* scale2, const float* bias2, const void* w3,
                          const float* scale3, const float* bias3, void* t1, void* t2, void* y,
                          void* stream) {
    FCM_TRY(check_plan(plan, FCM_KIND_PWDWPW));
    FCM_TRY(need(x, "x", 16));
    FCM_TRY(need(w1, "w1", 16));
    FCM_TRY(need(w2, "w2", 16));
    FCM_TRY(need(w3, "w3", 16));
    FCM_TRY(need(t1, "t1", 16));
    FCM_TRY(need(t2, "t2", 16));
    FCM_TRY(need(y, "y", 16));
    FCM_TRY(optional(scale1, "scale1"));
    FCM_TRY(optional(bias1, "bias1"));
    FCM_TRY(optional(scale2, "scale2"));
    FCM_TRY(optional(bias2, "bias2"));
    FCM_TRY(optional(scale3, "scale3"));
    FCM_TRY(optional(bias3, "bias3"));
    const fcm_problem& p = plan->prob;
    auto launched = [](int rc) {
        return rc == 0 ? ok()
                       : fail(FCM_ERR_HIP, std::string("kernel launch failed: ") +
                                               hipGetErrorString((hipError_t)rc));
    };
    // expansion: every input pixel, C -> K1, epilogue 1
    KArgs a = base_args(plan);
    a.Ho = p.H;
    a.Wo = p.W;
    a.K = p.K1;
    a.act2 = p.act1;
    a.x = x;
    a.w2 = w1;
    a.s2 = scale1;
    a.b2 = bias1;
    a.y = t1;
    a.residual = 0;
    a.num_ktiles = (p.K1 + lbl::PW_KT16 - 1) / lbl::PW_KT16;
    FCM_TRY(launched(launch_pw_lbl(p.dtype, a, stream)));
    // depthwise over the K1-channel expansion, epilogue 2
    a = base_args(plan);
    a.C = p.K1;
    a.act1 = p.act2;
    a.x = t1;
    a.w1 = w2;
    a.s1 = scale2;
    a.b1 = bias2;
    a.y = t2;
    a.residual = 0;
    set_tiles(&a, lbl::DW_TH, lbl::DW_TW, 1, 1);
    FCM_TRY(launched(launch_dw_lbl(p.dtype, p.stride_h, a, stream)));
    // projection K1 -> K, epilogue 3, the shortcut
    a = base_args(plan);
    a.C = p.K1;
    a.act2 = p.act3;
    a.x = t2;
    a.w2 = w3;
    a.s2 = scale3;
    a.b2 = bias3;
    a.res = p.residual ? x : nullptr;
    a.y = y;
    a.num_ktiles = (p.K + lbl::PW_KT16 - 1) / lbl::PW_KT16;
    return launched(launch_pw_lbl(p.dtype, a, stream));
}

// ---- no-allocation layer-by-layer PW->DW->PW -----------------------------------------
// The two intermediates of fcm_pwdwpw_lbl_noalloc live in this file-scope device array
// (one copy per GPU, at its own address).  Host code never uses the array's name as an
// address: the device address comes from hipGetSymbolAddress, once per device with that
// device current, and is kept per device.
static __device__ __align__(256) unsigned char scratch[FCM_NOALLOC_SCRATCH_BYTES];

namespace fcm {
namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// device address of `scratch` on the device that runs `stream` (the current device for
// the null stream)
fcm_status scratch_address(void* stream, void** out) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess)
        return fail(FCM_ERR_HIP, std::string("hipGetDevice failed: ") + hipGetErrorString(e));
    int dev = cur;
    if (stream) {
        hipDevice_t d = 0;
        e = hipStreamGetDevice((hipStream_t)stream, &d);
        if (e != hipSuccess)
            return fail(FCM_ERR_HIP,
                        std::string("hipStreamGetDevice failed: ") + hipGetErrorString(e));
        dev = (int)d;
    }
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(FCM_ERR_UNSUPPORTED, "device index beyond the static scratch table");
    std::lock_guard<std::mutex> guard(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
            return fail(FCM_ERR_HIP, std::string("hipSetDevice failed: ") + hipGetErrorString(e));
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (dev != cur) (void)hipSetDevice(cur);
        if (e != hipSuccess || !ptr)
            return fail(FCM_ERR_HIP, std::string("hipGetSymbolAddress(scratch) failed: ") +
                                         hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return ok();
}
}  // namespace
}  // namespace fcm

fcm_status fcm_pwdwpw_lbl_noalloc(const fcm_plan_t* plan, const void* x, const void* w1,
                                  const float* scale1, const float* bias1, const void* w2,
                                  const float* scale2, const float* bias2, const void* w3,
                                  const float* scale3, const float* bias3, void* y,
                                  void* stream) {
    using namespace fcm;
    FCM_TRY(check_plan(plan, FCM_KIND_PWDWPW));
    if (plan->workspace_bytes > FCM_NOALLOC_SCRATCH_BYTES)
        return fail(FCM_ERR_UNSUPPORTED,
                    "layer-by-layer intermediates need " +
                        std::to_string((long long)plan->workspace_bytes) +
                        " bytes, more than the " +
                        std::to_string((long long)FCM_NOALLOC_SCRATCH_BYTES) +
                        "-byte static scratch of the no-allocation entry point");
    void* base = nullptr;
    FCM_TRY(scratch_address(stream, &base));
    const fcm_problem& p = plan->prob;
    const int e = p.dtype == FCM_F32 ? 4 : p.dtype == FCM_I8 ? 1 : 2;
    const int64_t t1_bytes = (int64_t)p.N * p.H * p.W * p.K1 * e;
    return fcm_pwdwpw_lbl(plan, x, w1, scale1, bias1, w2, scale2, bias2, w3, scale3, bias3,
                          base, (char*)base + t1_bytes, y, stream);
}


fcm_status fcm_tune(const fcm_problem* prob, const fcm_device_spec* spec, int32_t nsets,
                    const void* const* x, const void* w1, const float* scale1,
                    const float* bias1, const void* w2, const float* scale2,
                    const float* bias2, void* const* y, void* stream, int32_t iters,
                    fcm_plan_t* out) {
    if (!out) return fail(FCM_ERR_INVALID_ARG, "plan output pointer is NULL");
    if (iters <= 0) return fail(FCM_ERR_INVALID_ARG, "iters must be positive");
    if (nsets < 1 || !x || !y) return fail(FCM_ERR_INVALID_ARG, "need nsets >= 1 and x, y arrays");
    if (prob && prob->kind == FCM_KIND_PWDWPW)
        return fail(FCM_ERR_INVALID_ARG, "a PW->DW->PW module is tuned with fcm_tune_pwdwpw");
    int call = 0;
    auto run = [&](const fcm_plan_t* pl) {
        const int i = call++ % nsets;
        switch (prob->kind) {
        case FCM_KIND_DWPW:
            return fcm_dwpw_fwd(pl, x[i], w1, scale1, bias1, w2, scale2, bias2, y[i], stream);
        case FCM_KIND_PWDW:
            return fcm_pwdw_fwd(pl, x[i], w1, scale1, bias1, w2, scale2, bias2, y[i], stream);
        case FCM_KIND_PWPW:
            return fcm_pwpw_fwd(pl, x[i], w1, scale1, bias1, w2, scale2, bias2, y[i], stream);
        default:
            return fcm_b2b_conv_fwd(pl, x[i], w1, scale1, bias1, w2, scale2, bias2, y[i],
                                    stream);
        }
    };
    return tune_impl(prob, spec, iters, stream, out, run);
}

fcm_status fcm_tune_pwdwpw(const fcm_problem* prob, const fcm_device_spec* spec, int32_t nsets,
                           const void* const* x, const void* w1, const float* scale1,
                           const float* bias1, const void* w2, const float* scale2,
                           const float* bias2, const void* w3, const float* scale3,
                           const float* bias3, void* const* y, void* stream, int32_t iters,
                           fcm_plan_t* out) {
    if (!out) return fail(FCM_ERR_INVALID_ARG, "plan output pointer is NULL");
    if (iters <= 0) return fail(FCM_ERR_INVALID_ARG, "iters must be positive");
    if (nsets < 1 || !x || !y) return fail(FCM_ERR_INVALID_ARG, "need nsets >= 1 and x, y arrays");
    if (!prob || prob->kind != FCM_KIND_PWDWPW)
        return fail(FCM_ERR_INVALID_ARG, "fcm_tune_pwdwpw takes a PW->DW->PW problem");
    int call = 0;
    auto run = [&](const fcm_plan_t* pl) {
        const int i = call++ % nsets;
        return fcm_pwdwpw_fwd(pl, x[i], w1, scale1, bias1, w2, scale2, bias2, w3, scale3, bias3,
                              y[i], stream);
    };
    return tune_impl(prob, spec, iters, stream, out, run);
}

fcm_status fcm_dw_fwd(const fcm_plan_t* plan, const void* x, const void* w_dw,
                      const float* scale1, const float* bias1, void* t, void* stream) {
    if (!plan) return fail(FCM_ERR_INVALID_ARG, "plan is NULL");
    FCM_TRY(check_plan(plan, plan->prob.kind == FCM_KIND_PWDW ? FCM_KIND_PWDW : FCM_KIND_DWPW));
    FCM_TRY(need(x, "x", 16));
    FCM_TRY(need(w_dw, "w_dw", 16));
    FCM_TRY(need(t, "t", 16));
    FCM_TRY(optional(scale1, "scale1"));
    FCM_TRY(optional(bias1, "bias1"));
    KArgs a = base_args(plan);
    if (plan->prob.kind == FCM_KIND_PWDW) {
        // the second layer of a PW->DW module: depthwise over the K1-channel
        // intermediate with the module's second epilogue
        a.C = plan->prob.K1;
        a.act1 = plan->prob.act2;
    }
    a.x = x;
    a.w1 = w_dw;
    a.s1 = scale1;
    a.b1 = bias1;
    a.y = t;
    if (prob_is_gen(plan->prob)) {
        // the generalised depthwise layer: the plan's variant names the kernel (filter,
        // dilation, multiplier, chunk); one workgroup per (tile, chunk)
        FCM_TRY(check_variant(plan));
        const VariantDesc& v = kVariants[plan->variant];
        // the layer-by-layer depthwise kernel depends on (storage type, stride, filter,
        // dilation, multiplier) only: a plan whose variant has none (a matrix-core variant
        // for dilated taps) takes that of a generalised variant with the same fields
        launch_fn lbl_dw = kImpls[plan->variant].lbl_first;
        for (int i = 0; !lbl_dw && i < kNumVariants; ++i) {
            const VariantDesc& g = kVariants[i];
            if (g.vkind == VK_DWPW_GEN && g.dtype == v.dtype && g.stride == v.stride &&
                g.fs == plan->prob.R && g.dil == prob_dil_h(plan->prob) &&
                g.mult == prob_mult(plan->prob))
                lbl_dw = kImpls[i].lbl_first;
        }
        if (!lbl_dw)
            return fail(FCM_ERR_UNSUPPORTED, "no layer-by-layer kernel for this depthwise layer");
        set_tiles(&a, lbl::DWG_TH, lbl::DWG_TW, 1, 1);
        const int64_t grid =
            (int64_t)a.num_ptiles * ((plan->prob.C + lbl::DWG_CC - 1) / lbl::DWG_CC);
        if (grid > INT32_MAX) return fail(FCM_ERR_UNSUPPORTED, "too many depthwise tiles");
        const int rc = lbl_dw(a, (int)grid, stream);
        if (rc != 0)
            return fail(FCM_ERR_HIP, std::string("kernel launch failed: ") +
                                         hipGetErrorString((hipError_t)rc));
        return ok();
    }
    set_tiles(&a, lbl::DW_TH, lbl::DW_TW, 1, 1);
    const int rc = plan->prob.dtype == FCM_I8
                       ? launch_dw_lbl_i8(plan->prob.stride_h, a, stream)
                       : launch_dw_lbl(plan->prob.dtype, plan->prob.stride_h, a, stream);
    if (rc != 0)
        return fail(FCM_ERR_HIP,
                    std::string("kernel launch failed: ") + hipGetErrorString((hipError_t)rc));
    return ok();
}

fcm_status fcm_pw_fwd(const fcm_plan_t* plan, const void* t, const void* w_pw,
                      const float* scale2, const float* bias2, void* y, void* stream) {
    if (!plan) return fail(FCM_ERR_INVALID_ARG, "plan is NULL");
    FCM_TRY(check_plan(plan, plan->prob.kind));
    FCM_TRY(need(t, "t", 16));
    FCM_TRY(need(w_pw, "w_pw", 16));
    FCM_TRY(need(y, "y", 16));
    FCM_TRY(optional(scale2, "scale2"));
    FCM_TRY(optional(bias2, "bias2"));
    KArgs a = base_args(plan);
    // the 1x1 layer reads the intermediate as its input: [N*Ho*Wo][C or K1]
    // (DW->PW: K1 = C * mult depthwise outputs)
    if (plan->prob.kind == FCM_KIND_B2B || plan->prob.kind == FCM_KIND_PWPW ||
        plan->prob.kind == FCM_KIND_DWPW)
        a.C = plan->prob.K1;
    if (plan->prob.kind == FCM_KIND_PWDW) {
        // the first layer of a PW->DW module: every input pixel, C -> K1, with the
        // module's first epilogue
        a.Ho = plan->prob.H;
        a.Wo = plan->prob.W;
        a.K = plan->prob.K1;
        a.act2 = plan->prob.act1;
    }
    a.x = t;
    a.w2 = w_pw;
    a.s2 = scale2;
    a.b2 = bias2;
    a.y = y;
    const int kt = plan->prob.dtype == FCM_F32 ? lbl::PW_KT32 : lbl::PW_KT16;
    a.num_ktiles = (plan->prob.K + kt - 1) / kt;
    const int rc = plan->prob.dtype == FCM_I8 ? launch_pw_lbl_i8(a, stream)
                                              : launch_pw_lbl(plan->prob.dtype, a, stream);
    if (rc != 0)
        return fail(FCM_ERR_HIP,
                    std::string("kernel launch failed: ") + hipGetErrorString((hipError_t)rc));
    return ok();
}

fcm_status fcm_conv_fwd(const fcm_plan_t* plan, const void* x, const void* w1,
                        const float* scale1, const float* bias1, void* t, void* stream) {
    if (plan && plan->prob.kind == FCM_KIND_PWPW) {
        // the first 1x1 layer of a PW->PW module: C -> K1 over every pixel, epilogue 1
        FCM_TRY(check_plan(plan, FCM_KIND_PWPW));
        FCM_TRY(need(x, "x", 16));
        FCM_TRY(need(w1, "w1", 16));
        FCM_TRY(need(t, "t", 16));
        FCM_TRY(optional(scale1, "scale1"));
        FCM_TRY(optional(bias1, "bias1"));
        KArgs a = base_args(plan);
        a.x = x;
        a.w2 = w1;
        a.s2 = scale1;
        a.b2 = bias1;
        a.act2 = plan->prob.act1;
        a.K = plan->prob.K1;
        a.y = t;
        a.num_ktiles = (plan->prob.K1 + lbl::PW_KT16 - 1) / lbl::PW_KT16;
        const int rc = launch_pw_lbl(plan->prob.dtype, a, stream);
        if (rc != 0)
            return fail(FCM_ERR_HIP,
                        std::string("kernel launch failed: ") + hipGetErrorString((hipError_t)rc));
        return ok();
    }
    FCM_TRY(check_plan(plan, FCM_KIND_B2B));
    FCM_TRY(need(x, "x", 16));
    FCM_TRY(need(w1, "w1", 16));
    FCM_TRY(need(t, "t", 16));
    FCM_TRY(optional(scale1, "scale1"));
    FCM_TRY(optional(bias1, "bias1"));
    KArgs a = base_args(plan);
    a.x = x;
    a.w1 = w1;
    a.s1 = scale1;
    a.b1 = bias1;
    a.y = t;
    set_tiles(&a, lbl::CV_TH, lbl::CV_TW, lbl::CV_KT, plan->prob.K1);
    const int rc = launch_conv_lbl(plan->prob.dtype, plan->prob.stride_h, a, stream);
    if (rc != 0)
        return fail(FCM_ERR_HIP,
                    std::string("kernel launch failed: ") + hipGetErrorString((hipError_t)rc));
    return ok();
}

}  // extern "C"
