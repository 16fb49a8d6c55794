// api.hip -- the extern "C" entry points of include/convmi.h: argument checking, kernel
// selection and launch.  No allocation, no synchronisation: every kernel goes on the
// caller's stream.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/convmi.h"
#include "internal.hpp"

using namespace convmi;

namespace {

thread_local std::string g_last_error;

convmi_status fail(convmi_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

convmi_status hip_fail(hipError_t e, const char* where) {
    return fail(CONVMI_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr int64_t kI32Max = 2147483647LL;

int64_t out_extent(int64_t in, int64_t k, int64_t s, int64_t p) {
    int64_t span = in + 2 * p - k;
    return span < 0 ? 0 : span / s + 1;
}

// Validate a descriptor; fills kernel dims.  `need_bn_params` checks momentum/eps.
convmi_status check_desc(const convmi_desc* d, ConvDims* out) {
    if (!d) return fail(CONVMI_ERR_INVALID_ARG, "desc is NULL");
    if (d->N < 1 || d->H < 1 || d->W < 1 || d->IC < 1 || d->OC < 1 || d->KH < 1 || d->KW < 1)
        return fail(CONVMI_ERR_INVALID_ARG, "sizes must be >= 1 (N=%lld H=%lld W=%lld IC=%lld OC=%lld KH=%lld KW=%lld)",
                    (long long)d->N, (long long)d->H, (long long)d->W, (long long)d->IC, (long long)d->OC,
                    (long long)d->KH, (long long)d->KW);
    if (d->stride_h < 1 || d->stride_w < 1) return fail(CONVMI_ERR_INVALID_ARG, "strides must be >= 1");
    if (d->pad_h < 0 || d->pad_w < 0) return fail(CONVMI_ERR_INVALID_ARG, "padding must be >= 0");
    if (d->dtype != CONVMI_F32 && d->dtype != CONVMI_BF16)
        return fail(CONVMI_ERR_INVALID_ARG, "unknown dtype %d", d->dtype);
    if (d->activation < CONVMI_ACT_IDENTITY || d->activation > CONVMI_ACT_GELU)
        return fail(CONVMI_ERR_INVALID_ARG, "unknown activation %d", d->activation);
    if (d->normalization < CONVMI_NORM_NONE || d->normalization > CONVMI_NORM_GROUP)
        return fail(CONVMI_ERR_INVALID_ARG, "unknown normalization %d", d->normalization);
    if (d->mode != CONVMI_MODE_TRAIN && d->mode != CONVMI_MODE_EVAL)
        return fail(CONVMI_ERR_INVALID_ARG, "unknown mode %d", d->mode);
    if (d->normalization == CONVMI_NORM_BATCH && !(d->momentum >= 0.0f && d->momentum <= 1.0f))
        return fail(CONVMI_ERR_INVALID_ARG, "momentum must be in [0, 1]");
    if (d->normalization != CONVMI_NORM_NONE && !(d->eps > 0.0f))
        return fail(CONVMI_ERR_INVALID_ARG, "eps must be > 0");
    if (d->normalization == CONVMI_NORM_GROUP && (d->groups < 1 || d->OC % d->groups != 0))
        return fail(CONVMI_ERR_INVALID_ARG, "groups (%d) must be >= 1 and divide OC (%lld)", d->groups,
                    (long long)d->OC);
    const int64_t OH = out_extent(d->H, d->KH, d->stride_h, d->pad_h);
    const int64_t OW = out_extent(d->W, d->KW, d->stride_w, d->pad_w);
    if (OH < 1 || OW < 1)
        return fail(CONVMI_ERR_INVALID_ARG, "kernel %lldx%lld does not fit the padded %lldx%lld input",
                    (long long)d->KH, (long long)d->KW, (long long)d->H, (long long)d->W);
    // Index arithmetic inside the kernels is int32 per image and for N*OH*OW rows.
    if (d->H * d->W * d->IC > kI32Max || OH * OW * d->OC > kI32Max || d->N * OH * OW > kI32Max ||
        d->N * d->H * d->W > kI32Max || d->OC * d->KH * d->KW * d->IC > kI32Max ||
        d->stride_h > 65535 || d->stride_w > 65535 || d->pad_h > 65535 || d->pad_w > 65535 ||
        d->H > kI32Max / 4 || d->W > kI32Max / 4)
        return fail(CONVMI_ERR_UNSUPPORTED, "problem exceeds the int32 index limits of the kernels");
    if (out) {
        *out = ConvDims{(int)d->N, (int)d->H, (int)d->W, (int)d->IC, (int)d->OC, (int)d->KH, (int)d->KW,
                        d->stride_h, d->stride_w, d->pad_h, d->pad_w, (int)OH, (int)OW};
    }
    return CONVMI_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

convmi_status need(const void* p, const char* name) {
    if (!p) return fail(CONVMI_ERR_INVALID_ARG, "%s is NULL", name);
    if (!aligned(p, 16)) return fail(CONVMI_ERR_MISALIGNED, "%s is not 16-byte aligned", name);
    return CONVMI_OK;
}

convmi_status need_vec(const float* p, const char* name) {
    if (!p) return fail(CONVMI_ERR_INVALID_ARG, "%s is NULL", name);
    if (!aligned(p, 4)) return fail(CONVMI_ERR_MISALIGNED, "%s is not 4-byte aligned", name);
    return CONVMI_OK;
}

convmi_status check_ws(void* ws, size_t have, size_t want, const char* op) {
    if (want == 0) return CONVMI_OK;
    if (have < want || !ws)
        return fail(CONVMI_ERR_WORKSPACE, "%s needs %zu workspace bytes, got %zu%s", op, want, have,
                    ws ? "" : " (NULL)");
    if (!aligned(ws, 256)) return fail(CONVMI_ERR_MISALIGNED, "workspace is not 256-byte aligned");
    return CONVMI_OK;
}

#define CHECK(expr)                        \
    do {                                   \
        convmi_status _st = (expr);        \
        if (_st != CONVMI_OK) return _st;  \
    } while (0)

int64_t rows_of(const ConvDims& d) { return (int64_t)d.N * d.OH * d.OW; }

// Layer norm and group norm: per-sample statistics over channel groups.
bool per_sample_norm(const convmi_desc* desc) {
    return desc->normalization == CONVMI_NORM_LAYER || desc->normalization == CONVMI_NORM_GROUP;
}
int norm_groups(const convmi_desc* desc) { return desc->normalization == CONVMI_NORM_GROUP ? desc->groups : 1; }

// Per-tile batch-norm statistics of the fused training forward, after its weight copy.
size_t stats_offset(const convmi_desc* desc, const ConvDims& d) { return halo_fwd_ws_bytes(desc->dtype, d); }
size_t stats_bytes(const convmi_desc* desc, const ConvDims& d) {
    return align_up((size_t)halo_fwd_stat_tiles(desc->dtype, d) * 4 * d.OC * sizeof(float), 256);
}

size_t ws_forward(const convmi_desc* desc, const ConvDims& d) {
    size_t a = igemm_fwd_supported(desc->dtype, d) ? igemm_fwd_ws_bytes(desc->dtype, d) : 0;
    size_t b = 0;
    if (desc->normalization != CONVMI_NORM_NONE) {
        b = per_sample_norm(desc) ? grp_stats_ws_bytes(d.N, (int64_t)d.OH * d.OW, d.OC, desc->dtype)
                                  : bn_stats_ws_bytes(rows_of(d), d.OC, desc->dtype);
        if (halo_fwd_supported(desc->dtype, d)) {
            const size_t c = stats_offset(desc, d) + stats_bytes(desc, d);
            if (c > b) b = c;
        }
    }
    return a > b ? a : b;
}
size_t ws_backward_data(const convmi_desc* desc, const ConvDims& d) {
    return igemm_dx_supported(desc->dtype, d) ? igemm_dx_ws_bytes(desc->dtype, d) : 0;
}
size_t ws_backward_weight(const convmi_desc* desc, const ConvDims& d) {
    return igemm_dw_supported(desc->dtype, d) ? igemm_dw_ws_bytes(desc->dtype, d) : 0;
}
size_t ws_bn_stats(const convmi_desc* desc, const ConvDims& d) {
    if (per_sample_norm(desc)) return grp_stats_ws_bytes(d.N, (int64_t)d.OH * d.OW, d.OC, desc->dtype);
    return bn_stats_ws_bytes(rows_of(d), d.OC, desc->dtype);
}
size_t ws_act_bwd(const convmi_desc* desc, const ConvDims& d) {
    if (per_sample_norm(desc))
        return grp_bwd_ws_bytes(d.N, (int64_t)d.OH * d.OW, d.OC, norm_groups(desc), desc->dtype);
    return desc->normalization == CONVMI_NORM_BATCH ? bn_bwd_ws_bytes(rows_of(d), d.OC, desc->dtype) : 0;
}

// backward_full: dz (unless the activation is the identity), then the weight-gradient
// workspace, then the input-gradient one (the two products run concurrently, so they
// cannot share bytes).
size_t dz_bytes_full(const convmi_desc* desc, const ConvDims& d) {
    return desc->activation == CONVMI_ACT_IDENTITY ? 0
                                                   : align_up((size_t)rows_of(d) * d.OC * dtype_size(desc->dtype), 256);
}
size_t ws_backward_full(const convmi_desc* desc, const ConvDims& d) {
    return dz_bytes_full(desc, d) + align_up(ws_backward_weight(desc, d), 256) + ws_backward_data(desc, d);
}

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
    if (!a || !b) return false;
    uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bn && b0 < a0 + an;
}

}  // namespace

#define CONVMI_API __attribute__((visibility("default")))

extern "C" {

CONVMI_API const char* convmi_last_error(void) { return g_last_error.c_str(); }

CONVMI_API const char* convmi_version(void) { return "convmi 0.1 (gfx950)"; }

CONVMI_API convmi_status convmi_output_dims(const convmi_desc* desc, int64_t* OH, int64_t* OW) {
    ConvDims d;
    CHECK(check_desc(desc, &d));
    if (!OH || !OW) return fail(CONVMI_ERR_INVALID_ARG, "OH/OW out-pointers are NULL");
    *OH = d.OH;
    *OW = d.OW;
    return CONVMI_OK;
}

CONVMI_API convmi_status convmi_workspace_size(const convmi_desc* desc, int32_t op, size_t* bytes) {
    ConvDims d;
    CHECK(check_desc(desc, &d));
    if (!bytes) return fail(CONVMI_ERR_INVALID_ARG, "bytes out-pointer is NULL");
    switch (op) {
    case CONVMI_OP_FORWARD: *bytes = ws_forward(desc, d); break;
    case CONVMI_OP_BACKWARD_DATA: *bytes = ws_backward_data(desc, d); break;
    case CONVMI_OP_BACKWARD_WEIGHT: *bytes = ws_backward_weight(desc, d); break;
    case CONVMI_OP_BN_STATS: *bytes = ws_bn_stats(desc, d); break;
    case CONVMI_OP_ACTIVATION_BACKWARD: *bytes = ws_act_bwd(desc, d); break;
    case CONVMI_OP_BACKWARD_FULL: *bytes = ws_backward_full(desc, d); break;
    default: return fail(CONVMI_ERR_INVALID_ARG, "unknown op %d", op);
    }
    return CONVMI_OK;
}

CONVMI_API convmi_status convmi_plan_name(const convmi_desc* desc, int32_t op, char* buf, size_t len) {
    ConvDims d;
    CHECK(check_desc(desc, &d));
    if (!buf || len == 0) return fail(CONVMI_ERR_INVALID_ARG, "buf is NULL or len is 0");
    const int dt = desc->dtype;
    if (op == CONVMI_OP_FORWARD) {
        if (!halo_plan_text(dt, d, true, buf, len))
            snprintf(buf, len, "%s", igemm_fwd_supported(dt, d) ? "implicit gemm" : "direct");
    } else if (op == CONVMI_OP_BACKWARD_DATA) {
        if (!igemm_dx_supported(dt, d))
            snprintf(buf, len, "direct");
        else if (!halo_plan_text(dt, d, false, buf, len))
            snprintf(buf, len, "implicit gemm");
    } else {
        return fail(CONVMI_ERR_INVALID_ARG, "plan names cover the forward and the input gradient, not op %d", op);
    }
    return CONVMI_OK;
}

}  // extern "C"

namespace {

// conv2d_forward after the descriptor check; shared by the allocation-free variant,
// which passes its static scratch array as the workspace.
convmi_status forward_impl(const convmi_desc* desc, const ConvDims& d, const void* x, const void* w,
                           const float* bias, const float* gamma, const float* beta, float* running_mean,
                           float* running_var, float* save_mean, float* save_inv_std, void* z, void* y,
                           void* workspace, size_t workspace_bytes, void* stream) {
    CHECK(need(x, "x"));
    CHECK(need(w, "w"));
    CHECK(need(y, "y"));
    if (bias) CHECK(need_vec(bias, "bias"));
    const bool bn = desc->normalization == CONVMI_NORM_BATCH;
    const bool psn = per_sample_norm(desc);
    const size_t es = dtype_size(desc->dtype);
    const size_t ybytes = (size_t)rows_of(d) * d.OC * es;
    if (bn) {
        CHECK(need(z, "z (required with batch norm)"));
        CHECK(need_vec(gamma, "gamma"));
        CHECK(need_vec(beta, "beta"));
        CHECK(need_vec(save_mean, "save_mean"));
        CHECK(need_vec(save_inv_std, "save_inv_std"));
        if ((running_mean == nullptr) != (running_var == nullptr))
            return fail(CONVMI_ERR_INVALID_ARG, "running_mean and running_var must be both given or both NULL");
        if (desc->mode == CONVMI_MODE_EVAL && running_mean == nullptr)
            return fail(CONVMI_ERR_INVALID_ARG, "evaluation mode normalises with running_mean/running_var: both required");
        if (running_mean) {
            CHECK(need_vec(running_mean, "running_mean"));
            CHECK(need_vec(running_var, "running_var"));
        }
    } else if (psn) {
        CHECK(need(z, "z (required with layer / group norm)"));
        CHECK(need_vec(gamma, "gamma"));
        CHECK(need_vec(beta, "beta"));
        CHECK(need_vec(save_mean, "save_mean"));
        CHECK(need_vec(save_inv_std, "save_inv_std"));
        if (running_mean || running_var)
            return fail(CONVMI_ERR_INVALID_ARG, "layer / group norm keep no running statistics: pass NULL");
    } else if (z) {
        CHECK(need(z, "z"));
    }
    if (z && z == y) return fail(CONVMI_ERR_INVALID_ARG, "z and y must be distinct buffers");
    if (overlaps(y, ybytes, x, (size_t)d.N * d.H * d.W * d.IC * es) || overlaps(z, ybytes, x, (size_t)d.N * d.H * d.W * d.IC * es))
        return fail(CONVMI_ERR_INVALID_ARG, "outputs overlap x");
    CHECK(check_ws(workspace, workspace_bytes, ws_forward(desc, d), "conv2d_forward"));
    hipStream_t s = (hipStream_t)stream;
    const int act = desc->activation;
    hipError_t e;
    // Layer / group norm: z (with per-tile statistics from the stride-1 epilogue when that
    // path runs), the per-sample group statistics, then normalise + activate.
    if (psn) {
        const int G = norm_groups(desc);
        const int64_t S = (int64_t)d.OH * d.OW;
        if (halo_fwd_supported(desc->dtype, d)) {
            float* part = (float*)((char*)workspace + stats_offset(desc, d));
            e = launch_halo_fwd(desc->dtype, x, w, bias, z, nullptr, d, act, workspace, s, nullptr, part);
            if (e != hipSuccess) return hip_fail(e, "conv2d_forward: convolution launch");
            e = launch_grp_tiles_finalize(part, halo_fwd_stat_tiles(desc->dtype, d), d.N, d.OC, G, S, desc->eps,
                                          save_mean, save_inv_std, s);
        } else {
            e = igemm_fwd_supported(desc->dtype, d)
                    ? launch_igemm_fwd(desc->dtype, x, w, bias, z, nullptr, d, act, workspace, s)
                    : launch_conv_fwd_direct(desc->dtype, x, w, bias, z, nullptr, d, act, s);
            if (e != hipSuccess) return hip_fail(e, "conv2d_forward: convolution launch");
            e = launch_grp_stats(desc->dtype, z, d.N, S, d.OC, G, desc->eps, save_mean, save_inv_std, workspace, s);
        }
        if (e != hipSuccess) return hip_fail(e, "conv2d_forward: normalisation statistics launch");
        e = launch_grp_apply(desc->dtype, z, y, d.N, S, d.OC, G, act, gamma, beta, save_mean, save_inv_std, s);
        if (e != hipSuccess) return hip_fail(e, "conv2d_forward: normalise/activate launch");
        return CONVMI_OK;
    }
    // Without batch norm the activation is fused into the convolution's epilogue; so is
    // evaluation-mode batch norm on the input-tile-reuse path (its statistics are known
    // before the convolution runs).
    if (bn && desc->mode == CONVMI_MODE_EVAL && halo_fwd_supported(desc->dtype, d)) {
        e = launch_bn_eval_stats(running_mean, running_var, d.OC, desc->eps, save_mean, save_inv_std, s);
        if (e != hipSuccess) return hip_fail(e, "conv2d_forward: batch-norm statistics launch");
        const float* bn_eval[4] = {save_mean, save_inv_std, gamma, beta};
        e = launch_halo_fwd(desc->dtype, x, w, bias, z, y, d, act, workspace, s, bn_eval);
        if (e != hipSuccess) return hip_fail(e, "conv2d_forward: convolution launch");
        return CONVMI_OK;
    }
    // Training-mode batch norm on the input-tile-reuse path: the convolution's epilogue
    // also reduces per-tile statistics of the stored z, so z is not read again for them.
    if (bn && desc->mode == CONVMI_MODE_TRAIN && halo_fwd_supported(desc->dtype, d)) {
        float* part = (float*)((char*)workspace + stats_offset(desc, d));
        e = launch_halo_fwd(desc->dtype, x, w, bias, z, nullptr, d, act, workspace, s, nullptr, part);
        if (e != hipSuccess) return hip_fail(e, "conv2d_forward: convolution launch");
        e = launch_bn_tiles_finalize(part, halo_fwd_stat_tiles(desc->dtype, d), (int)d.OC, rows_of(d),
                                     desc->momentum, desc->eps, save_mean, save_inv_std, running_mean, running_var, s);
        if (e != hipSuccess) return hip_fail(e, "conv2d_forward: batch-norm statistics launch");
        e = launch_apply_act(desc->dtype, z, y, rows_of(d), d.OC, act, 1, gamma, beta, save_mean, save_inv_std, s);
        if (e != hipSuccess) return hip_fail(e, "conv2d_forward: normalise/activate launch");
        return CONVMI_OK;
    }
    void* conv_y = bn ? nullptr : y;
    if (igemm_fwd_supported(desc->dtype, d))
        e = launch_igemm_fwd(desc->dtype, x, w, bias, z, conv_y, d, act, workspace, s);
    else
        e = launch_conv_fwd_direct(desc->dtype, x, w, bias, z, conv_y, d, act, s);
    if (e != hipSuccess) return hip_fail(e, "conv2d_forward: convolution launch");
    if (bn) {
        if (desc->mode == CONVMI_MODE_EVAL)  // running statistics, left unchanged
            e = launch_bn_eval_stats(running_mean, running_var, d.OC, desc->eps, save_mean, save_inv_std, s);
        else
            e = launch_bn_stats(desc->dtype, z, rows_of(d), d.OC, desc->momentum, desc->eps, save_mean,
                                save_inv_std, running_mean, running_var, workspace, s);
        if (e != hipSuccess) return hip_fail(e, "conv2d_forward: batch-norm statistics launch");
        e = launch_apply_act(desc->dtype, z, y, rows_of(d), d.OC, act, 1, gamma, beta, save_mean, save_inv_std, s);
        if (e != hipSuccess) return hip_fail(e, "conv2d_forward: normalise/activate launch");
    }
    return CONVMI_OK;
}

// Scratch for conv2d_forward_noalloc: one copy per GPU, held until the process ends.
// Host code never passes `scratch` itself to a kernel (in host code the name is a
// host-side stand-in): it uses the device address hipGetSymbolAddress returns, looked
// up once per device.
constexpr size_t kScratchBytes = CONVMI_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of this device's `scratch`, resolved on the first call made with the
// device current.
convmi_status scratch_for_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "conv2d_forward_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(CONVMI_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "conv2d_forward_noalloc: hipGetSymbolAddress(scratch)");
        if (!p || !aligned(p, 256)) return fail(CONVMI_ERR_HIP, "scratch array has no usable device address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return CONVMI_OK;
}

// A second stream per device for conv2d_backward_full: the weight gradient runs there
// while the input gradient runs on the caller's stream, forked and joined with events
// (default priority, non-blocking; created on the device's first such call and kept
// until the process ends).  The mutex covers the whole fork-join enqueue, so the shared
// events are never recorded by two calls at once.
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    std::mutex mu;
};
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];

convmi_status side_stream_for_current_device(SideStream** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "conv2d_backward_full: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(CONVMI_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_side_mu);
    SideStream& ss = g_side[dev];
    if (!ss.join) {
        if (!ss.s && (e = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking)) != hipSuccess)
            return hip_fail(e, "conv2d_backward_full: creating the weight-gradient stream");
        if (!ss.fork && (e = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming)) != hipSuccess)
            return hip_fail(e, "conv2d_backward_full: creating an event");
        if ((e = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming)) != hipSuccess)
            return hip_fail(e, "conv2d_backward_full: creating an event");
    }
    *out = &ss;
    return CONVMI_OK;
}

}  // namespace

extern "C" {

CONVMI_API convmi_status conv2d_forward(const convmi_desc* desc, const void* x, const void* w, const float* bias,
                             const float* gamma, const float* beta, float* running_mean, float* running_var,
                             float* save_mean, float* save_inv_std, void* z, void* y,
                             void* workspace, size_t workspace_bytes, void* stream) {
    ConvDims d;
    CHECK(check_desc(desc, &d));
    return forward_impl(desc, d, x, w, bias, gamma, beta, running_mean, running_var, save_mean, save_inv_std, z, y,
                        workspace, workspace_bytes, stream);
}

CONVMI_API convmi_status conv2d_forward_noalloc(const convmi_desc* desc, const void* x, const void* w,
                                                const float* bias, const float* gamma, const float* beta,
                                                float* running_mean, float* running_var, float* save_mean,
                                                float* save_inv_std, void* z, void* y, void* stream) {
    ConvDims d;
    CHECK(check_desc(desc, &d));
    const size_t want = ws_forward(desc, d);
    if (want > kScratchBytes)
        return fail(CONVMI_ERR_WORKSPACE,
                    "conv2d_forward_noalloc: this layer needs %zu bytes of scratch, above the static limit of %zu; "
                    "use conv2d_forward with a caller-owned workspace",
                    want, kScratchBytes);
    void* ws = nullptr;
    if (want > 0) CHECK(scratch_for_current_device(&ws));
    return forward_impl(desc, d, x, w, bias, gamma, beta, running_mean, running_var, save_mean, save_inv_std, z, y,
                        ws, want, stream);
}

CONVMI_API convmi_status conv2d_backward_data(const convmi_desc* desc, const void* dz, const void* w, void* dx,
                                   void* workspace, size_t workspace_bytes, void* stream) {
    ConvDims d;
    CHECK(check_desc(desc, &d));
    CHECK(need(dz, "dz"));
    CHECK(need(w, "w"));
    CHECK(need(dx, "dx"));
    const size_t es = dtype_size(desc->dtype);
    const size_t dxb = (size_t)d.N * d.H * d.W * d.IC * es;
    if (overlaps(dx, dxb, dz, (size_t)rows_of(d) * d.OC * es) || overlaps(dx, dxb, w, (size_t)d.OC * d.KH * d.KW * d.IC * es))
        return fail(CONVMI_ERR_INVALID_ARG, "dx overlaps an input");
    CHECK(check_ws(workspace, workspace_bytes, ws_backward_data(desc, d), "conv2d_backward_data"));
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = igemm_dx_supported(desc->dtype, d)
                       ? launch_igemm_dx(desc->dtype, dz, w, dx, d, workspace, s)
                       : launch_conv_dx_direct(desc->dtype, dz, w, dx, d, s);
    if (e != hipSuccess) return hip_fail(e, "conv2d_backward_data launch");
    return CONVMI_OK;
}

CONVMI_API convmi_status conv2d_backward_weight(const convmi_desc* desc, const void* x, const void* dz, float* dw,
                                     float* db, int32_t accumulate, void* workspace, size_t workspace_bytes,
                                     void* stream) {
    ConvDims d;
    CHECK(check_desc(desc, &d));
    CHECK(need(x, "x"));
    CHECK(need(dz, "dz"));
    CHECK(need(dw, "dw"));
    if (db) CHECK(need_vec(db, "db"));
    if (accumulate != 0 && accumulate != 1) return fail(CONVMI_ERR_INVALID_ARG, "accumulate must be 0 or 1");
    CHECK(check_ws(workspace, workspace_bytes, ws_backward_weight(desc, d), "conv2d_backward_weight"));
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = igemm_dw_supported(desc->dtype, d)
                       ? launch_igemm_dw(desc->dtype, x, dz, dw, db, accumulate, d, workspace, s)
                       : launch_conv_dw_direct(desc->dtype, x, dz, dw, db, accumulate, d, s);
    if (e != hipSuccess) return hip_fail(e, "conv2d_backward_weight launch");
    return CONVMI_OK;
}

CONVMI_API convmi_status bn_stats_training(const convmi_desc* desc, const void* z, float* save_mean, float* save_inv_std,
                                float* running_mean, float* running_var,
                                void* workspace, size_t workspace_bytes, void* stream) {
    ConvDims d;
    CHECK(check_desc(desc, &d));
    if (desc->normalization == CONVMI_NORM_NONE)
        return fail(CONVMI_ERR_INVALID_ARG, "bn_stats_training needs a normalization");
    if (per_sample_norm(desc)) {
        CHECK(need(z, "z"));
        CHECK(need_vec(save_mean, "save_mean"));
        CHECK(need_vec(save_inv_std, "save_inv_std"));
        if (running_mean || running_var)
            return fail(CONVMI_ERR_INVALID_ARG, "layer / group norm keep no running statistics: pass NULL");
        CHECK(check_ws(workspace, workspace_bytes, ws_bn_stats(desc, d), "bn_stats_training"));
        hipError_t e = launch_grp_stats(desc->dtype, z, d.N, (int64_t)d.OH * d.OW, d.OC, norm_groups(desc), desc->eps,
                                        save_mean, save_inv_std, workspace, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "bn_stats_training launch");
        return CONVMI_OK;
    }
    if (desc->mode != CONVMI_MODE_TRAIN)
        return fail(CONVMI_ERR_INVALID_ARG,
                    "bn_stats_training computes training statistics; in evaluation mode conv2d_forward uses the "
                    "running statistics");
    CHECK(need(z, "z"));
    CHECK(need_vec(save_mean, "save_mean"));
    CHECK(need_vec(save_inv_std, "save_inv_std"));
    if ((running_mean == nullptr) != (running_var == nullptr))
        return fail(CONVMI_ERR_INVALID_ARG, "running_mean and running_var must be both given or both NULL");
    if (running_mean) {
        CHECK(need_vec(running_mean, "running_mean"));
        CHECK(need_vec(running_var, "running_var"));
    }
    CHECK(check_ws(workspace, workspace_bytes, ws_bn_stats(desc, d), "bn_stats_training"));
    hipError_t e = launch_bn_stats(desc->dtype, z, rows_of(d), d.OC, desc->momentum, desc->eps, save_mean,
                                   save_inv_std, running_mean, running_var, workspace, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "bn_stats_training launch");
    return CONVMI_OK;
}

CONVMI_API convmi_status activation_backward(const convmi_desc* desc, const void* z, const void* dy,
                                  const float* gamma, const float* beta,
                                  const float* save_mean, const float* save_inv_std,
                                  void* dz, float* dgamma, float* dbeta, int32_t accumulate,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    ConvDims d;
    CHECK(check_desc(desc, &d));
    CHECK(need(z, "z"));
    CHECK(need(dy, "dy"));
    CHECK(need(dz, "dz"));
    if (accumulate != 0 && accumulate != 1) return fail(CONVMI_ERR_INVALID_ARG, "accumulate must be 0 or 1");
    const size_t bytes = (size_t)rows_of(d) * d.OC * dtype_size(desc->dtype);
    if (dz != dy && overlaps(dz, bytes, dy, bytes)) return fail(CONVMI_ERR_INVALID_ARG, "dz partially overlaps dy");
    if (overlaps(dz, bytes, z, bytes)) return fail(CONVMI_ERR_INVALID_ARG, "dz overlaps z");
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (per_sample_norm(desc)) {
        CHECK(need_vec(gamma, "gamma"));
        CHECK(need_vec(beta, "beta"));
        CHECK(need_vec(save_mean, "save_mean"));
        CHECK(need_vec(save_inv_std, "save_inv_std"));
        if (dgamma) CHECK(need_vec(dgamma, "dgamma"));
        if (dbeta) CHECK(need_vec(dbeta, "dbeta"));
        CHECK(check_ws(workspace, workspace_bytes, ws_act_bwd(desc, d), "activation_backward"));
        e = launch_grp_bwd(desc->dtype, z, dy, dz, d.N, (int64_t)d.OH * d.OW, d.OC, norm_groups(desc),
                           desc->activation, gamma, beta, save_mean, save_inv_std, dgamma, dbeta, accumulate,
                           workspace, s);
    } else if (desc->normalization == CONVMI_NORM_BATCH) {
        CHECK(need_vec(gamma, "gamma"));
        CHECK(need_vec(beta, "beta"));
        CHECK(need_vec(save_mean, "save_mean"));
        CHECK(need_vec(save_inv_std, "save_inv_std"));
        if (dgamma) CHECK(need_vec(dgamma, "dgamma"));
        if (dbeta) CHECK(need_vec(dbeta, "dbeta"));
        CHECK(check_ws(workspace, workspace_bytes, ws_act_bwd(desc, d), "activation_backward"));
        e = launch_bn_bwd(desc->dtype, z, dy, dz, rows_of(d), d.OC, desc->activation, gamma, beta, save_mean,
                          save_inv_std, dgamma, dbeta, accumulate, desc->mode == CONVMI_MODE_EVAL ? 1 : 0,
                          workspace, s);
    } else {
        e = launch_act_bwd(desc->dtype, z, dy, dz, rows_of(d), d.OC, desc->activation, s);
    }
    if (e != hipSuccess) return hip_fail(e, "activation_backward launch");
    return CONVMI_OK;
}

CONVMI_API convmi_status conv2d_backward_full(const convmi_desc* desc, const void* x, const void* w, const void* saved,
                                              int32_t saved_is_output, const void* dy, void* dx, float* dw, float* db,
                                              int32_t accumulate, void* workspace, size_t workspace_bytes,
                                              void* stream) {
    ConvDims d;
    CHECK(check_desc(desc, &d));
    if (desc->normalization != CONVMI_NORM_NONE)
        return fail(CONVMI_ERR_UNSUPPORTED,
                    "conv2d_backward_full takes unnormalised layers; with a normalisation call activation_backward, "
                    "then conv2d_backward_data and conv2d_backward_weight");
    if (saved_is_output != 0 && saved_is_output != 1)
        return fail(CONVMI_ERR_INVALID_ARG, "saved_is_output must be 0 or 1");
    if (saved_is_output && desc->activation == CONVMI_ACT_GELU)
        return fail(CONVMI_ERR_INVALID_ARG, "the GELU derivative is not a function of its output: pass z");
    CHECK(need(x, "x"));
    CHECK(need(w, "w"));
    CHECK(need(saved, saved_is_output ? "y" : "z"));
    CHECK(need(dy, "dy"));
    CHECK(need(dw, "dw"));
    if (dx) CHECK(need(dx, "dx"));
    if (db) CHECK(need_vec(db, "db"));
    if (accumulate != 0 && accumulate != 1) return fail(CONVMI_ERR_INVALID_ARG, "accumulate must be 0 or 1");
    const size_t es = dtype_size(desc->dtype);
    const size_t xb = (size_t)d.N * d.H * d.W * d.IC * es, yb = (size_t)rows_of(d) * d.OC * es;
    if (dx && (overlaps(dx, xb, x, xb) || overlaps(dx, xb, dy, yb) || overlaps(dx, xb, saved, yb) ||
               overlaps(dx, xb, w, (size_t)d.OC * d.KH * d.KW * d.IC * es)))
        return fail(CONVMI_ERR_INVALID_ARG, "dx overlaps an input");
    CHECK(check_ws(workspace, workspace_bytes, ws_backward_full(desc, d), "conv2d_backward_full"));
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    const void* dz = dy;  // identity: act' = 1
    const size_t zb = dz_bytes_full(desc, d);
    if (zb) {
        dz = workspace;
        e = saved_is_output
                ? launch_act_bwd_from_output(desc->dtype, saved, dy, workspace, rows_of(d), d.OC, desc->activation, s)
                : launch_act_bwd(desc->dtype, saved, dy, workspace, rows_of(d), d.OC, desc->activation, s);
        if (e != hipSuccess) return hip_fail(e, "conv2d_backward_full: activation backward launch");
    }
    void* ws_dw = (char*)workspace + zb;
    void* ws_dx = (char*)ws_dw + align_up(ws_backward_weight(desc, d), 256);
    auto weight_gradient = [&](hipStream_t st) {
        return igemm_dw_supported(desc->dtype, d) ? launch_igemm_dw(desc->dtype, x, dz, dw, db, accumulate, d, ws_dw, st)
                                                  : launch_conv_dw_direct(desc->dtype, x, dz, dw, db, accumulate, d, st);
    };
    auto input_gradient = [&](hipStream_t st) {
        return igemm_dx_supported(desc->dtype, d) ? launch_igemm_dx(desc->dtype, dz, w, dx, d, ws_dx, st)
                                                  : launch_conv_dx_direct(desc->dtype, dz, w, dx, d, st);
    };
    if (!dx || !dw_leaves_room(desc->dtype, d)) {
        if ((e = weight_gradient(s)) != hipSuccess) return hip_fail(e, "conv2d_backward_full: weight-gradient launch");
        if (dx && (e = input_gradient(s)) != hipSuccess)
            return hip_fail(e, "conv2d_backward_full: input-gradient launch");
        return CONVMI_OK;
    }
    // Fork: the weight gradient on the side stream, after everything before it on `s`
    // (dz included); the input gradient on `s`.  Join: `s` waits for the side stream, so
    // work the caller enqueues later sees both products.  Only where the weight-gradient
    // workgroups leave room on a CU do the two kernels fill each other's idle slots
    // (c5's backward 105 -> 91 us); elsewhere the fork and join cost more than they save.
    SideStream* side = nullptr;
    CHECK(side_stream_for_current_device(&side));
    std::lock_guard<std::mutex> lock(side->mu);
    if ((e = hipEventRecord(side->fork, s)) != hipSuccess) return hip_fail(e, "conv2d_backward_full: fork event");
    if ((e = hipStreamWaitEvent(side->s, side->fork, 0)) != hipSuccess)
        return hip_fail(e, "conv2d_backward_full: fork wait");
    const hipError_t ew = weight_gradient(side->s);
    // the join is enqueued even when a launch failed, so `s` never runs ahead of the side stream
    const hipError_t ex = input_gradient(s);
    if ((e = hipEventRecord(side->join, side->s)) != hipSuccess) return hip_fail(e, "conv2d_backward_full: join event");
    if ((e = hipStreamWaitEvent(s, side->join, 0)) != hipSuccess) return hip_fail(e, "conv2d_backward_full: join wait");
    if (ew != hipSuccess) return hip_fail(ew, "conv2d_backward_full: weight-gradient launch");
    if (ex != hipSuccess) return hip_fail(ex, "conv2d_backward_full: input-gradient launch");
    return CONVMI_OK;
}

}  // extern "C"
