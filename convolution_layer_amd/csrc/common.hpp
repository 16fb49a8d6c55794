// common.hpp -- device helpers shared by the gfx950 kernels of the conv2d layer library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convmi {

enum Act : int { ACT_IDENTITY = 0, ACT_RELU = 1, ACT_TANH = 2, ACT_SIGMOID = 3, ACT_GELU = 4 };

// bf16 values travel as raw 16-bit patterns.
typedef uint16_t bf16;

// Problem dimensions as the kernels see them (validated on the host to fit int32).
struct ConvDims {
    int N, H, W, IC, OC, KH, KW, sh, sw, ph, pw, OH, OW;
};

__device__ __forceinline__ float bf16_to_f32(bf16 h) { return __uint_as_float((uint32_t)h << 16); }

typedef __bf16 hw_bf16x2 __attribute__((ext_vector_type(2)));
typedef float hw_floatx2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even: the gfx950 conversion instruction
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16 f32_to_bf16(float f) { return __builtin_bit_cast(bf16, (__bf16)f); }

// Two fp32 values -> two bf16 packed in 32 bits (low half = a), one instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    hw_floatx2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, hw_bf16x2));
}

// Division by a divisor fixed for the whole launch, as a multiply-high and a shift
// (round-up method, Granlund & Montgomery 1994; valid for numerators below 2^31).
struct FastDiv {
    uint32_t d, m, s;
};
inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    const uint64_t m = ((1ull << 32) * ((1ull << s) - d)) / d + 1;
    return FastDiv{d, (uint32_t)m, s};
}
__device__ __forceinline__ int fdiv(int n, const FastDiv& f) {
    return (int)((__umulhi((uint32_t)n, f.m) + (uint32_t)n) >> f.s);
}

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return bf16_to_f32(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return f32_to_bf16(v); }

// Storage round trip: the value a stored T reads back as.
template <typename T> __device__ __forceinline__ float round_trip(float v) { return to_f32(from_f32<T>(v)); }

// tanh(a) = sign(a) * (1 - e) / (1 + e) with e = exp(-2|a|) in (0, 1]: no overflow, and
// the hardware exponential and reciprocal (v_exp_f32, v_rcp_f32) keep it to a handful of
// instructions.  Absolute error stays near fp32 rounding of values of order 1.
__device__ __forceinline__ float fast_tanh(float a) {
    // exp(-2|a|) = 2^(|a| * -2 log2 e): one multiply (with the |.| source modifier) and v_exp_f32
    const float e = __builtin_amdgcn_exp2f(__builtin_fabsf(a) * -2.8853900817779268f);
    const float t = (1.0f - e) * __builtin_amdgcn_rcpf(1.0f + e);
    return __builtin_copysignf(t, a);
}

// 1 / (1 + exp(-a)); the exponential saturates to inf for a < -88, giving 0.
__device__ __forceinline__ float fast_sigmoid(float a) { return __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }

// GELU, tanh form (the @simulatte/doppler "gelu_backward.wgsl" kernel):
// gelu(a) = a/2 (1 + tanh(u)), u = sqrt(2/pi) (a + 0.044715 a^3).  fast_tanh saturates
// to +-1 for large |u| without overflow, so no clamp of u is needed.
constexpr float kGeluK0 = 0.7978845608028654f;  // sqrt(2/pi)
constexpr float kGeluK1 = 0.044715f;
__device__ __forceinline__ float gelu_t(float a) { return fast_tanh(kGeluK0 * __builtin_fmaf(kGeluK1 * a, a * a, a)); }

// act(a)
template <int ACT> __device__ __forceinline__ float act_fwd(float a) {
    if constexpr (ACT == ACT_RELU) return a > 0.0f ? a : 0.0f;
    else if constexpr (ACT == ACT_TANH) return fast_tanh(a);
    else if constexpr (ACT == ACT_SIGMOID) return fast_sigmoid(a);
    else if constexpr (ACT == ACT_GELU) { const float h = 0.5f * a; return __builtin_fmaf(h, gelu_t(a), h); }
    else return a;
}

// d act / d a at a.  relu'(0) = 0.  gelu'(a) = (1 + t)/2 + a/2 (1 - t^2) du/da with
// du/da = sqrt(2/pi) (1 + 3 * 0.044715 a^2) (product and chain rules on the form above).
template <int ACT> __device__ __forceinline__ float act_slope(float a) {
    if constexpr (ACT == ACT_RELU) return a > 0.0f ? 1.0f : 0.0f;
    else if constexpr (ACT == ACT_TANH) { float t = fast_tanh(a); return 1.0f - t * t; }
    else if constexpr (ACT == ACT_SIGMOID) { float s = fast_sigmoid(a); return s * (1.0f - s); }
    else if constexpr (ACT == ACT_GELU) {
        const float t = gelu_t(a);
        const float du = kGeluK0 * __builtin_fmaf(3.0f * kGeluK1 * a, a, 1.0f);
        return __builtin_fmaf(0.5f * a * du, __builtin_fmaf(-t, t, 1.0f), 0.5f + 0.5f * t);
    }
    else return 1.0f;
}

// d act / d a written in terms of the output y = act(a) (identity, relu, tanh, sigmoid):
// 1, [y > 0], 1 - y^2, y (1 - y).  GELU has no such form; callers never pass it.
template <int ACT> __device__ __forceinline__ float act_slope_out(float y) {
    if constexpr (ACT == ACT_RELU) return y > 0.0f ? 1.0f : 0.0f;
    else if constexpr (ACT == ACT_TANH) return __builtin_fmaf(-y, y, 1.0f);
    else if constexpr (ACT == ACT_SIGMOID) return y * (1.0f - y);
    else return 1.0f;
}

// Normalised activation input a = gamma (z - mean) inv_std + beta, in one fixed fp32
// operation order (subtract, multiply, fused multiply-add) shared by every kernel that
// forms it, so the fused epilogues, the separate normalise pass and the backward passes
// agree bit for bit on a (and hence on the activation's derivative at a).
__device__ __forceinline__ float bn_affine(float z, float mean, float inv_std, float gamma, float beta,
                                           float* zhat_out) {
    float zh = (z - mean) * inv_std;
    *zhat_out = zh;
    return __builtin_fmaf(gamma, zh, beta);
}

// Dispatch a runtime activation id to a compile-time template argument.
#define CONVMI_ACT_SWITCH(act, ACTV, ...)                                   \
    switch (act) {                                                          \
    case ACT_RELU: { constexpr int ACTV = ACT_RELU; __VA_ARGS__; } break;   \
    case ACT_TANH: { constexpr int ACTV = ACT_TANH; __VA_ARGS__; } break;   \
    case ACT_SIGMOID: { constexpr int ACTV = ACT_SIGMOID; __VA_ARGS__; } break; \
    case ACT_GELU: { constexpr int ACTV = ACT_GELU; __VA_ARGS__; } break;   \
    default: { constexpr int ACTV = ACT_IDENTITY; __VA_ARGS__; } break;     \
    }

}  // namespace convmi
