// common.hpp -- device helpers shared by the gfx950 kernels of the conv2d layer library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convmi {

enum Act : int { ACT_IDENTITY = 0, ACT_RELU = 1, ACT_TANH = 2, ACT_SIGMOID = 3 };

// bf16 values travel as raw 16-bit patterns.
typedef uint16_t bf16;

// Problem dimensions as the kernels see them (validated on the host to fit int32).
struct ConvDims {
    int N, H, W, IC, OC, KH, KW, sh, sw, ph, pw, OH, OW;
};

__device__ __forceinline__ float bf16_to_f32(bf16 h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ bf16 f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (bf16)(u >> 16);
}

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return bf16_to_f32(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return f32_to_bf16(v); }

// Storage round trip: the value a stored T reads back as.
template <typename T> __device__ __forceinline__ float round_trip(float v) { return to_f32(from_f32<T>(v)); }

// act(a).  tanh and the exponential come from the device math library.
template <int ACT> __device__ __forceinline__ float act_fwd(float a) {
    if constexpr (ACT == ACT_RELU) return a > 0.0f ? a : 0.0f;
    else if constexpr (ACT == ACT_TANH) return tanhf(a);
    else if constexpr (ACT == ACT_SIGMOID) return 1.0f / (1.0f + expf(-a));
    else return a;
}

// d act / d a at a.  relu'(0) = 0.
template <int ACT> __device__ __forceinline__ float act_slope(float a) {
    if constexpr (ACT == ACT_RELU) return a > 0.0f ? 1.0f : 0.0f;
    else if constexpr (ACT == ACT_TANH) { float t = tanhf(a); return 1.0f - t * t; }
    else if constexpr (ACT == ACT_SIGMOID) { float s = 1.0f / (1.0f + expf(-a)); return s * (1.0f - s); }
    else return 1.0f;
}

// Batch-norm activation input, in a fixed fp32 operation order (subtract, multiply,
// fused multiply-add) so the ReLU mask can be reproduced exactly off the GPU.
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
    default: { constexpr int ACTV = ACT_IDENTITY; __VA_ARGS__; } break;     \
    }

}  // namespace convmi
