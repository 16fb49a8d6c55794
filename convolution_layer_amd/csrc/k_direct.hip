// k_direct.hip -- general-shape conv2d kernels for gfx950: one thread per output element.
//
// These take any channel count, kernel size, stride and padding.  The library uses
// them for layers too small or too irregular for the tiled MFMA kernels (e.g. three
// input channels) and they define the fallback behaviour for every shape the ABI
// accepts.  Accumulation is fp32; loops follow the operation definitions of the
// rl_tools conv2d generic listing ("operations_generic.h": forward, backward_input,
// backward).
#include "internal.hpp"

namespace convmi {
namespace {

constexpr int kThreads = 256;

// z = b + sum w*x over in-range taps; y = act(stored z).  One thread per (n,oh,ow,oc),
// oc fastest so a wave reads one weight row set and broadcasts the input pixel.
template <typename T, int ACT>
__global__ __launch_bounds__(kThreads) void conv_fwd_direct(const T* __restrict__ x, const T* __restrict__ w,
                                                            const float* __restrict__ bias, T* __restrict__ z,
                                                            T* __restrict__ y, ConvDims d, int64_t total) {
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kThreads) {
        int oc = (int)(i % d.OC);
        int64_t t = i / d.OC;
        int ow = (int)(t % d.OW);
        t /= d.OW;
        int oh = (int)(t % d.OH);
        int n = (int)(t / d.OH);
        float acc = bias ? bias[oc] : 0.0f;
        for (int kh = 0; kh < d.KH; ++kh) {
            int ih = oh * d.sh - d.ph + kh;
            if (ih < 0 || ih >= d.H) continue;
            for (int kw = 0; kw < d.KW; ++kw) {
                int iw = ow * d.sw - d.pw + kw;
                if (iw < 0 || iw >= d.W) continue;
                const T* xp = x + (((int64_t)n * d.H + ih) * d.W + iw) * d.IC;
                const T* wp = w + (((int64_t)oc * d.KH + kh) * d.KW + kw) * d.IC;
                for (int ic = 0; ic < d.IC; ++ic) acc = __builtin_fmaf(to_f32(wp[ic]), to_f32(xp[ic]), acc);
            }
        }
        T zs = from_f32<T>(acc);
        if (z) z[i] = zs;
        if (y) y[i] = from_f32<T>(act_fwd<ACT>(to_f32(zs)));
    }
}

// dx[n,ih,iw,ic] = sum over taps landing on (ih,iw) of w*dz (gather form of the
// scatter in backward_input).  ic fastest: a wave shares the dz pixel.  Eight lanes
// share an element and split its output channels (lane j takes oc = j, j + 8, ...); the
// eight partial sums are added across the lanes in a butterfly in which every lane adds
// the same pairs (IEEE addition is commutative), so the result depends only on the data.
// The chain per lane is an eighth as long as with one lane per element.
constexpr int kDxLanes = 8;

template <typename T>
__global__ __launch_bounds__(kThreads) void conv_dx_direct(const T* __restrict__ dz, const T* __restrict__ w,
                                                           T* __restrict__ dx, ConvDims d, int64_t total) {
    const int j = threadIdx.x & (kDxLanes - 1);
    const int64_t step = (int64_t)gridDim.x * (kThreads / kDxLanes);
    // the loop bound is uniform over each group of eight lanes (same element)
    for (int64_t i = ((int64_t)blockIdx.x * kThreads + threadIdx.x) / kDxLanes; i < total; i += step) {
        int ic = (int)(i % d.IC);
        int64_t t = i / d.IC;
        int iw = (int)(t % d.W);
        t /= d.W;
        int ih = (int)(t % d.H);
        int n = (int)(t / d.H);
        float acc = 0.0f;
        for (int kh = 0; kh < d.KH; ++kh) {
            int th = ih + d.ph - kh;
            if (th < 0 || th % d.sh) continue;
            int oh = th / d.sh;
            if (oh >= d.OH) continue;
            for (int kw = 0; kw < d.KW; ++kw) {
                int tw = iw + d.pw - kw;
                if (tw < 0 || tw % d.sw) continue;
                int ow = tw / d.sw;
                if (ow >= d.OW) continue;
                const T* gp = dz + (((int64_t)n * d.OH + oh) * d.OW + ow) * d.OC;
                const T* wp = w + ((int64_t)kh * d.KW + kw) * d.IC + ic;
                const int64_t wstride = (int64_t)d.KH * d.KW * d.IC;
                for (int oc = j; oc < d.OC; oc += kDxLanes)
                    acc = __builtin_fmaf(to_f32(wp[oc * wstride]), to_f32(gp[oc]), acc);
            }
        }
#pragma unroll
        for (int m = 1; m < kDxLanes; m <<= 1) acc += __shfl_xor(acc, m);
        if (j == 0) dx[i] = from_f32<T>(acc);
    }
}

// Fixed-order tree sum of one value per thread; every thread returns the total.
__device__ float block_sum(float v, float* red) {
    red[threadIdx.x] = v;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
        __syncthreads();
    }
    float r = red[0];
    __syncthreads();
    return r;
}

// One workgroup per dw element (oc, kh, kw, ic): threads stride over the output rows,
// then a fixed-order tree merge.  Row blockIdx.y == 1 computes db[oc] for blocks whose
// (kh, kw, ic) is (0, 0, 0).
template <typename T>
__global__ __launch_bounds__(kThreads) void conv_dw_direct(const T* __restrict__ x, const T* __restrict__ dz,
                                                           float* __restrict__ dw, float* __restrict__ db,
                                                           int accumulate, ConvDims d) {
    __shared__ float red[kThreads];
    const int K = d.KH * d.KW * d.IC;
    const int e = blockIdx.x;  // oc*K + k
    const int oc = e / K, k = e % K;
    const int kh = k / (d.KW * d.IC), kw = (k / d.IC) % d.KW, ic = k % d.IC;
    const int64_t P = (int64_t)d.N * d.OH * d.OW;
    float acc = 0.0f, bacc = 0.0f;
    const bool do_bias = db && k == 0;
    for (int64_t p = threadIdx.x; p < P; p += kThreads) {
        int ow = (int)(p % d.OW);
        int64_t t = p / d.OW;
        int oh = (int)(t % d.OH);
        int n = (int)(t / d.OH);
        float g = to_f32(dz[p * d.OC + oc]);
        bacc += g;
        int ih = oh * d.sh - d.ph + kh, iw = ow * d.sw - d.pw + kw;
        if (ih < 0 || ih >= d.H || iw < 0 || iw >= d.W) continue;
        acc = __builtin_fmaf(g, to_f32(x[(((int64_t)n * d.H + ih) * d.W + iw) * d.IC + ic]), acc);
    }
    float s = block_sum(acc, red);
    if (threadIdx.x == 0) dw[e] = accumulate ? dw[e] + s : s;
    if (do_bias) {
        float sb = block_sum(bacc, red);
        if (threadIdx.x == 0) db[oc] = accumulate ? db[oc] + sb : sb;
    }
}

int grid_for(int64_t total) {
    int64_t g = ceil_div(total, kThreads);
    return (int)(g < 65536 ? (g < 1 ? 1 : g) : 65536);
}

}  // namespace

hipError_t launch_conv_fwd_direct(int dt, const void* x, const void* w, const float* bias, void* z, void* y,
                                  const ConvDims& d, int act, hipStream_t s) {
    int64_t total = (int64_t)d.N * d.OH * d.OW * d.OC;
    dim3 grid(grid_for(total)), block(kThreads);
    if (dt == DT_BF16) {
        CONVMI_ACT_SWITCH(act, A, (conv_fwd_direct<bf16, A><<<grid, block, 0, s>>>(
                                      (const bf16*)x, (const bf16*)w, bias, (bf16*)z, (bf16*)y, d, total)));
    } else {
        CONVMI_ACT_SWITCH(act, A, (conv_fwd_direct<float, A><<<grid, block, 0, s>>>(
                                      (const float*)x, (const float*)w, bias, (float*)z, (float*)y, d, total)));
    }
    return hipGetLastError();
}

hipError_t launch_conv_dx_direct(int dt, const void* dz, const void* w, void* dx, const ConvDims& d,
                                 hipStream_t s) {
    int64_t total = (int64_t)d.N * d.H * d.W * d.IC;
    dim3 grid(grid_for(total * kDxLanes)), block(kThreads);
    if (dt == DT_BF16)
        conv_dx_direct<bf16><<<grid, block, 0, s>>>((const bf16*)dz, (const bf16*)w, (bf16*)dx, d, total);
    else
        conv_dx_direct<float><<<grid, block, 0, s>>>((const float*)dz, (const float*)w, (float*)dx, d, total);
    return hipGetLastError();
}

hipError_t launch_conv_dw_direct(int dt, const void* x, const void* dz, float* dw, float* db, int accumulate,
                                 const ConvDims& d, hipStream_t s) {
    dim3 grid((unsigned)(d.OC * d.KH * d.KW * d.IC)), block(kThreads);
    if (dt == DT_BF16)
        conv_dw_direct<bf16><<<grid, block, 0, s>>>((const bf16*)x, (const bf16*)dz, dw, db, accumulate, d);
    else
        conv_dw_direct<float><<<grid, block, 0, s>>>((const float*)x, (const float*)dz, dw, db, accumulate, d);
    return hipGetLastError();
}

}  // namespace convmi
