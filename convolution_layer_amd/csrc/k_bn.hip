// k_bn.hip -- bandwidth-bound kernels of the conv2d training layer for gfx950:
// batch-norm training statistics, normalise + activation, activation backward and the
// batch-norm training backward.
//
// All tensors are [M][C] rows (M = N*OH*OW, channels fastest).  Instead of one
// workgroup per channel reading a column with stride C (the layout of the
// bn_stats_training / bn_training_backward kernels in the rl_tools conv2d CUDA
// listing, "operations_cuda.h"), each workgroup streams a contiguous slab of rows with
// 16-byte loads across all channels, keeps per-lane partial sums, merges its rows in
// LDS in a fixed order and writes one partial per channel; a second small launch merges
// the slab partials per channel in fp64 in a fixed order.  (A single launch whose last
// workgroup merges, signalled through a device-scope atomic, measured several times
// slower here: the cross-XCD fences and atomics cost more than the second launch.)
// Summation order depends only on the shape: results are bitwise reproducible.
#include "internal.hpp"

namespace convmi {
namespace {

constexpr int kThreads = 256;
constexpr int kTargetBlocks = 512;  // row slabs: two workgroups per CU over 256 CUs

template <typename T, int VEC> struct Vec;
template <> struct Vec<float, 4> {
    using raw = float4;
    static __device__ __forceinline__ void load(const float* p, float* v) {
        float4 r = *(const float4*)p;
        v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
    }
    static __device__ __forceinline__ void store(float* p, const float* v) {
        *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
    }
};
template <> struct Vec<bf16, 8> {
    static __device__ __forceinline__ void load(const bf16* p, float* v) {
        uint4 r = *(const uint4*)p;
        uint32_t u[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float(u[j] << 16);
            v[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void store(bf16* p, const float* v) {
        uint32_t u[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) u[j] = (uint32_t)f32_to_bf16(v[2 * j]) | ((uint32_t)f32_to_bf16(v[2 * j + 1]) << 16);
        *(uint4*)p = make_uint4(u[0], u[1], u[2], u[3]);
    }
};
template <typename T> struct Vec<T, 1> {
    static __device__ __forceinline__ void load(const T* p, float* v) { v[0] = to_f32(*p); }
    static __device__ __forceinline__ void store(T* p, const float* v) { *p = from_f32<T>(v[0]); }
};

// Fixed-order merge of `rpi` row groups held in red[r][lane_slot] (any rpi >= 1):
// halve the count each step, adding the upper part onto the lower.  Result in red[0][*].
__device__ __forceinline__ void merge_rows(float* red, int rpi, int width, int r, int slot, int nvals,
                                           bool active) {
    int n = rpi;
    while (n > 1) {
        int h = (n + 1) / 2;
        if (active && r < n - h)
            for (int j = 0; j < nvals; ++j) red[r * width + slot + j] += red[(r + h) * width + slot + j];
        __syncthreads();
        n = h;
    }
}

// Per-slab sums of two quantities per channel over a slab of rows, merged across the
// workgroup's row groups in a fixed order and written to part[c][q][slab] (q = 0, 1).
// Each lane streams UNROLL 16-byte vectors per iteration.  An accumulator with kOut
// also produces one output element per input element (written to `out`, same layout).
template <typename T, int VEC, class Acc>
__device__ __forceinline__ void slab_partials(const T* __restrict__ a, const T* __restrict__ b, int64_t M, int C,
                                              int tpr, int rpi, int64_t rows_per_block, Acc accf,
                                              float* __restrict__ part, float* red, T* out = nullptr) {
    constexpr int UNROLL = 4;
    const int t = threadIdx.x, cv = t % tpr, r = t / tpr;
    const int c0 = (blockIdx.y * tpr + cv) * VEC;
    const bool active = r < rpi && c0 < C;
    const int64_t m0 = (int64_t)blockIdx.x * rows_per_block;
    const int64_t m1 = m0 + rows_per_block < M ? m0 + rows_per_block : M;
    float s1[VEC], s2[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) s1[j] = s2[j] = 0.0f;
    if (active) {
        accf.init(c0);
        int64_t m = m0 + r;
        for (; m + (UNROLL - 1) * rpi < m1; m += UNROLL * rpi) {
            float va[UNROLL][VEC], vb[UNROLL][VEC];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                Vec<T, VEC>::load(a + (m + u * rpi) * C + c0, va[u]);
                if (b) Vec<T, VEC>::load(b + (m + u * rpi) * C + c0, vb[u]);
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                if constexpr (Acc::kOut) {
                    float o[VEC];
                    accf.add_out(va[u], vb[u], s1, s2, o);
                    Vec<T, VEC>::store(out + (m + u * rpi) * C + c0, o);
                } else {
                    accf.add(va[u], vb[u], s1, s2);
                }
            }
        }
        for (; m < m1; m += rpi) {
            float va[VEC], vb[VEC];
            Vec<T, VEC>::load(a + m * C + c0, va);
            if (b) Vec<T, VEC>::load(b + m * C + c0, vb);
            if constexpr (Acc::kOut) {
                float o[VEC];
                accf.add_out(va, vb, s1, s2, o);
                Vec<T, VEC>::store(out + m * C + c0, o);
            } else {
                accf.add(va, vb, s1, s2);
            }
        }
    }
    const int width = tpr * VEC * 2, slot = cv * VEC * 2;
    if (active)
        for (int j = 0; j < VEC; ++j) {
            red[r * width + slot + 2 * j] = s1[j];
            red[r * width + slot + 2 * j + 1] = s2[j];
        }
    __syncthreads();
    merge_rows(red, rpi, width, r, slot, VEC * 2, active);
    if (active && r == 0)
        for (int j = 0; j < VEC; ++j) {
            const int c = c0 + j;
            part[((int64_t)c * 2 + 0) * gridDim.x + blockIdx.x] = red[slot + 2 * j];
            part[((int64_t)c * 2 + 1) * gridDim.x + blockIdx.x] = red[slot + 2 * j + 1];
        }
}

// Shifted sums for the statistics: shift_c = z[0][c] keeps E[(z-s)^2] - E[z-s]^2 free of
// cancellation when |mean| >> std.
template <typename T, int VEC> struct StatsAcc {
    static constexpr bool kOut = false;
    const T* z;
    float sh[VEC];
    __device__ __forceinline__ void init(int c0) { Vec<T, VEC>::load(z + c0, sh); }
    __device__ __forceinline__ void add(const float* v, const float*, float* s1, float* s2) const {
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            const float d = v[j] - sh[j];
            s1[j] += d;
            s2[j] = __builtin_fmaf(d, d, s2[j]);
        }
    }
};

// Sums of dno and dno*zhat for the batch-norm backward.
template <typename T, int VEC, int ACT> struct BwdAcc {
    static constexpr bool kOut = false;
    const float *gamma, *beta, *mean, *inv_std;
    float g[VEC], bt[VEC], mu[VEC], is[VEC];
    __device__ __forceinline__ void init(int c0) {
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            g[j] = gamma[c0 + j]; bt[j] = beta[c0 + j]; mu[j] = mean[c0 + j]; is[j] = inv_std[c0 + j];
        }
    }
    __device__ __forceinline__ void add(const float* zv, const float* gv, float* s1, float* s2) const {
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            float zh;
            const float a = bn_affine(zv[j], mu[j], is[j], g[j], bt[j], &zh);
            const float dno = act_slope<ACT>(a) * gv[j];
            s1[j] += dno;
            s2[j] = __builtin_fmaf(dno, zh, s2[j]);
        }
    }
};

// Evaluation mode: the same sums, and dz = dno * gamma * inv_std in the same pass (the
// statistics are constants, so dz needs no reduction).
template <typename T, int VEC, int ACT> struct EvalBwdAcc {
    static constexpr bool kOut = true;
    const float *gamma, *beta, *mean, *inv_std;
    float g[VEC], bt[VEC], mu[VEC], is[VEC];
    __device__ __forceinline__ void init(int c0) {
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            g[j] = gamma[c0 + j]; bt[j] = beta[c0 + j]; mu[j] = mean[c0 + j]; is[j] = inv_std[c0 + j];
        }
    }
    __device__ __forceinline__ void add_out(const float* zv, const float* gv, float* s1, float* s2,
                                            float* o) const {
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            float zh;
            const float a = bn_affine(zv[j], mu[j], is[j], g[j], bt[j], &zh);
            const float dno = act_slope<ACT>(a) * gv[j];
            s1[j] += dno;
            s2[j] = __builtin_fmaf(dno, zh, s2[j]);
            o[j] = dno * (g[j] * is[j]);
        }
    }
};

// Merge the slab partials per channel in fp64: each workgroup takes a contiguous group of
// channels; for each pass of up to kThreads of them, P2 threads per channel (a power of
// two) take slabs j, j + P2, ... in order and their sums are combined in thread order.
// fin(c, S1, S2) runs once per channel.
template <class Fin>
__device__ __forceinline__ void merge_slabs(const float* __restrict__ part, int slabs, int C, double* dred,
                                            Fin fin) {
    const int t = threadIdx.x;
    const int cpb = (C + gridDim.x - 1) / gridDim.x;  // channels of this workgroup
    const int c_lo = blockIdx.x * cpb, c_hi = c_lo + cpb < C ? c_lo + cpb : C;
    for (int cb = c_lo; cb < c_hi; cb += kThreads) {
        const int pass_c = c_hi - cb < kThreads ? c_hi - cb : kThreads;
        int p2 = 1;
        while (p2 * 2 * pass_c <= kThreads) p2 *= 2;
        const int cl = t / p2, j = t % p2, c = cb + cl;
        const bool own = cl < pass_c;
        double a = 0.0, b = 0.0;
        if (own) {
            const float* p1 = part + (int64_t)c * 2 * slabs;
            for (int k = j; k < slabs; k += p2) {
                a += (double)p1[k];
                b += (double)p1[slabs + k];
            }
        }
        dred[2 * t] = a;
        dred[2 * t + 1] = b;
        __syncthreads();
        for (int h = p2 / 2; h > 0; h >>= 1) {  // fixed-order tree over the P2 partial sums
            if (j < h) {
                dred[2 * t] += dred[2 * (t + h)];
                dred[2 * t + 1] += dred[2 * (t + h) + 1];
            }
            __syncthreads();
        }
        if (own && j == 0) fin(c, dred[2 * t], dred[2 * t + 1]);
        __syncthreads();
    }
}

template <typename T, int VEC>
__global__ __launch_bounds__(kThreads) void bn_stats_partials(const T* __restrict__ z, int64_t M, int C, int tpr,
                                                              int rpi, int64_t rows_per_block,
                                                              float* __restrict__ part) {
    extern __shared__ float red[];
    StatsAcc<T, VEC> acc{z, {}};
    slab_partials<T, VEC>(z, (const T*)nullptr, M, C, tpr, rpi, rows_per_block, acc, part, red);
}

// Statistics from the slab partials (one workgroup per kThreads/P2 channels):
// mean = shift + S1/M, biased var = S2/M - (S1/M)^2 (clamped at 0), inv_std =
// 1/sqrt(var + eps), running statistics with momentum.
template <typename T>
__global__ __launch_bounds__(kThreads) void bn_stats_finalize(const float* __restrict__ part, int slabs, int C,
                                                              const T* __restrict__ z, int64_t M, float momentum,
                                                              float eps, float* __restrict__ mean,
                                                              float* __restrict__ inv_std,
                                                              float* __restrict__ run_mean,
                                                              float* __restrict__ run_var) {
    __shared__ double dred[2 * kThreads];
    merge_slabs(part, slabs, C, dred, [&](int c, double S1, double S2) {
        const double d = S1 / (double)M;
        double var = S2 / (double)M - d * d;
        if (var < 0.0) var = 0.0;
        const double mu = (double)to_f32(z[c]) + d;
        mean[c] = (float)mu;
        inv_std[c] = (float)(1.0 / sqrt(var + (double)eps));
        if (run_mean) {
            run_mean[c] = (float)((1.0 - (double)momentum) * (double)run_mean[c] + (double)momentum * mu);
            run_var[c] = (float)((1.0 - (double)momentum) * (double)run_var[c] + (double)momentum * var);
        }
    });
}

// Statistics from per-tile partials of the convolution epilogue: tile t of channel c
// holds S1 = sum (z - s), S2 = sum (z - s)^2, its shift s and pixel count n at
// part[(c*4 + q)*ntiles + t].  One workgroup per channel; in fp64 and in a fixed order
// (thread j takes tiles j, j + kThreads, ..., then a tree over the threads):
// mean = sum (n*s + S1) / M, then var = sum [S2 - S1^2/n + n*(s + S1/n - mean)^2] / M
// (the tile's squared deviations about its own mean plus its mean's offset), so no
// term cancels.  Running statistics as in bn_stats_finalize.
__global__ __launch_bounds__(kThreads) void bn_tiles_finalize(const float* __restrict__ part, int ntiles, int64_t M,
                                                              float momentum, float eps, float* __restrict__ mean,
                                                              float* __restrict__ inv_std,
                                                              float* __restrict__ run_mean,
                                                              float* __restrict__ run_var) {
    __shared__ double dred[kThreads];
    const int c = blockIdx.x, t = threadIdx.x;
    const float* S1 = part + (int64_t)c * 4 * ntiles;
    const float* S2 = S1 + ntiles;
    const float* SH = S2 + ntiles;
    const float* CN = SH + ntiles;
    auto tree = [&](double v) {  // fixed-order sum over the workgroup; every thread gets it
        dred[t] = v;
        __syncthreads();
        for (int h = kThreads / 2; h > 0; h >>= 1) {
            if (t < h) dred[t] += dred[t + h];
            __syncthreads();
        }
        const double r = dred[0];
        __syncthreads();
        return r;
    };
    double a = 0.0;
    for (int j = t; j < ntiles; j += kThreads) a += (double)CN[j] * (double)SH[j] + (double)S1[j];
    const double mu = tree(a) / (double)M;
    double b = 0.0;
    for (int j = t; j < ntiles; j += kThreads) {
        const double n = (double)CN[j], s1 = (double)S1[j];
        const double dm = (double)SH[j] + s1 / n - mu;
        b += ((double)S2[j] - s1 * s1 / n) + n * dm * dm;
    }
    double var = tree(b) / (double)M;
    if (var < 0.0) var = 0.0;
    if (t == 0) {
        mean[c] = (float)mu;
        inv_std[c] = (float)(1.0 / sqrt(var + (double)eps));
        if (run_mean) {
            run_mean[c] = (float)((1.0 - (double)momentum) * (double)run_mean[c] + (double)momentum * mu);
            run_var[c] = (float)((1.0 - (double)momentum) * (double)run_var[c] + (double)momentum * var);
        }
    }
}

// Batch-norm backward, first launch: slab partials of A = sum dno and B = sum dno*zhat.
template <typename T, int VEC, int ACT>
__global__ __launch_bounds__(kThreads) void bn_bwd_partials(const T* __restrict__ z, const T* __restrict__ dy,
                                                            int64_t M, int C, int tpr, int rpi, int64_t rows_per_block,
                                                            const float* __restrict__ gamma,
                                                            const float* __restrict__ beta,
                                                            const float* __restrict__ mean,
                                                            const float* __restrict__ inv_std,
                                                            float* __restrict__ part) {
    extern __shared__ float red[];
    BwdAcc<T, VEC, ACT> acc{gamma, beta, mean, inv_std, {}, {}, {}, {}};
    slab_partials<T, VEC>(z, dy, M, C, tpr, rpi, rows_per_block, acc, part, red);
}

// Evaluation-mode batch-norm backward, first launch: dz and the slab partials of
// A = sum dno and B = sum dno*zhat in one pass over z and dy.
template <typename T, int VEC, int ACT>
__global__ __launch_bounds__(kThreads) void bn_bwd_eval(const T* __restrict__ z, const T* dy, T* dz, int64_t M, int C,
                                                        int tpr, int rpi, int64_t rows_per_block,
                                                        const float* __restrict__ gamma,
                                                        const float* __restrict__ beta,
                                                        const float* __restrict__ mean,
                                                        const float* __restrict__ inv_std,
                                                        float* __restrict__ part) {
    extern __shared__ float red[];
    EvalBwdAcc<T, VEC, ACT> acc{gamma, beta, mean, inv_std, {}, {}, {}, {}};
    slab_partials<T, VEC>(z, dy, M, C, tpr, rpi, rows_per_block, acc, part, red, dz);
}

// Second launch: dgamma (+)= B, dbeta (+)= A and the coefficients of
// dz = gamma*inv_std*(dno - A/M - zhat*B/M) into coef[c][3].  In evaluation mode the
// statistics are constants and dz = gamma*inv_std*dno: the two mean terms are zero.
__global__ __launch_bounds__(kThreads) void bn_bwd_finalize(const float* __restrict__ part, int slabs, int C, int64_t M,
                                                            const float* __restrict__ gamma,
                                                            const float* __restrict__ inv_std,
                                                            float* __restrict__ dgamma, float* __restrict__ dbeta,
                                                            int accumulate, int evaluation,
                                                            float* __restrict__ coef) {
    __shared__ double dred[2 * kThreads];
    merge_slabs(part, slabs, C, dred, [&](int c, double A, double B) {
        if (dgamma) dgamma[c] = accumulate ? (float)((double)dgamma[c] + B) : (float)B;
        if (dbeta) dbeta[c] = accumulate ? (float)((double)dbeta[c] + A) : (float)A;
        coef[3 * c + 0] = gamma[c] * inv_std[c];
        coef[3 * c + 1] = evaluation ? 0.0f : (float)(A / (double)M);
        coef[3 * c + 2] = evaluation ? 0.0f : (float)(B / (double)M);
    });
}

// Evaluation-mode statistics: mean = running_mean, inv_std = 1/sqrt(running_var + eps)
// (in fp64, then stored in fp32); the running statistics are left unchanged.
__global__ __launch_bounds__(kThreads) void bn_eval_stats(const float* __restrict__ run_mean,
                                                          const float* __restrict__ run_var, int C, float eps,
                                                          float* __restrict__ mean, float* __restrict__ inv_std) {
    const int c = blockIdx.x * kThreads + threadIdx.x;
    if (c >= C) return;
    mean[c] = run_mean[c];
    inv_std[c] = (float)(1.0 / sqrt((double)run_var[c] + (double)eps));
}

// y = act(a) with a = z or the batch-norm affine; grid-stride over 16-byte vectors.
template <typename T, int VEC, int ACT, bool BN>
__global__ __launch_bounds__(kThreads) void apply_act(const T* __restrict__ z, T* __restrict__ y, int64_t nvec, int C,
                                                      const float* __restrict__ gamma,
                                                      const float* __restrict__ beta,
                                                      const float* __restrict__ mean,
                                                      const float* __restrict__ inv_std) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    // channel of the first element, stepped by the grid stride (the per-channel
    // parameters are reloaded only when it changes: never, when C divides the stride)
    int c0 = (int)((v * VEC) % C), cached = -1;
    const int step = (int)((stride * VEC) % C);
    float mu[VEC], is[VEC], g[VEC], bt[VEC];
    for (; v < nvec; v += stride) {
        float a[VEC];
        Vec<T, VEC>::load(z + v * VEC, a);
        if constexpr (BN) {
            if (c0 != cached) {
#pragma unroll
                for (int j = 0; j < VEC; ++j) {
                    mu[j] = mean[c0 + j]; is[j] = inv_std[c0 + j]; g[j] = gamma[c0 + j]; bt[j] = beta[c0 + j];
                }
                cached = c0;
            }
        }
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            float in = a[j];
            if constexpr (BN) {
                float zh;
                in = bn_affine(in, mu[j], is[j], g[j], bt[j], &zh);
            }
            a[j] = act_fwd<ACT>(in);
        }
        Vec<T, VEC>::store(y + v * VEC, a);
        c0 += step;
        if (c0 >= C) c0 -= C;
    }
}

// dz = act'(z) * dy, no norm.
template <typename T, int VEC, int ACT>
__global__ __launch_bounds__(kThreads) void act_bwd(const T* __restrict__ z, const T* dy, T* dz, int64_t nvec) {
    for (int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x; v < nvec; v += (int64_t)gridDim.x * kThreads) {
        float a[VEC], g[VEC];
        Vec<T, VEC>::load(z + v * VEC, a);
        Vec<T, VEC>::load(dy + v * VEC, g);
#pragma unroll
        for (int j = 0; j < VEC; ++j) g[j] *= act_slope<ACT>(a[j]);
        Vec<T, VEC>::store(dz + v * VEC, g);
    }
}

// Third launch: dz = k0*(dno - k1 - zhat*k2) elementwise.
template <typename T, int VEC, int ACT>
__global__ __launch_bounds__(kThreads) void bn_bwd_apply(const T* __restrict__ z, const T* dy, T* dz, int64_t nvec,
                                                         int C, const float* __restrict__ gamma,
                                                         const float* __restrict__ beta,
                                                         const float* __restrict__ mean,
                                                         const float* __restrict__ inv_std,
                                                         const float* __restrict__ coef) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    int c0 = (int)((v * VEC) % C), cached = -1;
    const int step = (int)((stride * VEC) % C);
    float mu[VEC], is[VEC], g[VEC], bt[VEC], k0[VEC], k1[VEC], k2[VEC];
    for (; v < nvec; v += stride) {
        float zv[VEC], gv[VEC];
        Vec<T, VEC>::load(z + v * VEC, zv);
        Vec<T, VEC>::load(dy + v * VEC, gv);
        if (c0 != cached) {
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                const int c = c0 + j;
                mu[j] = mean[c]; is[j] = inv_std[c]; g[j] = gamma[c]; bt[j] = beta[c];
                k0[j] = coef[3 * c]; k1[j] = coef[3 * c + 1]; k2[j] = coef[3 * c + 2];
            }
            cached = c0;
        }
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            float zh, a = bn_affine(zv[j], mu[j], is[j], g[j], bt[j], &zh);
            float dno = act_slope<ACT>(a) * gv[j];
            gv[j] = k0[j] * (dno - k1[j] - zh * k2[j]);
        }
        Vec<T, VEC>::store(dz + v * VEC, gv);
        c0 += step;
        if (c0 >= C) c0 -= C;
    }
}

int elementwise_grid(int64_t nvec) {
    int64_t g = ceil_div(nvec, kThreads * 4);  // ~4 vectors per thread
    if (g < 1) g = 1;
    if (g > 8192) g = 8192;
    return (int)g;
}

size_t partial_bytes(const RowPlan& p, int C) { return align_up((size_t)C * 2 * p.blocks * sizeof(float), 256); }

// Workgroups for the per-channel merge: up to 64 channels each, at least 64 workgroups
// when there are that many channels.
int merge_grid(int C) {
    int g = (int)ceil_div(C, 64);
    const int g2 = C < 64 ? C : 64;
    return g > g2 ? g : g2;
}

}  // namespace

RowPlan row_plan(int64_t M, int C, int dt) {
    RowPlan p;
    const int full = dt == DT_BF16 ? 8 : 4;
    p.vec = (C % full == 0) ? full : 1;
    const int cv = C / p.vec;
    p.tpr = cv < kThreads ? cv : kThreads;
    p.rpi = kThreads / p.tpr;
    p.chunks = (int)ceil_div(cv, p.tpr);
    int64_t rpb = ceil_div(M, kTargetBlocks);
    rpb = ceil_div(rpb, p.rpi) * p.rpi;
    if (rpb < p.rpi) rpb = p.rpi;
    p.rows_per_block = rpb;
    p.blocks = (int)ceil_div(M, rpb);
    return p;
}

size_t bn_stats_ws_bytes(int64_t M, int C, int dt) { return partial_bytes(row_plan(M, C, dt), C); }

size_t bn_bwd_ws_bytes(int64_t M, int C, int dt) {
    return partial_bytes(row_plan(M, C, dt), C) + align_up((size_t)C * 3 * sizeof(float), 256);
}

#define CONVMI_VEC_SWITCH(dt, vec, T, VEC, ...)                                  \
    if (dt == DT_BF16) {                                                         \
        using T = bf16;                                                          \
        if (vec == 8) { constexpr int VEC = 8; __VA_ARGS__; }                    \
        else { constexpr int VEC = 1; __VA_ARGS__; }                             \
    } else {                                                                     \
        using T = float;                                                         \
        if (vec == 4) { constexpr int VEC = 4; __VA_ARGS__; }                    \
        else { constexpr int VEC = 1; __VA_ARGS__; }                             \
    }

hipError_t launch_bn_stats(int dt, const void* z, int64_t M, int C, float momentum, float eps, float* mean,
                           float* inv_std, float* run_mean, float* run_var, void* ws, hipStream_t s) {
    RowPlan p = row_plan(M, C, dt);
    float* part = (float*)ws;
    dim3 grid(p.blocks, p.chunks), block(kThreads);
    size_t lds = (size_t)p.rpi * p.tpr * p.vec * 2 * sizeof(float);
    CONVMI_VEC_SWITCH(dt, p.vec, T, VEC,
                      (bn_stats_partials<T, VEC><<<grid, block, lds, s>>>((const T*)z, M, C, p.tpr, p.rpi,
                                                                          p.rows_per_block, part)));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (dt == DT_BF16)
        bn_stats_finalize<bf16><<<merge_grid(C), block, 0, s>>>(part, p.blocks, C, (const bf16*)z, M, momentum, eps,
                                                                mean, inv_std, run_mean, run_var);
    else
        bn_stats_finalize<float><<<merge_grid(C), block, 0, s>>>(part, p.blocks, C, (const float*)z, M, momentum,
                                                                 eps, mean, inv_std, run_mean, run_var);
    return hipGetLastError();
}

hipError_t launch_apply_act(int dt, const void* z, void* y, int64_t M, int C, int act, int norm,
                            const float* gamma, const float* beta, const float* mean, const float* inv_std,
                            hipStream_t s) {
    const int full = dt == DT_BF16 ? 8 : 4;
    const int vec = (C % full == 0) ? full : 1;
    const int64_t nvec = M * C / vec;
    dim3 grid(elementwise_grid(nvec)), block(kThreads);
    CONVMI_VEC_SWITCH(dt, vec, T, VEC, CONVMI_ACT_SWITCH(act, A, {
        if (norm)
            apply_act<T, VEC, A, true><<<grid, block, 0, s>>>((const T*)z, (T*)y, nvec, C, gamma, beta, mean, inv_std);
        else
            apply_act<T, VEC, A, false><<<grid, block, 0, s>>>((const T*)z, (T*)y, nvec, C, gamma, beta, mean, inv_std);
    }));
    return hipGetLastError();
}

hipError_t launch_act_bwd(int dt, const void* z, const void* dy, void* dz, int64_t M, int C, int act,
                          hipStream_t s) {
    const int full = dt == DT_BF16 ? 8 : 4;
    const int vec = (C % full == 0) ? full : 1;
    const int64_t nvec = M * C / vec;
    dim3 grid(elementwise_grid(nvec)), block(kThreads);
    CONVMI_VEC_SWITCH(dt, vec, T, VEC, CONVMI_ACT_SWITCH(act, A, (act_bwd<T, VEC, A><<<grid, block, 0, s>>>(
                                                                   (const T*)z, (const T*)dy, (T*)dz, nvec))));
    return hipGetLastError();
}

hipError_t launch_bn_tiles_finalize(const float* part, int ntiles, int C, int64_t M, float momentum, float eps,
                                    float* mean, float* inv_std, float* run_mean, float* run_var, hipStream_t s) {
    bn_tiles_finalize<<<C, kThreads, 0, s>>>(part, ntiles, M, momentum, eps, mean, inv_std, run_mean, run_var);
    return hipGetLastError();
}

hipError_t launch_bn_eval_stats(const float* run_mean, const float* run_var, int C, float eps, float* mean,
                                float* inv_std, hipStream_t s) {
    bn_eval_stats<<<(C + kThreads - 1) / kThreads, kThreads, 0, s>>>(run_mean, run_var, C, eps, mean, inv_std);
    return hipGetLastError();
}

hipError_t launch_bn_bwd(int dt, const void* z, const void* dy, void* dz, int64_t M, int C, int act,
                         const float* gamma, const float* beta, const float* mean, const float* inv_std,
                         float* dgamma, float* dbeta, int accumulate, int evaluation, void* ws, hipStream_t s) {
    RowPlan p = row_plan(M, C, dt);
    float* part = (float*)ws;
    float* coef = (float*)((char*)ws + partial_bytes(p, C));
    dim3 grid(p.blocks, p.chunks), block(kThreads);
    size_t lds = (size_t)p.rpi * p.tpr * p.vec * 2 * sizeof(float);
    if (evaluation) {  // one pass for dz and the partials, then dgamma / dbeta
        CONVMI_VEC_SWITCH(dt, p.vec, T, VEC, CONVMI_ACT_SWITCH(act, A, (bn_bwd_eval<T, VEC, A><<<grid, block, lds, s>>>(
                                                                          (const T*)z, (const T*)dy, (T*)dz, M, C,
                                                                          p.tpr, p.rpi, p.rows_per_block, gamma, beta,
                                                                          mean, inv_std, part))));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        bn_bwd_finalize<<<merge_grid(C), block, 0, s>>>(part, p.blocks, C, M, gamma, inv_std, dgamma, dbeta,
                                                        accumulate, 1, coef);
        return hipGetLastError();
    }
    CONVMI_VEC_SWITCH(dt, p.vec, T, VEC, CONVMI_ACT_SWITCH(act, A, (bn_bwd_partials<T, VEC, A><<<grid, block, lds, s>>>(
                                                                      (const T*)z, (const T*)dy, M, C, p.tpr, p.rpi,
                                                                      p.rows_per_block, gamma, beta, mean, inv_std,
                                                                      part))));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    bn_bwd_finalize<<<merge_grid(C), block, 0, s>>>(part, p.blocks, C, M, gamma, inv_std, dgamma, dbeta, accumulate,
                                                    evaluation, coef);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nvec = M * C / p.vec;
    dim3 g2(elementwise_grid(nvec));
    CONVMI_VEC_SWITCH(dt, p.vec, T, VEC, CONVMI_ACT_SWITCH(act, A, (bn_bwd_apply<T, VEC, A><<<g2, block, 0, s>>>(
                                                                      (const T*)z, (const T*)dy, (T*)dz, nvec, C,
                                                                      gamma, beta, mean, inv_std, coef))));
    return hipGetLastError();
}

}  // namespace convmi
