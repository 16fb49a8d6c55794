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

// ---------------------------------------------------------------- cross-lane sums
// Lanes l and l + k of a wave64 exchange values without LDS memory: rotations within
// 16-lane rows through DPP (row_ror), the two halves of each 32-lane group through
// ds_swizzle (bit mode, xor 16), the two 32-lane halves through ds_bpermute (xor 32).
__device__ __forceinline__ float dpp_ror(float v, int k) {  // k in {1, 2, 4, 8}; lane i gets lane (i + k) % 16 of its row
    const int x = __builtin_bit_cast(int, v);
    int r;
    switch (k) {
    case 8: r = __builtin_amdgcn_update_dpp(0, x, 0x128, 0xf, 0xf, false); break;
    case 4: r = __builtin_amdgcn_update_dpp(0, x, 0x124, 0xf, 0xf, false); break;
    case 2: r = __builtin_amdgcn_update_dpp(0, x, 0x122, 0xf, 0xf, false); break;
    default: r = __builtin_amdgcn_update_dpp(0, x, 0x121, 0xf, 0xf, false); break;
    }
    return __builtin_bit_cast(float, r);
}
__device__ __forceinline__ float lane_xor16(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), (0x10 << 10) | 0x1f));
}
__device__ __forceinline__ float lane_xor32(float v) {
    const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __builtin_bit_cast(int, v)));
}

// Sum over the lanes of a wave congruent modulo `stride` (a power of two <= 64): every
// lane ends with the sum of its class.  Each lane adds the same terms in the same
// pairing (IEEE addition is commutative), so all lanes of a class agree bit for bit and
// the result depends only on the data.
__device__ __forceinline__ float wave_class_sum(float v, int stride) {
    for (int k = 8; k >= stride && k >= 1; k >>= 1) v += dpp_ror(v, k);
    if (stride <= 16) v += lane_xor16(v);
    if (stride <= 32) v += lane_xor32(v);
    return v;
}

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
// The rows form segments of `seg` rows (one segment of all M rows for batch norm, one
// per sample for layer and group norm), each cut into `bps` slabs of rows_per_block
// rows: slab b covers rows of segment b / bps only.  Each lane streams UNROLL 16-byte
// vectors per iteration.  An accumulator with kOut also produces one output element
// per input element (written to `out`, same layout).
template <typename T, int VEC, class Acc>
__device__ __forceinline__ void slab_partials(const T* __restrict__ a, const T* __restrict__ b, int64_t M, int C,
                                              int tpr, int rpi, int64_t rows_per_block, Acc accf,
                                              float* __restrict__ part, float* red, T* out = nullptr,
                                              int64_t seg = 0, int bps = 0) {
    constexpr int UNROLL = 8;
    const int t = threadIdx.x, cv = t % tpr, r = t / tpr;
    const int c0 = (blockIdx.y * tpr + cv) * VEC;
    const bool active = r < rpi && c0 < C;
    if (seg == 0) {
        seg = M;
        bps = gridDim.x;
    }
    const int sid = (int)(blockIdx.x / bps);
    const int64_t s0 = (int64_t)sid * seg, s1end = s0 + seg < M ? s0 + seg : M;
    const int64_t m0 = s0 + (int64_t)(blockIdx.x - sid * bps) * rows_per_block;
    const int64_t m1 = m0 + rows_per_block < s1end ? m0 + rows_per_block : s1end;
    float s1[VEC], s2[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) s1[j] = s2[j] = 0.0f;
    if (active) {
        accf.init(c0, sid, s0);
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
    if ((tpr & (tpr - 1)) == 0 && tpr <= 64) {
        // The row groups of a wave hold the same channels in lanes tpr apart: sum them
        // across lanes, then the kThreads/64 waves' sums in wave order (one barrier).
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            s1[j] = wave_class_sum(s1[j], tpr);
            s2[j] = wave_class_sum(s2[j], tpr);
        }
        const int lane = t & 63, wv = t >> 6, slot = cv * VEC * 2, width = tpr * VEC * 2;
        if (lane < tpr)
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                red[wv * width + slot + 2 * j] = s1[j];
                red[wv * width + slot + 2 * j + 1] = s2[j];
            }
        __syncthreads();
        if (t < tpr && c0 < C)
            for (int j = 0; j < VEC; ++j) {
                float a = 0.0f, b = 0.0f;
                for (int w = 0; w < kThreads / 64; ++w) {
                    a += red[w * width + slot + 2 * j];
                    b += red[w * width + slot + 2 * j + 1];
                }
                part[((int64_t)(c0 + j) * 2 + 0) * gridDim.x + blockIdx.x] = a;
                part[((int64_t)(c0 + j) * 2 + 1) * gridDim.x + blockIdx.x] = b;
            }
        return;
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
    int C;
    float sh[VEC];
    // shift: the segment's first row
    __device__ __forceinline__ void init(int c0, int, int64_t row0) { Vec<T, VEC>::load(z + row0 * C + c0, sh); }
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
    __device__ __forceinline__ void init(int c0, int, int64_t) {
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
    __device__ __forceinline__ void init(int c0, int, int64_t) {
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
            for (int k0 = j; k0 < slabs; k0 += 8 * p2) {  // eight slabs' loads in flight, then their sums in order
                float va[8], vb[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int k = k0 + u * p2;
                    va[u] = k < slabs ? p1[k] : 0.0f;
                    vb[u] = k < slabs ? p1[slabs + k] : 0.0f;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    a += (double)va[u];
                    b += (double)vb[u];
                }
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
                                                              float* __restrict__ part, int64_t seg, int bps) {
    extern __shared__ float red[];
    StatsAcc<T, VEC> acc{z, C, {}};
    slab_partials<T, VEC>(z, (const T*)nullptr, M, C, tpr, rpi, rows_per_block, acc, part, red, nullptr, seg, bps);
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

// ------------------------------------------------------------ layer norm / group norm
// Statistics per sample n and group g of Cg = C/G consecutive channels (layer norm:
// G = 1), over the S = OH*OW rows of the sample: the rows of a sample form one segment
// of the slab partials, and the merges below combine channels as well as slabs.

// Fixed-order sum over the workgroup; every thread gets the result.
__device__ __forceinline__ double block_sum(double v, double* dred) {
    const int t = threadIdx.x;
    dred[t] = v;
    __syncthreads();
    for (int h = kThreads / 2; h > 0; h >>= 1) {
        if (t < h) dred[t] += dred[t + h];
        __syncthreads();
    }
    const double r = dred[0];
    __syncthreads();
    return r;
}

// Group statistics from the per-sample slab partials (bps slabs per sample; shifts =
// each sample's first row): one workgroup per (n, g).  Channel c of the group:
// mean_c = s_c + S1_c/S, M2_c = S2_c - S1_c^2/S (fp64, slabs in order); then
// mean = sum mean_c / Cg and var = sum [M2_c + S (mean_c - mean)^2] / (S Cg).
template <typename T>
__global__ __launch_bounds__(kThreads) void grp_stats_finalize(const float* __restrict__ part, int bps, int C, int G,
                                                               const T* __restrict__ z, int64_t S, float eps,
                                                               float* __restrict__ mean, float* __restrict__ inv_std) {
    __shared__ double dred[kThreads];
    const int ng = blockIdx.x, n = ng / G, g = ng - n * G, cg = C / G, t = threadIdx.x;
    const int nslab = bps;
    const int64_t total_slabs = (int64_t)nslab * (gridDim.x / G);  // N * bps
    double msum = 0.0;
    for (int k = t; k < cg; k += kThreads) {
        const int c = g * cg + k;
        const float* p1 = part + (int64_t)c * 2 * total_slabs + (int64_t)n * nslab;
        double a = 0.0;
        for (int j = 0; j < nslab; ++j) a += (double)p1[j];
        msum += (double)to_f32(z[(int64_t)n * S * C + c]) + a / (double)S;
    }
    const double mu = block_sum(msum, dred) / (double)cg;
    double m2 = 0.0;
    for (int k = t; k < cg; k += kThreads) {
        const int c = g * cg + k;
        const float* p1 = part + (int64_t)c * 2 * total_slabs + (int64_t)n * nslab;
        double a = 0.0, b = 0.0;
        for (int j = 0; j < nslab; ++j) {
            a += (double)p1[j];
            b += (double)p1[total_slabs + j];
        }
        const double mc = (double)to_f32(z[(int64_t)n * S * C + c]) + a / (double)S;
        m2 += (b - a * a / (double)S) + (double)S * (mc - mu) * (mc - mu);
    }
    double var = block_sum(m2, dred) / ((double)S * cg);
    if (var < 0.0) var = 0.0;
    if (t == 0) {
        mean[ng] = (float)mu;
        inv_std[ng] = (float)(1.0 / sqrt(var + (double)eps));
    }
}

// Group statistics from the per-tile partials of the convolution epilogue (tiles of
// image n are tiles n*tpi .. (n+1)*tpi - 1; see bn_tiles_finalize for the quantities):
// one workgroup per (n, g); thread t takes (tile, channel) pairs t, t + kThreads, ...
__global__ __launch_bounds__(kThreads) void grp_tiles_finalize(const float* __restrict__ part, int ntiles, int tpi,
                                                               int C, int G, int64_t S, float eps,
                                                               float* __restrict__ mean,
                                                               float* __restrict__ inv_std) {
    __shared__ double dred[kThreads];
    const int ng = blockIdx.x, n = ng / G, g = ng - n * G, cg = C / G, t = threadIdx.x;
    const int pairs = tpi * cg;
    const double cnt_all = (double)S * cg;
    double a = 0.0;
    for (int q = t; q < pairs; q += kThreads) {
        const int k = q / tpi, tile = n * tpi + (q - k * tpi), c = g * cg + k;
        const float* p = part + (int64_t)c * 4 * ntiles + tile;
        a += (double)p[3 * (int64_t)ntiles] * (double)p[2 * (int64_t)ntiles] + (double)p[0];
    }
    const double mu = block_sum(a, dred) / cnt_all;
    double b = 0.0;
    for (int q = t; q < pairs; q += kThreads) {
        const int k = q / tpi, tile = n * tpi + (q - k * tpi), c = g * cg + k;
        const float* p = part + (int64_t)c * 4 * ntiles + tile;
        const double cn = (double)p[3 * (int64_t)ntiles], s1 = (double)p[0];
        if (cn > 0.0) {
            const double dm = (double)p[2 * (int64_t)ntiles] + s1 / cn - mu;
            b += ((double)p[ntiles] - s1 * s1 / cn) + cn * dm * dm;
        }
    }
    double var = block_sum(b, dred) / cnt_all;
    if (var < 0.0) var = 0.0;
    if (t == 0) {
        mean[ng] = (float)mu;
        inv_std[ng] = (float)(1.0 / sqrt(var + (double)eps));
    }
}

// Per-element statistics of sample n for channels c0 .. c0 + VEC - 1.
template <int VEC>
__device__ __forceinline__ void grp_params(const float* mean, const float* inv_std, int n, int G, int cg, int c0,
                                           float* mu, float* is) {
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
        const int st = n * G + (c0 + j) / cg;
        mu[j] = mean[st];
        is[j] = inv_std[st];
    }
}

// y = act(gamma_c (z - mean_ng) inv_std_ng + beta_c); grid (blocks per sample, N).
template <typename T, int VEC, int ACT>
__global__ __launch_bounds__(kThreads) void grp_apply(const T* __restrict__ z, T* __restrict__ y, int64_t per_sample,
                                                      int C, int G, const float* __restrict__ gamma,
                                                      const float* __restrict__ beta, const float* __restrict__ mean,
                                                      const float* __restrict__ inv_std) {
    const int n = blockIdx.y, cg = C / G;
    const int64_t nvec = per_sample / VEC, base = (int64_t)n * per_sample;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    int c0 = (int)((v * VEC) % C), cached = -1;
    const int step = (int)((stride * VEC) % C);
    float mu[VEC], is[VEC], g[VEC], bt[VEC];
    for (; v < nvec; v += stride) {
        float a[VEC];
        Vec<T, VEC>::load(z + base + v * VEC, a);
        if (c0 != cached) {
            grp_params<VEC>(mean, inv_std, n, G, cg, c0, mu, is);
#pragma unroll
            for (int j = 0; j < VEC; ++j) { g[j] = gamma[c0 + j]; bt[j] = beta[c0 + j]; }
            cached = c0;
        }
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            float zh;
            a[j] = act_fwd<ACT>(bn_affine(a[j], mu[j], is[j], g[j], bt[j], &zh));
        }
        Vec<T, VEC>::store(y + base + v * VEC, a);
        c0 += step;
        if (c0 >= C) c0 -= C;
    }
}

// Sums of dno and dno*zhat per channel over a slab of one sample's rows, with the
// sample's group statistics.
template <typename T, int VEC, int ACT> struct GrpBwdAcc {
    static constexpr bool kOut = false;
    const float *gamma, *beta, *mean, *inv_std;
    int G, cg;
    float g[VEC], bt[VEC], mu[VEC], is[VEC];
    __device__ __forceinline__ void init(int c0, int n, int64_t) {
        grp_params<VEC>(mean, inv_std, n, G, cg, c0, mu, is);
#pragma unroll
        for (int j = 0; j < VEC; ++j) { g[j] = gamma[c0 + j]; bt[j] = beta[c0 + j]; }
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

template <typename T, int VEC, int ACT>
__global__ __launch_bounds__(kThreads) void grp_bwd_partials(const T* __restrict__ z, const T* __restrict__ dy,
                                                             int64_t M, int C, int tpr, int rpi, int64_t rows_per_block,
                                                             int64_t seg, int bps, int G,
                                                             const float* __restrict__ gamma,
                                                             const float* __restrict__ beta,
                                                             const float* __restrict__ mean,
                                                             const float* __restrict__ inv_std,
                                                             float* __restrict__ part) {
    extern __shared__ float red[];
    GrpBwdAcc<T, VEC, ACT> acc{gamma, beta, mean, inv_std, G, C / G, {}, {}, {}, {}};
    slab_partials<T, VEC>(z, dy, M, C, tpr, rpi, rows_per_block, acc, part, red, nullptr, seg, bps);
}

// Per (n, c): A = sum dno, B = sum dno*zhat over the sample's slabs, in order, as fp64
// into ab[(n*C + c)*2 + {0,1}].
__global__ __launch_bounds__(kThreads) void grp_bwd_merge(const float* __restrict__ part, int bps, int N, int C,
                                                          double* __restrict__ ab) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= (int64_t)N * C) return;
    const int n = (int)(i / C), c = (int)(i - (int64_t)n * C);
    const int64_t slabs = (int64_t)N * bps;
    const float* p1 = part + (int64_t)c * 2 * slabs + (int64_t)n * bps;
    double a = 0.0, b = 0.0;
    for (int j = 0; j < bps; ++j) {
        a += (double)p1[j];
        b += (double)p1[slabs + j];
    }
    ab[2 * i] = a;
    ab[2 * i + 1] = b;
}

// Workgroups 0 .. N*G-1: per (n, g) S1 = sum_c gamma_c A_nc, S2 = sum_c gamma_c B_nc
// (channels of the group, fixed order) -> coef[(n*G + g)*2] = S1/cnt, [+1] = S2/cnt.
// Workgroups N*G .. N*G+C-1: channel c = blockIdx - N*G, dgamma (+)= sum_n B_nc,
// dbeta (+)= sum_n A_nc (thread t takes samples t, t + kThreads, ..., then a fixed-order
// tree over the threads).
__global__ __launch_bounds__(kThreads) void grp_bwd_coef(const double* __restrict__ ab, int N, int C, int G,
                                                         double cnt, const float* __restrict__ gamma,
                                                         float* __restrict__ dgamma, float* __restrict__ dbeta,
                                                         int accumulate, float* __restrict__ coef) {
    __shared__ double dred[kThreads];
    const int t = threadIdx.x, cg = C / G;
    if ((int)blockIdx.x < N * G) {
        const int ng = blockIdx.x, n = ng / G, g = ng - n * G;
        double a = 0.0, b = 0.0;
        for (int k = t; k < cg; k += kThreads) {
            const int c = g * cg + k;
            const double* p = ab + ((int64_t)n * C + c) * 2;
            a += (double)gamma[c] * p[0];
            b += (double)gamma[c] * p[1];
        }
        a = block_sum(a, dred);
        b = block_sum(b, dred);
        if (t == 0) {
            coef[2 * ng] = (float)(a / cnt);
            coef[2 * ng + 1] = (float)(b / cnt);
        }
        return;
    }
    const int c = blockIdx.x - N * G;
    if (!dgamma && !dbeta) return;  // uniform per workgroup
    double a = 0.0, b = 0.0;
    for (int n = t; n < N; n += kThreads) {
        a += ab[((int64_t)n * C + c) * 2];
        b += ab[((int64_t)n * C + c) * 2 + 1];
    }
    a = block_sum(a, dred);
    b = block_sum(b, dred);
    if (t == 0) {
        if (dgamma) dgamma[c] = accumulate ? (float)((double)dgamma[c] + b) : (float)b;
        if (dbeta) dbeta[c] = accumulate ? (float)((double)dbeta[c] + a) : (float)a;
    }
}

// dz = inv_std_ng (gamma_c dno - k1_ng - zhat k2_ng); grid (blocks per sample, N).
template <typename T, int VEC, int ACT>
__global__ __launch_bounds__(kThreads) void grp_bwd_apply(const T* __restrict__ z, const T* dy, T* dz,
                                                          int64_t per_sample, int C, int G,
                                                          const float* __restrict__ gamma,
                                                          const float* __restrict__ beta,
                                                          const float* __restrict__ mean,
                                                          const float* __restrict__ inv_std,
                                                          const float* __restrict__ coef) {
    const int n = blockIdx.y, cg = C / G;
    const int64_t nvec = per_sample / VEC, base = (int64_t)n * per_sample;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    int c0 = (int)((v * VEC) % C), cached = -1;
    const int step = (int)((stride * VEC) % C);
    float mu[VEC], is[VEC], g[VEC], bt[VEC], k1[VEC], k2[VEC];
    for (; v < nvec; v += stride) {
        float zv[VEC], gv[VEC];
        Vec<T, VEC>::load(z + base + v * VEC, zv);
        Vec<T, VEC>::load(dy + base + v * VEC, gv);
        if (c0 != cached) {
            grp_params<VEC>(mean, inv_std, n, G, cg, c0, mu, is);
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                const int st = n * G + (c0 + j) / cg;
                g[j] = gamma[c0 + j]; bt[j] = beta[c0 + j];
                k1[j] = coef[2 * st]; k2[j] = coef[2 * st + 1];
            }
            cached = c0;
        }
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            float zh, a = bn_affine(zv[j], mu[j], is[j], g[j], bt[j], &zh);
            const float dno = act_slope<ACT>(a) * gv[j];
            gv[j] = is[j] * (__builtin_fmaf(g[j], dno, -k1[j]) - zh * k2[j]);
        }
        Vec<T, VEC>::store(dz + base + v * VEC, gv);
        c0 += step;
        if (c0 >= C) c0 -= C;
    }
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

// dz = act'(z) * dy, no norm; FROM_OUT: the derivative from the stored output y instead.
template <typename T, int VEC, int ACT, bool FROM_OUT = false>
__global__ __launch_bounds__(kThreads) void act_bwd(const T* __restrict__ z, const T* dy, T* dz, int64_t nvec) {
    for (int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x; v < nvec; v += (int64_t)gridDim.x * kThreads) {
        float a[VEC], g[VEC];
        Vec<T, VEC>::load(z + v * VEC, a);
        Vec<T, VEC>::load(dy + v * VEC, g);
#pragma unroll
        for (int j = 0; j < VEC; ++j) g[j] *= FROM_OUT ? act_slope_out<ACT>(a[j]) : act_slope<ACT>(a[j]);
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
    p.seg = 0;
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
    p.bps = p.blocks;
    return p;
}

RowPlan seg_plan(int N, int64_t S, int C, int dt) {
    RowPlan p = row_plan(S, C, dt);
    int bps = (int)ceil_div(kTargetBlocks, N);
    int64_t rpb = ceil_div(S, bps);
    rpb = ceil_div(rpb, p.rpi) * p.rpi;
    if (rpb < p.rpi) rpb = p.rpi;
    p.rows_per_block = rpb;
    p.bps = (int)ceil_div(S, rpb);
    p.blocks = N * p.bps;
    p.seg = S;
    return p;
}

size_t bn_stats_ws_bytes(int64_t M, int C, int dt) { return partial_bytes(row_plan(M, C, dt), C); }

size_t bn_bwd_ws_bytes(int64_t M, int C, int dt) {
    return partial_bytes(row_plan(M, C, dt), C) + align_up((size_t)C * 3 * sizeof(float), 256);
}

size_t grp_stats_ws_bytes(int N, int64_t S, int C, int dt) { return partial_bytes(seg_plan(N, S, C, dt), C); }

size_t grp_bwd_ws_bytes(int N, int64_t S, int C, int G, int dt) {
    return partial_bytes(seg_plan(N, S, C, dt), C) + align_up((size_t)N * C * 2 * sizeof(double), 256) +
           align_up((size_t)N * G * 2 * sizeof(float), 256);
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
                                                                          p.rows_per_block, part, 0, 0)));
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

hipError_t launch_act_bwd_from_output(int dt, const void* y, const void* dy, void* dz, int64_t M, int C, int act,
                                      hipStream_t s) {
    const int full = dt == DT_BF16 ? 8 : 4;
    const int vec = (C % full == 0) ? full : 1;
    const int64_t nvec = M * C / vec;
    dim3 grid(elementwise_grid(nvec)), block(kThreads);
    if (act == ACT_GELU) return hipErrorInvalidValue;
    CONVMI_VEC_SWITCH(dt, vec, T, VEC, CONVMI_ACT_SWITCH(act, A, (act_bwd<T, VEC, A, true><<<grid, block, 0, s>>>(
                                                                   (const T*)y, (const T*)dy, (T*)dz, nvec))));
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

hipError_t launch_grp_stats(int dt, const void* z, int N, int64_t S, int C, int G, float eps, float* mean,
                            float* inv_std, void* ws, hipStream_t s) {
    RowPlan p = seg_plan(N, S, C, dt);
    float* part = (float*)ws;
    dim3 grid(p.blocks, p.chunks), block(kThreads);
    size_t lds = (size_t)p.rpi * p.tpr * p.vec * 2 * sizeof(float);
    const int64_t M = (int64_t)N * S;
    CONVMI_VEC_SWITCH(dt, p.vec, T, VEC,
                      (bn_stats_partials<T, VEC><<<grid, block, lds, s>>>((const T*)z, M, C, p.tpr, p.rpi,
                                                                          p.rows_per_block, part, p.seg, p.bps)));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (dt == DT_BF16)
        grp_stats_finalize<bf16><<<N * G, block, 0, s>>>(part, p.bps, C, G, (const bf16*)z, S, eps, mean, inv_std);
    else
        grp_stats_finalize<float><<<N * G, block, 0, s>>>(part, p.bps, C, G, (const float*)z, S, eps, mean, inv_std);
    return hipGetLastError();
}

hipError_t launch_grp_tiles_finalize(const float* part, int ntiles, int N, int C, int G, int64_t S, float eps,
                                     float* mean, float* inv_std, hipStream_t s) {
    grp_tiles_finalize<<<N * G, kThreads, 0, s>>>(part, ntiles, ntiles / N, C, G, S, eps, mean, inv_std);
    return hipGetLastError();
}

static int per_sample_grid(int N, int64_t nvec_per_sample) {
    int64_t g = ceil_div(nvec_per_sample, kThreads * 4);
    const int64_t cap = ceil_div(8192, N);
    if (g > cap) g = cap;
    return g < 1 ? 1 : (int)g;
}

hipError_t launch_grp_apply(int dt, const void* z, void* y, int N, int64_t S, int C, int G, int act,
                            const float* gamma, const float* beta, const float* mean, const float* inv_std,
                            hipStream_t s) {
    const int full = dt == DT_BF16 ? 8 : 4;
    const int vec = (C % full == 0) ? full : 1;
    const int64_t per_sample = S * C;
    dim3 grid(per_sample_grid(N, per_sample / vec), N), block(kThreads);
    CONVMI_VEC_SWITCH(dt, vec, T, VEC, CONVMI_ACT_SWITCH(act, A, (grp_apply<T, VEC, A><<<grid, block, 0, s>>>(
                                                                   (const T*)z, (T*)y, per_sample, C, G, gamma, beta,
                                                                   mean, inv_std))));
    return hipGetLastError();
}

hipError_t launch_grp_bwd(int dt, const void* z, const void* dy, void* dz, int N, int64_t S, int C, int G, int act,
                          const float* gamma, const float* beta, const float* mean, const float* inv_std,
                          float* dgamma, float* dbeta, int accumulate, void* ws, hipStream_t s) {
    RowPlan p = seg_plan(N, S, C, dt);
    float* part = (float*)ws;
    double* ab = (double*)((char*)ws + partial_bytes(p, C));
    float* coef = (float*)((char*)ab + align_up((size_t)N * C * 2 * sizeof(double), 256));
    dim3 grid(p.blocks, p.chunks), block(kThreads);
    size_t lds = (size_t)p.rpi * p.tpr * p.vec * 2 * sizeof(float);
    const int64_t M = (int64_t)N * S;
    CONVMI_VEC_SWITCH(dt, p.vec, T, VEC, CONVMI_ACT_SWITCH(act, A, (grp_bwd_partials<T, VEC, A><<<grid, block, lds, s>>>(
                                                                      (const T*)z, (const T*)dy, M, C, p.tpr, p.rpi,
                                                                      p.rows_per_block, p.seg, p.bps, G, gamma, beta,
                                                                      mean, inv_std, part))));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    grp_bwd_merge<<<(int)ceil_div((int64_t)N * C, kThreads), block, 0, s>>>(part, p.bps, N, C, ab);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    grp_bwd_coef<<<N * G + C, block, 0, s>>>(ab, N, C, G, (double)S * (C / G), gamma, dgamma, dbeta, accumulate,
                                             coef);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t per_sample = S * C;
    dim3 g2(per_sample_grid(N, per_sample / p.vec), N);
    CONVMI_VEC_SWITCH(dt, p.vec, T, VEC, CONVMI_ACT_SWITCH(act, A, (grp_bwd_apply<T, VEC, A><<<g2, block, 0, s>>>(
                                                                      (const T*)z, (const T*)dy, (T*)dz, per_sample, C,
                                                                      G, gamma, beta, mean, inv_std, coef))));
    return hipGetLastError();
}

}  // namespace convmi
