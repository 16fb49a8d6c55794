// k_halo.hip -- stride-1 convolution forward and input gradient with input-tile reuse.
//
// For a stride-1 layer the implicit-GEMM operand A of every tap (kh, kw) is one input
// rectangle shifted by (kh, kw).  The per-tap gather of the generic MFMA kernel reads that
// rectangle KH*KW times.  Here an output tile is an R x Q rectangle of one image; for each
// 128-byte channel chunk the tile's input rectangle plus its halo, (R + KH - 1) x
// (Q + KW - 1) positions, is copied into LDS once, and every tap reads its MFMA fragments
// from it at shifted positions.  Only the weights stream per tap.  With four whole
// 56-pixel rows per tile this loads about a third of the bytes per FLOP of the per-tap
// gather; on gfx950 the vector-memory address path, not the MFMA or the LDS, is what the
// gather saturates first.
//
// Forward: out(n, oh, ow, oc) = sum_{kh,kw,ic} w[oc, kh, kw, ic] x[n, oh - ph + kh, ow - pw + kw, ic]
//   halo origin (oh0 - ph, ow0 - pw); tap (kh, kw) sits at halo offset (kh, kw).
// Input gradient: dx(n, ih, iw, ic) = sum_{kh,kw,oc} w[oc, kh, kw, ic] dz[n, ih + ph - kh, iw + pw - kw, oc]
//   halo origin (ih0 + ph - KH + 1, iw0 + pw - KW + 1); tap (kh, kw) sits at offset
//   (KH - 1 - kh, KW - 1 - kw); the weight operand is the rearranged copy
//   Bt[ic][(kh, kw, oc)] = w[oc, kh, kw, ic] that the generic input-gradient path builds.
// Definitions: rl_tools conv2d listings "operations_generic.h" (forward, backward_input)
// and "operations_cuda.h" (forward with bias and activation; backward_input).
//
// Pipeline: steps (chunk c, tap t), c outer.  The weights are laid out in MFMA fragment
// order beforehand and each wave streams its own fragments into registers one step ahead;
// LDS holds only the input halo.  With two halo buffers the halo of chunk c + 1 is copied
// during chunk c; with one it is copied after the last tap of chunk c and a second
// workgroup on the CU covers the gap.  Halo copies are 16-byte LDS-DMA with XOR-swizzled
// 16-byte chunks.  The epilogue stages the tile in LDS in the storage type (the
// activation reads the stored pre-activation, so staging the rounded value loses nothing)
// and writes 16-byte vectors.
#include <stdio.h>

#include <algorithm>

#include "internal.hpp"
#include "lds_dma.hpp"

namespace convmi {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

typedef float floatx16 __attribute__((ext_vector_type(16)));

// MFMA flavours.  MF = rows (and columns) of one output fragment.  A lane of group
// lg = lane / MF holds row lane % MF of its operand fragments, one 16-byte chunk of k;
// the 128-byte k chunk of a step is covered in 8 / (64 / MF) MFMA k-steps.
//   MF = 16: fp32, 4 x v_mfma_f32_16x16x4_f32 per 16-byte vector (the four k of a lane's
//            vector go to four MFMAs; A and B use the same order); accumulator element e
//            of lane group lg is output row 4*lg + e.
//   MF = 32: v_mfma_f32_32x32x16_bf16; accumulator element e of lane group lg is output
//            row 8*(e/4) + 4*lg + e%4.
template <typename T, int MF> struct HMma;
template <> struct HMma<float, 16> {
    typedef floatx4 Acc;
    static constexpr int NE = 4;
    static __device__ __forceinline__ void run(Acc& c, const uint4& a, const uint4& b) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    }
    static __device__ __forceinline__ int row(int lg, int e) { return 4 * lg + e; }
};
template <> struct HMma<bf16, 32> {
    typedef floatx16 Acc;
    static constexpr int NE = 16;
    static __device__ __forceinline__ void run(Acc& c, const uint4& a, const uint4& b) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                    0, 0, 0);
    }
    static __device__ __forceinline__ int row(int lg, int e) { return 8 * (e >> 2) + 4 * lg + (e & 3); }
};

template <> struct HMma<bf16, 16> {
    typedef floatx4 Acc;
    static constexpr int NE = 4;
    static __device__ __forceinline__ void run(Acc& c, const uint4& a, const uint4& b) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                    0, 0);
    }
    static __device__ __forceinline__ int row(int lg, int e) { return 4 * lg + e; }
};

// 16-byte chunk swizzle of a 128-byte LDS row (one halo position): the slot of logical
// chunk k at position p is k ^ swz<MF>(key(p)).  A ds_read_b128 runs in four passes of 16
// lanes (measured on gfx950 with the bank-conflict counters): lanes 0-7 with 24-31, 8-15
// with 16-23, 32-39 with 56-63 and 40-47 with 48-55; the 64 banks take 16 distinct 16-byte
// (position parity, slot) pairs per pass.  With fragments of 16 pixels a pass holds 8
// consecutive pixels reading chunk L and the next 8 reading chunk L ^ 1, so the slot is
// 2 * ((key >> 1) & 3): one slot of each XOR-1 pair, the pair's other slot left to the
// other half.  With 32-pixel fragments both halves read one chunk and pixels 24 apart
// share a pass: slot (key >> 1) & 7.  Either is conflict-free when a fragment's 16 or 32
// keys are consecutive integers of its positions' parity.  key = halo row * QS + halo
// column with QS = HQ - 2*((KW-1)/2) (Q for odd KW): the keys of consecutive tile pixels
// under one tap are then consecutive even where a fragment crosses a tile row (its raw
// positions skip the KW-1 halo columns there), and QS, of HQ's parity, keeps the key's
// parity the position's.
template <int MF> __device__ __forceinline__ int swz(int key) {
    return MF == 16 ? ((key >> 1) & 3) << 1 : (key >> 1) & 7;
}

constexpr int kCUs = 256;

struct HaloGeom {
    int Hin, Win, Cin;     // gathered tensor: x (forward) or dz (input gradient)
    int KH, KW;
    int Hout, Wout, Nn;    // output image size and output channels
    int R, Q;              // output tile: R rows x Q columns
    int R2;                // paired bands: rows of the short bands (0: one tile per workgroup)
    int HQ, HP, GH;        // halo row length (Q + KW - 1), positions, 8-position copy groups
    int QS;                // row length of the swizzle key (HQ - 2*((KW-1)/2))
    int org_r, org_c;      // halo origin relative to the tile origin
    int tiles_r, tiles_c;  // tile rows (paired: pairs of bands) and columns per image
    int nchunks;           // Cin / channels per 128-byte chunk
    int Kb;                // weight row length KH*KW*Cin
    int sign;              // +1 forward (tap at (kh, kw)), -1 input gradient (flipped)
    int hb;                // halo buffers (1 or 2)
    int par_off;           // LDS byte offset of the per-column epilogue parameters
    int64_t img_stride;    // Hin*Win*Cin
    FastDiv fQ, fHQ, fTR, fTC;
};

template <typename T> __device__ __forceinline__ void put16(T* p, const float* v);
template <> __device__ __forceinline__ void put16<float>(float* p, const float* v) {
    *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
}
template <> __device__ __forceinline__ void put16<bf16>(bf16* p, const float* v) {
    *(uint4*)p = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                            pack_bf16x2(v[6], v[7]));
}

// Per-column epilogue parameters (bias, batch-norm statistics) go to LDS, kPar arrays of
// BN floats (0 past the last column): a workgroup loads them into registers while its
// first halo is in flight and writes them to LDS after the prologue barrier, so the
// epilogue reads them at LDS latency instead of waiting on global loads after the main
// loop.  `par_src(k)` is parameter array k (nullable); `colbias` takes a column of the
// tile; `prep` loads a thread's parameters for its 8 columns once.
template <class Out, int BN, int NTH> struct ParStage {
    static constexpr int N = Out::kPar * BN;
    static constexpr int R = N > 0 ? (N + NTH - 1) / NTH : 1;  // registers per thread
    float v[R];
    __device__ __forceinline__ void load(const Out& out, int n0, int t) {
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int idx = t + k * NTH;
            v[k] = 0.0f;
            if (idx < N) {
                const int kind = idx / BN, c = idx - kind * BN;
                const float* src = out.par_src(kind);
                if (src && n0 + c < out.ncols()) v[k] = src[n0 + c];
            }
        }
    }
    __device__ __forceinline__ void store(float* par, int t) const {
#pragma unroll
        for (int k = 0; k < R; ++k)
            if (t + k * NTH < N) par[t + k * NTH] = v[k];
    }
};

// z = stored(acc + bias), y = act(z).  `raw` holds 16 bytes of stored z of one pixel.
struct HFwdOut {
    void* z;            // nullable
    void* y;            // nullable
    const float* bias;  // nullable
    int OC;
    static constexpr int kPar = 1;
    static constexpr bool kStats = false;
    struct Cache {};
    __device__ __forceinline__ int ncols() const { return OC; }
    __device__ __forceinline__ const float* par_src(int) const { return bias; }
    __device__ __forceinline__ float colbias(const float* par, int cl) const { return par[cl]; }
    __device__ __forceinline__ Cache prep(const float*, int, int, int) const { return Cache{}; }
    template <typename T, int ACT>
    __device__ __forceinline__ void put(int64_t pix, int col, const uint4& raw, int nv, const Cache&) const {
        constexpr int VEC = 16 / (int)sizeof(T);
        T v[VEC];
        __builtin_memcpy(v, &raw, 16);
        const int64_t off = pix * OC + col;
        if (nv == VEC && OC % VEC == 0) {
            if (z) *(uint4*)((T*)z + off) = raw;
            if (y) {
                float yr[VEC];
#pragma unroll
                for (int j = 0; j < VEC; ++j) yr[j] = act_fwd<ACT>(to_f32(v[j]));
                put16<T>((T*)y + off, yr);
            }
        } else {
            for (int j = 0; j < nv; ++j) {
                if (z) ((T*)z)[off + j] = v[j];
                if (y) ((T*)y)[off + j] = from_f32<T>(act_fwd<ACT>(to_f32(v[j])));
            }
        }
    }
};

// Evaluation-mode batch norm in the epilogue (its statistics are known before the
// convolution): z = stored(acc + bias), y = act(gamma*(z - mean)*inv_std + beta), with
// the same fp32 operation order as the separate normalise/activate pass.
struct HFwdBnOut {
    void* z;            // nullable
    void* y;
    const float* bias;  // nullable
    int OC;
    const float *mean, *inv_std, *gamma, *beta;
    static constexpr int kPar = 5;  // bias, mean, inv_std, gamma, beta
    static constexpr bool kStats = false;
    struct Cache {
        float m[8], i[8], g[8], b[8];
    };
    __device__ __forceinline__ int ncols() const { return OC; }
    __device__ __forceinline__ const float* par_src(int k) const {
        return k == 0 ? bias : k == 1 ? mean : k == 2 ? inv_std : k == 3 ? gamma : beta;
    }
    __device__ __forceinline__ float colbias(const float* par, int cl) const { return par[cl]; }
    // columns cl .. cl + nv - 1 lie inside the tile; the unused entries repeat column cl
    __device__ __forceinline__ Cache prep(const float* par, int bn, int cl, int nv) const {
        Cache c;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int cc = cl + (j < nv ? j : 0);
            c.m[j] = par[bn + cc];
            c.i[j] = par[2 * bn + cc];
            c.g[j] = par[3 * bn + cc];
            c.b[j] = par[4 * bn + cc];
        }
        return c;
    }
    template <int ACT> __device__ __forceinline__ float yval(float zv, const Cache& c, int j) const {
        float zh;
        return act_fwd<ACT>(bn_affine(zv, c.m[j], c.i[j], c.g[j], c.b[j], &zh));
    }
    template <typename T, int ACT>
    __device__ __forceinline__ void put(int64_t pix, int col, const uint4& raw, int nv, const Cache& c) const {
        constexpr int VEC = 16 / (int)sizeof(T);
        T v[VEC];
        __builtin_memcpy(v, &raw, 16);
        const int64_t off = pix * OC + col;
        if (nv == VEC && OC % VEC == 0) {
            if (z) *(uint4*)((T*)z + off) = raw;
            float yr[VEC];
#pragma unroll
            for (int j = 0; j < VEC; ++j) yr[j] = yval<ACT>(to_f32(v[j]), c, j);
            put16<T>((T*)y + off, yr);
        } else {
            for (int j = 0; j < nv; ++j) {
                if (z) ((T*)z)[off + j] = v[j];
                ((T*)y)[off + j] = from_f32<T>(yval<ACT>(to_f32(v[j]), c, j));
            }
        }
    }
};

// Training-mode batch norm: z = stored(acc + bias) only (the normalisation needs the
// batch statistics, so y comes from a later pass), plus per-tile statistics of the
// stored z for each column: with shift s = the tile's first pixel, S1 = sum (z - s),
// S2 = sum (z - s)^2 and the pixel count, at part[((c * 4 + q) * ntiles) + tile] for
// q = S1, S2, s, count.  The shift keeps S2 free of cancellation when |mean| >> std;
// bn_tiles_finalize merges the tiles in a fixed order.
struct HFwdStatsOut {
    void* z;
    const float* bias;  // nullable
    int OC;
    float* part;
    int ntiles;  // spatial tiles (images x tile rows x tile columns)
    static constexpr int kPar = 1;
    static constexpr bool kStats = true;
    struct Cache {};
    __device__ __forceinline__ int ncols() const { return OC; }
    __device__ __forceinline__ const float* par_src(int) const { return bias; }
    __device__ __forceinline__ float colbias(const float* par, int cl) const { return par[cl]; }
    __device__ __forceinline__ Cache prep(const float*, int, int, int) const { return Cache{}; }
    template <typename T, int ACT>
    __device__ __forceinline__ void put(int64_t pix, int col, const uint4& raw, int nv, const Cache&) const {
        constexpr int VEC = 16 / (int)sizeof(T);
        const int64_t off = pix * OC + col;
        if (nv == VEC && OC % VEC == 0) {
            *(uint4*)((T*)z + off) = raw;
        } else {
            T v[VEC];
            __builtin_memcpy(v, &raw, 16);
            for (int j = 0; j < nv; ++j) ((T*)z)[off + j] = v[j];
        }
    }
};

struct HDxOut {
    void* dx;
    int IC;
    static constexpr int kPar = 0;
    static constexpr bool kStats = false;
    struct Cache {};
    __device__ __forceinline__ int ncols() const { return IC; }
    __device__ __forceinline__ const float* par_src(int) const { return nullptr; }
    __device__ __forceinline__ float colbias(const float*, int) const { return 0.0f; }
    __device__ __forceinline__ Cache prep(const float*, int, int, int) const { return Cache{}; }
    template <typename T, int ACT>
    __device__ __forceinline__ void put(int64_t pix, int col, const uint4& raw, int nv, const Cache&) const {
        constexpr int VEC = 16 / (int)sizeof(T);
        const int64_t off = pix * IC + col;
        if (nv == VEC && IC % VEC == 0) {
            *(uint4*)((T*)dx + off) = raw;
        } else {
            T v[VEC];
            __builtin_memcpy(v, &raw, 16);
            for (int j = 0; j < nv; ++j) ((T*)dx)[off + j] = v[j];
        }
    }
};

constexpr int kThreadsH = 256;  // four waves, WM x WN

// Waves per SIMD the register budget of halo_rb_kernel is set for: 64-channel bf16 tiles
// of 16-row fragments fit four workgroups on a CU (128 VGPRs), the others two.
constexpr int rb_waves(int esize, int bn, int mf) { return esize == 2 && bn == 64 && mf == 16 ? 4 : 2; }

// Second half of the epilogue: the tile's stored values sit in LDS (Cs, rows of LDC
// elements, pixel m = rr*Q + qq of the tile at row m); thread t writes columns
// (t % OVR)*VEC .. +VEC of rows t/OVR, t/OVR + NTH/OVR, ...  With Out::kStats it also
// reduces the per-tile column statistics (every thread of the workgroup reaches the
// barriers below, active or not).
template <typename T, int ACT, int BM, int BN, int NTH, class Out>
__device__ __forceinline__ void epilogue_store(const T* Cs, const Out& out, const float* par, const HaloGeom& g,
                                               int n, int r0, int c0, int n0, int sp, int R) {
    constexpr int VEC = 16 / (int)sizeof(T);
    constexpr int LDC = BN + VEC;
    constexpr int OVR = BN / VEC;
    constexpr int RG = NTH / OVR;  // row groups
    static_assert(NTH % OVR == 0, "each thread keeps one column range");
    static_assert((2 * RG * BN + BN + RG) * 4 <= BM * LDC * (int)sizeof(T), "statistics fit the staging area");
    const int t = threadIdx.x;
    const int cv = t % OVR, col = n0 + cv * VEC;
    const bool active = col < g.Nn;
    if (!Out::kStats && !active) return;
    const int nv = g.Nn - col < VEC ? g.Nn - col : VEC;
    const int RQ = R * g.Q;
    const typename Out::Cache cache = out.prep(par, BN, cv * VEC, nv);
    float s1[VEC], s2[VEC], sh[VEC];
    int cnt = 0;
    if constexpr (Out::kStats) {
        // pixel 0 of the tile (its first row and column) always lies inside the image
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            sh[j] = to_f32(Cs[cv * VEC + j]);
            s1[j] = s2[j] = 0.0f;
        }
    }
    if (active) {
        for (int m = t / OVR; m < RQ; m += RG) {
            const int rr = fdiv(m, g.fQ);
            const int oh = r0 + rr, ow = c0 + (m - rr * g.Q);
            if (oh >= g.Hout || ow >= g.Wout) continue;
            const int64_t pix = ((int64_t)n * g.Hout + oh) * g.Wout + ow;
            const uint4 raw = *(const uint4*)(Cs + m * LDC + cv * VEC);
            out.template put<T, ACT>(pix, col, raw, nv, cache);
            if constexpr (Out::kStats) {
                T v[VEC];
                __builtin_memcpy(v, &raw, 16);
#pragma unroll
                for (int j = 0; j < VEC; ++j) {
                    const float d = to_f32(v[j]) - sh[j];
                    s1[j] += d;
                    s2[j] = __builtin_fmaf(d, d, s2[j]);
                }
                ++cnt;
            }
        }
    }
    if constexpr (Out::kStats) {
        // fixed-order merge of the RG row groups per column (the staged tile is no longer read)
        __syncthreads();
        float* red = (float*)(void*)Cs;  // [2][RG][BN] sums, [BN] shifts, [RG] counts
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            red[(t / OVR) * BN + cv * VEC + j] = s1[j];
            red[(RG + t / OVR) * BN + cv * VEC + j] = s2[j];
        }
        if (t < OVR)
#pragma unroll
            for (int j = 0; j < VEC; ++j) red[2 * RG * BN + cv * VEC + j] = sh[j];
        if (cv == 0) red[2 * RG * BN + BN + t / OVR] = (float)cnt;
        __syncthreads();
        if (t < BN && n0 + t < g.Nn) {
            float a = 0.0f, b = 0.0f, c = 0.0f;
            for (int k = 0; k < RG; ++k) {
                a += red[k * BN + t];
                b += red[(RG + k) * BN + t];
                c += red[2 * RG * BN + BN + k];
            }
            float* p = out.part + (int64_t)(n0 + t) * 4 * out.ntiles + sp;
            p[0] = a;
            p[out.ntiles] = b;
            p[2 * (int64_t)out.ntiles] = red[2 * RG * BN + t];
            p[3 * (int64_t)out.ntiles] = c;
        }
    }
}

// The tile kernel, bf16 or fp32, without a per-step barrier.  The weights are first laid
// out in MFMA fragment order (frag_weights below): the B fragment that a wave needs for
// one MFMA k-step (32 or 16 rows x 32 bytes of k) is 1 KB contiguous, so every weight
// load instruction reads whole cache lines.  Each wave loads its own B fragments straight into registers one step
// ahead; LDS holds only the input halo, whose next chunk is copied during the current one
// (two buffers) or after it (one buffer).  Waves therefore only meet at chunk
// boundaries, where each waits for all of its outstanding vector-memory operations:
// LDS-DMA copies and register loads need not complete in issue order with respect to
// each other, so a count that mixes the two kinds proves nothing.
//
// rb_tile computes one tile: R x Q pixels from row r0, column c0 of image n, output
// channels n0 .. n0 + BN - 1, in BM = TM*WM*MF fragment rows; sp is the tile's index in
// the per-tile statistics.  Two calls in one workgroup need a barrier between them (the
// epilogue stages the tile in the halo's LDS).
template <typename T, int BM, int BN, int WM, int WN, int ACT, class Out, int MF>
__device__ __forceinline__ void rb_tile(const T* __restrict__ A, const HaloGeom& g, const uint4* __restrict__ Bf,
                                        const Out& out, int n, int r0, int c0, int n0, int R, int sp) {
    using MM = HMma<T, MF>;
    using Acc = typename MM::Acc;
    constexpr int NWAVE = 4, NTH = kThreadsH;
    static_assert(WM * WN == NWAVE, "four waves");
    constexpr int TM = BM / (WM * MF), TN = BN / (WN * MF);
    static_assert(TM * WM * MF == BM && TN * WN * MF == BN, "tile shape");
    // 16-byte chunk = 8 bf16 or 4 fp32; a 128-byte chunk (64 bf16 or 32 fp32 channels) is 4
    // k-steps of 32 bytes (32x32x16: lane groups of 32 take 2 chunks per k-step) or 2 of 64
    // bytes (16x16x32 bf16, 4 x 16x16x4 fp32: lane groups of 16 take 4 chunks)
    static_assert(sizeof(T) == 2 || MF == 16, "fp32 tiles use 16-row fragments");
    constexpr int VEC = 16 / (int)sizeof(T), CK = 128 / (int)sizeof(T), KST = MF == 32 ? 4 : 2,
                  LGS = MF == 32 ? 5 : 4;
    extern __shared__ __align__(1024) unsigned char smem[];
    // Swizzle key: row*QS + column (conflict-free also for fragments that cross a tile
    // row) in the bf16 two-wave kernels; the raw position in the others, which have no
    // register to spare for it and whose plans use 16-pixel rows (16-pixel fragments
    // never cross one).
    constexpr bool KEYED = sizeof(T) == 2 && rb_waves(2, BN, MF) == 2;

    const int t = threadIdx.x, lane = t & 63;
    const int wid = __builtin_amdgcn_readfirstlane(t >> 6);
    const int halo_bytes = g.GH * 1024;  // buffer stride: the plan's largest halo
    const int HPt = (R + g.KH - 1) * g.HQ, GHt = (HPt + 7) / 8;  // this tile's halo
    const bool two = g.hb == 2;
    const uint32_t smem_base = __builtin_amdgcn_readfirstlane(lds_addr(smem));
    const int hr0 = r0 + g.org_r, hc0 = c0 + g.org_c;
    const T* Aimg = A + (int64_t)n * g.img_stride;
    ParStage<Out, BN, NTH> pst;  // stored to LDS after the main loop
    pst.load(out, n0, t);
    const int taps = g.KH * g.KW;
    const int nsteps = g.nchunks * taps;

    // Halo copy: a chunk's halo is JH copy instructions per wave; instruction j of this
    // wave covers halo positions 8*(wid + 4j) .. +7, lane l chunk l%8 of position l/8.
    const int rg = lane >> 3, pc = lane & 7;
    const int JH = (GHt + NWAVE - 1) / NWAVE;
    auto issue_halo = [&](int c, int j0, int j1) {
        const uint32_t dstb = smem_base + (uint32_t)((two ? (c & 1) : 0) * halo_bytes);
        for (int j = j0; j < j1; ++j) {
            const int grp = wid + NWAVE * j;
            if (grp >= GHt) break;
            const int p = grp * 8 + rg;
            const void* src = &kZero16;
            if (p < HPt) {
                const int hr = fdiv(p, g.fHQ), hc = p - hr * g.HQ;
                const int ih = hr0 + hr, iw = hc0 + hc, key = KEYED ? hr * g.QS + hc : p;
                if ((unsigned)ih < (unsigned)g.Hin && (unsigned)iw < (unsigned)g.Win)
                    src = Aimg + ((int64_t)ih * g.Win + iw) * g.Cin + c * CK + (pc ^ swz<MF>(key)) * VEC;
            }
            dma16(src, __builtin_amdgcn_readfirstlane(dstb + grp * 1024));
        }
    };
    const int wm = wid / WN, wn = wid % WN;
    const int lr = lane & (MF - 1), lg = lane >> LGS;
    // halo position of each fragment's pixel at tap 0 (KEYED: in the low 16 bits, the
    // swizzle key in the high 16)
    int hpos[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        int m = wm * TM * MF + i * MF + lr;
        // rows past the tile read a valid pixel (never stored); KEYED: one whose key keeps
        // the lane's residue mod 16, so it does not collide with the fragment's other lanes
        if (m >= R * g.Q) m = KEYED && R * g.Q >= 16 ? (m & 15) : 0;
        const int rr = fdiv(m, g.fQ), cc = m - rr * g.Q;
        hpos[i] = KEYED ? (rr * g.HQ + cc) | ((rr * g.QS + cc) << 16) : rr * g.HQ + cc;
    }
    // B fragments: 32-row group (n0 + wn*TN*32)/32 + j, step st, k-step kk at
    // ((group * nsteps + st) * 4 + kk) * 64 + lane
    const uint4* bq = Bf + (int64_t)((n0 + wn * TN * MF) / MF) * nsteps * (KST * 64) + lane;
    const int64_t gstride = (int64_t)nsteps * (KST * 64);
    auto load_b = [&](int st, uint4 (&dst)[TN][KST]) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int kk = 0; kk < KST; ++kk) dst[j][kk] = bq[j * gstride + (st * KST + kk) * 64];
    };

    Acc acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < MM::NE; ++e) acc[i][j][e] = 0.0f;

    uint4 bA[TN][KST], bB[TN][KST];
    issue_halo(0, 0, JH);
    load_b(0, bA);
    // The first fragments are waited for here, while the halo copies are in flight;
    // otherwise the compiler sinks their loads below the barrier and the first step
    // waits for them on its own.
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int kk = 0; kk < KST; ++kk) asm volatile("" ::"v"(bA[j][kk].x));
    wait_dma(0);
    __syncthreads();

    // Step st = (chunk c, tap (kh, kw)), advanced incrementally (no divisions per step).
    int c = 0, kh = 0, kw = 0;
    auto step = [&](int st, const uint4 (&cur)[TN][KST], uint4 (&nxt)[TN][KST]) {
        const int tap = kh * g.KW + kw;
        // Always issued (the last step reloads its own fragments): a load on only some
        // paths makes the compiler wait for it at the merge as if it were on every path,
        // which would stall each step on the next step's fragments.
        load_b(st + 1 < nsteps ? st + 1 : st, nxt);
        const int th = g.sign > 0 ? kh : g.KH - 1 - kh, tw = g.sign > 0 ? kw : g.KW - 1 - kw;
        const int toff = th * g.HQ + tw, tkey = th * g.QS + tw;
        const int hbase = __builtin_amdgcn_readfirstlane((two ? (c & 1) : 0) * halo_bytes);
        // LDS offset of the A fragment at k-step 0; the halo buffer and every 128-byte row
        // start are 128-byte aligned, so k-step kk (chunk G*kk + lg = G*kk ^ lg, G = 2 or 4
        // chunks per k-step) is the same offset XOR (G*kk) << 4.
        uint32_t fo[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int p = (KEYED ? hpos[i] & 0xffff : hpos[i]) + toff;
            const int key = KEYED ? (hpos[i] >> 16) + tkey : p;
            fo[i] = (uint32_t)(hbase + p * 128 + ((lg ^ swz<MF>(key)) << 4));
        }
        // A fragments of k-step kk + 1 are read during kk's MFMAs (two buffers) where two
        // waves share a SIMD; with four, the other waves cover the read latency and one
        // buffer keeps the register budget.
        constexpr int NFA = rb_waves((int)sizeof(T), BN, MF) > 2 ? 1 : 2;
        uint4 fa[NFA][TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[0][i] = *(const uint4*)(smem + fo[i]);
#pragma unroll
        for (int kk = 0; kk < KST; ++kk) {
            if (NFA == 2 && kk + 1 < KST) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    fa[(kk + 1) % NFA][i] = *(const uint4*)(smem + (fo[i] ^ ((kk + 1) << (MF == 32 ? 5 : 6))));
            } else if (NFA == 1 && kk > 0) {
#pragma unroll
                for (int i = 0; i < TM; ++i) fa[0][i] = *(const uint4*)(smem + (fo[i] ^ (kk << (MF == 32 ? 5 : 6))));
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) MM::run(acc[i][j], cur[j][kk], fa[kk % NFA][i]);
            // The next chunk's halo, issued once this chunk's first MFMAs are under way.
            if (kk == 0 && two && c + 1 < g.nchunks && tap == 0) issue_halo(c + 1, 0, JH);
        }
        if (tap == taps - 1 && c + 1 < g.nchunks) {
            if (two) {
                wait_dma(0);      // this wave's slices of the next halo have landed
                __syncthreads();  // ... and every wave's; the old halo is free again
            } else {
                __syncthreads();  // every wave is done with the halo of chunk c
                issue_halo(c + 1, 0, JH);
                wait_dma(0);
                __syncthreads();
            }
        }
        if (++kw == g.KW) {
            kw = 0;
            if (++kh == g.KH) {
                kh = 0;
                ++c;
            }
        }
    };
    for (int st = 0; st < nsteps; st += 2) {
        step(st, bA, bB);
        if (st + 1 < nsteps) step(st + 1, bB, bA);
    }
    float* par = (float*)(smem + g.par_off);
    pst.store(par, t);
    __syncthreads();

    // epilogue: stored values -> LDS (rows of BN + 16 bytes) -> 16-byte vectors.  The
    // accumulators hold the transposed tile (MFMA rows are channels, columns pixels), so
    // a lane owns 4 consecutive channels of one pixel per row group: one 8-byte write.
    constexpr int LDC = BN + VEC;
    T* Cs = (T*)smem;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int g4 = 0; g4 < MM::NE / 4; ++g4) {
            const int cl = wn * TN * MF + j * MF + MM::row(lg, 4 * g4);  // 4 consecutive channels
            float bj[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) bj[q] = out.colbias(par, cl + q);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int m = wm * TM * MF + i * MF + lr;
                const float v0 = acc[i][j][4 * g4] + bj[0], v1 = acc[i][j][4 * g4 + 1] + bj[1];
                const float v2 = acc[i][j][4 * g4 + 2] + bj[2], v3 = acc[i][j][4 * g4 + 3] + bj[3];
                if constexpr (sizeof(T) == 2)
                    *(uint2*)(Cs + m * LDC + cl) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
                else
                    *(float4*)(Cs + m * LDC + cl) = make_float4(v0, v1, v2, v3);
            }
        }
    }
    __syncthreads();
    epilogue_store<T, ACT, BM, BN, NTH>(Cs, out, par, g, n, r0, c0, n0, sp, R);
}

// One tile per workgroup (BM2 = 0), or paired bands (BM2 > 0): the image's rows are cut
// into tiles_r bands of R rows followed by tiles_r bands of R2 rows, and workgroup
// (n, band b, column tile, channel tile) computes band b of each kind, the long one
// first, the short one in BM2 fragment rows.  Every workgroup then carries the same
// work, where equal tiles would leave the last round of workgroup slots partly empty.
// (Running the short band first on half of the workgroups, so that co-resident
// workgroups reach their epilogues at different times, measured slower on c4.)
template <typename T, int BM, int BN, int WM, int WN, int ACT, class Out, int MF, int BM2>
__global__ __launch_bounds__(kThreadsH) __attribute__((amdgpu_waves_per_eu(rb_waves(sizeof(T), BN, MF)))) void halo_rb_kernel(
    const T* __restrict__ A, HaloGeom g, const uint4* __restrict__ Bf, Out out, int tiles_n) {
    const int tile = xcd_tile(blockIdx.x, gridDim.x);
    const int tn = tile % tiles_n;
    const int sp = tile / tiles_n;
    const int qsp = fdiv(sp, g.fTC);
    const int tc = sp - qsp * g.tiles_c;
    const int n = fdiv(qsp, g.fTR);
    const int tr = qsp - n * g.tiles_r;
    const int c0 = tc * g.Q, n0 = tn * BN;
    if constexpr (BM2 == 0) {
        rb_tile<T, BM, BN, WM, WN, ACT, Out, MF>(A, g, Bf, out, n, tr * g.R, c0, n0, g.R, sp);
    } else {
        // statistics index: the 2*tiles_r bands of image n are contiguous, long ones first
        const int bands = 2 * g.tiles_r;
        rb_tile<T, BM, BN, WM, WN, ACT, Out, MF>(A, g, Bf, out, n, tr * g.R, c0, n0, g.R,
                                                 (n * bands + tr) * g.tiles_c + tc);
        __syncthreads();  // the first tile's epilogue is done with the LDS
        rb_tile<T, BM2, BN, WM, WN, ACT, Out, MF>(A, g, Bf, out, n, g.tiles_r * g.R + tr * g.R2, c0, n0, g.R2,
                                                  (n * bands + g.tiles_r + tr) * g.tiles_c + tc);
    }
}

// Weights in B-fragment order for halo_rb_kernel with fragments of mf = 32 or 16 rows.
// Output 16-byte unit  ((group * nsteps + st) * kst + kk) * 64 + lane,  st = chunk * KH*KW
// + tap, kst = 4 (mf 32) or 2 (mf 16), holds, for row = mf*group + lane%mf, the 8
// consecutive k of channel chunk*64 + kk*16 + (lane/32)*8 (mf 32) or chunk*64 + kk*32 +
// (lane/16)*8 (mf 16) at tap.  Forward rows are output channels:
// w[row, tap, ch]; input-gradient rows are input channels: w[ch, tap, row].  Rows past
// the matrix are zero.
template <typename T>
__global__ __launch_bounds__(256) void frag_weights(const T* __restrict__ w, uint4* __restrict__ dst, int Nn,
                                                    int taps, int Cin, int nsteps, int fwd, int mf) {
    // block (st, group) writes the kst*64 units of one step of one row group; thread
    // kk*64 + lane writes unit (..., kk) * 64 + lane (no per-unit index division)
    constexpr int EV = 16 / (int)sizeof(T), CK = 128 / (int)sizeof(T);  // per 16 bytes, per 128-byte chunk
    const int kst = mf == 32 ? 4 : 2;
    const int st = blockIdx.x, grp = blockIdx.y;
    const int l = threadIdx.x & 63, kk = threadIdx.x >> 6;
    const int row = grp * mf + (l & (mf - 1));
    const int chunk = st / taps, tap = st - chunk * taps;
    const int ch0 = chunk * CK + kk * (CK / kst) + (l / mf) * EV;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < Nn) {
        if (fwd) {
            v = *(const uint4*)(w + ((int64_t)row * taps + tap) * Cin + ch0);
        } else {
            T e[EV];
#pragma unroll
            for (int k = 0; k < EV; ++k) e[k] = w[((int64_t)(ch0 + k) * taps + tap) * Nn + row];
            __builtin_memcpy(&v, e, 16);
        }
    }
    dst[((int64_t)((int64_t)grp * nsteps + st) * kst + kk) * 64 + l] = v;
}

// ------------------------------------------------------------------ host side
constexpr int kLdsMax = 160 * 1024;

struct HaloPlan {
    int bm, bn, hb;
    int R, Q;
    int lds;     // dynamic LDS bytes per workgroup
    int mf = 32; // MFMA fragment height: bf16 32 (32x32x16) or 16 (16x16x32, 224-row blocks); fp32 16
    int R2 = 0;  // paired bands: rows of the short bands, computed in bm2 fragment rows
    int bm2 = 0;
};

int halo_groups(int R, int Q, int KH, int KW) { return ((R + KH - 1) * (Q + KW - 1) + 7) / 8; }

// Bytes before the per-column parameters: the halo buffers (the weights stream through
// registers), reused by the epilogue's staged tile.
int plan_main(int bm, int bn, int hb, int gh, int esize) {
    const int ring = hb * gh * 1024;
    const int epi = bm * (bn + 16 / esize) * esize;
    return (int)align_up((size_t)(ring > epi ? ring : epi), 16);
}

struct Sides {
    int Hout, Wout, Cin, Nn;
    int par;  // per-column epilogue parameter arrays (forward: bias and four batch-norm ones)
};

int plan_lds(int bm, int bn, int hb, int gh, int esize, const Sides& sd) {
    return plan_main(bm, bn, hb, gh, esize) + sd.par * bn * 4;
}

// Estimated time of a tile layout: rounds of workgroups times the slower of the bytes a
// CU loads (16-byte loads of whole cache lines run at about 34-60 B/clk per CU) and its
// MFMA work (about 3700 bf16 flop/clk per CU measured for 32x32x16 fed from LDS; 256
// fp32 flop/clk peak).  A single halo buffer exposes the copy of every later chunk's
// halo, half hidden when a second workgroup shares the CU.  Only the ranking matters.
double plan_cost(int dt, const ConvDims& d, const Sides& sd, int bm, int bn, int hb, int R, int Q, int occ) {
    const int64_t tiles = (int64_t)d.N * ceil_div(sd.Hout, R) * ceil_div(sd.Wout, Q) * ceil_div(sd.Nn, bn);
    const double rounds = fmax(1.0, (double)tiles / ((double)kCUs * occ));
    const int chunks = sd.Cin * (int)dtype_size(dt) / 128;
    const double halo = halo_groups(R, Q, d.KH, d.KW) * 1024.0;
    const double copy = chunks * (halo + (double)d.KH * d.KW * bn * 128) / 34.0;
    const double mfma = 2.0 * bm * bn * d.KH * d.KW * sd.Cin / (dt == DT_BF16 ? 3700.0 : 256.0);
    double clk = fmax(copy, mfma) + 0.05 * (copy + mfma);  // the smaller one still costs a little
    if (hb == 1 && chunks > 1) clk += (chunks - 1) * halo / 34.0 * (occ == 1 ? 1.0 : 0.5);
    if (occ == 1) clk *= 1.6;  // a lone workgroup per CU leaves every stall exposed (measured)
    return rounds * occ * clk;
}

// Paired bands for 224-row tiles (halo_rb_kernel): each workgroup also takes a band of
// R2 = 192 / Q rows (at most 12 fragments of 16 pixels, 192 rows).  Taken when the plain
// tiles leave the last round of workgroup slots partly empty and the pairs need fewer
// fragment-row rounds (7 per 224-row tile, 6 per short one); the bands must tile the
// image with every band starting inside it.  c4 (64 images of 56 x 56, Q = 28): 896
// tiles of 8 rows on 512 slots take two rounds of 7; 512 pairs of 8 + 6 rows take 13.
void pair_bands(const ConvDims& d, const Sides& sd, HaloPlan* p) {
    const int R = p->R, Q = p->Q, R2 = 192 / Q;
    if (R2 < 1 || R2 >= R) return;
    const int occ = std::min(rb_waves(2, p->bn, p->mf), kLdsMax / p->lds);  // workgroups per CU
    const int64_t slots = (int64_t)kCUs * occ;
    const int64_t per_band = (int64_t)d.N * ceil_div(sd.Wout, Q) * ceil_div(sd.Nn, p->bn);
    const int64_t plain = ceil_div(per_band * ceil_div(sd.Hout, R), slots) * 7;
    const int nb = (int)ceil_div(sd.Hout, R + R2);
    if (nb * R + (nb - 1) * R2 >= sd.Hout) return;  // the last short band would start below the image
    const int64_t paired = ceil_div(per_band * nb, slots) * (7 + ceil_div(R2 * Q, 32));
    if (paired >= plain) return;
    p->R2 = R2;
    p->bm2 = 192;
}

// Output tiles are R x Q rectangles: Q is the whole row or an even split of it, and the
// R*Q pixels fill at least three quarters of the block's MFMA rows.  Block heights are
// tried in a fixed order (a taller block loads each weight fragment for more pixels):
// bf16 256 or 128 rows for 128 output channels; 256, 512 or 128 rows for 64 (256-row
// blocks keep two workgroups on a CU, so one's halo copy overlaps the other's MFMAs:
// c5's forward 52 -> 49 us and input gradient 44 -> 40 us against 512-row blocks with
// one workgroup per CU); fp32 256 or 224.
// Within the first height that fits, the layout with the lowest estimated time wins.
bool pick_halo(int dt, const ConvDims& d, const Sides& sd, HaloPlan* best) {
    const int es = (int)dtype_size(dt);
    if ((sd.Cin * es) % 128) return false;
    const int chunks = sd.Cin * es / 128;
    const int bn = sd.Nn <= 64 ? 64 : 128;
    bool found = false;
    double best_cost = 0.0;
    auto try_bm = [&](int bm, int mf) {
        for (int R = 1; R <= bm && R <= sd.Hout; ++R) {
            int Q = bm / R;
            if (Q > sd.Wout) Q = sd.Wout;
            const int nseg = (int)ceil_div(sd.Wout, Q);
            Q = (int)ceil_div(sd.Wout, nseg);
            if (R * Q * 4 < bm * 3) continue;
            const int gh = halo_groups(R, Q, d.KH, d.KW);
            for (int hb = 1; hb <= (chunks > 1 ? 2 : 1); ++hb) {
                const int lds = plan_lds(bm, bn, hb, gh, es, sd);
                if (lds > kLdsMax) continue;
                const int occ = lds <= kLdsMax / 2 ? 2 : 1;
                const double cost = plan_cost(dt, d, sd, bm, bn, hb, R, Q, occ);
                if (!found || cost < best_cost) {
                    *best = HaloPlan{bm, bn, hb, R, Q, lds, mf};
                    best_cost = cost;
                    found = true;
                }
            }
        }
    };
    if (dt == DT_BF16 && bn == 128) {
        // 256-row blocks of 32x32x16 fragments, or 224-row blocks of 16x16x32 ones (rows
        // of 28 or 56 pixels fill 224 exactly): the cheaper estimate wins
        try_bm(256, 32);
        try_bm(224, 16);
        if (!found) try_bm(128, 32);
        if (found && best->bm == 224) pair_bands(d, sd, best);
        return found;
    }
    if (dt == DT_BF16) {
        // 64 channels: 224-row blocks of 16-row fragments (four workgroups per CU) when
        // paired bands fill whole rounds of slots; otherwise the 32-row-fragment blocks below
        try_bm(224, 16);
        if (found) {
            pair_bands(d, sd, best);
            if (best->R2) return true;
            found = false;
        }
    }
    // fp32 with 128 output channels: 224-row blocks first (256 rows of 16x16x4 fragments
    // exceed the register budget of two workgroups per CU)
    static const int bms_b64[] = {256, 512, 128, 0}, bms_f32[] = {256, 224, 0}, bms_f32w[] = {224, 256, 0};
    const int* bms0 = dt == DT_BF16 ? bms_b64 : (bn == 128 ? bms_f32w : bms_f32);
    for (const int* bms = bms0; *bms && !found; ++bms) try_bm(*bms, dt == DT_BF16 ? 32 : 16);
    return found;
}

HaloGeom make_geom(const ConvDims& d, const Sides& sd, const HaloPlan& p, int dt, bool fwd) {
    HaloGeom g;
    g.Hin = fwd ? d.H : d.OH;
    g.Win = fwd ? d.W : d.OW;
    g.Cin = sd.Cin;
    g.KH = d.KH;
    g.KW = d.KW;
    g.Hout = sd.Hout;
    g.Wout = sd.Wout;
    g.Nn = sd.Nn;
    g.R = p.R;
    g.R2 = p.R2;
    g.Q = p.Q;
    g.HQ = p.Q + d.KW - 1;
    g.QS = g.HQ - 2 * ((d.KW - 1) / 2);
    g.HP = (p.R + d.KH - 1) * g.HQ;
    g.GH = (g.HP + 7) / 8;
    g.org_r = fwd ? -d.ph : d.ph - d.KH + 1;
    g.org_c = fwd ? -d.pw : d.pw - d.KW + 1;
    g.tiles_r = p.R2 ? (int)ceil_div(sd.Hout, p.R + p.R2) : (int)ceil_div(sd.Hout, p.R);
    g.tiles_c = (int)ceil_div(sd.Wout, p.Q);
    g.nchunks = sd.Cin * (int)dtype_size(dt) / 128;
    g.Kb = d.KH * d.KW * sd.Cin;
    g.sign = fwd ? 1 : -1;
    g.hb = p.hb;
    g.par_off = plan_main(p.bm, p.bn, p.hb, g.GH, (int)dtype_size(dt));
    g.img_stride = (int64_t)g.Hin * g.Win * g.Cin;
    g.fQ = make_fastdiv(p.Q);
    g.fHQ = make_fastdiv(g.HQ);
    g.fTR = make_fastdiv(g.tiles_r);
    g.fTC = make_fastdiv(g.tiles_c);
    return g;
}

template <class K> hipError_t raise_lds(K kern, bool& raised) {
    if (raised) return hipSuccess;  // the dynamic LDS limit is raised once per instantiation
    const hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax);
    if (e == hipSuccess) raised = true;
    return e;
}

template <typename T, int BM, int BN, int WM, int WN, int ACT, class Out, int MF, int BM2 = 0>
hipError_t launch_rb(const T* A, const HaloGeom& g, const uint4* Bf, const Out& out, int images, int lds,
                     hipStream_t s) {
    auto kern = halo_rb_kernel<T, BM, BN, WM, WN, ACT, Out, MF, BM2>;
    static bool raised = false;
    const hipError_t e = raise_lds(kern, raised);
    if (e != hipSuccess) return e;
    const int tiles_n = (int)ceil_div(g.Nn, BN);
    const int64_t grid = (int64_t)images * g.tiles_r * g.tiles_c * tiles_n;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreadsH), lds, s, A, g, Bf, out, tiles_n);
    return hipGetLastError();
}

template <int ACT, class Out>
hipError_t dispatch_f32(const float* A, const HaloGeom& g, const uint4* Bf, const Out& out, const HaloPlan& p,
                        int images, hipStream_t s) {
#define CONVMI_HP(BM_, BN_)                                                                                      \
    if (p.bm == BM_ && p.bn == BN_ && p.mf == 16 && p.bm2 == 0)                                                \
        return launch_rb<float, BM_, BN_, 2, 2, ACT, Out, 16>(A, g, Bf, out, images, p.lds, s);
    CONVMI_HP(224, 128) CONVMI_HP(224, 64) CONVMI_HP(256, 128) CONVMI_HP(256, 64)
#undef CONVMI_HP
    return hipErrorInvalidValue;
}

// bf16 wave layouts: 128 output channels as 2 x 64 (waves 2 x 2; TN = 2 fragments of 32 per
// wave, or with 224-row blocks 7 x 4 fragments of 16); 64 output channels as 1 x 64 (waves
// 4 x 1).
template <int ACT, class Out>
hipError_t dispatch_bf16(const bf16* A, const HaloGeom& g, const uint4* Bf, const Out& out, const HaloPlan& p,
                         int images, hipStream_t s) {
#define CONVMI_RB(BM_, BN_, WM_, WN_, MF_)                                                                  \
    if (p.bm == BM_ && p.bn == BN_ && p.mf == MF_ && p.bm2 == 0)                                              \
        return launch_rb<bf16, BM_, BN_, WM_, WN_, ACT, Out, MF_>(A, g, Bf, out, images, p.lds, s);
    if (p.bm == 224 && p.bn == 128 && p.mf == 16 && p.bm2 == 192)
        return launch_rb<bf16, 224, 128, 2, 2, ACT, Out, 16, 192>(A, g, Bf, out, images, p.lds, s);
    if (p.bm == 224 && p.bn == 64 && p.mf == 16 && p.bm2 == 192)
        return launch_rb<bf16, 224, 64, 2, 2, ACT, Out, 16, 192>(A, g, Bf, out, images, p.lds, s);
    CONVMI_RB(256, 128, 2, 2, 32) CONVMI_RB(224, 128, 2, 2, 16) CONVMI_RB(128, 128, 2, 2, 32)
    CONVMI_RB(224, 64, 2, 2, 16)
    CONVMI_RB(512, 64, 4, 1, 32) CONVMI_RB(256, 64, 4, 1, 32) CONVMI_RB(128, 64, 4, 1, 32)
#undef CONVMI_RB
    return hipErrorInvalidValue;
}

Sides fwd_sides(const ConvDims& d) { return Sides{d.OH, d.OW, d.IC, d.OC, HFwdBnOut::kPar}; }
Sides dx_sides(const ConvDims& d) { return Sides{d.H, d.W, d.OC, d.IC, HDxOut::kPar}; }

// Fragment-ordered weights: every column tile's rows, KH*KW*Cin k each, in the element type.
size_t frag_bytes(const ConvDims& d, const Sides& sd, const HaloPlan& p, int es) {
    return align_up((size_t)ceil_div(sd.Nn, p.bn) * p.bn * d.KH * d.KW * sd.Cin * es, 256);
}

hipError_t launch_frag_weights(int dt, const void* w, uint4* dst, const ConvDims& d, const Sides& sd,
                               const HaloPlan& p, bool fwd, hipStream_t s) {
    const int taps = d.KH * d.KW;
    const int nsteps = (sd.Cin * (int)dtype_size(dt) / 128) * taps;
    const int64_t groups = ceil_div(sd.Nn, p.bn) * (p.bn / p.mf);
    if (groups > 65535) return hipErrorInvalidValue;  // grid y limit (Nn above a million channels)
    const dim3 grid((unsigned)nsteps, (unsigned)groups);
    const int threads = (p.mf == 32 ? 4 : 2) * 64;
    if (dt == DT_BF16)
        frag_weights<bf16><<<grid, threads, 0, s>>>((const bf16*)w, dst, sd.Nn, taps, sd.Cin, nsteps, fwd ? 1 : 0,
                                                     p.mf);
    else
        frag_weights<float><<<grid, threads, 0, s>>>((const float*)w, dst, sd.Nn, taps, sd.Cin, nsteps, fwd ? 1 : 0,
                                                      p.mf);
    return hipGetLastError();
}

}  // namespace

bool halo_fwd_supported(int dt, const ConvDims& d) {
    HaloPlan p;
    return d.sh == 1 && d.sw == 1 && pick_halo(dt, d, fwd_sides(d), &p);
}

bool halo_dx_supported(int dt, const ConvDims& d) {
    HaloPlan p;
    return d.sh == 1 && d.sw == 1 && pick_halo(dt, d, dx_sides(d), &p);
}

bool halo_plan_text(int dt, const ConvDims& d, bool fwd, char* buf, size_t len) {
    HaloPlan p;
    if (d.sh != 1 || d.sw != 1 || !pick_halo(dt, d, fwd ? fwd_sides(d) : dx_sides(d), &p)) return false;
    if (p.R2)
        snprintf(buf, len, "halo %s %dx%d mf%d tile %dx%d hb%d paired %dx%d in %d rows", dt == DT_BF16 ? "bf16" : "f32",
                 p.bm, p.bn, p.mf, p.R, p.Q, p.hb, p.R2, p.Q, p.bm2);
    else
        snprintf(buf, len, "halo %s %dx%d mf%d tile %dx%d hb%d", dt == DT_BF16 ? "bf16" : "f32", p.bm, p.bn, p.mf,
                 p.R, p.Q, p.hb);
    return true;
}

size_t halo_fwd_ws_bytes(int dt, const ConvDims& d) {
    HaloPlan p;
    if (!halo_fwd_supported(dt, d) || !pick_halo(dt, d, fwd_sides(d), &p)) return 0;
    return frag_bytes(d, fwd_sides(d), p, (int)dtype_size(dt));
}

size_t halo_dx_ws_bytes(int dt, const ConvDims& d) {
    HaloPlan p;
    if (!halo_dx_supported(dt, d) || !pick_halo(dt, d, dx_sides(d), &p)) return 0;
    return frag_bytes(d, dx_sides(d), p, (int)dtype_size(dt));
}

int halo_fwd_stat_tiles(int dt, const ConvDims& d) {
    const Sides sd = fwd_sides(d);
    HaloPlan p;
    if (d.sh != 1 || d.sw != 1 || !pick_halo(dt, d, sd, &p)) return 0;
    const int64_t bands = p.R2 ? 2 * ceil_div(sd.Hout, p.R + p.R2) : ceil_div(sd.Hout, p.R);
    return (int)(d.N * bands * ceil_div(sd.Wout, p.Q));
}

hipError_t launch_halo_fwd(int dt, const void* x, const void* w, const float* bias, void* z, void* y,
                           const ConvDims& d, int act, void* ws, hipStream_t s, const float* const* bn_eval,
                           float* stats_part) {
    const Sides sd = fwd_sides(d);
    HaloPlan p;
    if (d.sh != 1 || d.sw != 1 || !pick_halo(dt, d, sd, &p)) return hipErrorInvalidValue;
    const HaloGeom g = make_geom(d, sd, p, dt, true);
    if (stats_part) {
        if (bn_eval || !z) return hipErrorInvalidValue;
        const int ntiles = d.N * (g.R2 ? 2 : 1) * g.tiles_r * g.tiles_c;
        const HFwdStatsOut os{z, bias, d.OC, stats_part, ntiles};
        const hipError_t e = launch_frag_weights(dt, w, (uint4*)ws, d, sd, p, true, s);
        if (e != hipSuccess) return e;
        if (dt == DT_BF16)
            return dispatch_bf16<ACT_IDENTITY, HFwdStatsOut>((const bf16*)x, g, (const uint4*)ws, os, p, d.N, s);
        return dispatch_f32<ACT_IDENTITY, HFwdStatsOut>((const float*)x, g, (const uint4*)ws, os, p, d.N, s);
    }
    const HFwdOut o{z, y, bias, d.OC};
    const HFwdBnOut ob{z, y, bias, d.OC, bn_eval ? bn_eval[0] : nullptr, bn_eval ? bn_eval[1] : nullptr,
                       bn_eval ? bn_eval[2] : nullptr, bn_eval ? bn_eval[3] : nullptr};
    if (bn_eval && (!y || !bn_eval[0] || !bn_eval[1] || !bn_eval[2] || !bn_eval[3])) return hipErrorInvalidValue;
    const hipError_t e = launch_frag_weights(dt, w, (uint4*)ws, d, sd, p, true, s);
    if (e != hipSuccess) return e;
    const uint4* wf = (const uint4*)ws;
    if (dt == DT_BF16) {
        if (bn_eval)
            CONVMI_ACT_SWITCH(act, A_, return (dispatch_bf16<A_, HFwdBnOut>((const bf16*)x, g, wf, ob, p, d.N, s)));
        CONVMI_ACT_SWITCH(act, A_, return (dispatch_bf16<A_, HFwdOut>((const bf16*)x, g, wf, o, p, d.N, s)));
    } else {
        if (bn_eval)
            CONVMI_ACT_SWITCH(act, A_, return (dispatch_f32<A_, HFwdBnOut>((const float*)x, g, wf, ob, p, d.N, s)));
        CONVMI_ACT_SWITCH(act, A_, return (dispatch_f32<A_, HFwdOut>((const float*)x, g, wf, o, p, d.N, s)));
    }
    return hipErrorInvalidValue;
}

hipError_t launch_halo_dx(int dt, const void* dz, const void* w, void* dx, const ConvDims& d, void* ws,
                          hipStream_t s) {
    const Sides sd = dx_sides(d);
    HaloPlan p;
    if (d.sh != 1 || d.sw != 1 || !pick_halo(dt, d, sd, &p)) return hipErrorInvalidValue;
    const HaloGeom g = make_geom(d, sd, p, dt, false);
    const HDxOut o{dx, d.IC};
    const hipError_t e = launch_frag_weights(dt, w, (uint4*)ws, d, sd, p, false, s);
    if (e != hipSuccess) return e;
    if (dt == DT_BF16) return dispatch_bf16<ACT_IDENTITY, HDxOut>((const bf16*)dz, g, (const uint4*)ws, o, p, d.N, s);
    return dispatch_f32<ACT_IDENTITY, HDxOut>((const float*)dz, g, (const uint4*)ws, o, p, d.N, s);
}

}  // namespace convmi
