// k_igemm.hip -- convolution forward and input gradient as implicit GEMM on gfx950 MFMA.
//
// Forward (convolution + bias, with the activation epilogue fused when there is no
// normalisation):  C[m][n] = sum_k A[m][k] * B[n][k]
//   m = (n_img, oh, ow)  rows of z, y         (M = N*OH*OW)
//   n = oc                                     (N = OC)
//   k = (kh, kw, ic)     ic fastest            (K = KH*KW*IC)
//   A[m][k] = x[n_img, oh*sh - ph + kh, ow*sw - pw + kw, ic] (0 outside)   -- gathered
//   B[n][k] = w[oc, kh, kw, ic]                                            -- w as stored
//
// Input gradient, any stride, as one GEMM over "phase blocks":  write
// ih + ph = sh*qh + rh (0 <= rh < sh), likewise for w.  A tap kh reaches input row ih
// only from oh = qh - a where kh = rh + sh*a, so with KHs = ceil(KH/sh):
//   m = (n_img, qh, qw)                       rows   (qh over the blocks that touch the image)
//   n = (rh, rw, ic)     ic fastest            (N = sh*sw*IC)
//   k = (a, b, oc)       oc fastest            (K = KHs*KWs*OC)
//   A[m][k] = dz[n_img, qh - a, qw - b, oc] (0 outside)                   -- gathered
//   B[n][k] = w[oc, rh + sh*a, rw + sw*b, ic] (0 past the kernel)          -- rearranged copy
//   dx[n_img, sh*qh + rh - ph, sw*qw + rw - pw, ic] = C[m][n]  where in range
// For stride 1 this is the usual gather form of the transposed convolution; for stride s
// it keeps every MFMA column useful even when IC is tiny (4 channels, stride 4: N = 64).
//
// Kernel structure: 256 threads (4 waves), block tile BM x BN, K step BK.  Global
// operands are read as 16-byte vectors (8 bf16 or 4 fp32 consecutive k), staged through
// registers into double-buffered LDS tiles stored K-contiguous with a 16-byte row pad,
// and consumed by 16x16 MFMA tiles: v_mfma_f32_16x16x32_bf16 for bf16,
// 4 x v_mfma_f32_16x16x4_f32 per 16-byte vector for fp32 (the four k of a lane vector are
// spread over four MFMAs; A and B use the same order, so the sum is unchanged).  The
// accumulators (fp32) go through LDS once more so the epilogue writes 16-byte vectors.
// Blocks are renumbered so consecutive M tiles share one XCD's L2.
//
// Definitions followed: rl_tools conv2d listings "operations_generic.h" (forward:
// convolution + bias into pre_activations; backward_input: scatter of w * d_pre_act) and
// "operations_cuda.h" (forward with bias + activation; backward_input = BackwardData).
#include "internal.hpp"
#include "lds_dma.hpp"

namespace convmi {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int NT = 256;

template <typename T> struct Mma;
template <> struct Mma<bf16> {
    static constexpr int VEC = 8;   // elements per 16-byte lane vector
    static constexpr int KM = 32;   // k consumed per MFMA step (4 lane groups x VEC)
    static __device__ __forceinline__ void run(floatx4& c, const uint4& a, const uint4& b) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                    0, 0, 0);
    }
};
template <> struct Mma<float> {
    static constexpr int VEC = 4;
    static constexpr int KM = 16;
    static __device__ __forceinline__ void run(floatx4& c, const uint4& a, const uint4& b) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    }
};

// Gathered operand: rows m = (n_img, r1, r2) over an R1 x R2 grid per image; a row's
// window origin is (r1*rs1 + ro1, r2*rs2 + ro2) in a [Hin][Win][Cin] image; k = (kh, kw, c)
// with c fastest over a kernel KWk taps wide; tap (kh, kw) reads (ih0 + SIGN*kh,
// iw0 + SIGN*kw).
struct GatherGeom {
    int Hin, Win, Cin, KWk;
    int R1, R2, rs1, ro1, rs2, ro2;
    int M;
    int64_t img_stride;  // Hin*Win*Cin
    FastDiv fR1, fR2, fCin, fKWC;
};

// Epilogue targets.  For each 16-byte output vector (VEC columns from col) of row m:
// colinit() once per thread for its fixed column range, store() per row.
template <typename T> __device__ __forceinline__ void store_vec(T* p, const float* v);
template <> __device__ __forceinline__ void store_vec<float>(float* p, const float* v) {
    *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
}
template <> __device__ __forceinline__ void store_vec<bf16>(bf16* p, const float* v) {
    *(uint4*)p = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                            pack_bf16x2(v[6], v[7]));
}

// z = acc + bias (stored in T), y = act(stored z).
struct FwdOut {
    void* z;            // nullable
    void* y;            // nullable
    const float* bias;  // nullable
    int OC;
    int act;
    template <int VEC> __device__ __forceinline__ void colinit(int col, float* bv) const {
#pragma unroll
        for (int j = 0; j < VEC; ++j) bv[j] = (bias && col + j < OC) ? bias[col + j] : 0.0f;
    }
    template <typename T, int ACT, int VEC>
    __device__ __forceinline__ void store(int m, int col, const float* v, const float* bv) const {
        float zr[VEC], yr[VEC];
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            zr[j] = round_trip<T>(v[j] + bv[j]);
            yr[j] = act_fwd<ACT>(zr[j]);
        }
        const int64_t base = (int64_t)m * OC + col;
        if (col + VEC <= OC && (OC % VEC) == 0) {
            if (z) store_vec<T>((T*)z + base, zr);
            if (y) store_vec<T>((T*)y + base, yr);
        } else {
            for (int j = 0; j < VEC && col + j < OC; ++j) {
                if (z) ((T*)z)[base + j] = from_f32<T>(zr[j]);
                if (y) ((T*)y)[base + j] = from_f32<T>(yr[j]);
            }
        }
    }
};

// dx[n, sh*qh + rh - ph, sw*qw + rw - pw, ic] = C[(n, qh, qw)][(rh, rw, ic)] where in range.
struct DxOut {
    void* dx;
    int N, H, W, IC;
    int QH, QW, qh0, qw0;  // row grid and its origin in block units
    int sh, sw, ph, pw;
    FastDiv fQW, fQH, fIC, fsw;
    template <int VEC> __device__ __forceinline__ void colinit(int, float*) const {}
    template <typename T, int ACT, int VEC>
    __device__ __forceinline__ void store(int m, int col, const float* v, const float*) const {
        // IC is a multiple of VEC, so the vector stays inside one phase (rh, rw)
        const int phs = fdiv(col, fIC);
        const int ic = col - phs * IC;
        const int rh = fdiv(phs, fsw), rw = phs - rh * sw;
        const int q = fdiv(m, fQW);
        const int qw = m - q * QW;
        const int n = fdiv(q, fQH);
        const int qh = q - n * QH;
        const int ih = (qh + qh0) * sh + rh - ph;
        const int iw = (qw + qw0) * sw + rw - pw;
        if (ih < 0 || ih >= H || iw < 0 || iw >= W) return;
        store_vec<T>((T*)dx + (((int64_t)n * H + ih) * W + iw) * IC + ic, v);
    }
};

template <typename T, int BM, int BN, int BK, int WM, int WN, int SIGN, int ACT, class Out>
__global__ __launch_bounds__(NT) void igemm_kernel(const T* __restrict__ A, GatherGeom g, const T* __restrict__ B,
                                                   int Nn, int Kb, Out out, int tiles_n) {
    using MM = Mma<T>;
    constexpr int VEC = MM::VEC, KM = MM::KM;
    static_assert(WM * WN == 4, "four waves");
    constexpr int TM = BM / (WM * 16), TN = BN / (WN * 16);
    static_assert(TM * WM * 16 == BM && TN * WN * 16 == BN, "tile shape");
    static_assert(BK % KM == 0, "K step");
    constexpr int LDK = BK + VEC;  // padded LDS row (elements)
    constexpr int KV = BK / VEC;   // 16-byte vectors per row per K step
    constexpr int RPP = NT / KV;   // rows loaded per pass
    static_assert(BM % RPP == 0, "load passes");
    constexpr int AP = BM / RPP, BP = (BN + RPP - 1) / RPP;  // B rows may not fill the last pass
    constexpr int STAGE = (BM + BN) * LDK;                 // elements per LDS stage
    constexpr int LDS_AB = 2 * STAGE * (int)sizeof(T);
    constexpr int LDC = BN + 4;                            // fp32 staging row
    constexpr int LDS_C = BM * LDC * 4;
    constexpr int LDS_BYTES = LDS_AB > LDS_C ? LDS_AB : LDS_C;
    __shared__ __align__(16) unsigned char smem[LDS_BYTES];
    T* lds = (T*)smem;

    const int t = threadIdx.x;
    const int tile = xcd_tile(blockIdx.x, gridDim.x);
    const int m0 = (tile / tiles_n) * BM, n0 = (tile % tiles_n) * BN;

    // ---- per-thread gather state (fixed for the whole K loop)
    const int kv = t % KV, rr = t / KV;
    const int kofs = kv * VEC;
    const int kq = fdiv(kofs, g.fCin), kr = kofs - kq * g.Cin;  // tap and channel offset of this vector
    int64_t a_base[AP];
    int a_h[AP], a_w[AP];
    bool a_ok[AP];
#pragma unroll
    for (int p = 0; p < AP; ++p) {
        const int m = m0 + p * RPP + rr;
        a_ok[p] = m < g.M;
        const int mm = a_ok[p] ? m : 0;
        const int q = fdiv(mm, g.fR2);
        const int r2 = mm - q * g.R2;
        const int n = fdiv(q, g.fR1);
        const int r1 = q - n * g.R1;
        a_h[p] = r1 * g.rs1 + g.ro1;
        a_w[p] = r2 * g.rs2 + g.ro2 + SIGN * kq;
        a_base[p] = (int64_t)n * g.img_stride + ((int64_t)a_h[p] * g.Win + a_w[p]) * g.Cin + kr;
    }
    const T* b_ptr[BP];
    bool b_ok[BP];
    const bool b_row = (BN % RPP == 0) || rr < BN % RPP;  // this thread owns a row in the last pass
#pragma unroll
    for (int p = 0; p < BP; ++p) {
        const int n = n0 + p * RPP + rr;
        b_ok[p] = n < Nn && (p * RPP + rr) < BN;
        b_ptr[p] = B + (int64_t)(b_ok[p] ? n : 0) * Kb + kofs;
    }
    const int KWC = g.KWk * g.Cin;

    uint4 ra[AP], rb[BP];
    auto load = [&](int k0) {
        const int kh = fdiv(k0, g.fKWC);
        const int rem = k0 - kh * KWC;
        const int kw = fdiv(rem, g.fCin);
        const int c0 = rem - kw * g.Cin;
        const int dh = SIGN * kh, dw = SIGN * kw;
        const int64_t U = ((int64_t)dh * g.Win + dw) * g.Cin + c0;
#pragma unroll
        for (int p = 0; p < AP; ++p) {
            const int ih = a_h[p] + dh, iw = a_w[p] + dw;
            const bool ok = a_ok[p] && (unsigned)ih < (unsigned)g.Hin && (unsigned)iw < (unsigned)g.Win;
            ra[p] = ok ? *(const uint4*)(A + a_base[p] + U) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int p = 0; p < BP; ++p) rb[p] = b_ok[p] ? *(const uint4*)(b_ptr[p] + k0) : make_uint4(0, 0, 0, 0);
    };
    auto stash = [&](int buf) {
        T* As = lds + buf * STAGE;
        T* Bs = As + BM * LDK;
#pragma unroll
        for (int p = 0; p < AP; ++p) *(uint4*)(As + (p * RPP + rr) * LDK + kofs) = ra[p];
#pragma unroll
        for (int p = 0; p < BP; ++p)
            if (p + 1 < BP || b_row) *(uint4*)(Bs + (p * RPP + rr) * LDK + kofs) = rb[p];
    };

    const int lane = t & 63, wid = t >> 6;
    const int wm = wid / WN, wn = wid % WN;
    const int lr = lane & 15, lk = (lane >> 4) * VEC;
    floatx4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int KT = Kb / BK;
    load(0);
    stash(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) load((kt + 1) * BK);
        const T* As = lds + buf * STAGE;
        const T* Bs = As + BM * LDK;
#pragma unroll
        for (int kk = 0; kk < BK; kk += KM) {
            uint4 af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) af[i] = *(const uint4*)(As + (wm * TM * 16 + i * 16 + lr) * LDK + kk + lk);
#pragma unroll
            for (int j = 0; j < TN; ++j) bfr[j] = *(const uint4*)(Bs + (wn * TN * 16 + j * 16 + lr) * LDK + kk + lk);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) MM::run(acc[i][j], af[i], bfr[j]);
        }
        if (kt + 1 < KT) stash(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: accumulators -> LDS (fp32) -> 16-byte vectors
    float* Cs = (float*)smem;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                Cs[(wm * TM * 16 + i * 16 + (lane >> 4) * 4 + e) * LDC + wn * TN * 16 + j * 16 + lr] = acc[i][j][e];
    __syncthreads();
    constexpr int OVR = BN / VEC;  // output vectors per row
    static_assert(NT % OVR == 0, "each thread keeps one column range");
    const int cv = t % OVR, col = n0 + cv * VEC;
    float bv[VEC];
    out.template colinit<VEC>(col, bv);
    if (col < Nn)
        for (int r = t / OVR; r < BM; r += NT / OVR) {
            const int m = m0 + r;
            if (m >= g.M) break;
            out.template store<T, ACT, VEC>(m, col, Cs + r * LDC + cv * VEC, bv);
        }
}

// ------------------------------------------------------------------ asynchronous-copy kernel
// The same GEMM with the operand tiles brought into LDS by the gfx950 LDS-DMA path
// (global_load_lds_dwordx4: lane i writes 16 bytes at M0 + 16*i), so no registers stage
// the tiles and STAGES-1 K steps are in flight while one is consumed.  A K step is one
// 128-byte row per tile row (64 bf16 or 32 fp32 of k); each group of 8 rows is one DMA
// instruction.  16-byte chunks are XOR-swizzled within a row (chunk c of row r lives at
// c ^ ((r >> 1) & 7)) so that 16 lanes reading the same chunk of 16 consecutive rows hit
// distinct LDS banks.  Rows outside the image or the matrix load a 16-byte zero page.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

template <typename T, int BM, int BN, int WM, int WN, int STAGES, int SIGN, int ACT, class Out>
__global__ __launch_bounds__(WM * WN * 64) void igemm2_kernel(const T* __restrict__ A, GatherGeom g,
                                                              const T* __restrict__ B, int Nn, int Kb, Out out,
                                                              int tiles_n) {
    using MM = Mma<T>;
    constexpr int NWAVE = WM * WN, NTH = NWAVE * 64;
    constexpr int VEC = MM::VEC;
    constexpr int BK = 128 / (int)sizeof(T);
    constexpr int TM = BM / (WM * 16), TN = BN / (WN * 16);
    static_assert(TM * WM * 16 == BM && TN * WN * 16 == BN, "tile shape");
    static_assert(BM % 8 == 0 && BN % 8 == 0, "8-row copy groups");
    constexpr int GA = BM / 8, GB = BN / 8;
    constexpr int GPW = (GA + GB + NWAVE - 1) / NWAVE;
    constexpr int STAGE_BYTES = (BM + BN) * 128;
    constexpr int RING = STAGES * STAGE_BYTES;
    constexpr int LDC = BN + 4;
    constexpr int EPI = BM * LDC * 4;
    constexpr int LDS_BYTES = RING > EPI ? RING : EPI;
    __shared__ __align__(1024) unsigned char smem[LDS_BYTES];

    const int t = threadIdx.x, lane = t & 63;
    const int wid = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform, kept in an SGPR
    const int tile = xcd_tile(blockIdx.x, gridDim.x);
    const int m0 = (tile / tiles_n) * BM, n0 = (tile % tiles_n) * BN;
    const uint32_t smem_base = __builtin_amdgcn_readfirstlane(lds_addr(smem));

    // per-lane copy state for each 8-row group this wave owns
    const int rg = lane >> 3, pc = lane & 7;
    int64_t cbase[GPW];
    int ch[GPW], cw[GPW];
    bool cok[GPW];
    int n_w = 0;  // copies this wave issues per stage (wave-uniform)
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
        const int grp = wid + NWAVE * j;
        cbase[j] = 0; ch[j] = 0; cw[j] = 0; cok[j] = false;
        if (grp >= GA + GB) continue;
        ++n_w;
        const int rl = (grp < GA ? grp : grp - GA) * 8 + rg;  // row within its tile
        const int kofs = (pc ^ swz(rl)) * VEC;                // logical k offset of this lane's chunk
        if (grp < GA) {
            const int m = m0 + rl;
            const int kq = fdiv(kofs, g.fCin), kr = kofs - kq * g.Cin;
            cok[j] = m < g.M;
            const int mm = cok[j] ? m : 0;
            const int q = fdiv(mm, g.fR2);
            const int r2 = mm - q * g.R2;
            const int n = fdiv(q, g.fR1);
            const int r1 = q - n * g.R1;
            ch[j] = r1 * g.rs1 + g.ro1;
            cw[j] = r2 * g.rs2 + g.ro2 + SIGN * kq;
            cbase[j] = (int64_t)n * g.img_stride + ((int64_t)ch[j] * g.Win + cw[j]) * g.Cin + kr;
        } else {
            const int n = n0 + rl;
            cok[j] = n < Nn;
            cbase[j] = (int64_t)(cok[j] ? n : 0) * Kb + kofs;
        }
    }
    const int KWC = g.KWk * g.Cin;

    auto issue = [&](int st) {  // copy K step st into ring slot st % STAGES
        const int k0 = st * BK;
        const int kh = fdiv(k0, g.fKWC);
        const int rem = k0 - kh * KWC;
        const int kw = fdiv(rem, g.fCin);
        const int c0 = rem - kw * g.Cin;
        const int dh = SIGN * kh, dw = SIGN * kw;
        const int64_t U = ((int64_t)dh * g.Win + dw) * g.Cin + c0;
        const uint32_t slot = smem_base + (uint32_t)((st % STAGES) * STAGE_BYTES);
#pragma unroll
        for (int j = 0; j < GPW; ++j) {
            const int grp = wid + NWAVE * j;
            if (grp >= GA + GB) break;
            const void* src;
            uint32_t dst;
            if (grp < GA) {
                const int ih = ch[j] + dh, iw = cw[j] + dw;
                const bool ok = cok[j] && (unsigned)ih < (unsigned)g.Hin && (unsigned)iw < (unsigned)g.Win;
                src = ok ? (const void*)(A + cbase[j] + U) : (const void*)&kZero16;
                dst = slot + grp * 1024;
            } else {
                src = cok[j] ? (const void*)(B + cbase[j] + k0) : (const void*)&kZero16;
                dst = slot + BM * 128 + (grp - GA) * 1024;
            }
            dma16(src, __builtin_amdgcn_readfirstlane(dst));
        }
    };

    const int wm = wid / WN, wn = wid % WN;
    const int lr = lane & 15, lg = lane >> 4;
    floatx4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int st) {
        const unsigned char* As = smem + (st % STAGES) * STAGE_BYTES;
        const unsigned char* Bs = As + BM * 128;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int lc = kk * 4 + lg;
            uint4 af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = wm * TM * 16 + i * 16 + lr;
                af[i] = *(const uint4*)(As + r * 128 + ((lc ^ swz(r)) << 4));
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int r = wn * TN * 16 + j * 16 + lr;
                bfr[j] = *(const uint4*)(Bs + r * 128 + ((lc ^ swz(r)) << 4));
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) MM::run(acc[i][j], af[i], bfr[j]);
        }
    };

    const int KT = Kb / BK;
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        if (st < KT) issue(st);
    for (int k = 0; k < KT; ++k) {
        const int later = (KT - 1 - k) < (STAGES - 2) ? (KT - 1 - k) : (STAGES - 2);
        wait_dma(later * n_w);
        __syncthreads();
        if (k + STAGES - 1 < KT) issue(k + STAGES - 1);
        compute(k);
    }
    __syncthreads();

    float* Cs = (float*)smem;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                Cs[(wm * TM * 16 + i * 16 + lg * 4 + e) * LDC + wn * TN * 16 + j * 16 + lr] = acc[i][j][e];
    __syncthreads();
    constexpr int OVR = BN / VEC;
    static_assert(NTH % OVR == 0, "each thread keeps one column range");
    const int cv = t % OVR, col = n0 + cv * VEC;
    float bv[VEC];
    out.template colinit<VEC>(col, bv);
    if (col < Nn)
        for (int r = t / OVR; r < BM; r += NTH / OVR) {
            const int m = m0 + r;
            if (m >= g.M) break;
            out.template store<T, ACT, VEC>(m, col, Cs + r * LDC + cv * VEC, bv);
        }
}

// B for the input gradient: Bt[(rh, rw, ic)][(a, b, oc)] = w[oc, rh + sh*a, rw + sw*b, ic].
template <typename T>
__global__ __launch_bounds__(NT) void dx_weights(const T* __restrict__ w, T* __restrict__ bt, ConvDims d, int KHs,
                                                 int KWs) {
    const int Ncol = d.sh * d.sw * d.IC;
    const int Kb = KHs * KWs * d.OC;
    const int total = Ncol * Kb;  // below 2^31 (checked by the launcher): 32-bit index arithmetic
    for (int i = blockIdx.x * NT + threadIdx.x; i < total; i += gridDim.x * NT) {
        const int col = i / Kb, k = i - col * Kb;
        const int oc = k % d.OC, ab = k / d.OC;
        const int b = ab % KWs, a = ab / KWs;
        const int ic = col % d.IC, ph_ = col / d.IC;
        const int rw = ph_ % d.sw, rh = ph_ / d.sw;
        const int kh = rh + d.sh * a, kw = rw + d.sw * b;
        T v = from_f32<T>(0.0f);
        if (kh < d.KH && kw < d.KW) v = w[(((int64_t)oc * d.KH + kh) * d.KW + kw) * d.IC + ic];
        bt[i] = v;
    }
}

// ------------------------------------------------------------------ host side
struct Cfg {
    int bm, bn, bk;
};

// Can a gathered operand with Cin channels and a kernel KWk taps wide be read in K steps
// of bk elements as whole 16-byte vectors that never straddle a tap?
bool gather_ok(int Cin, int KWk, int bk, int vec) {
    if (Cin % vec) return false;
    if (Cin % bk == 0) return true;
    return bk % Cin == 0 && (KWk * Cin) % bk == 0;
}

int pick_bk(int dt, int Cin, int KWk) {
    const int vec = dt == DT_BF16 ? 8 : 4;
    const int km = dt == DT_BF16 ? 32 : 16;
    if (gather_ok(Cin, KWk, 2 * km, vec)) return 2 * km;
    if (gather_ok(Cin, KWk, km, vec)) return km;
    return 0;
}

int pick_bn(int N) { return N <= 32 ? 32 : (N <= 64 ? 64 : 128); }

template <typename T, int BM, int BN, int BK, int SIGN, int ACT, class Out>
hipError_t launch_cfg(const T* A, const GatherGeom& g, const T* B, int Nn, int Kb, const Out& out,
                      hipStream_t s) {
    constexpr int WN = BN >= 64 ? 2 : 1;
    constexpr int WM = 4 / WN;
    const int tiles_m = (int)ceil_div(g.M, BM), tiles_n = (int)ceil_div(Nn, BN);
    igemm_kernel<T, BM, BN, BK, WM, WN, SIGN, ACT, Out><<<tiles_m * tiles_n, NT, 0, s>>>(A, g, B, Nn, Kb, out,
                                                                                         tiles_n);
    return hipGetLastError();
}

// Two ring stages (one K step in flight while one is consumed) keep a 128x128 block
// under 80 KB of LDS, so two workgroups share a CU and cover each other's load latency
// and epilogue; measured on MI355X this beats three stages at one workgroup per CU.
constexpr int kStages = 2;

// Asynchronous-copy kernel: pick the block tile whose last wave of workgroups leaves
// the fewest CUs idle (tiles are 16-row multiples so e.g. 200704 rows split evenly).
template <typename T, int BM, int BN, int WM, int WN, int SIGN, int ACT, class Out>
hipError_t launch2_cfg(const T* A, const GatherGeom& g, const T* B, int Nn, int Kb, const Out& out,
                       hipStream_t s) {
    const int tiles_m = (int)ceil_div(g.M, BM), tiles_n = (int)ceil_div(Nn, BN);
    igemm2_kernel<T, BM, BN, WM, WN, kStages, SIGN, ACT, Out><<<tiles_m * tiles_n, WM * WN * 64, 0, s>>>(
        A, g, B, Nn, Kb, out, tiles_n);
    return hipGetLastError();
}

double tile_cost(int M, int Nn, int bm, int bn, int lds_bytes, double eff) {
    int occ = 163840 / lds_bytes;
    occ = occ < 1 ? 1 : (occ > 2 ? 2 : occ);
    const int64_t tiles = ceil_div(M, bm) * ceil_div(Nn, bn);
    const int64_t rounds = ceil_div(tiles, 256LL * occ);
    return (double)rounds * occ * bm * bn / eff;
}

int lds2(int bm, int bn) {
    const int ring = kStages * (bm + bn) * 128, epi = bm * (bn + 4) * 4;
    return ring > epi ? ring : epi;
}

template <typename T, int SIGN, int ACT, class Out>
hipError_t launch2_any(const T* A, const GatherGeom& g, const T* B, int Nn, int Kb, const Out& out,
                       hipStream_t s) {
    const int bn = pick_bn(Nn);
    // fp32 grids of fewer 112-row tiles than CUs (small images, few channels): 32-row
    // tiles spread the work over every CU (measured 33 -> 22 us on 256 x 7x7x64 outputs).
    if (sizeof(T) == 4 && bn == 64 && ceil_div(g.M, 112) * ceil_div(Nn, 64) < 256)
        return launch2_cfg<T, 32, 64, 2, 2, SIGN, ACT, Out>(A, g, B, Nn, Kb, out, s);
    if (bn == 128) {
        const double c128 = tile_cost(g.M, Nn, 128, 128, lds2(128, 128), 1.0);
        const double c112 = tile_cost(g.M, Nn, 112, 128, lds2(112, 128), 0.97);
        if (c112 < c128) return launch2_cfg<T, 112, 128, 1, 4, SIGN, ACT, Out>(A, g, B, Nn, Kb, out, s);
        return launch2_cfg<T, 128, 128, 2, 2, SIGN, ACT, Out>(A, g, B, Nn, Kb, out, s);
    }
    if (bn == 64) {
        // fp32 grids that fill the CUs anyway: 64-row tiles (measured over 32, 64, 112 and
        // 128 rows: c2a's input gradient, 112896 x 64, 29.9 -> 28.4 us)
        if (sizeof(T) == 4) return launch2_cfg<T, 64, 64, 2, 2, SIGN, ACT, Out>(A, g, B, Nn, Kb, out, s);
        const double c128 = tile_cost(g.M, Nn, 128, 64, lds2(128, 64), 1.0);
        const double c112 = tile_cost(g.M, Nn, 112, 64, lds2(112, 64), 0.97);
        if (c112 < c128) return launch2_cfg<T, 112, 64, 1, 4, SIGN, ACT, Out>(A, g, B, Nn, Kb, out, s);
        return launch2_cfg<T, 128, 64, 2, 2, SIGN, ACT, Out>(A, g, B, Nn, Kb, out, s);
    }
    // fp32 with at most 32 columns: 64-row tiles always (the grids are latency-bound; more,
    // smaller workgroups beat the round count the cost model ranks by: c2a's forward,
    // 102400 x 32, 30.0 -> 27.7 us)
    const double c128 = tile_cost(g.M, Nn, 128, 32, lds2(128, 32), 1.0);
    const double c64 = tile_cost(g.M, Nn, 64, 32, lds2(64, 32), 0.85);
    if (sizeof(T) == 4 || c64 < c128) return launch2_cfg<T, 64, 32, 4, 1, SIGN, ACT, Out>(A, g, B, Nn, Kb, out, s);
    return launch2_cfg<T, 128, 32, 4, 1, SIGN, ACT, Out>(A, g, B, Nn, Kb, out, s);
}

template <typename T, int SIGN, int ACT, class Out>
hipError_t launch_any(const T* A, const GatherGeom& g, const T* B, int Nn, int Kb, int bk, const Out& out,
                      hipStream_t s) {
    constexpr int KM = Mma<T>::KM;
    if (bk == 2 * KM) return launch2_any<T, SIGN, ACT, Out>(A, g, B, Nn, Kb, out, s);
    const int bn = pick_bn(Nn);
#define CONVMI_IG(BN_, BK_)                                                                        \
    if (bn == BN_ && bk == BK_) return launch_cfg<T, 128, BN_, BK_, SIGN, ACT, Out>(A, g, B, Nn, Kb, out, s);
    CONVMI_IG(32, KM) CONVMI_IG(64, KM) CONVMI_IG(128, KM)
#undef CONVMI_IG
    return hipErrorInvalidValue;
}

void set_divs(GatherGeom& g) {
    g.fR1 = make_fastdiv(g.R1);
    g.fR2 = make_fastdiv(g.R2);
    g.fCin = make_fastdiv(g.Cin);
    g.fKWC = make_fastdiv(g.KWk * g.Cin);
}

int dx_khs(const ConvDims& d) { return (int)ceil_div(d.KH, d.sh); }
int dx_kws(const ConvDims& d) { return (int)ceil_div(d.KW, d.sw); }

}  // namespace

bool igemm_fwd_supported(int dt, const ConvDims& d) {
    if (d.IC * (dt == DT_BF16 ? 2 : 4) < 16) return false;
    return pick_bk(dt, d.IC, d.KW) != 0 && d.OC >= 16;
}

bool igemm_dx_supported(int dt, const ConvDims& d) {
    const int vec = dt == DT_BF16 ? 8 : 4;
    if (d.IC % vec) return false;
    if (d.sh * d.sw * d.IC < 16) return false;
    return pick_bk(dt, d.OC, dx_kws(d)) != 0;
}

size_t igemm_fwd_ws_bytes(int dt, const ConvDims& d) { return halo_fwd_ws_bytes(dt, d); }

size_t igemm_dx_ws_bytes(int dt, const ConvDims& d) {
    const size_t n = (size_t)d.sh * d.sw * d.IC * dx_khs(d) * dx_kws(d) * d.OC;
    const size_t bt = align_up(n * dtype_size(dt), 256), frag = halo_dx_ws_bytes(dt, d);
    return bt > frag ? bt : frag;
}

hipError_t launch_igemm_fwd(int dt, const void* x, const void* w, const float* bias, void* z, void* y,
                            const ConvDims& d, int act, void* ws, hipStream_t s) {
    if (halo_fwd_supported(dt, d)) return launch_halo_fwd(dt, x, w, bias, z, y, d, act, ws, s);
    GatherGeom g;
    g.Hin = d.H; g.Win = d.W; g.Cin = d.IC; g.KWk = d.KW;
    g.R1 = d.OH; g.R2 = d.OW; g.rs1 = d.sh; g.ro1 = -d.ph; g.rs2 = d.sw; g.ro2 = -d.pw;
    g.M = d.N * d.OH * d.OW;
    g.img_stride = (int64_t)d.H * d.W * d.IC;
    set_divs(g);
    FwdOut o{z, y, bias, d.OC, act};
    const int Kb = d.KH * d.KW * d.IC;
    const int bk = pick_bk(dt, d.IC, d.KW);
    if (dt == DT_BF16) {
        CONVMI_ACT_SWITCH(act, A_, return (launch_any<bf16, 1, A_, FwdOut>((const bf16*)x, g, (const bf16*)w, d.OC,
                                                                           Kb, bk, o, s)));
    } else {
        CONVMI_ACT_SWITCH(act, A_, return (launch_any<float, 1, A_, FwdOut>((const float*)x, g, (const float*)w,
                                                                            d.OC, Kb, bk, o, s)));
    }
    return hipErrorInvalidValue;
}

hipError_t launch_igemm_dx(int dt, const void* dz, const void* w, void* dx, const ConvDims& d, void* ws,
                           hipStream_t s) {
    // stride 1: the tile-reuse kernel reads the weights in its own fragment order
    if (halo_dx_supported(dt, d)) return launch_halo_dx(dt, dz, w, dx, d, ws, s);
    const int KHs = dx_khs(d), KWs = dx_kws(d);
    const int Ncol = d.sh * d.sw * d.IC, Kb = KHs * KWs * d.OC;
    // rearranged weights into the workspace
    {
        const int64_t total = (int64_t)Ncol * Kb;
        if (total > INT32_MAX - 4096 * (int64_t)NT) return hipErrorInvalidValue;
        const int grid = (int)(ceil_div(total, NT) < 4096 ? ceil_div(total, NT) : 4096);
        if (dt == DT_BF16)
            dx_weights<bf16><<<grid, NT, 0, s>>>((const bf16*)w, (bf16*)ws, d, KHs, KWs);
        else
            dx_weights<float><<<grid, NT, 0, s>>>((const float*)w, (float*)ws, d, KHs, KWs);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // rows: phase blocks (qh, qw) that touch the image
    const int qh0 = d.ph / d.sh, qh1 = (d.H - 1 + d.ph) / d.sh;
    const int qw0 = d.pw / d.sw, qw1 = (d.W - 1 + d.pw) / d.sw;
    GatherGeom g;
    g.Hin = d.OH; g.Win = d.OW; g.Cin = d.OC; g.KWk = KWs;
    g.R1 = qh1 - qh0 + 1; g.R2 = qw1 - qw0 + 1;
    g.rs1 = 1; g.ro1 = qh0; g.rs2 = 1; g.ro2 = qw0;
    g.M = d.N * g.R1 * g.R2;
    g.img_stride = (int64_t)d.OH * d.OW * d.OC;
    set_divs(g);
    DxOut o{dx, d.N, d.H, d.W, d.IC, g.R1, g.R2, qh0, qw0, d.sh, d.sw, d.ph, d.pw,
            make_fastdiv(g.R2), make_fastdiv(g.R1), make_fastdiv(d.IC), make_fastdiv(d.sw)};
    const int bk = pick_bk(dt, d.OC, KWs);
    if (dt == DT_BF16)
        return launch_any<bf16, -1, ACT_IDENTITY, DxOut>((const bf16*)dz, g, (const bf16*)ws, Ncol, Kb, bk, o, s);
    return launch_any<float, -1, ACT_IDENTITY, DxOut>((const float*)dz, g, (const float*)ws, Ncol, Kb, bk, o, s);
}

}  // namespace convmi
