// k_dw.hip -- weight and bias gradients as a split-K GEMM on gfx950 MFMA.
//
//   dw[oc][k] = sum_p dz[p][oc] * x_col[p][k],   db[oc] = sum_p dz[p][oc]
//   p = (n, oh, ow) over the N*OH*OW output positions (the reduction),
//   k = (kh, kw, ic), x_col[p][k] = x[n, oh*sh - ph + kh, ow*sw - pw + kw, ic] (0 outside).
// This is the per-weight sum over output positions of the weight-gradient WGSL kernel
// ("conv2d_backward_weight.wgsl", @simulatte/doppler) and of the rl_tools generic
// listing's backward, extended over the batch.
//
// Both operands arrive with the reduction index p strided (channels are contiguous in
// NHWC), while the MFMA wants each lane's 16-byte operand vector to hold consecutive p.
// Each thread therefore loads a VEC x VEC block (VEC consecutive positions x VEC
// consecutive channels, one 16-byte load per position), transposes it in registers and
// writes VEC position-contiguous vectors into the LDS tiles.  Tiles are then consumed
// exactly as in the forward kernel (16x16 MFMA, lane vector = 8 bf16 / 4 fp32 of k).
//
// The P reduction is split over S slabs (grid.z) to fill the 256 CUs; each slab writes an
// fp32 partial tile, and a second kernel adds the S partials in slab order (and into the
// existing gradient when accumulating).  No atomics: results are bitwise reproducible.
// The bias gradient comes from the same dz loads: workgroups of the first k tile keep
// per-channel sums of their dz block and write them beside the partial tile.
#include <type_traits>

#include "internal.hpp"
#include "lds_dma.hpp"

namespace convmi {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int NT = 256;

template <typename T> struct Mma;
template <> struct Mma<bf16> {
    static constexpr int VEC = 8, KM = 32;
    static __device__ __forceinline__ void run(floatx4& c, const uint4& a, const uint4& b) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                    0, 0, 0);
    }
    // r[i] = 8 channels of position i  ->  o[j] = 8 positions of channel j
    static __device__ __forceinline__ void transpose(const uint4* r, uint4* o) {
        uint32_t in[8][4], out[8][4];
#pragma unroll
        for (int i = 0; i < 8; ++i) { in[i][0] = r[i].x; in[i][1] = r[i].y; in[i][2] = r[i].z; in[i][3] = r[i].w; }
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t lo = in[2 * d][j >> 1], hi = in[2 * d + 1][j >> 1];
                out[j][d] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
            }
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = make_uint4(out[j][0], out[j][1], out[j][2], out[j][3]);
    }
    static __device__ __forceinline__ void add_channels(const uint4& v, float* s) {
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            s[2 * d] += __uint_as_float(u[d] << 16);
            s[2 * d + 1] += __uint_as_float(u[d] & 0xffff0000u);
        }
    }
};
template <> struct Mma<float> {
    static constexpr int VEC = 4, KM = 16;
    static __device__ __forceinline__ void run(floatx4& c, const uint4& a, const uint4& b) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    }
    static __device__ __forceinline__ void transpose(const uint4* r, uint4* o) {
        o[0] = make_uint4(r[0].x, r[1].x, r[2].x, r[3].x);
        o[1] = make_uint4(r[0].y, r[1].y, r[2].y, r[3].y);
        o[2] = make_uint4(r[0].z, r[1].z, r[2].z, r[3].z);
        o[3] = make_uint4(r[0].w, r[1].w, r[2].w, r[3].w);
    }
    static __device__ __forceinline__ void add_channels(const uint4& v, float* s) {
        s[0] += __uint_as_float(v.x); s[1] += __uint_as_float(v.y);
        s[2] += __uint_as_float(v.z); s[3] += __uint_as_float(v.w);
    }
};

struct DwGeom {
    int N, H, W, IC, OC, KW, sh, sw, ph, pw, OH, OW;
    int Kdim;       // KH*KW*IC
    int P;          // N*OH*OW
    int Pc;         // positions per slab (multiple of BK)
    int tiles_n;    // k tiles
    int S;          // slabs
};

template <typename T, int BM, int BN, int BK, int WM, int WN>
__global__ __launch_bounds__(NT) void dw_kernel(const T* __restrict__ x, const T* __restrict__ dz, DwGeom g,
                                                float* __restrict__ part, float* __restrict__ part_db,
                                                int want_db) {
    using MM = Mma<T>;
    constexpr int VEC = MM::VEC, KM = MM::KM;
    static_assert(WM * WN == 4, "four waves");
    constexpr int TM = BM / (WM * 16), TN = BN / (WN * 16);
    static_assert(TM * WM * 16 == BM && TN * WN * 16 == BN, "tile shape");
    constexpr int LDK = BK + VEC;
    constexpr int PG = BK / VEC;                 // position groups per K step
    constexpr int NBA = PG * (BM / VEC);         // VEC x VEC blocks of the dz tile
    constexpr int NBB = PG * (BN / VEC);         // blocks of the x tile
    constexpr int ITER = (NBA + NBB + NT - 1) / NT;
    constexpr int STAGE = (BM + BN) * LDK;
    constexpr int LDS_AB = 2 * STAGE * (int)sizeof(T);
    constexpr int LDS_R = PG * BM * 4;           // bias partials
    constexpr int LDS_BYTES = LDS_AB > LDS_R ? LDS_AB : LDS_R;
    __shared__ __align__(16) unsigned char smem[LDS_BYTES];
    T* lds = (T*)smem;

    const int t = threadIdx.x;
    const int tn = blockIdx.x % g.tiles_n, tm = blockIdx.x / g.tiles_n;
    const int oc0 = tm * BM, k0 = tn * BN;
    const int p_begin = blockIdx.z * g.Pc;
    const int p_end = min(g.P, p_begin + g.Pc);
    const bool do_db = want_db && tn == 0;

    // Static per-thread block assignment.  Block b < NBA: dz block (channel group
    // fastest so a wave reads whole dz rows); otherwise an x block (k group fastest).
    int kind[ITER], cg[ITER], pg[ITER];
    int tap_h[ITER], tap_w[ITER], tap_c[ITER];
    bool col_ok[ITER];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        const int b = t + it * NT;
        if (b < NBA) {
            kind[it] = 0;
            cg[it] = b % (BM / VEC);
            pg[it] = b / (BM / VEC);
            col_ok[it] = oc0 + cg[it] * VEC < g.OC;
            tap_h[it] = tap_w[it] = tap_c[it] = 0;
        } else if (b < NBA + NBB) {
            const int bb = b - NBA;
            kind[it] = 1;
            cg[it] = bb % (BN / VEC);
            pg[it] = bb / (BN / VEC);
            const int k = k0 + cg[it] * VEC;
            col_ok[it] = k < g.Kdim;
            const int kk = col_ok[it] ? k : 0;
            const int tap = kk / g.IC;
            tap_c[it] = kk - tap * g.IC;
            tap_h[it] = tap / g.KW;
            tap_w[it] = tap - tap_h[it] * g.KW;
        } else {
            kind[it] = 2;
            cg[it] = pg[it] = 0;
            col_ok[it] = false;
            tap_h[it] = tap_w[it] = tap_c[it] = 0;
        }
    }

    uint4 reg[ITER][VEC];
    float dbs[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) dbs[j] = 0.0f;

    auto load = [&](int pk) {  // pk: first position of this K step
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
            if (kind[it] == 2) continue;
            const int p0 = pk + pg[it] * VEC;
            if (kind[it] == 0) {
                const T* src = dz + (int64_t)p0 * g.OC + oc0 + cg[it] * VEC;
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    const bool ok = col_ok[it] && p0 + i < p_end;
                    reg[it][i] = ok ? *(const uint4*)(src + (int64_t)i * g.OC) : make_uint4(0, 0, 0, 0);
                }
            } else {
                // decompose the first position once, then step along ow with carry
                int ow = p0 % g.OW;
                int q = p0 / g.OW;
                int oh = q % g.OH;
                int n = q / g.OH;
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    const int ih = oh * g.sh - g.ph + tap_h[it];
                    const int iw = ow * g.sw - g.pw + tap_w[it];
                    const bool ok = col_ok[it] && p0 + i < p_end && (unsigned)ih < (unsigned)g.H &&
                                    (unsigned)iw < (unsigned)g.W;
                    reg[it][i] = ok ? *(const uint4*)(x + (((int64_t)n * g.H + ih) * g.W + iw) * g.IC + tap_c[it])
                                    : make_uint4(0, 0, 0, 0);
                    if (++ow == g.OW) {
                        ow = 0;
                        if (++oh == g.OH) { oh = 0; ++n; }
                    }
                }
            }
        }
    };
    auto stash = [&](int buf) {
        T* As = lds + buf * STAGE;
        T* Bs = As + BM * LDK;
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
            if (kind[it] == 2) continue;
            if (kind[it] == 0 && do_db)
#pragma unroll
                for (int i = 0; i < VEC; ++i) MM::add_channels(reg[it][i], dbs);
            uint4 o[VEC];
            MM::transpose(reg[it], o);
            T* base = (kind[it] == 0 ? As : Bs) + (cg[it] * VEC) * LDK + pg[it] * VEC;
#pragma unroll
            for (int j = 0; j < VEC; ++j) *(uint4*)(base + j * LDK) = o[j];
        }
    };

    const int lane = t & 63, wid = t >> 6;
    const int wm = wid / WN, wn = wid % WN;
    const int lr = lane & 15, lk = (lane >> 4) * VEC;
    floatx4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int KT = (p_end - p_begin + BK - 1) / BK;
    if (KT > 0) {
        load(p_begin);
        stash(0);
    }
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) load(p_begin + (kt + 1) * BK);
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

    // partial tile: part[slab][oc][k], only the in-range part
    float* dst = part + (int64_t)blockIdx.z * g.OC * g.Kdim;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int oc = oc0 + wm * TM * 16 + i * 16 + (lane >> 4) * 4 + e;
                const int k = k0 + wn * TN * 16 + j * 16 + lr;
                if (oc < g.OC && k < g.Kdim) dst[(int64_t)oc * g.Kdim + k] = acc[i][j][e];
            }

    if (do_db) {  // uniform per workgroup
        float* red = (float*)smem;  // [PG][BM], free after the last barrier of the loop
#pragma unroll
        for (int it = 0; it < ITER; ++it)
            if (kind[it] == 0)
#pragma unroll
                for (int j = 0; j < VEC; ++j) red[pg[it] * BM + cg[it] * VEC + j] = dbs[j];
        __syncthreads();
        if (t < BM && oc0 + t < g.OC) {
            float s = 0.0f;
            for (int q = 0; q < PG; ++q) s += red[q * BM + t];
            part_db[(int64_t)blockIdx.z * g.OC + oc0 + t] = s;
        }
    }
}

// ------------------------------------------------------------------ LDS-DMA variant
// Tiles keep their natural layout -- rows are output positions (the reduction index),
// columns are channels -- so they are copied global -> LDS with 16-byte DMA, no staging
// registers and no register transpose.  The MFMA operands, which need consecutive
// positions per lane, are read back transposed: for bf16 with ds_read_b64_tr_b16, whose
// 16-lane groups return out[i][j] = row(4j + i/4)[i % 4] of the 8-byte rows the lanes
// address (so lane r pointing at row kb + r/4, column c0 + 4*(r%4) makes lane i receive
// positions kb..kb+3 of column c0 + i); for fp32 with one 4-byte read per position.
// 16-byte chunks are XOR-swizzled by (row & 3) << 1 so the four rows a 16-lane group
// touches fall in distinct banks; in rows of 256 bytes or more read as fp32 or as 32-row
// bf16 fragments by (row & 3) << 2, since there the four rows' 64-byte column pieces
// (fp32) or 32-byte pieces of both lane halves (bf16) only stay apart with steps of four
// chunks (the steps of two left those reads 2-way conflicted on the bank-conflict
// counters).  Two ring stages, two workgroups per CU.
template <int ES, int MF> __device__ __forceinline__ int dswz(int row, int R) {
    return (row & 3) << (R >= 256 && (ES == 4 || MF == 32) ? 2 : 1);
}

typedef short dw_short4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) dw_short4* dw_lds4_t;

template <typename T, int BM, int BN, int WM, int WN, int MF>
__global__ __launch_bounds__(NT) void dw2_kernel(const T* __restrict__ x, const T* __restrict__ dz, DwGeom g,
                                                 FastDiv fOW, FastDiv fOH, FastDiv fIC, FastDiv fKW,
                                                 float* __restrict__ part, float* __restrict__ part_db,
                                                 int want_db) {
    using MM = Mma<T>;
    constexpr int ES = (int)sizeof(T), VEC = 16 / ES;
    constexpr int BK = 64;                       // positions per stage
    constexpr int RA = BM * ES, RB = BN * ES;    // row bytes
    constexpr int CA = RA / 16, CB = RB / 16;    // 16-byte chunks per row
    static_assert(CA >= 8 && CB >= 8 && RA <= 1024 && RB <= 1024, "row size");
    constexpr int ROWS_A = 1024 / RA, ROWS_B = 1024 / RB;  // rows per DMA instruction
    constexpr int IA = BK / ROWS_A, IB = BK / ROWS_B;      // DMA instructions per stage
    static_assert((IA + IB) % 4 == 0, "copies split evenly over the four waves");
    constexpr int IPW = (IA + IB) / 4;
    constexpr int STAGE = BK * (RA + RB);
    constexpr int TM = BM / (WM * MF), TN = BN / (WN * MF);
    static_assert(TM * WM * MF == BM && TN * WN * MF == BN, "tile shape");
    static_assert(MF == 16 || (MF == 32 && sizeof(T) == 2), "32x32 fragments are bf16 only");
    using Acc = typename std::conditional<MF == 32, floatx16, floatx4>::type;
    constexpr int NE = MF == 32 ? 16 : 4;
    __shared__ __align__(1024) unsigned char smem[2 * STAGE];

    const int t = threadIdx.x, lane = t & 63;
    const int wid = __builtin_amdgcn_readfirstlane(t >> 6);
    // One-dimensional grid over (slab, tile), renumbered so each XCD gets whole slabs:
    // the tiles of one slab read the same dz rows and overlapping x rows, which then
    // stay in that XCD's L2.
    const int tiles = gridDim.x / g.S;
    const int lin = xcd_tile(blockIdx.x, gridDim.x);
    const int slab = lin / tiles, tile = lin - slab * tiles;
    const int tn = tile % g.tiles_n, tm = tile / g.tiles_n;
    const int oc0 = tm * BM, k0 = tn * BN;
    const int p_begin = slab * g.Pc;
    const int p_end = min(g.P, p_begin + g.Pc);
    const bool do_db = want_db && tn == 0;
    const uint32_t smem_base = __builtin_amdgcn_readfirstlane(lds_addr(smem));

    // per-lane copy plan; instruction j of the stage (A for j < IA) belongs to wave j % 4
    int rowi[IPW], colo[IPW], tkh[IPW], tkw[IPW], tic[IPW];
    bool cok[IPW];
#pragma unroll
    for (int q = 0; q < IPW; ++q) {
        const int j = wid + 4 * q;
        if (j < IA) {
            const int row = j * ROWS_A + lane / CA;
            const int lc = (lane % CA) ^ dswz<ES, MF>(row, RA);
            rowi[q] = row;
            colo[q] = oc0 + lc * VEC;
            cok[q] = colo[q] < g.OC;
            tkh[q] = tkw[q] = tic[q] = 0;
        } else {
            const int jb = j - IA;
            const int row = jb * ROWS_B + lane / CB;
            const int lc = (lane % CB) ^ dswz<ES, MF>(row, RB);
            const int k = k0 + lc * VEC;
            rowi[q] = row;
            colo[q] = k;
            cok[q] = k < g.Kdim;
            const int kk = cok[q] ? k : 0;
            const int tap = fdiv(kk, fIC);
            tic[q] = kk - tap * g.IC;
            tkh[q] = fdiv(tap, fKW);
            tkw[q] = tap - tkh[q] * g.KW;
        }
    }

    auto issue = [&](int st) {
        const int pst = p_begin + st * BK;
        const uint32_t slot = smem_base + (uint32_t)((st & 1) * STAGE);
#pragma unroll
        for (int q = 0; q < IPW; ++q) {
            const int j = wid + 4 * q;
            const int p = pst + rowi[q];
            const void* src = &kZero16;
            uint32_t dst;
            if (j < IA) {
                if (cok[q] && p < p_end) src = dz + (int64_t)p * g.OC + colo[q];
                dst = slot + j * 1024;
            } else {
                if (cok[q] && p < p_end) {
                    const int q1 = fdiv(p, fOW);
                    const int ow = p - q1 * g.OW;
                    const int n = fdiv(q1, fOH);
                    const int oh = q1 - n * g.OH;
                    const int ih = oh * g.sh - g.ph + tkh[q], iw = ow * g.sw - g.pw + tkw[q];
                    if ((unsigned)ih < (unsigned)g.H && (unsigned)iw < (unsigned)g.W)
                        src = x + (((int64_t)n * g.H + ih) * g.W + iw) * g.IC + tic[q];
                }
                dst = slot + BK * RA + (j - IA) * 1024;
            }
            dma16(src, __builtin_amdgcn_readfirstlane(dst));
        }
    };

    const int wm = wid / WN, wn = wid % WN;
    const int lr = lane & 15, lg = lane >> 4;
    Acc acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < NE; ++e) acc[i][j][e] = 0.0f;

    // operand vector of 16 consecutive-in-position bytes for column c (tile-local) at
    // positions kb.. of a tile with row bytes R
    auto frag = [&](const unsigned char* base, int R, int kb, int c) -> uint4 {
        if constexpr (sizeof(T) == 2) {
            uint4 v;
            dw_short4 h[2];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int row = kb + 4 * half + (lr >> 2);
                const int cb = 2 * (c + 4 * (lr & 3));  // byte offset of the lane's 8-byte piece
                const int off = row * R + ((((cb >> 4) ^ dswz<ES, MF>(row, R)) << 4) | (cb & 15));
                h[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dw_lds4_t)(base + off));
            }
            v.x = __builtin_bit_cast(uint2, h[0]).x; v.y = __builtin_bit_cast(uint2, h[0]).y;
            v.z = __builtin_bit_cast(uint2, h[1]).x; v.w = __builtin_bit_cast(uint2, h[1]).y;
            return v;
        } else {
            uint32_t r[4];
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const int row = kb + 4 * s4;
                const int cb = 4 * (c + lr);
                const int off = row * R + ((((cb >> 4) ^ dswz<ES, MF>(row, R)) << 4) | (cb & 15));
                r[s4] = *(const uint32_t*)(base + off);
            }
            return make_uint4(r[0], r[1], r[2], r[3]);
        }
    };
    // 32x32x16 operand: lane l holds column c + l%32 at positions kb + 8*(l/32) .. +7.  In
    // each 16-lane group the transposing read gives lane i the column (group's first) + i,
    // so lane i addresses position kb + 4*half + i/4, columns 4*(i%4) .. +3 of the group.
    auto frag32 = [&](const unsigned char* base, int R, int kk, int c) -> uint4 {
        const int l16 = lane & 15, hi = (lane >> 4) & 1, kb = kk + 8 * (lane >> 5);
        uint4 v;
        dw_short4 h[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int row = kb + 4 * half + (l16 >> 2);
            const int cb = 2 * (c + 16 * hi + 4 * (l16 & 3));
            const int off = row * R + ((((cb >> 4) ^ dswz<ES, MF>(row, R)) << 4) | (cb & 15));
            h[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dw_lds4_t)(base + off));
        }
        v.x = __builtin_bit_cast(uint2, h[0]).x; v.y = __builtin_bit_cast(uint2, h[0]).y;
        v.z = __builtin_bit_cast(uint2, h[1]).x; v.w = __builtin_bit_cast(uint2, h[1]).y;
        return v;
    };
    auto compute = [&](int st) {
        const unsigned char* As = smem + (st & 1) * STAGE;
        const unsigned char* Bs = As + BK * RA;
        if constexpr (MF == 32) {
#pragma unroll
            for (int kk = 0; kk < BK; kk += 16) {
                uint4 af[TM], bfr[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) af[i] = frag32(As, RA, kk, wm * TM * 32 + i * 32);
#pragma unroll
                for (int j = 0; j < TN; ++j) bfr[j] = frag32(Bs, RB, kk, wn * TN * 32 + j * 32);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[i]),
                                                                            __builtin_bit_cast(bf16x8, bfr[j]),
                                                                            acc[i][j], 0, 0, 0);
            }
            return;
        }
        constexpr int KM = MM::KM;
#pragma unroll
        for (int kk = 0; kk < BK; kk += KM) {
            // bf16: lane group lg covers positions kk + 8*lg .. +7; fp32: kk + lg + 4*s
            const int kb = (sizeof(T) == 2) ? kk + 8 * lg : kk + lg;
            uint4 af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) af[i] = frag(As, RA, kb, wm * TM * 16 + i * 16);
#pragma unroll
            for (int j = 0; j < TN; ++j) bfr[j] = frag(Bs, RB, kb, wn * TN * 16 + j * 16);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    if constexpr (MF == 16) MM::run(acc[i][j], af[i], bfr[j]);
                }
        }
    };

    // Column sums of dz for the bias gradient (first k tile only): thread t owns the
    // 16-byte chunk t % CA of rows t / CA, t / CA + NT / CA, ...
    float dbs[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) dbs[j] = 0.0f;
    const int db_chunk = t % CA;
    const int KT = (p_end - p_begin + BK - 1) / BK;
    if (KT > 0) issue(0);
    for (int k = 0; k < KT; ++k) {
        wait_dma(0);
        __syncthreads();
        if (k + 1 < KT) issue(k + 1);
        if (do_db) {
            const unsigned char* As = smem + (k & 1) * STAGE;
            for (int row = t / CA; row < BK; row += NT / CA) {
                const uint4 v = *(const uint4*)(As + row * RA + ((db_chunk ^ dswz<ES, MF>(row, RA)) << 4));
                MM::add_channels(v, dbs);
            }
        }
        compute(k);
    }

    // accumulator element e of a lane: row (oc) 4*(lane/16) + e (16x16) or
    // 8*(e/4) + 4*(lane/32) + e%4 (32x32), column lane % MF
    float* dst = part + (int64_t)slab * g.OC * g.Kdim;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                const int row = MF == 32 ? 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3) : lg * 4 + e;
                const int oc = oc0 + wm * TM * MF + i * MF + row;
                const int k = k0 + wn * TN * MF + j * MF + lane % MF;
                if (oc < g.OC && k < g.Kdim) dst[(int64_t)oc * g.Kdim + k] = acc[i][j][e];
            }
    if (do_db) {  // uniform per workgroup
        __syncthreads();
        float* red = (float*)smem;  // [NT/CA][BM]; the ring is no longer needed
#pragma unroll
        for (int j = 0; j < VEC; ++j) red[(t / CA) * BM + db_chunk * VEC + j] = dbs[j];
        __syncthreads();
        if (t < BM && oc0 + t < g.OC) {
            float s_ = 0.0f;
            for (int q = 0; q < NT / CA; ++q) s_ += red[q * BM + t];
            part_db[(int64_t)slab * g.OC + oc0 + t] = s_;
        }
    }
}

// ------------------------------------------------------------------ stride-1 bf16 kernel
// For stride 1 the KW taps of one kernel row read the same input row shifted by one
// position each.  A workgroup owns a whole kernel row kh: CH output channels x (KW taps
// x CH input channels), CH = 128 or 64.  It streams stages of RS output-row segments of
// SEG positions: the dz rows (positions x CH oc) and, once, the input rows they touch
// (SEG + KW - 1 positions x CH ic); tap kw reads the input tile at a row offset of kw.
// That loads about a third of the bytes per FLOP of the per-tap gather above.  Operands
// are read with transposing LDS reads into 32x32x16 MFMA fragments (lane l: column l%32,
// positions 8*(l/32) .. +7 of the k-step).  Each wave holds 2 x KW accumulator fragments
// (64 oc x KW*32 columns).  CH = 128: eight waves (2 x 4), one workgroup per CU (the
// stage ring is ~115 KB).  CH = 64 (64-channel layers): two waves (1 x 2) per workgroup
// and shorter stages, four workgroups per CU.
struct Dw3Geom {
    int N, H, W, IC, OC, KH, KW, OH, OW, ph, pw;
    int SEG, RS, nseg;  // stage: RS segments of SEG positions of output rows
    int SEGp;           // LDS row of the second segment's first dz row (SEG rounded up to a copy's rows)
    int SPp;            // positions per stage, padded to a multiple of 16
    int XW, XR;         // input positions per segment (SEG + KW - 1), input rows per stage
    int XWp;            // LDS row of the second segment's first input row (SEGp + a multiple of a copy's rows)
    int G;              // segments in all (N*OH*nseg)
    int nst;            // stages in all (ceil(G / RS))
    int spb;            // stages per slab
    int S, tiles, ict, oct;
    int Kdim;           // KH*KW*IC
    FastDiv fnseg, fOH;
};

// 16-byte chunk swizzle of an LDS row of ROWB bytes: 4 consecutive rows read at the same
// 32-byte column piece (bf16 transposing reads) or 64-byte piece (fp32 reads) land in
// different slots of the 256 bytes the banks span.  256-byte rows: chunk ^ 4*(row%4).
// 128-byte rows (two rows per bank span): chunk ^ 4*((row/2)%2).  An XOR with 2 there
// left the transposing reads 2-way conflicted on the bank-conflict counters; the XOR
// with 4 is conflict-free under each lane-pass grouping of ds_read_b64_tr_b16 that is
// consistent with the counters, at every row offset the taps and k-steps produce.  The
// swizzle has period 4 in the row, so the second segment's rows, a multiple of 4
// further, keep it.
template <int ROWB> __device__ __forceinline__ int sw3(int row) {
    return ROWB == 256 ? (row & 3) << 2 : ((row >> 1) & 1) << 2;
}

// Stage copies of the stride-1 weight-gradient kernels, for tiles of CH channels of T
// (LDS rows of ROWB = CH*sizeof(T) bytes, RPI rows per 1-KB copy) and NT threads.
// Copy instructions of a stage: NA for dz (RPI LDS rows each), then NB for the input
// rows, split into per-segment streams (below).  Lane l copies 16-byte chunk l%CPR of
// row RPI*j + l/CPR; the swizzle of that row depends on l/CPR only.  Segment r of a
// stage (RS <= 2 of them) holds its dz rows at LDS rows r*SEGp + q and its input row at
// LDS rows r*XWp + c (c = input column + pw - w0); a copy never spans two segments.
// Each segment's dz rows and its input row are raw buffers sized to the valid data, so
// dz rows past the segment's length, input columns left or right of the image (offsets
// below the start wrap to huge values) and input rows above or below it (an empty
// buffer) all read as zeros.
template <typename T, int CH, int NT> struct Dw3Copies {
    static constexpr int ES = (int)sizeof(T), ROWB = CH * ES, CPR = ROWB / 16, RPI = 1024 / ROWB, NW = NT / 64;
    // A stage's copies c = 0 .. NA+NB-1 land at LDS byte c*1024 of its slot and form four
    // streams: k = 0 the dz rows of segment 0 ([0, A0)), 1 those of segment 1 ([A0, NA)),
    // 2 the input row of segment 0 ([NA, NA+B0)), 3 that of segment 1 ([NA+B0, NA+NB)).
    // With four or more waves, wave w copies part w/4 of stream w%4; with two, wave w
    // copies streams w and w+2 (both of segment w).  Either way a wave needs the geometry
    // of one segment and one or two buffer descriptors per stage, which keeps the scalar
    // work and registers of the copies small next to the MFMA loop.
    static_assert(NW == 2 || NW % 4 == 0, "two waves or a multiple of four");
    static constexpr int SPW = NW >= 4 ? 1 : 2;  // streams per wave
    struct Segs {
        dma_rsrc rs[SPW];
        int xo;  // byte offset of the segment's LDS input row 0 from its buffer: (w0 - pw)*IC*ES
        uint32_t slot;
    };
    const T* x;
    const T* dz;
    int kh, oc0, ic0, s_begin, seg, nmine, stage_bytes;
    int kind[SPW], c_lo[SPW], c_hi[SPW], row_lo[SPW];  // stream, copy range, row of its first copy
    uint32_t lane_off[SPW];                             // per-lane source offset of the first copy's row
    int stride[SPW];                                    // source bytes per row

    __device__ __forceinline__ Dw3Copies(const Dw3Geom& g, const T* x_, const T* dz_, int kh_, int oc0_, int ic0_,
                                         int s_begin_, int wid, int lane, uint32_t smem_base)
        : x(x_), dz(dz_), kh(kh_), oc0(oc0_), ic0(ic0_), s_begin(s_begin_) {
        const int NA = g.SPp / RPI, NB = g.XR / RPI;
        const int A0 = g.SEGp / RPI, B0 = g.XWp / RPI;  // SEGp <= SPp, XWp <= XR, multiples of RPI
        const int lo[4] = {0, A0, NA, NA + B0}, hi[4] = {A0, NA, NA + B0, NA + NB};
        const int rsub = lane / CPR;
        const int choff = ((lane % CPR) ^ sw3<ROWB>(rsub)) * 16;  // source byte offset of the chunk
        stage_bytes = (g.SPp + g.XR) * ROWB;
        nmine = 0;
        seg = NW >= 4 ? (wid & 1) : wid;
#pragma unroll
        for (int q = 0; q < SPW; ++q) {
            const int k = NW >= 4 ? (wid & 3) : wid + 2 * q;
            const int parts = NW >= 4 ? NW / 4 : 1, part = NW >= 4 ? wid / 4 : 0;
            const int per = (hi[k] - lo[k] + parts - 1) / parts;
            kind[q] = k;
            c_lo[q] = min(hi[k], lo[k] + part * per);
            c_hi[q] = min(hi[k], c_lo[q] + per);
            row_lo[q] = RPI * (c_lo[q] - lo[k]);
            stride[q] = (k >= 2 ? g.IC : g.OC) * ES;
            lane_off[q] = (uint32_t)(rsub * stride[q] + choff) + (uint32_t)(row_lo[q] * stride[q]);
            nmine += c_hi[q] - c_lo[q];
        }
        smem_base_ = smem_base;
    }
    uint32_t smem_base_;
    __device__ __forceinline__ Segs segs_of(const Dw3Geom& g, int st) const {
        Segs sg;
        sg.slot = smem_base_ + (uint32_t)((st & 1) * stage_bytes);
        sg.xo = 0;
        // this wave's segment of the stage; none (every copy reads zeros) past the last one
        const int gr = seg == 0 || g.RS == 2 ? (s_begin + st) * g.RS + seg : g.G;
        int f = 0, w0 = 0;
        const bool valid = gr < g.G;
        if (valid) {
            f = fdiv(gr, g.fnseg);
            w0 = (gr - f * g.nseg) * g.SEG;
        }
#pragma unroll
        for (int q = 0; q < SPW; ++q) {
            const bool is_x = SPW == 2 ? q == 1 : kind[q] >= 2;
            const T* b = is_x ? x : dz;
            uint32_t bytes = 0;
            if (valid && !is_x) {
                const int len = min(g.SEG, g.OW - w0);
                b = dz + ((int64_t)f * g.OW + w0) * g.OC + oc0;
                bytes = (uint32_t)((len * g.OC - oc0) * ES);
            } else if (valid) {
                const int n = fdiv(f, g.fOH), oh = f - n * g.OH;
                const int ih = oh + kh - g.ph;
                if ((unsigned)ih < (unsigned)g.H) {
                    b = x + ((int64_t)n * g.H + ih) * g.W * g.IC + ic0;
                    bytes = (uint32_t)((g.W * g.IC - ic0) * ES);
                }
                sg.xo = (w0 - g.pw) * g.IC * ES;
            }
            sg.rs[q] = make_rsrc(b, bytes);
        }
        return sg;
    }
    // this wave's copy instructions i0 .. i1-1 of a stage (counted over its streams in order)
    __device__ __forceinline__ void issue(const Dw3Geom&, const Segs& sg, int i0, int i1) const {
        int done = 0;
#pragma unroll
        for (int q = 0; q < SPW; ++q) {
            const bool is_x = SPW == 2 ? q == 1 : kind[q] >= 2;
            const int n = c_hi[q] - c_lo[q];
            const int a = max(i0 - done, 0), b = min(i1 - done, n);
            uint32_t voff = lane_off[q] + (uint32_t)(RPI * a * stride[q] + (is_x ? sg.xo : 0));
            for (int i = a; i < b; ++i) {
                dma16_buf(voff, sg.rs[q], __builtin_amdgcn_readfirstlane(sg.slot + (uint32_t)(c_lo[q] + i) * 1024u));
                voff += (uint32_t)(RPI * stride[q]);
            }
            done += n;
        }
    }
};

// Threads per workgroup: eight waves for 128-channel tiles (two per SIMD, so one wave's
// address work overlaps the other's MFMAs); two waves for 64-channel tiles, four
// workgroups per CU.
template <int CH> constexpr int dw3_threads() { return CH == 128 ? 512 : 128; }

// NK: k-steps per stage when known at compile time (0: read from the geometry); with a
// fixed count every LDS offset of a k-step is an immediate.
template <int CH, int KW_, int NK>
__global__ __launch_bounds__(dw3_threads<CH>()) __attribute__((amdgpu_waves_per_eu(2, 2))) void dw3_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ dz, Dw3Geom g, float* __restrict__ part,
    float* __restrict__ part_db, int want_db) {
    constexpr int NT = dw3_threads<CH>();
    constexpr int ROWB = CH * 2;         // LDS row bytes (one position)
    constexpr int CPR = ROWB / 16;       // 16-byte chunks per row
    constexpr int WN = CH == 128 ? 4 : 2;  // waves: (CH/64) x WN
    constexpr int TM = 2, TN = KW_;        // wave tile 64 oc x KW*32 columns
    extern __shared__ __align__(1024) unsigned char smem[];
    const int t = threadIdx.x, lane = t & 63;
    const int wid = __builtin_amdgcn_readfirstlane(t >> 6);
    const int stage_bytes = (g.SPp + g.XR) * ROWB;
    const uint32_t smem_base = __builtin_amdgcn_readfirstlane(lds_addr(smem));

    // (slab, tile); the tiles of one slab share its dz rows and stay on one XCD
    const int lin = xcd_tile(blockIdx.x, gridDim.x);
    const int slab = lin / g.tiles, tile = lin - slab * g.tiles;
    const int oct_i = tile % g.oct, r1 = tile / g.oct;
    const int ict_i = r1 % g.ict, kh = r1 / g.ict;
    const int oc0 = oct_i * CH, ic0 = ict_i * CH;
    const int s_begin = slab * g.spb;
    const int s_end = min(g.nst, s_begin + g.spb);
    const int KT = s_end - s_begin;
    // every kernel row's workgroup sums every KH-th dz row of a stage for the bias gradient
    const bool do_db = want_db && ict_i == 0;

    const Dw3Copies<bf16, CH, NT> cp(g, x, dz, kh, oc0, ic0, s_begin, wid, lane, smem_base);
    const int nmine = cp.nmine;
    using Segs = typename Dw3Copies<bf16, CH, NT>::Segs;
    auto segs_of = [&](int st) { return cp.segs_of(g, st); };
    auto issue = [&](const Segs& sg, int i0, int i1) { cp.issue(g, sg, i0, i1); };

    const int wm = wid / WN, wn = wid % WN;
    floatx16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // Transposing fragment read: lane l gets column c + l%32 at positions
    // kk + 8*(l/32) .. +7; in each 16-lane group lane i addresses position +i/4 of a
    // half and the 8-byte piece 4*(i%4) of the group's 16 columns.  Input rows of tap kw
    // sit kw rows further; the second segment's rows start XWp - SEGp rows later, a
    // multiple of 4, so the swizzle is unchanged.  k-steps start at multiples of 16, so
    // every offset is a per-lane constant plus kk*ROWB (plus the second-segment shift).
    typedef short dw_short8 __attribute__((ext_vector_type(8)));
    const int l16 = lane & 15, hi = (lane >> 4) & 1, kb8 = 8 * (lane >> 5);
    auto lds_off = [&](int row, int c) {
        const int cb = 2 * (c + 16 * hi + 4 * (l16 & 3));
        return row * ROWB + ((((cb >> 4) ^ sw3<ROWB>(row)) << 4) | (cb & 15));
    };
    int a_off[TM][2], b_off[TN][2];
    int prow[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        prow[half] = kb8 + 4 * half + (l16 >> 2);
#pragma unroll
        for (int i = 0; i < TM; ++i) a_off[i][half] = lds_off(prow[half], wm * 64 + i * 32);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = wn * KW_ * 32 + j * 32;  // tap col/CH, input channel col%CH
            b_off[j][half] = lds_off(prow[half] + col / CH, col % CH);
        }
    }
    const int seg_shift = (g.XWp - g.SEGp) * ROWB;
    auto read_frags = [&](const unsigned char* As, const unsigned char* Xs, int kk, dw_short8 (&af)[TM],
                          dw_short8 (&bf)[TN]) {
        const unsigned char* Ak = As + kk * ROWB;
        const unsigned char* Xk = Xs + kk * ROWB;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const dw_short4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dw_lds4_t)(Ak + a_off[i][0]));
            const dw_short4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dw_lds4_t)(Ak + a_off[i][1]));
            af[i] = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
        }
        const int sh0 = kk + prow[0] >= g.SEGp ? seg_shift : 0;
        const int sh1 = kk + prow[1] >= g.SEGp ? seg_shift : 0;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const dw_short4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dw_lds4_t)(Xk + b_off[j][0] + sh0));
            const dw_short4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dw_lds4_t)(Xk + b_off[j][1] + sh1));
            bf[j] = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };
    auto mfmas = [&](const dw_short8 (&af)[TM], const dw_short8 (&bf)[TN]) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[i]),
                                                                    __builtin_bit_cast(bf16x8, bf[j]), acc[i][j],
                                                                    0, 0, 0);
    };

    // Column sums of dz for the bias gradient: thread t owns chunk t%CPR (8 channels) of
    // rows kh + KH*(t/CPR), kh + KH*(t/CPR + RG), ...
    constexpr int RG = NT / CPR;  // row groups
    float dbs[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) dbs[j] = 0.0f;
    auto db_sum = [&](const unsigned char* As) {
        for (int row = kh + g.KH * (t / CPR); row < g.SPp; row += RG * g.KH) {
            const uint4 v = *(const uint4*)(As + row * ROWB + (((t % CPR) ^ sw3<ROWB>(row)) << 4));
            const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                dbs[2 * d] += __uint_as_float(u[d] << 16);
                dbs[2 * d + 1] += __uint_as_float(u[d] & 0xffff0000u);
            }
        }
    };

    // Stage k: the copies of stage k + 1 go out in slices over the first k-steps of stage
    // k, between MFMA groups, so their address arithmetic overlaps the MFMAs; the reads
    // of k-step kk + 1 are issued before the MFMAs of kk.
    const int nk = NK > 0 ? NK : g.SPp / 16;
    // k-steps that carry the next stage's copies, early to leave them time to land; the
    // two-wave 64-channel workgroups issue theirs at once before the first MFMAs (measured
    // ~2 us faster on c5, ~1 us slower for the eight-wave 128-channel kernel)
    const int spread = CH == 64 ? 0 : (nk > 2 ? 2 : 1);
    const int sdiv = spread > 0 ? spread : 1;  // divisor of the slices (unused when spread is 0)
    if (KT > 0) issue(segs_of(0), 0, nmine);
    for (int k = 0; k < KT; ++k) {
        wait_dma(0);
        __syncthreads();
        const bool next = k + 1 < KT;
        const Segs sg = segs_of(next ? k + 1 : k);
        const unsigned char* As = smem + (k & 1) * stage_bytes;
        const unsigned char* Xs = As + g.SPp * ROWB;
        if (CH == 64 && next) issue(sg, 0, nmine);
        if (do_db) db_sum(As);
        dw_short8 fa[2][TM], fb[2][TN];
        read_frags(As, Xs, 0, fa[0], fb[0]);
        if constexpr (NK > 0) {
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                if (kk + 1 < NK) read_frags(As, Xs, (kk + 1) * 16, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
                mfmas(fa[kk & 1], fb[kk & 1]);
                if (next && kk < spread) issue(sg, kk * nmine / sdiv, (kk + 1) * nmine / sdiv);
            }
        } else {
            int kk = 0;
            for (; kk + 1 < nk; kk += 2) {
                read_frags(As, Xs, (kk + 1) * 16, fa[1], fb[1]);
                mfmas(fa[0], fb[0]);
                if (next && kk < spread) issue(sg, kk * nmine / sdiv, (kk + 1) * nmine / sdiv);
                if (kk + 2 < nk) read_frags(As, Xs, (kk + 2) * 16, fa[0], fb[0]);
                mfmas(fa[1], fb[1]);
                if (next && kk + 1 < spread) issue(sg, (kk + 1) * nmine / sdiv, (kk + 2) * nmine / sdiv);
            }
            if (kk < nk) {
                mfmas(fa[0], fb[0]);
                if (next && kk < spread) issue(sg, kk * nmine / sdiv, nmine);
            }
        }
    }

    // partial tile: row (oc) 8*(e/4) + 4*(lane/32) + e%4 of fragment i, column lane%32
    float* dst = part + (int64_t)slab * g.OC * g.Kdim;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = wn * KW_ * 32 + j * 32;
            const int k = (kh * g.KW + col / CH) * g.IC + ic0 + col % CH + (lane & 31);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int oc = oc0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                dst[(int64_t)oc * g.Kdim + k] = acc[i][j][e];
            }
        }
    if (do_db) {  // uniform per workgroup
        __syncthreads();
        float* red = (float*)smem;  // [RG][CH]; the ring is no longer needed
#pragma unroll
        for (int j = 0; j < 8; ++j) red[(t / CPR) * CH + (t % CPR) * 8 + j] = dbs[j];
        __syncthreads();
        if (t < CH) {
            float s_ = 0.0f;
            for (int q = 0; q < RG; ++q) s_ += red[q * CH + t];
            part_db[((int64_t)slab * g.KH + kh) * g.OC + oc0 + t] = s_;
        }
    }
}

// fp32 variant of the stride-1 weight-gradient kernel: 64-channel tiles (256-byte LDS
// rows, the same stage copies), four waves of 64 oc x KW*16 columns, two workgroups per
// CU.  v_mfma_f32_16x16x4_f32 takes 4 positions per k-step with one fp32 value of each
// operand per lane (A: channel l%16 at position l/16; B likewise), so the operands are
// read from the natural position-major tiles with plain 4-byte LDS reads; the row
// swizzle keeps the four positions a read touches in different banks.
template <int KW_, int NK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void dw3f_kernel(
    const float* __restrict__ x, const float* __restrict__ dz, Dw3Geom g, float* __restrict__ part,
    float* __restrict__ part_db, int want_db) {
    constexpr int CH = 64, NT = 256, ROWB = 256, CPR = 16;
    constexpr int TM = 4, TN = KW_;  // wave tile 64 oc x KW*16 columns (waves 1 x 4)
    extern __shared__ __align__(1024) unsigned char smem[];
    const int t = threadIdx.x, lane = t & 63;
    const int wid = __builtin_amdgcn_readfirstlane(t >> 6);
    const int stage_bytes = (g.SPp + g.XR) * ROWB;
    const uint32_t smem_base = __builtin_amdgcn_readfirstlane(lds_addr(smem));

    const int lin = xcd_tile(blockIdx.x, gridDim.x);
    const int slab = lin / g.tiles, tile = lin - slab * g.tiles;
    const int oct_i = tile % g.oct, r1 = tile / g.oct;
    const int ict_i = r1 % g.ict, kh = r1 / g.ict;
    const int oc0 = oct_i * CH, ic0 = ict_i * CH;
    const int s_begin = slab * g.spb;
    const int s_end = min(g.nst, s_begin + g.spb);
    const int KT = s_end - s_begin;
    const bool do_db = want_db && ict_i == 0;

    const Dw3Copies<float, CH, NT> cp(g, x, dz, kh, oc0, ic0, s_begin, wid, lane, smem_base);
    const int nmine = cp.nmine;

    floatx4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    // Lane l reads position kq = l/16 of the k-step and channel c16 = l%16 of its fragment.
    // k-steps start at multiples of 4 positions, so a read's row is kk + kq (+ the tap)
    // and its swizzle depends on kq (+ the tap) only: offsets are per-lane constants plus
    // kk*ROWB (plus the second-segment shift, a multiple of 4 rows, uniform per k-step
    // since segments start at multiples of 4).
    const int kq = lane >> 4, c16 = lane & 15;
    auto lds_off = [&](int row, int c) {  // byte offset of channel c in LDS row `row`
        return row * ROWB + ((((c >> 2) ^ sw3<ROWB>(row)) << 4) | ((c & 3) << 2));
    };
    int a_off[TM], b_off[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) a_off[i] = lds_off(kq, i * 16 + c16);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int col = wid * KW_ * 16 + j * 16;  // tap col/64, input channel col%64
        b_off[j] = lds_off(kq + col / CH, col % CH + c16);
    }
    const int seg_shift = (g.XWp - g.SEGp) * ROWB;
    auto read_frags = [&](const unsigned char* As, const unsigned char* Xs, int kk, float (&af)[TM],
                          float (&bf)[TN]) {
        const unsigned char* Ak = As + kk * ROWB;
        const unsigned char* Xk = Xs + kk * ROWB + (kk >= g.SEGp ? seg_shift : 0);
#pragma unroll
        for (int i = 0; i < TM; ++i) af[i] = *(const float*)(Ak + a_off[i]);
#pragma unroll
        for (int j = 0; j < TN; ++j) bf[j] = *(const float*)(Xk + b_off[j]);
    };
    auto mfmas = [&](const float (&af)[TM], const float (&bf)[TN]) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i], bf[j], acc[i][j], 0, 0, 0);
    };

    // Column sums of dz for the bias gradient: thread t owns chunk t%CPR (4 channels) of
    // rows kh + KH*(t/CPR), kh + KH*(t/CPR + RG), ...
    constexpr int RG = NT / CPR;
    float dbs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    auto db_sum = [&](const unsigned char* As) {
        for (int row = kh + g.KH * (t / CPR); row < g.SPp; row += RG * g.KH) {
            const float4 v = *(const float4*)(As + row * ROWB + (((t % CPR) ^ sw3<ROWB>(row)) << 4));
            dbs[0] += v.x;
            dbs[1] += v.y;
            dbs[2] += v.z;
            dbs[3] += v.w;
        }
    };

    // Stage k: the copies of stage k + 1 go out in slices over the first two k-steps of
    // stage k (measured ~2% faster than four on c3); the reads of k-step kk + 4 are issued
    // before the MFMAs of kk.
    const int nk = NK > 0 ? NK : g.SPp / 4;
    const int spread = nk > 2 ? 2 : nk;
    const int sdiv = spread > 0 ? spread : 1;  // divisor of the slices (unused when spread is 0)
    if (KT > 0) cp.issue(g, cp.segs_of(g, 0), 0, nmine);
    for (int k = 0; k < KT; ++k) {
        wait_dma(0);
        __syncthreads();
        const bool next = k + 1 < KT;
        const typename Dw3Copies<float, CH, NT>::Segs sg = cp.segs_of(g, next ? k + 1 : k);
        const unsigned char* As = smem + (k & 1) * stage_bytes;
        const unsigned char* Xs = As + g.SPp * ROWB;
        if (do_db) db_sum(As);
        float fa[2][TM], fb[2][TN];
        read_frags(As, Xs, 0, fa[0], fb[0]);
        if constexpr (NK > 0) {
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                if (kk + 1 < NK) read_frags(As, Xs, (kk + 1) * 4, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
                mfmas(fa[kk & 1], fb[kk & 1]);
                if (next && kk < spread) cp.issue(g, sg, kk * nmine / sdiv, (kk + 1) * nmine / sdiv);
            }
        } else {
            int kk = 0;
            for (; kk + 1 < nk; kk += 2) {
                read_frags(As, Xs, (kk + 1) * 4, fa[1], fb[1]);
                mfmas(fa[0], fb[0]);
                if (next && kk < spread) cp.issue(g, sg, kk * nmine / sdiv, (kk + 1) * nmine / sdiv);
                if (kk + 2 < nk) read_frags(As, Xs, (kk + 2) * 4, fa[0], fb[0]);
                mfmas(fa[1], fb[1]);
                if (next && kk + 1 < spread) cp.issue(g, sg, (kk + 1) * nmine / sdiv, (kk + 2) * nmine / sdiv);
            }
            if (kk < nk) {
                mfmas(fa[0], fb[0]);
                if (next && kk < spread) cp.issue(g, sg, kk * nmine / sdiv, nmine);
            }
        }
    }

    // partial tile: row (oc) 4*(lane/16) + e of fragment i, column lane%16 of fragment j
    float* dst = part + (int64_t)slab * g.OC * g.Kdim;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = wid * KW_ * 16 + j * 16;
            const int k = (kh * g.KW + col / CH) * g.IC + ic0 + col % CH + c16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int oc = oc0 + i * 16 + 4 * kq + e;
                dst[(int64_t)oc * g.Kdim + k] = acc[i][j][e];
            }
        }
    if (do_db) {  // uniform per workgroup
        __syncthreads();
        float* red = (float*)smem;  // [RG][CH]; the ring is no longer needed
#pragma unroll
        for (int j = 0; j < 4; ++j) red[(t / CPR) * CH + (t % CPR) * 4 + j] = dbs[j];
        __syncthreads();
        if (t < CH) {
            float s_ = 0.0f;
            for (int q = 0; q < RG; ++q) s_ += red[q * CH + t];
            part_db[((int64_t)slab * g.KH + kh) * g.OC + oc0 + t] = s_;
        }
    }
}

// dw = (accumulate ? dw : 0) + sum over slabs; four slab groups (s = q mod 4) per output
// vector are summed in slab order and then merged in group order: fixed order, so
// bitwise reproducible.  Blocks past the dw blocks finish db the same way (64 channels
// each).  count is a multiple of 4.
// sum_strided: a thread's slabs s = first, first + STEP, ... < S go out in batches of U
// loads before their in-order adds (a batch costs one memory latency, not U); past the
// last slab the index is clamped to an in-bounds re-read and zero is added instead.
template <int U, int STEP = 4>
__device__ __forceinline__ float4 sum_strided(const float4* __restrict__ p, int64_t stride4, int first, int S) {
    float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = first; s < S; s += STEP * U) {
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = p[(int64_t)(s + STEP * u < S ? s + STEP * u : S - 1) * stride4];
#pragma unroll
        for (int u = 0; u < U; ++u) {  // selects, not branches (a branch would let the load sink into it)
            const bool in = s + STEP * u < S;
            r.x += in ? v[u].x : 0.f; r.y += in ? v[u].y : 0.f; r.z += in ? v[u].z : 0.f; r.w += in ? v[u].w : 0.f;
        }
    }
    return r;
}

// (register budget for two waves per SIMD: a batch of 24 float4 loads stays in flight)
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 2))) void dw_reduce4(
    const float* __restrict__ part, const float* __restrict__ part_db, float* __restrict__ dw, float* __restrict__ db,
    int64_t count, int OC, int S, int Sdb, int accumulate) {
    __shared__ float4 red[4][64];
    const int q = threadIdx.x >> 6, o = threadIdx.x & 63;
    const int64_t n4 = count >> 2;
    const int nb_dw = (int)((n4 + 63) / 64);
    if ((int)blockIdx.x < nb_dw) {
        const int64_t i4 = (int64_t)blockIdx.x * 64 + o;
        float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i4 < n4) r = sum_strided<24>((const float4*)part + i4, n4, q, S);
        red[q][o] = r;
        __syncthreads();
        if (q == 0 && i4 < n4) {
            float4 a = red[0][o];
#pragma unroll
            for (int k = 1; k < 4; ++k) { a.x += red[k][o].x; a.y += red[k][o].y; a.z += red[k][o].z; a.w += red[k][o].w; }
            if (accumulate) {
                const float4 d = ((const float4*)dw)[i4];
                a.x += d.x; a.y += d.y; a.z += d.z; a.w += d.w;
            }
            ((float4*)dw)[i4] = a;
        }
        return;
    }
    // bias: block nb_dw + b sums channels 64b .. 64b+63 (as 16 float4 of 4 channels)
    if (db == nullptr) return;
    const int c4 = ((int)blockIdx.x - nb_dw) * 16 + (o & 15), sub = o >> 4;
    const int oc4 = OC >> 2;
    // 16 thread groups (q, sub) split the slabs: group g = 4q + sub takes s = g mod 16
    float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
    const int grp = q * 4 + sub;
    if (c4 < oc4) r = sum_strided<8, 16>((const float4*)part_db + c4, oc4, grp, Sdb);
    __shared__ float4 rdb[16][16];
    rdb[grp][o & 15] = r;
    __syncthreads();
    if (threadIdx.x < 16 && c4 - (o & 15) + (int)threadIdx.x < oc4) {
        const int cc = ((int)blockIdx.x - nb_dw) * 16 + (int)threadIdx.x;
        float4 a = rdb[0][threadIdx.x];
        for (int k = 1; k < 16; ++k) {
            a.x += rdb[k][threadIdx.x].x; a.y += rdb[k][threadIdx.x].y;
            a.z += rdb[k][threadIdx.x].z; a.w += rdb[k][threadIdx.x].w;
        }
        // db is only 4-byte aligned: scalar accesses
        float* o4 = db + 4 * cc;
        const float v4[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) o4[k] = accumulate ? o4[k] + v4[k] : v4[k];
    }
}

// grid of the reduction: dw blocks, then one block per 64 bias channels
unsigned reduce_grid(int64_t count, int OC, bool with_db) {
    const int64_t nb_dw = ceil_div(count / 4, 64);
    return (unsigned)(nb_dw + (with_db ? ceil_div(OC, 64) : 0));
}

struct Plan {
    int bm, bn, bk, tiles_m, tiles_n, S, Pc;
    bool dma;  // LDS-DMA kernel (dw2_kernel) rather than the register-transpose one
};

Plan plan(int dt, const ConvDims& d) {
    Plan p;
    const int P = d.N * d.OH * d.OW;
    const int Kdim = d.KH * d.KW * d.IC;
    p.bm = d.OC <= 32 ? 32 : (d.OC <= 64 ? 64 : 128);
    p.bn = dt == DT_BF16 ? 128 : 64;
    if (Kdim <= 64) p.bn = 64;
    p.dma = dt == DT_BF16 ? p.bm >= 64 : true;  // DMA tiles need rows of >= 128 bytes
    p.bk = (p.dma || dt == DT_BF16) ? 64 : 32;
    p.tiles_m = (int)ceil_div(d.OC, p.bm);
    p.tiles_n = (int)ceil_div(Kdim, p.bn);
    const int tiles = p.tiles_m * p.tiles_n;
    const int steps = (int)ceil_div(P, p.bk);
    int S = (int)ceil_div(512, tiles);       // about two workgroups per CU
    if (S > steps) S = steps;
    if (S < 1) S = 1;
    p.Pc = (int)ceil_div(ceil_div(P, S), p.bk) * p.bk;
    p.S = (int)ceil_div(P, p.Pc);
    return p;
}

// bf16 uses 32x32x16 MFMA fragments (waves 2 x 2), fp32 16x16x4.
template <typename T, int BM, int BN>
hipError_t launch_dw2(const T* x, const T* dz, const DwGeom& g, const ConvDims& d, const Plan& p, float* part,
                      float* part_db, int want_db, hipStream_t s) {
    constexpr int MF = sizeof(T) == 2 ? 32 : 16;
    constexpr int WN = MF == 32 ? 2 : ((BM == 128 || BN == 64) ? 2 : 4);
    constexpr int WM = 4 / WN;
    dim3 grid(p.tiles_m * p.tiles_n * p.S);
    dw2_kernel<T, BM, BN, WM, WN, MF><<<grid, NT, 0, s>>>(x, dz, g, make_fastdiv(d.OW), make_fastdiv(d.OH),
                                                      make_fastdiv(d.IC), make_fastdiv(d.KW), part, part_db,
                                                      want_db);
    return hipGetLastError();
}

template <typename T, int BM, int BN, int BK>
hipError_t launch_cfg(const T* x, const T* dz, const DwGeom& g, const Plan& p, float* part, float* part_db,
                      int want_db, hipStream_t s) {
    constexpr int WN = BN >= 64 ? (BM >= 64 ? 2 : 4) : 1;
    constexpr int WM = 4 / WN;
    dim3 grid(p.tiles_m * p.tiles_n, 1, p.S);
    dw_kernel<T, BM, BN, BK, WM, WN><<<grid, NT, 0, s>>>(x, dz, g, part, part_db, want_db);
    return hipGetLastError();
}

// Channel width of the stride-1 bf16 kernel for this layer: 128 when both channel counts
// are multiples of 128, else 64 when both are multiples of 64; 0: not taken (kernels at
// most 3 wide).
int dw3_ch(int dt, const ConvDims& d) {
    if (dt != DT_BF16 || d.sh != 1 || d.sw != 1 || d.KW < 1 || d.KW > 3) return 0;
    if (d.OC % 128 == 0 && d.IC % 128 == 0) return 128;
    if (d.OC % 64 == 0 && d.IC % 64 == 0) return 64;
    return 0;
}
bool dw3_ok(int dt, const ConvDims& d) { return dw3_ch(dt, d) != 0; }
}  // namespace

// The 64-channel stride-1 kernel runs two-wave workgroups with a small LDS ring, so a CU
// that holds some of them still has room for input-gradient workgroups.
bool dw_leaves_room(int dt, const ConvDims& d) { return dw3_ch(dt, d) == 64; }

namespace {
// fp32 stride-1 layers with 64-channel multiples and kernels at most 3 wide, on output
// rows of at least 16 positions (shorter rows leave most of a 16-position stage padding;
// the per-tap kernel is faster there: c2c's 7-wide rows).
bool dw3f_ok(int dt, const ConvDims& d) {
    return dt == DT_F32 && d.sh == 1 && d.sw == 1 && d.KW >= 1 && d.KW <= 3 && d.OC % 64 == 0 && d.IC % 64 == 0 &&
           d.OW >= 16;
}

// Stage geometry.  bf16, 128 channels: two whole output rows when they fit in 128
// positions, else one row split into equal segments of at most 128; about one workgroup
// per CU.  bf16, 64 channels: two segments of at most 32 positions (or two whole rows of
// at most 32); about four workgroups per CU.  fp32 (64 channels, 256-byte rows): two
// whole rows when they fit in 64 positions, else one segment of at most 64; about two
// workgroups per CU.  Segment starts are aligned to a copy's rows.
Dw3Geom plan3(const ConvDims& d, int ch, int es = 2) {
    Dw3Geom g;
    g.N = d.N; g.H = d.H; g.W = d.W; g.IC = d.IC; g.OC = d.OC; g.KH = d.KH; g.KW = d.KW;
    g.OH = d.OH; g.OW = d.OW; g.ph = d.ph; g.pw = d.pw;
    const bool f32 = es == 4;
    const int seg_max = f32 ? 64 : (ch == 128 ? 128 : 32), rpi = 1024 / (es * ch);
    if (2 * d.OW <= (f32 ? 64 : (ch == 128 ? 128 : 64))) {
        g.RS = 2;
        g.nseg = 1;
        g.SEG = d.OW;
    } else {
        g.RS = (ch == 128 || f32) ? 1 : 2;
        g.nseg = (int)ceil_div(d.OW, seg_max);
        g.SEG = (int)ceil_div(d.OW, g.nseg);
    }
    g.SEGp = (int)ceil_div(g.SEG, rpi) * rpi;
    g.SPp = (int)ceil_div(g.RS == 2 ? g.SEGp + g.SEG : g.SEG, 16) * 16;
    g.XW = g.SEG + d.KW - 1;
    g.XWp = g.SEGp + (int)ceil_div(d.KW - 1, rpi) * rpi;  // same swizzle phase as the first segment
    const int need_rows = g.RS == 2 ? g.XWp + g.XW : g.XW;
    const int read_rows = g.SPp + (g.XWp - g.SEGp) + d.KW - 1;  // padded positions included
    g.XR = (int)ceil_div(need_rows > read_rows ? need_rows : read_rows, rpi) * rpi;
    g.G = d.N * d.OH * g.nseg;
    g.nst = (int)ceil_div(g.G, g.RS);
    g.ict = d.IC / ch;
    g.oct = d.OC / ch;
    g.tiles = d.KH * g.ict * g.oct;
    int S = (f32 ? 512 : (ch == 128 ? 256 : 1024)) / g.tiles;
    if (S < 1) S = 1;
    if (S > g.nst) S = g.nst;
    g.spb = (int)ceil_div(g.nst, S);
    g.S = (int)ceil_div(g.nst, g.spb);
    g.Kdim = d.KH * d.KW * d.IC;
    g.fnseg = make_fastdiv(g.nseg);
    g.fOH = make_fastdiv(d.OH);
    return g;
}

size_t dw3_lds(const Dw3Geom& g, int ch, int es = 2) { return (size_t)2 * (g.SPp + g.XR) * es * ch; }

template <int CH, int KW_, int NK>
hipError_t launch_dw3_kw(const bf16* x, const bf16* dz, const Dw3Geom& g, float* part, float* part_db, int want_db,
                         hipStream_t s) {
    auto kern = dw3_kernel<CH, KW_, NK>;
    static bool raised = false;  // the dynamic LDS limit is raised once per instantiation
    if (!raised) {
        const hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 160 * 1024);
        if (e != hipSuccess) return e;
        raised = true;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)(g.S * g.tiles)), dim3(dw3_threads<CH>()), dw3_lds(g, CH), s, x, dz, g,
                       part, part_db, want_db);
    return hipGetLastError();
}

template <int KW_, int NK>
hipError_t launch_dw3f_kw(const float* x, const float* dz, const Dw3Geom& g, float* part, float* part_db,
                          int want_db, hipStream_t s) {
    auto kern = dw3f_kernel<KW_, NK>;
    static bool raised = false;  // the dynamic LDS limit is raised once per instantiation
    if (!raised) {
        const hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 160 * 1024);
        if (e != hipSuccess) return e;
        raised = true;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)(g.S * g.tiles)), dim3(256), dw3_lds(g, 64, 4), s, x, dz, g, part,
                       part_db, want_db);
    return hipGetLastError();
}

}  // namespace

bool igemm_dw_supported(int dt, const ConvDims& d) {
    const int vec = dt == DT_BF16 ? 8 : 4;
    return d.IC % vec == 0 && d.OC % vec == 0 && d.OC >= 16;
}

size_t igemm_dw_ws_bytes(int dt, const ConvDims& d) {
    const bool s1 = dw3_ok(dt, d) || dw3f_ok(dt, d);
    const int S = dw3_ok(dt, d) ? plan3(d, dw3_ch(dt, d)).S : dw3f_ok(dt, d) ? plan3(d, 64, 4).S : plan(dt, d).S;
    const int Sdb = s1 ? S * d.KH : S;  // bias partials: one per slab (and kernel row)
    const size_t Kdim = (size_t)d.KH * d.KW * d.IC;
    return align_up((size_t)S * d.OC * Kdim * 4, 256) + align_up((size_t)Sdb * d.OC * 4, 256);
}

hipError_t launch_igemm_dw(int dt, const void* x, const void* dz, float* dw, float* db, int accumulate,
                           const ConvDims& d, void* ws, hipStream_t s) {
    if (dw3f_ok(dt, d)) {
        const Dw3Geom g = plan3(d, 64, 4);
        float* part = (float*)ws;
        float* part_db = (float*)((char*)ws + align_up((size_t)g.S * d.OC * g.Kdim * 4, 256));
        const int want_db = db != nullptr;
        const float *xf = (const float*)x, *zf = (const float*)dz;
        hipError_t e;
        if (d.KW == 3 && g.SPp == 64) e = launch_dw3f_kw<3, 16>(xf, zf, g, part, part_db, want_db, s);
        else if (d.KW == 3) e = launch_dw3f_kw<3, 0>(xf, zf, g, part, part_db, want_db, s);
        else if (d.KW == 2) e = launch_dw3f_kw<2, 0>(xf, zf, g, part, part_db, want_db, s);
        else e = launch_dw3f_kw<1, 0>(xf, zf, g, part, part_db, want_db, s);
        if (e != hipSuccess) return e;
        const int64_t count = (int64_t)d.OC * g.Kdim;
        dw_reduce4<<<reduce_grid(count, d.OC, db != nullptr), NT, 0, s>>>(part, part_db, dw, db, count, d.OC, g.S,
                                                                          g.S * g.KH, accumulate);
        return hipGetLastError();
    }
    if (dw3_ok(dt, d)) {
        const int ch = dw3_ch(dt, d);
        const Dw3Geom g = plan3(d, ch);
        float* part = (float*)ws;
        float* part_db = (float*)((char*)ws + align_up((size_t)g.S * d.OC * g.Kdim * 4, 256));
        const int want_db = db != nullptr;
        const bf16 *xb = (const bf16*)x, *zb = (const bf16*)dz;
        hipError_t e = hipErrorInvalidValue;
        const int nk = g.SPp / 16;
        if (ch == 128) {
            if (d.KW == 3 && nk == 7) e = launch_dw3_kw<128, 3, 7>(xb, zb, g, part, part_db, want_db, s);
            else if (d.KW == 3 && nk == 8) e = launch_dw3_kw<128, 3, 8>(xb, zb, g, part, part_db, want_db, s);
            else if (d.KW == 3) e = launch_dw3_kw<128, 3, 0>(xb, zb, g, part, part_db, want_db, s);
            else if (d.KW == 2) e = launch_dw3_kw<128, 2, 0>(xb, zb, g, part, part_db, want_db, s);
            else e = launch_dw3_kw<128, 1, 0>(xb, zb, g, part, part_db, want_db, s);
        } else {
            if (d.KW == 3 && nk == 4) e = launch_dw3_kw<64, 3, 4>(xb, zb, g, part, part_db, want_db, s);
            else if (d.KW == 3) e = launch_dw3_kw<64, 3, 0>(xb, zb, g, part, part_db, want_db, s);
            else if (d.KW == 2) e = launch_dw3_kw<64, 2, 0>(xb, zb, g, part, part_db, want_db, s);
            else e = launch_dw3_kw<64, 1, 0>(xb, zb, g, part, part_db, want_db, s);
        }
        if (e != hipSuccess) return e;
        const int64_t count = (int64_t)d.OC * g.Kdim;
        dw_reduce4<<<reduce_grid(count, d.OC, db != nullptr), NT, 0, s>>>(part, part_db, dw, db, count, d.OC, g.S,
                                                                          g.S * g.KH, accumulate);
        return hipGetLastError();
    }
    const Plan p = plan(dt, d);
    DwGeom g{d.N, d.H, d.W, d.IC, d.OC, d.KW, d.sh, d.sw, d.ph, d.pw, d.OH, d.OW,
             d.KH * d.KW * d.IC, d.N * d.OH * d.OW, p.Pc, p.tiles_n, p.S};
    float* part = (float*)ws;
    float* part_db = (float*)((char*)ws + align_up((size_t)p.S * d.OC * g.Kdim * 4, 256));
    const int want_db = db != nullptr;
    hipError_t e = hipErrorInvalidValue;
    if (p.dma) {
        if (dt == DT_BF16) {
            const bf16 *xb = (const bf16*)x, *zb = (const bf16*)dz;
            if (p.bm == 128 && p.bn == 128) e = launch_dw2<bf16, 128, 128>(xb, zb, g, d, p, part, part_db, want_db, s);
            else if (p.bm == 128) e = launch_dw2<bf16, 128, 64>(xb, zb, g, d, p, part, part_db, want_db, s);
            else if (p.bn == 128) e = launch_dw2<bf16, 64, 128>(xb, zb, g, d, p, part, part_db, want_db, s);
            else e = launch_dw2<bf16, 64, 64>(xb, zb, g, d, p, part, part_db, want_db, s);
        } else {
            const float *xf = (const float*)x, *zf = (const float*)dz;
            if (p.bm == 128) e = launch_dw2<float, 128, 64>(xf, zf, g, d, p, part, part_db, want_db, s);
            else if (p.bm == 64) e = launch_dw2<float, 64, 64>(xf, zf, g, d, p, part, part_db, want_db, s);
            else e = launch_dw2<float, 32, 64>(xf, zf, g, d, p, part, part_db, want_db, s);
        }
    } else if (dt == DT_BF16) {
        if (p.bm == 128) e = launch_cfg<bf16, 128, 128, 64>((const bf16*)x, (const bf16*)dz, g, p, part, part_db, want_db, s);
        else if (p.bm == 64 && p.bn == 128) e = launch_cfg<bf16, 64, 128, 64>((const bf16*)x, (const bf16*)dz, g, p, part, part_db, want_db, s);
        else if (p.bm == 64) e = launch_cfg<bf16, 64, 64, 64>((const bf16*)x, (const bf16*)dz, g, p, part, part_db, want_db, s);
        else if (p.bn == 128) e = launch_cfg<bf16, 32, 128, 64>((const bf16*)x, (const bf16*)dz, g, p, part, part_db, want_db, s);
        else e = launch_cfg<bf16, 32, 64, 64>((const bf16*)x, (const bf16*)dz, g, p, part, part_db, want_db, s);
    } else {
        if (p.bm == 128) e = launch_cfg<float, 128, 64, 32>((const float*)x, (const float*)dz, g, p, part, part_db, want_db, s);
        else if (p.bm == 64) e = launch_cfg<float, 64, 64, 32>((const float*)x, (const float*)dz, g, p, part, part_db, want_db, s);
        else e = launch_cfg<float, 32, 64, 32>((const float*)x, (const float*)dz, g, p, part, part_db, want_db, s);
    }
    if (e != hipSuccess) return e;
    const int64_t count = (int64_t)d.OC * g.Kdim;
    dw_reduce4<<<reduce_grid(count, d.OC, db != nullptr), NT, 0, s>>>(part, part_db, dw, db, count, d.OC, p.S, p.S,
                                                                      accumulate);
    return hipGetLastError();
}

}  // namespace convmi
