// k_dw.hip -- weight and bias gradients (a6) as a split-K GEMM on gfx950 MFMA.
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
#include "internal.hpp"
#include "lds_dma.hpp"

namespace convmi {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
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
// touches fall in distinct banks.  Two ring stages, two workgroups per CU.
__device__ __forceinline__ int dswz(int row) { return (row & 3) << 1; }

typedef short dw_short4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) dw_short4* dw_lds4_t;

template <typename T, int BM, int BN, int WM, int WN>
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
    constexpr int TM = BM / (WM * 16), TN = BN / (WN * 16);
    static_assert(TM * WM * 16 == BM && TN * WN * 16 == BN, "tile shape");
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
            const int lc = (lane % CA) ^ dswz(row);
            rowi[q] = row;
            colo[q] = oc0 + lc * VEC;
            cok[q] = colo[q] < g.OC;
            tkh[q] = tkw[q] = tic[q] = 0;
        } else {
            const int jb = j - IA;
            const int row = jb * ROWS_B + lane / CB;
            const int lc = (lane % CB) ^ dswz(row);
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
    floatx4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

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
                const int off = row * R + ((((cb >> 4) ^ dswz(row)) << 4) | (cb & 15));
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
                const int off = row * R + ((((cb >> 4) ^ dswz(row)) << 4) | (cb & 15));
                r[s4] = *(const uint32_t*)(base + off);
            }
            return make_uint4(r[0], r[1], r[2], r[3]);
        }
    };
    auto compute = [&](int st) {
        const unsigned char* As = smem + (st & 1) * STAGE;
        const unsigned char* Bs = As + BK * RA;
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
                for (int j = 0; j < TN; ++j) MM::run(acc[i][j], af[i], bfr[j]);
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
                const uint4 v = *(const uint4*)(As + row * RA + ((db_chunk ^ dswz(row)) << 4));
                MM::add_channels(v, dbs);
            }
        }
        compute(k);
    }

    float* dst = part + (int64_t)slab * g.OC * g.Kdim;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int oc = oc0 + wm * TM * 16 + i * 16 + lg * 4 + e;
                const int k = k0 + wn * TN * 16 + j * 16 + lr;
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

// dw = (accumulate ? dw : 0) + sum over slabs; four slab groups (s = q mod 4) per output
// vector are summed in slab order and then merged in group order: fixed order, so
// bitwise reproducible.  Block 0 also finishes db.  count is a multiple of 4.
__global__ __launch_bounds__(NT) void dw_reduce4(const float* __restrict__ part, const float* __restrict__ part_db,
                                                 float* __restrict__ dw, float* __restrict__ db, int64_t count,
                                                 int OC, int S, int accumulate) {
    __shared__ float4 red[4][64];
    const int q = threadIdx.x >> 6, o = threadIdx.x & 63;
    const int64_t i4 = (int64_t)blockIdx.x * 64 + o, n4 = count >> 2;
    float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i4 < n4)
        for (int s = q; s < S; s += 4) {
            const float4 v = ((const float4*)(part + (int64_t)s * count))[i4];
            r.x += v.x; r.y += v.y; r.z += v.z; r.w += v.w;
        }
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
    if (db && blockIdx.x == 0)
        for (int c = threadIdx.x; c < OC; c += NT) {
            float v = 0.0f;
            for (int k = 0; k < S; ++k) v += part_db[(int64_t)k * OC + c];
            db[c] = accumulate ? db[c] + v : v;
        }
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

template <typename T, int BM, int BN>
hipError_t launch_dw2(const T* x, const T* dz, const DwGeom& g, const ConvDims& d, const Plan& p, float* part,
                      float* part_db, int want_db, hipStream_t s) {
    constexpr int WN = (BM == 128 || BN == 64) ? 2 : 4;
    constexpr int WM = 4 / WN;
    dim3 grid(p.tiles_m * p.tiles_n * p.S);
    dw2_kernel<T, BM, BN, WM, WN><<<grid, NT, 0, s>>>(x, dz, g, make_fastdiv(d.OW), make_fastdiv(d.OH),
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

}  // namespace

bool igemm_dw_supported(int dt, const ConvDims& d) {
    const int vec = dt == DT_BF16 ? 8 : 4;
    return d.IC % vec == 0 && d.OC % vec == 0 && d.OC >= 16;
}

size_t igemm_dw_ws_bytes(int dt, const ConvDims& d) {
    const Plan p = plan(dt, d);
    const size_t Kdim = (size_t)d.KH * d.KW * d.IC;
    return align_up((size_t)p.S * d.OC * Kdim * 4, 256) + align_up((size_t)p.S * d.OC * 4, 256);
}

hipError_t launch_igemm_dw(int dt, const void* x, const void* dz, float* dw, float* db, int accumulate,
                           const ConvDims& d, void* ws, hipStream_t s) {
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
    dw_reduce4<<<(unsigned)ceil_div(count / 4, 64), NT, 0, s>>>(part, part_db, dw, db, count, d.OC, p.S,
                                                                accumulate);
    return hipGetLastError();
}

}  // namespace convmi
