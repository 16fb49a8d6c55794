// internal.hpp -- host-side interface between the C-ABI front end (api.hip) and the
// kernel translation units.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.hpp"

namespace convmi {

enum DType : int { DT_F32 = 0, DT_BF16 = 1 };

inline size_t dtype_size(int dt) { return dt == DT_BF16 ? 2 : 4; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---------------------------------------------------------------- direct kernels
// General-shape kernels (any IC, stride, padding): one thread per output element.
// They serve small layers and shapes the tiled MFMA kernels do not take.
hipError_t launch_conv_fwd_direct(int dt, const void* x, const void* w, const float* bias, void* z, void* y,
                                  const ConvDims& d, int act, hipStream_t s);
hipError_t launch_conv_dx_direct(int dt, const void* dz, const void* w, void* dx, const ConvDims& d,
                                 hipStream_t s);
hipError_t launch_conv_dw_direct(int dt, const void* x, const void* dz, float* dw, float* db, int accumulate,
                                 const ConvDims& d, hipStream_t s);

// ---------------------------------------------------------------- row reductions
// Per-channel reductions over the M = N*OH*OW rows of a [M][C] tensor are split into
// row slabs (one workgroup each) that write fp32 partials, then merged per channel in
// a fixed order.  The plan depends only on (M, C, dtype), so the workspace size and the
// summation order are reproducible.
struct RowPlan {
    int vec;              // elements per vector access (16 bytes, or 1 when C is not a multiple)
    int tpr;              // threads per row slice
    int rpi;              // rows per iteration of a workgroup
    int chunks;           // channel slices (grid.y)
    int64_t rows_per_block;
    int blocks;           // row slabs (grid.x)
    int bps;              // slabs per segment (all of them for batch norm)
    int64_t seg;          // rows per segment: 0 = all M rows (batch norm), S (per-sample norms)
};
RowPlan row_plan(int64_t M, int C, int dt);
// Layer / group norm: each sample's S = OH*OW rows are a segment of their own.
RowPlan seg_plan(int N, int64_t S, int C, int dt);
size_t bn_stats_ws_bytes(int64_t M, int C, int dt);
size_t bn_bwd_ws_bytes(int64_t M, int C, int dt);

hipError_t launch_bn_stats(int dt, const void* z, int64_t M, int C, float momentum, float eps, float* mean,
                           float* inv_std, float* run_mean, float* run_var, void* ws, hipStream_t s);
// y = act(a), a = z (norm 0) or the batch-norm affine (norm 1).
hipError_t launch_apply_act(int dt, const void* z, void* y, int64_t M, int C, int act, int norm,
                            const float* gamma, const float* beta, const float* mean, const float* inv_std,
                            hipStream_t s);
// dz = act'(z) * dy (no norm).
hipError_t launch_act_bwd(int dt, const void* z, const void* dy, void* dz, int64_t M, int C, int act,
                          hipStream_t s);
// dz = act'(a) * dy with the derivative taken from the output y = act(a) (no norm;
// identity, relu, tanh, sigmoid).
hipError_t launch_act_bwd_from_output(int dt, const void* y, const void* dy, void* dz, int64_t M, int C, int act,
                                      hipStream_t s);
// Batch-norm training backward (+ activation derivative), dgamma/dbeta optional.
hipError_t launch_bn_bwd(int dt, const void* z, const void* dy, void* dz, int64_t M, int C, int act,
                         const float* gamma, const float* beta, const float* mean, const float* inv_std,
                         float* dgamma, float* dbeta, int accumulate, int evaluation, void* ws, hipStream_t s);
hipError_t launch_bn_eval_stats(const float* run_mean, const float* run_var, int C, float eps, float* mean,
                                float* inv_std, hipStream_t s);

// Layer norm (G = 1) and group norm: statistics per sample n and group of C/G
// consecutive channels over the sample's S = OH*OW rows of z [N][S][C], stored at
// [n*G + g]; gamma/beta per channel.
size_t grp_stats_ws_bytes(int N, int64_t S, int C, int dt);
size_t grp_bwd_ws_bytes(int N, int64_t S, int C, int G, int dt);
hipError_t launch_grp_stats(int dt, const void* z, int N, int64_t S, int C, int G, float eps, float* mean,
                            float* inv_std, void* ws, hipStream_t s);
// From the per-tile statistics of the stride-1 forward's epilogue (tiles of one image
// are consecutive, ntiles / N of them per image).
hipError_t launch_grp_tiles_finalize(const float* part, int ntiles, int N, int C, int G, int64_t S, float eps,
                                     float* mean, float* inv_std, hipStream_t s);
hipError_t launch_grp_apply(int dt, const void* z, void* y, int N, int64_t S, int C, int G, int act,
                            const float* gamma, const float* beta, const float* mean, const float* inv_std,
                            hipStream_t s);
hipError_t launch_grp_bwd(int dt, const void* z, const void* dy, void* dz, int N, int64_t S, int C, int G, int act,
                          const float* gamma, const float* beta, const float* mean, const float* inv_std,
                          float* dgamma, float* dbeta, int accumulate, void* ws, hipStream_t s);

// ---------------------------------------------------------------- MFMA implicit GEMM
// Returns false (and launches nothing) when the shape is outside what the tiled
// kernels take; the caller then uses the direct kernels.
bool igemm_fwd_supported(int dt, const ConvDims& d);
bool igemm_dx_supported(int dt, const ConvDims& d);
bool igemm_dw_supported(int dt, const ConvDims& d);
size_t igemm_fwd_ws_bytes(int dt, const ConvDims& d);
size_t igemm_dx_ws_bytes(int dt, const ConvDims& d);
size_t igemm_dw_ws_bytes(int dt, const ConvDims& d);
// True when the weight-gradient kernel's workgroups leave room on a CU for others.
bool dw_leaves_room(int dt, const ConvDims& d);
hipError_t launch_igemm_fwd(int dt, const void* x, const void* w, const float* bias, void* z, void* y,
                            const ConvDims& d, int act, void* ws, hipStream_t s);
hipError_t launch_igemm_dx(int dt, const void* dz, const void* w, void* dx, const ConvDims& d, void* ws,
                           hipStream_t s);
hipError_t launch_igemm_dw(int dt, const void* x, const void* dz, float* dw, float* db, int accumulate,
                           const ConvDims& d, void* ws, hipStream_t s);

// ---------------------------------------------------------------- stride-1 input-tile reuse
// Forward and input gradient of stride-1 layers whose gathered channels fill 128-byte
// chunks: each input tile + halo is copied to LDS once per chunk and shared by all taps.
// bf16 rearranges the weights into MFMA fragment order in the workspace first (ws bytes
// below); fp32 reads w (forward) or the rearranged input-gradient weights of the generic
// path (backward, passed as w) directly.
bool halo_fwd_supported(int dt, const ConvDims& d);
bool halo_dx_supported(int dt, const ConvDims& d);
// Text naming the stride-1 tile plan (block, fragments, tile, halo buffers, paired bands),
// written into buf (at most len bytes, NUL-terminated); false when the layer takes no
// tile plan.
bool halo_plan_text(int dt, const ConvDims& d, bool fwd, char* buf, size_t len);
size_t halo_fwd_ws_bytes(int dt, const ConvDims& d);
size_t halo_dx_ws_bytes(int dt, const ConvDims& d);
// bn_eval: null, or {mean, inv_std, gamma, beta} of evaluation-mode batch norm, applied
// before the activation in the epilogue (y = act(gamma*(z - mean)*inv_std + beta)).
// stats_part: null, or room for 4 * C * halo_fwd_stat_tiles floats of per-tile training
// batch-norm statistics of z; then only z is written (y and act are ignored) and
// launch_bn_tiles_finalize turns the statistics into the batch mean and inverse std.
hipError_t launch_halo_fwd(int dt, const void* x, const void* w, const float* bias, void* z, void* y,
                           const ConvDims& d, int act, void* ws, hipStream_t s,
                           const float* const* bn_eval = nullptr, float* stats_part = nullptr);
int halo_fwd_stat_tiles(int dt, const ConvDims& d);  // spatial tiles of the forward (0: path not taken)
// part[(c*4 + q)*ntiles + tile], q = S1, S2, shift, count (see the forward epilogue).
hipError_t launch_bn_tiles_finalize(const float* part, int ntiles, int C, int64_t M, float momentum, float eps,
                                    float* mean, float* inv_std, float* run_mean, float* run_var, hipStream_t s);
hipError_t launch_halo_dx(int dt, const void* dz, const void* w, void* dx, const ConvDims& d, void* ws,
                          hipStream_t s);

}  // namespace convmi
