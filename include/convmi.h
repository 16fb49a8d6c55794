/*
 * convmi.h -- C ABI of the MI355X (gfx950) conv2d training-layer library.
 *
 * One 2D convolution layer for training, NHWC activations and OHWI weights:
 *   forward    z = conv(x, w) + b;  [batch norm: batch statistics, then
 *              a = gamma*(z-mean)*inv_std + beta, else a = z];  y = act(a)
 *   backward   dz = d act / d a * dy  (+ batch-norm training backward, dgamma, dbeta)
 *              dx = conv^T(dz, w)     dw (+)= sum dz * x,  db (+)= sum dz
 *
 * Pages the operations come from (source listings; a function name stands in for a
 * section):
 *   [generic] "rl_tools/nn/layers/conv2d/operations_generic.h" (hyperray 0.0.1 wheel)
 *   [cuda]    "rl_tools/nn/layers/conv2d/operations_cuda.h"    (hyperray 0.0.1 wheel)
 *   [mkl]     "rl_tools/nn/layers/conv2d/operations_cpu_mkl.h" (hyperray 0.0.1 wheel)
 *   [wgsl]    "conv2d_backward_weight.wgsl" (@simulatte/doppler 0.1.0)
 *   [doppler] the same package's backward kernels "groupnorm_backward.wgsl" and
 *             "gelu_backward.wgsl"
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller (for example the
 *     data_ptr() of torch tensors on the same GPU).  The library never allocates or
 *     frees device memory and never waits on the host: every kernel is enqueued on
 *     `stream` (a hipStream_t; NULL means the default stream) and the call returns
 *     before the work is done.  (conv2d_backward_full may also run part of its work on
 *     one library stream per device, ordered with `stream` by events; see there.)
 *   - Layouts are dense and row-major, as the [cuda] listing requires of its inputs:
 *       x, dx          [N][H][W][IC]
 *       w              [OC][KH][KW][IC]
 *       z, y, dy, dz   [N][OH][OW][OC],  OH = (H + 2*pad_h - KH)/stride_h + 1 (floor),
 *                                          OW likewise
 *       bias, gamma, beta, running_*, save_*, db, dgamma, dbeta   [OC]
 *       dw             [OC][KH][KW][IC]
 *   - Element type: x, w, z, y, dy, dz, dx are `desc->dtype` (fp32 or bf16, the latter
 *     as raw IEEE bfloat16 bits).  bias, gamma, beta, running and saved statistics,
 *     dw, db, dgamma, dbeta are always fp32.  Accumulation is fp32.
 *   - Data tensors (x, w, z, y, dy, dz, dx, dw) must be 16-byte aligned; the workspace
 *     must be 256-byte aligned.  Otherwise CONVMI_ERR_MISALIGNED.
 *   - `workspace` is caller-owned device scratch of at least the size that
 *     convmi_workspace_size() reports for the operation (may be NULL when that size
 *     is 0).  Its contents on entry do not matter.  Too small: CONVMI_ERR_WORKSPACE.
 *   - Every argument is checked on the host before any device work is enqueued; on a
 *     non-OK status nothing has been enqueued, except CONVMI_ERR_HIP (a launch
 *     failed).  convmi_last_error() then returns a message for the calling thread.
 *   - Results are deterministic: the same inputs give bitwise identical outputs
 *     (fixed-order reductions, no floating-point atomics; the [cuda] listing likewise
 *     insists on deterministic backward algorithms).
 *   - Output buffers must not overlap inputs, except dz == dy in activation_backward
 *     (the pages apply the activation derivative in place).
 */
#ifndef CONVMI_H
#define CONVMI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CONVMI_OK = 0,
    CONVMI_ERR_INVALID_ARG = 1, /* bad size, stride, pad, enum value, NULL pointer, aliasing */
    CONVMI_ERR_UNSUPPORTED = 2, /* valid request the library does not implement */
    CONVMI_ERR_WORKSPACE = 3,   /* workspace smaller than convmi_workspace_size() */
    CONVMI_ERR_MISALIGNED = 4,  /* a pointer violates the alignment rule above */
    CONVMI_ERR_HIP = 5          /* a HIP launch or runtime call failed */
} convmi_status;

typedef enum { CONVMI_F32 = 0, CONVMI_BF16 = 1 } convmi_dtype;

/* The activation set of the [mkl] listing's post-op table: identity, relu, tanh,
 * sigmoid; relu'(0) is taken as 0.  Plus GELU in its tanh form, as the [doppler]
 * gelu_backward kernel differentiates it: gelu(a) = a/2 (1 + tanh(u)),
 * u = sqrt(2/pi) (a + 0.044715 a^3). */
typedef enum {
    CONVMI_ACT_IDENTITY = 0,
    CONVMI_ACT_RELU = 1,
    CONVMI_ACT_TANH = 2,
    CONVMI_ACT_SIGMOID = 3,
    CONVMI_ACT_GELU = 4
} convmi_act;

/* Normalisation of z before the activation, a = gamma[c]*(z - mean)*inv_std + beta[c]:
 *   BATCH  per channel over the N*OH*OW rows (training or running statistics, see mode);
 *   LAYER  per sample over its OH*OW*OC values ([generic] layer-norm branches);
 *   GROUP  per sample and group of OC/groups consecutive channels over OH*OW*OC/groups
 *          values ([doppler] groupnorm_backward); LAYER is GROUP with one group.
 * LAYER and GROUP have no running statistics and use the sample's own statistics in
 * both modes; their save_mean / save_inv_std hold [N][groups] values. */
typedef enum {
    CONVMI_NORM_NONE = 0,
    CONVMI_NORM_BATCH = 1,
    CONVMI_NORM_LAYER = 2,
    CONVMI_NORM_GROUP = 3
} convmi_norm;

/* Batch-norm mode.  TRAIN: batch statistics, running statistics updated.  EVAL: the
 * running statistics normalise (mean = running_mean, inv_std = 1/sqrt(running_var +
 * eps)), nothing is updated, and the backward treats the statistics as constants
 * ([generic] forward and backward_input / backward, evaluation-mode branches).  Without
 * batch norm the two modes compute the same thing. */
typedef enum { CONVMI_MODE_TRAIN = 0, CONVMI_MODE_EVAL = 1 } convmi_mode;

typedef enum {
    CONVMI_OP_FORWARD = 0,
    CONVMI_OP_BACKWARD_DATA = 1,
    CONVMI_OP_BACKWARD_WEIGHT = 2,
    CONVMI_OP_BN_STATS = 3,
    CONVMI_OP_ACTIVATION_BACKWARD = 4,
    CONVMI_OP_BACKWARD_FULL = 5
} convmi_op;

/* The layer's problem statement: the [generic] listing's compile-time layer spec
 * (batch, input height/width/channels, output channels, kernel height/width, stride,
 * padding, activation, normalisation, batch-norm momentum and epsilon), here as a
 * runtime descriptor.  Padding is symmetric and zero-filled; the operation is a
 * cross-correlation (the [cuda] descriptor uses CUDNN_CROSS_CORRELATION).
 * Limits: all sizes >= 1, strides >= 1, pads >= 0, OH and OW >= 1, each tensor of one
 * image below 2^31 elements, N*OH*OW below 2^31.  momentum in [0,1] (BATCH); eps > 0
 * with any normalisation; groups >= 1 dividing OC (GROUP; ignored otherwise). */
typedef struct convmi_desc {
    int64_t N, H, W, IC, OC, KH, KW;
    int32_t stride_h, stride_w, pad_h, pad_w;
    int32_t activation;    /* convmi_act */
    int32_t normalization; /* convmi_norm */
    int32_t mode;          /* convmi_mode */
    int32_t dtype;         /* convmi_dtype */
    float momentum;        /* running <- (1-momentum)*running + momentum*batch */
    float eps;             /* inv_std = 1/sqrt(var + eps) */
    int32_t groups;        /* channel groups of CONVMI_NORM_GROUP */
} convmi_desc;

/* OH, OW for a descriptor (floor formula above).  Checks the descriptor. */
convmi_status convmi_output_dims(const convmi_desc* desc, int64_t* OH, int64_t* OW);

/* Bytes of workspace `op` needs for `desc` (0 is possible). */
convmi_status convmi_workspace_size(const convmi_desc* desc, int32_t op, size_t* bytes);

/* Forward: convolution + bias, then (batch norm) training statistics and the
 * normalise/affine step, then the activation.  [generic] forward (conv + bias into
 * pre_activations; batch-norm or layer-norm statistics; normalise + activate); [cuda]
 * forward (conv, add bias, bn_stats_training, bn_forward_affine, activation).
 * LAYER / GROUP: gamma, beta, save_mean, save_inv_std ([N][groups]) and z required;
 * running_mean / running_var must be NULL.
 *   x, w: inputs.  bias: fp32 [OC] or NULL (no bias).
 *   gamma, beta, running_mean, running_var, save_mean, save_inv_std: batch norm only
 *     (NULL otherwise).  TRAIN: running_* (optional, both or neither) are updated in
 *     place with the biased batch variance (as on the pages); save_mean / save_inv_std
 *     receive the batch mean and 1/sqrt(var+eps) for the backward pass.  EVAL:
 *     running_* are required and only read; save_mean / save_inv_std receive
 *     running_mean and 1/sqrt(running_var+eps).
 *   z: pre-activation output (conv + bias).  Required with batch norm; may be NULL
 *     without it.  y: the layer output act(a).  Both overwritten. */
convmi_status conv2d_forward(const convmi_desc* desc, const void* x, const void* w, const float* bias,
                             const float* gamma, const float* beta, float* running_mean, float* running_var,
                             float* save_mean, float* save_inv_std, void* z, void* y,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Allocation-free forward, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, results and errors as conv2d_forward, minus the workspace: its scratch is a
 * static device array of CONVMI_NOALLOC_SCRATCH_BYTES that the library holds on each GPU
 * it runs on until the process ends (its address is looked up on the first call made
 * with that device current).  A layer needing more scratch than that returns
 * CONVMI_ERR_WORKSPACE before any device work; use conv2d_forward with a workspace then.
 * The call allocates nothing and calls no allocating routine.  Every call on one GPU
 * shares that GPU's array (whose contents on entry do not matter): calls that overlap
 * in time on the same GPU, from any stream or thread, race on it and must be ordered by
 * the caller. */
#define CONVMI_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
convmi_status conv2d_forward_noalloc(const convmi_desc* desc, const void* x, const void* w, const float* bias,
                                     const float* gamma, const float* beta, float* running_mean,
                                     float* running_var, float* save_mean, float* save_inv_std, void* z, void* y,
                                     void* stream);

/* Input gradient: dx[n,ih,iw,ic] = sum over (oc,kh,kw) with oh*stride_h - pad_h + kh == ih and
 * ow*stride_w - pad_w + kw == iw of w[oc,kh,kw,ic] * dz[n,oh,ow,oc].  Linear in dz:
 * the activation / batch-norm derivative is applied beforehand by
 * activation_backward.  dx is overwritten.  [generic] backward_input (the scatter
 * after the activation derivative); [cuda] backward_input (BackwardData, beta 0). */
convmi_status conv2d_backward_data(const convmi_desc* desc, const void* dz, const void* w, void* dx,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* Weight and bias gradients: dw[oc,kh,kw,ic] = sum_{n,oh,ow} dz[n,oh,ow,oc] * x[n, oh*sh-ph+kh, ow*sw-pw+kw, ic]
 * (zero outside the image); db[oc] = sum_{n,oh,ow} dz[n,oh,ow,oc].  accumulate = 0
 * overwrites dw/db, 1 adds into them (the pages accumulate parameter gradients).
 * db may be NULL.  [generic] backward; [wgsl] conv2d_backward_weight; [cuda]
 * BackwardFilter and bias_backward_partial/finalize. */
convmi_status conv2d_backward_weight(const convmi_desc* desc, const void* x, const void* dz, float* dw,
                                     float* db, int32_t accumulate, void* workspace, size_t workspace_bytes,
                                     void* stream);

/* Training statistics: per-channel statistics of z over the N*OH*OW rows: mean, biased var,
 * save_inv_std = 1/sqrt(var+eps); running_mean/var (nullable, both or neither)
 * updated with momentum.  [generic] forward, batch-norm training statistics; [cuda]
 * bn_stats_training.  TRAIN mode only (INVALID_ARG in EVAL mode, where
 * conv2d_forward takes the running statistics).  With LAYER / GROUP normalisation the
 * same call gives the per-sample (per-group) statistics, [N][groups] values, in either
 * mode; running_mean / running_var must then be NULL. */
convmi_status bn_stats_training(const convmi_desc* desc, const void* z, float* save_mean, float* save_inv_std,
                                float* running_mean, float* running_var,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Activation backward, plus the batch-norm training backward when
 * desc->normalization is BATCH.
 *   No norm:   dz = act'(z) * dy.
 *   Batch norm: zhat = (z-mean)*inv_std, a = gamma*zhat + beta, dno = act'(a)*dy,
 *     per channel over M = N*OH*OW rows: S1 = sum dno*gamma, S2 = sum dno*gamma*zhat,
 *     dz = inv_std/M * (M*dno*gamma - S1 - zhat*S2), dgamma (+)= sum dno*zhat,
 *     dbeta (+)= sum dno.  gamma, beta, save_mean, save_inv_std are required and
 *     dgamma, dbeta optional (NULL skips them); `accumulate` as for dw.
 *   Batch norm, EVAL mode (constant statistics): dz = dno * gamma * inv_std, with
 *     dgamma, dbeta as above.
 *   LAYER / GROUP (either mode): the training formula above per sample and group, with
 *     cnt = OH*OW*OC/groups values in place of M, save_* [N][groups]; dgamma and dbeta
 *     per channel over all samples and pixels.
 * dz may equal dy (in place).  [generic] backward_input / backward (training-mode
 * two-phase normalisation backward, evaluation-mode branch); [cuda]
 * activation_backward, bn_training_backward. */
convmi_status activation_backward(const convmi_desc* desc, const void* z, const void* dy,
                                  const float* gamma, const float* beta,
                                  const float* save_mean, const float* save_inv_std,
                                  void* dz, float* dgamma, float* dbeta, int32_t accumulate,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Activation backward, input gradient and weight/bias gradients of an unnormalised
 * layer in one call, as the [generic] listing's backward_full (input gradient and
 * parameter gradients from the output gradient):
 *   dz = act'(.) * dy;  dx = conv^T(dz, w) (overwritten);  dw (+)= sum dz * x;
 *   db (+)= sum dz  -- the results of activation_backward followed by
 * conv2d_backward_data and conv2d_backward_weight, without dz in the caller's memory.
 *   saved: what the forward kept of the activation input: z (saved_is_output = 0), or
 *     the output y (saved_is_output = 1) for identity, relu, tanh and sigmoid, whose
 *     derivative is a function of y -- 1, [y > 0], 1 - y^2, y (1 - y) -- as the [cuda]
 *     listing's activation backward reads y.  GELU needs z.
 *   dx may be NULL (no input gradient, as for a network's first layer); dw is
 *   required, db may be NULL; accumulate as for conv2d_backward_weight.
 * normalization must be NONE (CONVMI_ERR_UNSUPPORTED otherwise: normalised layers call
 * activation_backward and then the two products).  Workspace: the size
 * convmi_workspace_size reports for CONVMI_OP_BACKWARD_FULL (it holds dz unless the
 * activation is the identity, when dz = dy, and the two products' own workspaces side
 * by side).
 * Streams: with dx requested on a bf16 stride-1 layer whose weight gradient takes
 * 64-channel tiles (small workgroups that leave room on a CU), the weight gradient runs
 * on a second stream that the library creates once per device (default priority),
 * forked from `stream` after dz and joined back into it with events, while the input
 * gradient runs on `stream`; every other layer runs both on `stream`.  For the
 * caller the call stays ordered on `stream` like any other, and it can be captured into
 * a HIP graph (the fork and join become graph dependencies).  Calls on one device share
 * that second stream, so their weight gradients run in issue order. */
convmi_status conv2d_backward_full(const convmi_desc* desc, const void* x, const void* w, const void* saved,
                                   int32_t saved_is_output, const void* dy, void* dx, float* dw, float* db,
                                   int32_t accumulate, void* workspace, size_t workspace_bytes, void* stream);

/* Name of the kernel plan that `op` (CONVMI_OP_FORWARD or CONVMI_OP_BACKWARD_DATA) takes
 * for `desc`: "halo <dtype> <block rows>x<block channels> mf<fragment rows> tile <R>x<Q>
 * hb<halo buffers>" for the stride-1 tile kernel (with " paired <R2>x<Q> in <rows> rows"
 * when every workgroup also computes a short band of R2 rows), "implicit gemm" or
 * "direct".  Host-only: no device work, for tests and tuning.  Written into buf, at most
 * len bytes including the terminating NUL (longer names are cut).  Errors: invalid
 * descriptor, NULL buf or len 0, another op (CONVMI_ERR_INVALID_ARG). */
convmi_status convmi_plan_name(const convmi_desc* desc, int32_t op, char* buf, size_t len);

/* Message describing the last non-OK status returned on the calling thread. */
const char* convmi_last_error(void);

/* Library version string. */
const char* convmi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CONVMI_H */
