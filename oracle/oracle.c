/*
 * oracle.c -- plain, slow, fp64 CPU reference for the conv2d training layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load this
 * file: only the tests, the smoke check and the bench's cpu_baseline leg use it.  It
 * shares no code, header, table or helper with the HIP library in
 * convolution_layer_amd/csrc; the two meet only through the seeded inputs of
 * workloads.py.
 *
 * Every routine is the textbook definition written out with fp64 accumulation, one
 * output element at a time, with no blocking, fusion or reordering.  Parallelism
 * (OpenMP) is only over independent outer indices, so results do not depend on the
 * thread count.
 *
 * Pages cited (each is a source listing; the function name stands in for a section):
 *   [generic] "rl_tools/nn/layers/conv2d/operations_generic.h" (hyperray 0.0.1 wheel)
 *   [cuda]    "rl_tools/nn/layers/conv2d/operations_cuda.h"    (hyperray 0.0.1 wheel)
 *   [mkl]     "rl_tools/nn/layers/conv2d/operations_cpu_mkl.h" (hyperray 0.0.1 wheel)
 *   [wgsl]    "conv2d_backward_weight.wgsl" (@simulatte/doppler 0.1.0)
 *   [doppler] the @simulatte/doppler 0.1.0 backward kernels "groupnorm_backward.wgsl"
 *             and "gelu_backward.wgsl" (same page as [wgsl])
 *
 * Layouts (the pages' dense row-major NHWC activations and OHWI weights):
 *   x  [N][H][W][IC], w [OC][KH][KW][IC], z/y/dy/dz [N][OH][OW][OC], dx like x,
 *   dw like w, per-channel vectors [OC].
 *
 * Parity pinned by tests/test_oracle_pins.py: scipy correlate2d and torch fp64 conv
 * (library routines), delta kernel, 1x1 = matmul, closed forms for constant inputs,
 * adjoint identities, central finite differences, batch-norm invariants and torch fp64
 * autograd through batch_norm + activation.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef int64_t i64;

enum { ACT_IDENTITY = 0, ACT_RELU = 1, ACT_TANH = 2, ACT_SIGMOID = 3, ACT_GELU = 4 };
enum { NORM_NONE = 0, NORM_BATCH = 1, NORM_LAYER = 2, NORM_GROUP = 3 };

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Output extent along one axis: floor((in + 2p - k)/s) + 1 (symmetric zero padding,
 * cross-correlation; [cuda] descriptor set-up uses symmetric padding and
 * CUDNN_CROSS_CORRELATION; [generic] forward accepts a tap when p <= o*s+k < in+p).
 * Returns 0 when the window does not fit, -1 for invalid s/k/p. */
i64 oracle_out_extent(i64 in, i64 k, i64 s, i64 p) {
    if (in <= 0 || k <= 0 || s <= 0 || p < 0) return -1;
    i64 span = in + 2 * p - k;
    if (span < 0) return 0;
    return span / s + 1;
}

/* ---------------------------------------------------------------- activations ---- */
/* [mkl] make_activation_post_ops: the activation set is identity, relu, tanh, sigmoid.
 * [doppler] gelu_backward adds GELU in its tanh form:
 *   gelu(a) = a/2 * (1 + tanh(u)),  u = sqrt(2/pi) * (a + 0.044715 a^3). */
static const double GELU_K1 = 0.044715;
static const double ORACLE_PI = 3.14159265358979323846;

static double gelu_u(double a) { return sqrt(2.0 / ORACLE_PI) * (a + GELU_K1 * a * a * a); }

static double act_value(int act, double a) {
    switch (act) {
    case ACT_RELU: return a > 0.0 ? a : 0.0;
    case ACT_TANH: return tanh(a);
    case ACT_SIGMOID: return 1.0 / (1.0 + exp(-a));
    case ACT_GELU: return 0.5 * a * (1.0 + tanh(gelu_u(a)));
    default: return a;
    }
}

/* Derivative d act(a) / da, evaluated at the activation input a ([generic]
 * backward_input applies d_activation_d_x to the pre-activation).  relu'(0) = 0.
 * GELU, by the product and chain rules on the definition above:
 *   gelu'(a) = (1 + t)/2 + a/2 * (1 - t^2) * du/da,  t = tanh(u),
 *   du/da = sqrt(2/pi) * (1 + 3 * 0.044715 a^2). */
static double act_slope(int act, double a) {
    switch (act) {
    case ACT_RELU: return a > 0.0 ? 1.0 : 0.0;
    case ACT_TANH: { double t = tanh(a); return 1.0 - t * t; }
    case ACT_SIGMOID: { double s = 1.0 / (1.0 + exp(-a)); return s * (1.0 - s); }
    case ACT_GELU: {
        double t = tanh(gelu_u(a));
        double du = sqrt(2.0 / ORACLE_PI) * (1.0 + 3.0 * GELU_K1 * a * a);
        return 0.5 * (1.0 + t) + 0.5 * a * (1.0 - t * t) * du;
    }
    default: return 1.0;
    }
}

/* ------------------------------------------------------------------- forward ---- */
/* z[n,oh,ow,oc] = b[oc] + sum_{kh,kw,ic} w[oc,kh,kw,ic] * x[n, oh*sh-ph+kh, ow*sw-pw+kw, ic]
 * with out-of-range taps contributing zero.  [generic] forward, phase 1 (conv + bias
 * into pre_activations). */
static double conv_point(const double* x, const double* w, const double* b,
                         i64 H, i64 W, i64 IC, i64 KH, i64 KW, i64 sh, i64 sw, i64 ph, i64 pw,
                         i64 n, i64 oh, i64 ow, i64 oc) {
    double acc = b ? b[oc] : 0.0;
    for (i64 kh = 0; kh < KH; ++kh) {
        i64 ih = oh * sh - ph + kh;
        if (ih < 0 || ih >= H) continue;
        for (i64 kw = 0; kw < KW; ++kw) {
            i64 iw = ow * sw - pw + kw;
            if (iw < 0 || iw >= W) continue;
            const double* xp = x + ((n * H + ih) * W + iw) * IC;
            const double* wp = w + ((oc * KH + kh) * KW + kw) * IC;
            for (i64 ic = 0; ic < IC; ++ic) acc += wp[ic] * xp[ic];
        }
    }
    return acc;
}

void oracle_conv2d_forward(const double* x, const double* w, const double* b, double* z,
                           i64 N, i64 H, i64 W, i64 IC, i64 OC, i64 KH, i64 KW,
                           i64 sh, i64 sw, i64 ph, i64 pw) {
    i64 OH = oracle_out_extent(H, KH, sh, ph), OW = oracle_out_extent(W, KW, sw, pw);
    if (OH <= 0 || OW <= 0) return;
#pragma omp parallel for collapse(2) schedule(static)
    for (i64 n = 0; n < N; ++n)
        for (i64 oh = 0; oh < OH; ++oh)
            for (i64 ow = 0; ow < OW; ++ow)
                for (i64 oc = 0; oc < OC; ++oc)
                    z[((n * OH + oh) * OW + ow) * OC + oc] =
                        conv_point(x, w, b, H, W, IC, KH, KW, sh, sw, ph, pw, n, oh, ow, oc);
}

/* The same definition evaluated only at listed outputs idx[i] = (n, oh, ow, oc). */
void oracle_conv2d_forward_at(const double* x, const double* w, const double* b,
                              const i64* idx, i64 count, double* out,
                              i64 N, i64 H, i64 W, i64 IC, i64 OC, i64 KH, i64 KW,
                              i64 sh, i64 sw, i64 ph, i64 pw) {
    (void)N; (void)OC;
#pragma omp parallel for schedule(dynamic, 16)
    for (i64 i = 0; i < count; ++i)
        out[i] = conv_point(x, w, b, H, W, IC, KH, KW, sh, sw, ph, pw,
                            idx[4 * i], idx[4 * i + 1], idx[4 * i + 2], idx[4 * i + 3]);
}

/* --------------------------------------------------- batch-norm statistics ---- */
/* Per channel c over the M = N*OH*OW rows of z [M][C]:
 *   mean = sum z / M;  var = sum (z - mean)^2 / M  (biased);  inv_std = 1/sqrt(var+eps)
 *   running_mean <- (1-momentum)*running_mean + momentum*mean
 *   running_var  <- (1-momentum)*running_var  + momentum*var   (the biased var)
 * [generic] forward, batch-norm training branch (two passes); [cuda] bn_stats_training
 * (same update rule, biased variance).  Running pointers may be NULL. */
void oracle_bn_stats(const double* z, i64 M, i64 C, double momentum, double eps,
                     double* mean, double* var, double* inv_std,
                     double* running_mean, double* running_var) {
#pragma omp parallel for schedule(static)
    for (i64 c = 0; c < C; ++c) {
        double s = 0.0;
        for (i64 m = 0; m < M; ++m) s += z[m * C + c];
        double mu = s / (double)M;
        double q = 0.0;
        for (i64 m = 0; m < M; ++m) {
            double d = z[m * C + c] - mu;
            q += d * d;
        }
        double v = q / (double)M;
        mean[c] = mu;
        if (var) var[c] = v;
        inv_std[c] = 1.0 / sqrt(v + eps);
        if (running_mean) running_mean[c] = (1.0 - momentum) * running_mean[c] + momentum * mu;
        if (running_var) running_var[c] = (1.0 - momentum) * running_var[c] + momentum * v;
    }
}

/* Evaluation mode: the running statistics stand in for the batch ones.
 *   mean = running_mean,  inv_std = 1 / sqrt(running_var + eps);  nothing is updated.
 * [generic] forward, evaluation-mode branch of the batch-norm statistics. */
void oracle_bn_eval_stats(const double* running_mean, const double* running_var, i64 C, double eps,
                          double* mean, double* inv_std) {
    for (i64 c = 0; c < C; ++c) {
        mean[c] = running_mean[c];
        inv_std[c] = 1.0 / sqrt(running_var[c] + eps);
    }
}

/* ---------------------------------------------------- normalise + activate ---- */
/* a = z (no norm) or gamma*(z-mean)*inv_std + beta (batch norm); y = act(a).
 * [generic] forward phase 3 and the no-norm branch; [cuda] bn_forward_affine. */
void oracle_apply_activation(const double* z, i64 M, i64 C, int act, int norm,
                             const double* gamma, const double* beta,
                             const double* mean, const double* inv_std, double* y) {
#pragma omp parallel for schedule(static)
    for (i64 m = 0; m < M; ++m)
        for (i64 c = 0; c < C; ++c) {
            double a = z[m * C + c];
            if (norm == NORM_BATCH) a = gamma[c] * ((a - mean[c]) * inv_std[c]) + beta[c];
            y[m * C + c] = act_value(act, a);
        }
}

/* ----------------------------------------------------- activation backward ---- */
/* No norm:  dz = act'(z) * dy.
 * Batch norm, training mode, per channel c over M rows:
 *   zhat = (z - mean) * inv_std,  a = gamma*zhat + beta,  dno = act'(a) * dy,
 *   dzhat = dno * gamma,  S1 = sum dzhat,  S2 = sum dzhat * zhat,
 *   dz = inv_std / M * (M*dzhat - S1 - zhat*S2),
 *   dgamma = sum dno * zhat,  dbeta = sum dno   (written, not accumulated).
 * [generic] backward_input / backward, training-mode two-phase normalisation backward;
 * [cuda] activation_backward and bn_training_backward.  dgamma/dbeta may be NULL. */
void oracle_activation_backward(const double* z, const double* dy, i64 M, i64 C, int act, int norm,
                                const double* gamma, const double* beta,
                                const double* mean, const double* inv_std,
                                double* dz, double* dgamma, double* dbeta) {
    if (norm != NORM_BATCH) {
#pragma omp parallel for schedule(static)
        for (i64 i = 0; i < M * C; ++i) dz[i] = act_slope(act, z[i]) * dy[i];
        return;
    }
#pragma omp parallel for schedule(static)
    for (i64 c = 0; c < C; ++c) {
        double g = gamma[c], mu = mean[c], is = inv_std[c];
        double s1 = 0.0, s2 = 0.0, sg = 0.0, sb = 0.0;
        for (i64 m = 0; m < M; ++m) {
            i64 i = m * C + c;
            double zh = (z[i] - mu) * is;
            double a = g * zh + beta[c];
            double dno = act_slope(act, a) * dy[i];
            double dzh = dno * g;
            s1 += dzh;
            s2 += dzh * zh;
            sg += dno * zh;
            sb += dno;
        }
        for (i64 m = 0; m < M; ++m) {
            i64 i = m * C + c;
            double zh = (z[i] - mu) * is;
            double a = g * zh + beta[c];
            double dzh = act_slope(act, a) * dy[i] * g;
            dz[i] = is / (double)M * ((double)M * dzh - s1 - zh * s2);
        }
        if (dgamma) dgamma[c] = sg;
        if (dbeta) dbeta[c] = sb;
    }
}

/* The same derivative for the unnormalised layer, taken from the layer output y = act(z)
 * instead of z (the [cuda] listing's cuDNN activation backward reads the output y):
 *   identity 1,  relu [y > 0] (= [z > 0]),  tanh 1 - y^2,  sigmoid y (1 - y);
 *   dz = act'(y) * dy.  GELU has no such form (it is not invertible) and is rejected (-1). */
int oracle_activation_backward_from_output(const double* y, const double* dy, i64 n, int act, double* dz) {
    if (act == ACT_GELU) return -1;
#pragma omp parallel for schedule(static)
    for (i64 i = 0; i < n; ++i) {
        double s = 1.0, v = y[i];
        if (act == ACT_RELU) s = v > 0.0 ? 1.0 : 0.0;
        else if (act == ACT_TANH) s = 1.0 - v * v;
        else if (act == ACT_SIGMOID) s = v * (1.0 - v);
        dz[i] = s * dy[i];
    }
    return 0;
}

/* Evaluation-mode batch-norm backward: the statistics are constants, so each element
 * stands alone:
 *   zhat = (z - mean) * inv_std,  a = gamma*zhat + beta,  dno = act'(a) * dy,
 *   dz = dno * gamma * inv_std;   per channel dgamma = sum dno*zhat, dbeta = sum dno
 * (written, not accumulated).  [generic] backward_input and backward, evaluation-mode
 * branches.  dgamma/dbeta may be NULL. */
void oracle_activation_backward_eval(const double* z, const double* dy, i64 M, i64 C, int act,
                                     const double* gamma, const double* beta,
                                     const double* mean, const double* inv_std,
                                     double* dz, double* dgamma, double* dbeta) {
#pragma omp parallel for schedule(static)
    for (i64 c = 0; c < C; ++c) {
        double g = gamma[c], mu = mean[c], is = inv_std[c];
        double sg = 0.0, sb = 0.0;
        for (i64 m = 0; m < M; ++m) {
            i64 i = m * C + c;
            double zh = (z[i] - mu) * is;
            double a = g * zh + beta[c];
            double dno = act_slope(act, a) * dy[i];
            dz[i] = dno * g * is;
            sg += dno * zh;
            sb += dno;
        }
        if (dgamma) dgamma[c] = sg;
        if (dbeta) dbeta[c] = sb;
    }
}

/* ------------------------------------------- layer norm and group norm ---- */
/* Statistics per sample n and channel group g (channels g*C/G .. (g+1)*C/G - 1) over the
 * S = OH*OW pixels of the sample, z [N][S][C]:
 *   cnt = S*C/G,  mean = sum z / cnt,  var = sum (z - mean)^2 / cnt (biased),
 *   inv_std = 1/sqrt(var + eps);  stored at [n*G + g].
 * LayerNorm is G = 1: all OH*OW*OC values of a sample ([generic] forward, layer-norm
 * branch: per-sample mean, then variance, two passes).  [doppler] groupnorm_backward
 * recomputes the same per-group statistics of its input.  No running statistics. */
void oracle_group_stats(const double* z, i64 N, i64 S, i64 C, i64 G, double eps,
                        double* mean, double* var, double* inv_std) {
    const i64 cg = C / G;
    const double cnt = (double)(S * cg);
#pragma omp parallel for collapse(2) schedule(static)
    for (i64 n = 0; n < N; ++n)
        for (i64 g = 0; g < G; ++g) {
            double s = 0.0;
            for (i64 p = 0; p < S; ++p)
                for (i64 k = 0; k < cg; ++k) s += z[(n * S + p) * C + g * cg + k];
            double mu = s / cnt;
            double q = 0.0;
            for (i64 p = 0; p < S; ++p)
                for (i64 k = 0; k < cg; ++k) {
                    double d = z[(n * S + p) * C + g * cg + k] - mu;
                    q += d * d;
                }
            double v = q / cnt;
            mean[n * G + g] = mu;
            if (var) var[n * G + g] = v;
            inv_std[n * G + g] = 1.0 / sqrt(v + eps);
        }
}

/* a = gamma[c] * (z - mean[n,g]) * inv_std[n,g] + beta[c];  y = act(a), g = c / (C/G).
 * gamma and beta are per channel, as the [generic] layer-norm branch indexes them. */
void oracle_apply_group_norm(const double* z, i64 N, i64 S, i64 C, i64 G, int act,
                             const double* gamma, const double* beta,
                             const double* mean, const double* inv_std, double* y) {
    const i64 cg = C / G;
#pragma omp parallel for schedule(static)
    for (i64 n = 0; n < N; ++n)
        for (i64 p = 0; p < S; ++p)
            for (i64 c = 0; c < C; ++c) {
                i64 i = (n * S + p) * C + c, st = n * G + c / cg;
                double a = gamma[c] * ((z[i] - mean[st]) * inv_std[st]) + beta[c];
                y[i] = act_value(act, a);
            }
}

/* Training backward through the group normalisation and the activation, per sample n
 * and group g over its cnt = S*C/G values ([generic] backward_input / backward,
 * two-phase normalisation backward with the per-sample statistics index; [doppler]
 * groupnorm_backward, whose dx has the same form):
 *   zhat = (z - mean) * inv_std,  a = gamma[c]*zhat + beta[c],  dno = act'(a) * dy,
 *   dzhat = dno * gamma[c],  S1 = sum dzhat,  S2 = sum dzhat*zhat   (over the group),
 *   dz = inv_std / cnt * (cnt*dzhat - S1 - zhat*S2);
 *   per channel over all samples and pixels: dgamma = sum dno*zhat, dbeta = sum dno
 * (written, not accumulated).  dgamma/dbeta may be NULL. */
void oracle_group_norm_backward(const double* z, const double* dy, i64 N, i64 S, i64 C, i64 G, int act,
                                const double* gamma, const double* beta,
                                const double* mean, const double* inv_std,
                                double* dz, double* dgamma, double* dbeta) {
    const i64 cg = C / G;
    const double cnt = (double)(S * cg);
#pragma omp parallel for collapse(2) schedule(static)
    for (i64 n = 0; n < N; ++n)
        for (i64 g = 0; g < G; ++g) {
            const i64 st = n * G + g;
            const double mu = mean[st], is = inv_std[st];
            double s1 = 0.0, s2 = 0.0;
            for (i64 p = 0; p < S; ++p)
                for (i64 k = 0; k < cg; ++k) {
                    i64 c = g * cg + k, i = (n * S + p) * C + c;
                    double zh = (z[i] - mu) * is;
                    double dzh = act_slope(act, gamma[c] * zh + beta[c]) * dy[i] * gamma[c];
                    s1 += dzh;
                    s2 += dzh * zh;
                }
            for (i64 p = 0; p < S; ++p)
                for (i64 k = 0; k < cg; ++k) {
                    i64 c = g * cg + k, i = (n * S + p) * C + c;
                    double zh = (z[i] - mu) * is;
                    double dzh = act_slope(act, gamma[c] * zh + beta[c]) * dy[i] * gamma[c];
                    dz[i] = is / cnt * (cnt * dzh - s1 - zh * s2);
                }
        }
    if (!dgamma && !dbeta) return;
#pragma omp parallel for schedule(static)
    for (i64 c = 0; c < C; ++c) {
        double sg = 0.0, sb = 0.0;
        for (i64 n = 0; n < N; ++n)
            for (i64 p = 0; p < S; ++p) {
                i64 i = (n * S + p) * C + c, st = n * G + c / cg;
                double zh = (z[i] - mean[st]) * inv_std[st];
                double dno = act_slope(act, gamma[c] * zh + beta[c]) * dy[i];
                sg += dno * zh;
                sb += dno;
            }
        if (dgamma) dgamma[c] = sg;
        if (dbeta) dbeta[c] = sb;
    }
}

/* ------------------------------------------------------ input gradient dX ---- */
/* Scatter form of the adjoint of the forward: for every output (n,oh,ow,oc) and every in-range
 * tap (kh,kw), dx[n, oh*sh-ph+kh, ow*sw-pw+kw, ic] += w[oc,kh,kw,ic] * dz[n,oh,ow,oc].
 * dx is overwritten (zeroed first).  [generic] backward_input (the scatter loop after
 * the activation derivative); [cuda] backward_input = BackwardData with beta 0. */
void oracle_conv2d_backward_data(const double* dz, const double* w, double* dx,
                                 i64 N, i64 H, i64 W, i64 IC, i64 OC, i64 KH, i64 KW,
                                 i64 sh, i64 sw, i64 ph, i64 pw) {
    i64 OH = oracle_out_extent(H, KH, sh, ph), OW = oracle_out_extent(W, KW, sw, pw);
    memset(dx, 0, sizeof(double) * (size_t)(N * H * W * IC));
    if (OH <= 0 || OW <= 0) return;
#pragma omp parallel for schedule(static)
    for (i64 n = 0; n < N; ++n)
        for (i64 oh = 0; oh < OH; ++oh)
            for (i64 ow = 0; ow < OW; ++ow)
                for (i64 oc = 0; oc < OC; ++oc) {
                    double g = dz[((n * OH + oh) * OW + ow) * OC + oc];
                    for (i64 kh = 0; kh < KH; ++kh) {
                        i64 ih = oh * sh - ph + kh;
                        if (ih < 0 || ih >= H) continue;
                        for (i64 kw = 0; kw < KW; ++kw) {
                            i64 iw = ow * sw - pw + kw;
                            if (iw < 0 || iw >= W) continue;
                            double* xp = dx + ((n * H + ih) * W + iw) * IC;
                            const double* wp = w + ((oc * KH + kh) * KW + kw) * IC;
                            for (i64 ic = 0; ic < IC; ++ic) xp[ic] += wp[ic] * g;
                        }
                    }
                }
}

/* One dx element: the sum over every (oc, kh, kw) whose tap lands on (ih, iw), i.e.
 * oh*sh - ph + kh == ih and ow*sw - pw + kw == iw with (oh, ow) in range. */
void oracle_conv2d_backward_data_at(const double* dz, const double* w, const i64* idx, i64 count,
                                    double* out, i64 N, i64 H, i64 W, i64 IC, i64 OC, i64 KH, i64 KW,
                                    i64 sh, i64 sw, i64 ph, i64 pw) {
    (void)N; (void)H; (void)W;
    i64 OH = oracle_out_extent(H, KH, sh, ph), OW = oracle_out_extent(W, KW, sw, pw);
#pragma omp parallel for schedule(dynamic, 16)
    for (i64 i = 0; i < count; ++i) {
        i64 n = idx[4 * i], ih = idx[4 * i + 1], iw = idx[4 * i + 2], ic = idx[4 * i + 3];
        double acc = 0.0;
        for (i64 oc = 0; oc < OC; ++oc)
            for (i64 kh = 0; kh < KH; ++kh) {
                i64 th = ih + ph - kh;
                if (th < 0 || th % sh != 0 || th / sh >= OH) continue;
                for (i64 kw = 0; kw < KW; ++kw) {
                    i64 tw = iw + pw - kw;
                    if (tw < 0 || tw % sw != 0 || tw / sw >= OW) continue;
                    acc += w[((oc * KH + kh) * KW + kw) * IC + ic] *
                           dz[((n * OH + th / sh) * OW + tw / sw) * OC + oc];
                }
            }
        out[i] = acc;
    }
}

/* ---------------------------------------------- weight and bias gradients ---- */
/* dw[oc,kh,kw,ic] = sum_{n,oh,ow} dz[n,oh,ow,oc] * x[n, oh*sh-ph+kh, ow*sw-pw+kw, ic]
 * (out-of-range taps contribute zero);  db[oc] = sum_{n,oh,ow} dz[n,oh,ow,oc].
 * Written, not accumulated.  [generic] backward (weight and bias accumulators);
 * [wgsl] conv2d_backward_weight (per-element sum over output positions); [cuda]
 * bias_backward_partial/finalize.  db may be NULL. */
void oracle_conv2d_backward_weight(const double* x, const double* dz, double* dw, double* db,
                                   i64 N, i64 H, i64 W, i64 IC, i64 OC, i64 KH, i64 KW,
                                   i64 sh, i64 sw, i64 ph, i64 pw) {
    i64 OH = oracle_out_extent(H, KH, sh, ph), OW = oracle_out_extent(W, KW, sw, pw);
    i64 K = KH * KW * IC;
#pragma omp parallel for schedule(dynamic, 1)
    for (i64 oc = 0; oc < OC; ++oc) {
        double* row = dw + oc * K;
        for (i64 k = 0; k < K; ++k) row[k] = 0.0;
        double bsum = 0.0;
        for (i64 n = 0; n < N; ++n)
            for (i64 oh = 0; oh < OH; ++oh)
                for (i64 ow = 0; ow < OW; ++ow) {
                    double g = dz[((n * OH + oh) * OW + ow) * OC + oc];
                    bsum += g;
                    for (i64 kh = 0; kh < KH; ++kh) {
                        i64 ih = oh * sh - ph + kh;
                        if (ih < 0 || ih >= H) continue;
                        for (i64 kw = 0; kw < KW; ++kw) {
                            i64 iw = ow * sw - pw + kw;
                            if (iw < 0 || iw >= W) continue;
                            const double* xp = x + ((n * H + ih) * W + iw) * IC;
                            double* rp = row + (kh * KW + kw) * IC;
                            for (i64 ic = 0; ic < IC; ++ic) rp[ic] += g * xp[ic];
                        }
                    }
                }
        if (db) db[oc] = bsum;
    }
}

/* One dw element (oc, kh, kw, ic), same definition. */
void oracle_conv2d_backward_weight_at(const double* x, const double* dz, const i64* idx, i64 count,
                                      double* out, i64 N, i64 H, i64 W, i64 IC, i64 OC, i64 KH, i64 KW,
                                      i64 sh, i64 sw, i64 ph, i64 pw) {
    i64 OH = oracle_out_extent(H, KH, sh, ph), OW = oracle_out_extent(W, KW, sw, pw);
#pragma omp parallel for schedule(dynamic, 1)
    for (i64 i = 0; i < count; ++i) {
        i64 oc = idx[4 * i], kh = idx[4 * i + 1], kw = idx[4 * i + 2], ic = idx[4 * i + 3];
        double acc = 0.0;
        for (i64 n = 0; n < N; ++n)
            for (i64 oh = 0; oh < OH; ++oh) {
                i64 ih = oh * sh - ph + kh;
                if (ih < 0 || ih >= H) continue;
                for (i64 ow = 0; ow < OW; ++ow) {
                    i64 iw = ow * sw - pw + kw;
                    if (iw < 0 || iw >= W) continue;
                    acc += dz[((n * OH + oh) * OW + ow) * OC + oc] * x[((n * H + ih) * W + iw) * IC + ic];
                }
            }
        out[i] = acc;
    }
}

/* db alone: db[oc] = sum over all rows of dz. */
void oracle_bias_grad(const double* dz, i64 M, i64 C, double* db) {
#pragma omp parallel for schedule(static)
    for (i64 c = 0; c < C; ++c) {
        double s = 0.0;
        for (i64 m = 0; m < M; ++m) s += dz[m * C + c];
        db[c] = s;
    }
}
