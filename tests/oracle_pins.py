"""Pins for the fp64 oracle: each check ties an oracle routine to something other than
itself -- a library routine (scipy correlate2d, numpy matmul/mean/var, torch fp64 conv
and autograd), a closed form, an identity of the mathematics (adjoints, linearity,
translation equivariance, batch-norm invariants) or central finite differences.

Every check raises AssertionError on failure.  They are collected as tests in
test_oracle_pins.py and re-run against deliberately broken builds of oracle.c in
test_oracle_mutants.py, which shows each plausible mistake fails at least one pin.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F
from scipy import signal

import oracle as O

# (N, H, W, IC, OC, KH, KW, sh, sw, ph, pw): small shapes covering odd/even/rectangular
# kernels, strides 1-3, padding 0-2, kernels larger than stride, non-square inputs.
SMALL_SHAPES = [
    (2, 5, 6, 3, 4, 3, 3, 1, 1, 1, 1),
    (1, 7, 5, 2, 3, 2, 3, 2, 1, 0, 1),
    (2, 6, 6, 4, 2, 1, 1, 1, 1, 0, 0),
    (1, 9, 8, 2, 2, 4, 4, 2, 2, 0, 0),
    (2, 7, 7, 1, 3, 3, 2, 3, 2, 2, 1),
    (1, 8, 9, 3, 2, 5, 3, 1, 2, 2, 0),
    (2, 12, 12, 2, 3, 8, 8, 4, 4, 0, 0),
]


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_problem(shape, seed, bias=True):
    N, H, W, IC, OC, KH, KW, sh, sw, ph, pw = shape
    r = _rng(seed)
    x = r.uniform(-1, 1, (N, H, W, IC))
    w = r.uniform(-1, 1, (OC, KH, KW, IC))
    b = r.uniform(-1, 1, (OC,)) if bias else None
    return x, w, b, (sh, sw), (ph, pw)


def _torch_conv(x, w, b, stride, pad):
    xt = torch.from_numpy(x).permute(0, 3, 1, 2)
    wt = torch.from_numpy(w).permute(0, 3, 1, 2)
    bt = None if b is None else torch.from_numpy(b)
    y = F.conv2d(xt, wt, bt, stride=stride, padding=pad)
    return y.permute(0, 2, 3, 1).numpy()


def _close(a, b, rtol=1e-12, what=""):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= rtol * scale, f"{what}: max abs err {err:.3e} > {rtol:.1e} * {scale:.3e}"


# ---------------------------------------------------------------- forward
def pin_forward_vs_scipy():
    """Multi-channel cross-correlation = sum over ic of scipy correlate2d on the
    zero-padded plane, subsampled by the stride, plus the bias."""
    for i, sh_ in enumerate(SMALL_SHAPES):
        x, w, b, (sh, sw), (ph, pw) = _rand_problem(sh_, 100 + i)
        z = O.conv2d_forward(x, w, b, (sh, sw), (ph, pw))
        N, OC = x.shape[0], w.shape[0]
        ref = np.zeros_like(z)
        for n in range(N):
            for oc in range(OC):
                acc = None
                for ic in range(x.shape[3]):
                    plane = np.pad(x[n, :, :, ic], ((ph, ph), (pw, pw)))
                    full = signal.correlate2d(plane, w[oc, :, :, ic], mode="valid")
                    acc = full if acc is None else acc + full
                ref[n, :, :, oc] = acc[::sh, ::sw][: z.shape[1], : z.shape[2]] + b[oc]
        _close(z, ref, 1e-12, f"forward vs scipy {sh_}")


def pin_forward_vs_torch():
    for i, sh_ in enumerate(SMALL_SHAPES):
        x, w, b, st, pd = _rand_problem(sh_, 200 + i)
        _close(O.conv2d_forward(x, w, b, st, pd), _torch_conv(x, w, b, st, pd), 1e-12, f"fwd vs torch {sh_}")


def pin_forward_delta_kernel():
    """w[oc,kh,kw,ic] = [oc==ic][kh==p][kw==p] with K odd, s=1, p=(K-1)/2 reproduces x;
    with s=2 it returns x[:, ::2, ::2, :]."""
    r = _rng(3)
    for K in (1, 3, 5):
        p = (K - 1) // 2
        C = 3
        x = r.standard_normal((2, 7, 6, C))
        w = np.zeros((C, K, K, C))
        for c in range(C):
            w[c, p, p, c] = 1.0
        np.testing.assert_array_equal(O.conv2d_forward(x, w, None, (1, 1), (p, p)), x)
        np.testing.assert_array_equal(O.conv2d_forward(x, w, None, (2, 2), (p, p)), x[:, ::2, ::2, :])


def pin_forward_1x1_is_matmul():
    r = _rng(4)
    x = r.standard_normal((3, 5, 4, 6))
    w = r.standard_normal((7, 1, 1, 6))
    b = r.standard_normal(7)
    ref = (x.reshape(-1, 6) @ w.reshape(7, 6).T + b).reshape(3, 5, 4, 7)
    _close(O.conv2d_forward(x, w, b), ref, 1e-12, "1x1 matmul")


def pin_forward_constant_closed_form():
    """x = c, w = 1: z[n,oh,ow,oc] = b[oc] + c*IC*(#valid kh)*(#valid kw)."""
    for sh_ in SMALL_SHAPES:
        N, H, W, IC, OC, KH, KW, sh, sw, ph, pw = sh_
        c = 0.75
        b = np.arange(OC, dtype=float)
        z = O.conv2d_forward(np.full((N, H, W, IC), c), np.ones((OC, KH, KW, IC)), b, (sh, sw), (ph, pw))
        OH, OW = z.shape[1:3]
        for oh in range(OH):
            nh = sum(1 for kh in range(KH) if 0 <= oh * sh - ph + kh < H)
            for ow in range(OW):
                nw = sum(1 for kw in range(KW) if 0 <= ow * sw - pw + kw < W)
                np.testing.assert_allclose(z[:, oh, ow, :], np.broadcast_to(b + c * IC * nh * nw, (N, OC)),
                                           rtol=0, atol=1e-12)


def pin_forward_linearity_and_translation():
    r = _rng(5)
    x1, x2 = r.standard_normal((2, 2, 8, 9, 3))
    w1, w2 = r.standard_normal((2, 4, 3, 3, 3))
    a, c = 0.3, -1.7
    f = lambda x, w: O.conv2d_forward(x, w, None, (1, 1), (1, 1))
    _close(f(a * x1 + c * x2, w1), a * f(x1, w1) + c * f(x2, w1), 1e-12, "linear in x")
    _close(f(x1, a * w1 + c * w2), a * f(x1, w1) + c * f(x1, w2), 1e-12, "linear in w")
    # shifting the input by (1, 2) shifts interior outputs (no padding, stride 1)
    g = lambda x: O.conv2d_forward(x, w1, None, (1, 1), (0, 0))
    xs = np.zeros_like(x1)
    xs[:, 1:, 2:, :] = x1[:, :-1, :-2, :]
    y, ys = g(x1), g(xs)
    _close(ys[:, 1 + 2:, 2 + 2:, :], y[:, 2:-1, 2:-2, :], 1e-12, "translation")


def pin_forward_at_matches_full():
    for i, sh_ in enumerate(SMALL_SHAPES):
        x, w, b, st, pd = _rand_problem(sh_, 300 + i)
        z = O.conv2d_forward(x, w, b, st, pd)
        idx = np.array(list(np.ndindex(*z.shape)))
        np.testing.assert_array_equal(O.conv2d_forward_at(x, w, b, idx, st, pd), z.reshape(-1))


# ---------------------------------------------------------------- dX, dW, db
def pin_adjoint_identities():
    """<conv(x,w), dy> = <x, dX(dy)> = <w, dW(x,dy)> (bias 0); <1, dy> summed per oc = db."""
    for i, sh_ in enumerate(SMALL_SHAPES):
        x, w, _, st, pd = _rand_problem(sh_, 400 + i, bias=False)
        z = O.conv2d_forward(x, w, None, st, pd)
        dy = _rng(500 + i).standard_normal(z.shape)
        dx = O.conv2d_backward_data(dy, w, x.shape, st, pd)
        dw, db = O.conv2d_backward_weight(x, dy, w.shape, st, pd)
        lhs = float(np.sum(z * dy))
        for rhs, what in ((float(np.sum(x * dx)), "dX"), (float(np.sum(w * dw)), "dW")):
            assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs)) * 10, (sh_, what, lhs, rhs)
        np.testing.assert_allclose(db, dy.reshape(-1, w.shape[0]).sum(0), rtol=1e-12, atol=1e-12)


def pin_backward_vs_torch_autograd():
    for i, sh_ in enumerate(SMALL_SHAPES):
        x, w, b, st, pd = _rand_problem(sh_, 600 + i)
        xt = torch.from_numpy(x).permute(0, 3, 1, 2).clone().requires_grad_(True)
        wt = torch.from_numpy(w).permute(0, 3, 1, 2).clone().requires_grad_(True)
        bt = torch.from_numpy(b).clone().requires_grad_(True)
        y = F.conv2d(xt, wt, bt, stride=st, padding=pd)
        dy = _rng(700 + i).standard_normal(y.shape)
        y.backward(torch.from_numpy(dy))
        dy_nhwc = np.ascontiguousarray(dy.transpose(0, 2, 3, 1))
        _close(O.conv2d_backward_data(dy_nhwc, w, x.shape, st, pd),
               xt.grad.permute(0, 2, 3, 1).numpy(), 1e-12, f"dX vs torch {sh_}")
        dw, db = O.conv2d_backward_weight(x, dy_nhwc, w.shape, st, pd)
        _close(dw, wt.grad.permute(0, 2, 3, 1).numpy(), 1e-12, f"dW vs torch {sh_}")
        _close(db, bt.grad.numpy(), 1e-12, f"db vs torch {sh_}")


def pin_backward_finite_differences():
    """L(x, w, b) = <conv(x,w)+b, dy> is linear in each argument, so central
    differences are exact up to rounding."""
    sh_ = (1, 6, 5, 2, 3, 3, 2, 2, 1, 1, 0)
    x, w, b, st, pd = _rand_problem(sh_, 8)
    dy = _rng(9).standard_normal(O.conv2d_forward(x, w, b, st, pd).shape)
    L = lambda x_, w_, b_: float(np.sum(O.conv2d_forward(x_, w_, b_, st, pd) * dy))
    dx = O.conv2d_backward_data(dy, w, x.shape, st, pd)
    dw, db = O.conv2d_backward_weight(x, dy, w.shape, st, pd)
    h = 1e-3
    for idx in np.ndindex(*x.shape):
        e = np.zeros_like(x); e[idx] = h
        fd = (L(x + e, w, b) - L(x - e, w, b)) / (2 * h)
        assert abs(fd - dx[idx]) < 1e-9, ("dx", idx, fd, dx[idx])
    for idx in np.ndindex(*w.shape):
        e = np.zeros_like(w); e[idx] = h
        fd = (L(x, w + e, b) - L(x, w - e, b)) / (2 * h)
        assert abs(fd - dw[idx]) < 1e-9, ("dw", idx, fd, dw[idx])
    for oc in range(len(b)):
        e = np.zeros_like(b); e[oc] = h
        fd = (L(x, w, b + e) - L(x, w, b - e)) / (2 * h)
        assert abs(fd - db[oc]) < 1e-9, ("db", oc, fd, db[oc])


def pin_backward_closed_forms():
    """dY = 1, x = 1: dW[oc,kh,kw,ic] = N*cnt_h(kh)*cnt_w(kw) where cnt counts outputs
    whose tap kh lands inside; db = N*OH*OW.  dY = 1, w = 1: dX = OC*(#covering taps)."""
    for sh_ in SMALL_SHAPES:
        N, H, W, IC, OC, KH, KW, sh, sw, ph, pw = sh_
        OH, OW = O.out_extent(H, KH, sh, ph), O.out_extent(W, KW, sw, pw)
        dy = np.ones((N, OH, OW, OC))
        dw, db = O.conv2d_backward_weight(np.ones((N, H, W, IC)), dy, (OC, KH, KW, IC), (sh, sw), (ph, pw))
        for kh in range(KH):
            ch = sum(1 for oh in range(OH) if 0 <= oh * sh - ph + kh < H)
            for kw in range(KW):
                cw = sum(1 for ow in range(OW) if 0 <= ow * sw - pw + kw < W)
                np.testing.assert_array_equal(dw[:, kh, kw, :], N * ch * cw)
        np.testing.assert_array_equal(db, N * OH * OW)
        dx = O.conv2d_backward_data(dy, np.ones((OC, KH, KW, IC)), (N, H, W, IC), (sh, sw), (ph, pw))
        for ih in range(H):
            th = sum(1 for oh in range(OH) for kh in range(KH) if oh * sh - ph + kh == ih)
            for iw in range(W):
                tw = sum(1 for ow in range(OW) for kw in range(KW) if ow * sw - pw + kw == iw)
                np.testing.assert_array_equal(dx[:, ih, iw, :], OC * th * tw)


def pin_backward_at_matches_full():
    for i, sh_ in enumerate(SMALL_SHAPES):
        x, w, _, st, pd = _rand_problem(sh_, 800 + i, bias=False)
        dy = _rng(900 + i).standard_normal(O.conv2d_forward(x, w, None, st, pd).shape)
        dx = O.conv2d_backward_data(dy, w, x.shape, st, pd)
        idx = np.array(list(np.ndindex(*x.shape)))
        _close(O.conv2d_backward_data_at(dy, w, x.shape, idx, st, pd), dx.reshape(-1), 1e-12, "dx_at")
        dw, db = O.conv2d_backward_weight(x, dy, w.shape, st, pd)
        idx = np.array(list(np.ndindex(*w.shape)))
        _close(O.conv2d_backward_weight_at(x, dy, w.shape, idx, st, pd), dw.reshape(-1), 1e-12, "dw_at")
        _close(O.bias_grad(dy), db, 1e-12, "bias_grad")


# ---------------------------------------------------------------- batch norm
def pin_bn_stats_vs_numpy():
    r = _rng(10)
    z = r.standard_normal((3, 5, 4, 6)) * r.uniform(0.1, 3, 6) + r.uniform(-2, 2, 6)
    rm0, rv0 = r.standard_normal(6), r.uniform(0.5, 2, 6)
    mom, eps = 0.1, 1e-5
    mean, var, inv, rm, rv = O.bn_stats(z, mom, eps, rm0, rv0)
    flat = z.reshape(-1, 6)
    _close(mean, flat.mean(0), 1e-13, "mean")
    _close(var, flat.var(0, ddof=0), 1e-13, "biased var")
    _close(inv, 1.0 / np.sqrt(flat.var(0) + eps), 1e-13, "inv_std")
    _close(rm, 0.9 * rm0 + 0.1 * flat.mean(0), 1e-13, "running mean")
    _close(rv, 0.9 * rv0 + 0.1 * flat.var(0), 1e-13, "running var (biased, as on the pages)")


def pin_bn_stats_special_cases():
    eps = 1e-5
    z = np.full((4, 3, 3, 2), 2.5)
    mean, var, inv, rm, rv = O.bn_stats(z, 0.1, eps, np.zeros(2), np.ones(2))
    np.testing.assert_array_equal(mean, 2.5)
    np.testing.assert_array_equal(var, 0.0)
    np.testing.assert_allclose(inv, 316.22776601683796, rtol=1e-14)
    np.testing.assert_allclose(rm, 0.25, rtol=1e-15)
    np.testing.assert_allclose(rv, 0.9, rtol=1e-15)
    a = 1.7
    z = np.empty((2, 1, 5, 1)); z[0] = -a; z[1] = a
    mean, var, *_ = O.bn_stats(z, 0.1, eps)
    np.testing.assert_allclose(mean, 0.0, atol=1e-15)
    np.testing.assert_allclose(var, a * a, rtol=1e-14)


def pin_bn_apply_normalises():
    """Identity activation, gamma=1, beta=0: per channel mean 0 and variance
    var/(var+eps); with general gamma/beta, matches torch batch_norm (training) in fp64."""
    r = _rng(11)
    z = r.standard_normal((4, 6, 5, 3)) * np.array([0.5, 2.0, 7.0]) + np.array([1.0, -3.0, 0.2])
    mean, var, inv, *_ = O.bn_stats(z, 0.1, 1e-5)
    y = O.apply_activation(z, O.ACT_IDENTITY, O.NORM_BATCH, np.ones(3), np.zeros(3), mean, inv)
    flat = y.reshape(-1, 3)
    np.testing.assert_allclose(flat.mean(0), 0.0, atol=1e-13)
    np.testing.assert_allclose(flat.var(0), var / (var + 1e-5), rtol=1e-12)
    g, bt = r.uniform(0.5, 1.5, 3), r.normal(0, 0.1, 3)
    zt = torch.from_numpy(z).permute(0, 3, 1, 2)
    for act, fn in ((O.ACT_IDENTITY, lambda t: t), (O.ACT_RELU, torch.relu), (O.ACT_TANH, torch.tanh),
                    (O.ACT_SIGMOID, torch.sigmoid)):
        ref = fn(F.batch_norm(zt, None, None, torch.from_numpy(g), torch.from_numpy(bt), training=True,
                              eps=1e-5)).permute(0, 2, 3, 1).numpy()
        _close(O.apply_activation(z, act, O.NORM_BATCH, g, bt, mean, inv), ref, 1e-12, f"bn apply act {act}")


def pin_activation_values():
    a = np.linspace(-6, 6, 121).reshape(1, 11, 11, 1)
    _close(O.apply_activation(a, O.ACT_IDENTITY), a, 0, "identity")
    _close(O.apply_activation(a, O.ACT_RELU), np.maximum(a, 0), 0, "relu")
    _close(O.apply_activation(a, O.ACT_TANH), np.tanh(a), 1e-15, "tanh")
    _close(O.apply_activation(a, O.ACT_SIGMOID), 0.5 * (1 + np.tanh(a / 2)), 1e-15, "sigmoid")


# ---------------------------------------------------------------- activation backward
def pin_act_backward_no_norm():
    """dz = act'(z)*dy against torch fp64 autograd; tanh' = 1 - tanh^2 identity."""
    r = _rng(12)
    z = r.standard_normal((2, 4, 5, 3)) * 2
    dy = r.standard_normal(z.shape)
    for act, fn in ((O.ACT_IDENTITY, lambda t: t), (O.ACT_RELU, torch.relu), (O.ACT_TANH, torch.tanh),
                    (O.ACT_SIGMOID, torch.sigmoid)):
        zt = torch.from_numpy(z).clone().requires_grad_(True)
        fn(zt).backward(torch.from_numpy(dy))
        dz, dg, dbt = O.activation_backward(z, dy, act)
        assert dg is None and dbt is None
        _close(dz, zt.grad.numpy(), 1e-13, f"act bwd {act}")
    dz, *_ = O.activation_backward(z, dy, O.ACT_TANH)
    _close(dz, (1 - np.tanh(z) ** 2) * dy, 1e-14, "tanh identity")
    np.testing.assert_array_equal(O.activation_backward(np.zeros((1, 1, 1, 1)), np.ones((1, 1, 1, 1)),
                                                        O.ACT_RELU)[0], 0.0)


def _bn_problem(seed, shape=(3, 5, 4, 4)):
    r = _rng(seed)
    C = shape[-1]
    z = r.standard_normal(shape) * r.uniform(0.3, 3, C) + r.uniform(-1, 1, C)
    g, bt = r.uniform(0.5, 1.5, C), r.normal(0, 0.3, C)
    dy = r.standard_normal(shape)
    return z, g, bt, dy


def pin_bn_backward_vs_torch_autograd():
    """BN(train) + act backward: dz, dgamma, dbeta against torch fp64 autograd."""
    for act, fn in ((O.ACT_IDENTITY, lambda t: t), (O.ACT_RELU, torch.relu), (O.ACT_TANH, torch.tanh),
                    (O.ACT_SIGMOID, torch.sigmoid)):
        z, g, bt, dy = _bn_problem(13 + act)
        mean, _, inv, *_ = O.bn_stats(z, 0.1, 1e-5)
        dz, dg, dbt = O.activation_backward(z, dy, act, O.NORM_BATCH, g, bt, mean, inv)
        zt = torch.from_numpy(z).permute(0, 3, 1, 2).clone().requires_grad_(True)
        gt = torch.from_numpy(g).clone().requires_grad_(True)
        btt = torch.from_numpy(bt).clone().requires_grad_(True)
        y = fn(F.batch_norm(zt, None, None, gt, btt, training=True, eps=1e-5))
        y.backward(torch.from_numpy(dy).permute(0, 3, 1, 2))
        _close(dz, zt.grad.permute(0, 2, 3, 1).numpy(), 1e-11, f"bn dz act {act}")
        _close(dg, gt.grad.numpy(), 1e-11, f"dgamma act {act}")
        _close(dbt, btt.grad.numpy(), 1e-11, f"dbeta act {act}")


def pin_bn_backward_invariants_and_fd():
    """Per channel sum dz = 0, and with eps = 0 also sum dz*zhat = 0 (dz is the
    projection removing the directions BN is invariant to; with eps > 0 the second sum is
    inv_std*S2*eps/(var+eps)); central differences of L(z, gamma, beta) =
    <act(BN(z)), dy> (stats recomputed from z) match dz, dgamma, dbeta."""
    act = O.ACT_SIGMOID
    z, g, bt, dy = _bn_problem(21, (2, 3, 3, 3))
    mean, _, inv, *_ = O.bn_stats(z, 0.1, 0.0)
    dz, dg, dbt = O.activation_backward(z, dy, act, O.NORM_BATCH, g, bt, mean, inv)
    flat, zh = dz.reshape(-1, 3), ((z - mean) * inv).reshape(-1, 3)
    np.testing.assert_allclose(flat.sum(0), 0.0, atol=1e-12)
    np.testing.assert_allclose((flat * zh).sum(0), 0.0, atol=1e-12)
    mean, _, inv, *_ = O.bn_stats(z, 0.1, 1e-5)
    dz, dg, dbt = O.activation_backward(z, dy, act, O.NORM_BATCH, g, bt, mean, inv)
    np.testing.assert_allclose(dz.reshape(-1, 3).sum(0), 0.0, atol=1e-12)

    def L(z_, g_, b_):
        m_, _, i_, *_ = O.bn_stats(z_, 0.1, 1e-5)
        return float(np.sum(O.apply_activation(z_, act, O.NORM_BATCH, g_, b_, m_, i_) * dy))

    h = 1e-6
    for idx in np.ndindex(*z.shape):
        e = np.zeros_like(z); e[idx] = h
        fd = (L(z + e, g, bt) - L(z - e, g, bt)) / (2 * h)
        assert abs(fd - dz[idx]) < 1e-7, ("dz", idx, fd, dz[idx])
    for c in range(3):
        e = np.zeros(3); e[c] = h
        assert abs((L(z, g + e, bt) - L(z, g - e, bt)) / (2 * h) - dg[c]) < 1e-7, ("dgamma", c)
        assert abs((L(z, g, bt + e) - L(z, g, bt - e)) / (2 * h) - dbt[c]) < 1e-7, ("dbeta", c)


def pin_bn_bias_invariance():
    """A per-channel shift of z (a conv bias) leaves the BN output and dz unchanged."""
    z, g, bt, dy = _bn_problem(22)
    shift = np.array([3.0, -1.0, 0.5, 10.0])
    for zz in (z, z + shift):
        mean, _, inv, *_ = O.bn_stats(zz, 0.1, 1e-5)
        y = O.apply_activation(zz, O.ACT_TANH, O.NORM_BATCH, g, bt, mean, inv)
        dz, *_ = O.activation_backward(zz, dy, O.ACT_TANH, O.NORM_BATCH, g, bt, mean, inv)
        if zz is z:
            y0, dz0 = y, dz
    _close(y, y0, 1e-12, "bias invariance y")
    _close(dz, dz0, 1e-10, "bias invariance dz")


def _eval_running(C, seed):
    r = _rng(seed)
    return r.normal(0, 0.5, C), r.uniform(0.2, 3.0, C)


def pin_bn_eval_stats_closed_form():
    """Evaluation-mode statistics: mean passes the running mean through; running_var =
    1 - eps gives inv_std = 1 exactly, running_var = 4 - eps gives 1/2, and in general
    inv_std**2 * (running_var + eps) = 1."""
    eps = 1e-5
    rm = np.array([0.25, -3.0, 7.5, 0.0])
    rv = np.array([1.0 - eps, 4.0 - eps, 0.5, 9.0])
    mean, inv = O.bn_eval_stats(rm, rv, eps)
    np.testing.assert_array_equal(mean, rm)
    assert inv[0] == 1.0 and inv[1] == 0.5
    _close(inv ** 2 * (rv + eps), np.ones(4), 1e-15, "inv_std^2 (var + eps)")


def pin_bn_eval_forward_matches_training_forward():
    """With running statistics equal to the batch statistics of z (var biased, as the
    training statistics), the evaluation forward reproduces the training forward."""
    z, g, bt, _ = _bn_problem(31)
    mean, var, inv, *_ = O.bn_stats(z, 0.1, 1e-5)
    em, ei = O.bn_eval_stats(mean, var, 1e-5)
    for act in (O.ACT_IDENTITY, O.ACT_RELU, O.ACT_TANH, O.ACT_SIGMOID):
        yt = O.apply_activation(z, act, O.NORM_BATCH, g, bt, mean, inv)
        ye = O.apply_activation(z, act, O.NORM_BATCH, g, bt, em, ei)
        _close(ye, yt, 1e-14, f"eval forward act {act}")


def pin_bn_eval_backward_vs_torch_autograd():
    """Evaluation-mode BN + act backward: dz, dgamma, dbeta against torch fp64 autograd
    through batch_norm(training=False) with the running statistics."""
    for act, fn in ((O.ACT_IDENTITY, lambda t: t), (O.ACT_RELU, torch.relu), (O.ACT_TANH, torch.tanh),
                    (O.ACT_SIGMOID, torch.sigmoid)):
        z, g, bt, dy = _bn_problem(41 + act)
        rm, rv = _eval_running(z.shape[-1], 45 + act)
        mean, inv = O.bn_eval_stats(rm, rv, 1e-5)
        dz, dg, dbt = O.activation_backward(z, dy, act, O.NORM_BATCH, g, bt, mean, inv, evaluation=True)
        zt = torch.from_numpy(z).permute(0, 3, 1, 2).clone().requires_grad_(True)
        gt = torch.from_numpy(g).clone().requires_grad_(True)
        btt = torch.from_numpy(bt).clone().requires_grad_(True)
        y = fn(F.batch_norm(zt, torch.from_numpy(rm), torch.from_numpy(rv), gt, btt, training=False, eps=1e-5))
        y.backward(torch.from_numpy(dy).permute(0, 3, 1, 2))
        _close(dz, zt.grad.permute(0, 2, 3, 1).numpy(), 1e-11, f"eval dz act {act}")
        _close(dg, gt.grad.numpy(), 1e-11, f"eval dgamma act {act}")
        _close(dbt, btt.grad.numpy(), 1e-11, f"eval dbeta act {act}")


def pin_bn_eval_backward_fd_and_closed_form():
    """Central differences of L(z, gamma, beta) = <act(gamma*(z - m)*s + beta), dy> with
    fixed (m, s) match dz, dgamma, dbeta; with gamma = 1, identity activation and s = 1
    the backward passes dy through: dz = dy, dbeta = sum dy, dgamma = sum dy*(z - m)."""
    act = O.ACT_TANH
    z, g, bt, dy = _bn_problem(51, (2, 3, 3, 3))
    rm, rv = _eval_running(3, 52)
    mean, inv = O.bn_eval_stats(rm, rv, 1e-5)
    dz, dg, dbt = O.activation_backward(z, dy, act, O.NORM_BATCH, g, bt, mean, inv, evaluation=True)

    def L(z_, g_, b_):
        return float(np.sum(O.apply_activation(z_, act, O.NORM_BATCH, g_, b_, mean, inv) * dy))

    h = 1e-6
    for idx in np.ndindex(*z.shape):
        e = np.zeros_like(z); e[idx] = h
        fd = (L(z + e, g, bt) - L(z - e, g, bt)) / (2 * h)
        assert abs(fd - dz[idx]) < 1e-7, ("eval dz", idx, fd, dz[idx])
    for c in range(3):
        e = np.zeros(3); e[c] = h
        assert abs((L(z, g + e, bt) - L(z, g - e, bt)) / (2 * h) - dg[c]) < 1e-7, ("eval dgamma", c)
        assert abs((L(z, g, bt + e) - L(z, g, bt - e)) / (2 * h) - dbt[c]) < 1e-7, ("eval dbeta", c)
    ones, one_inv = np.ones(3), np.ones(3)
    dz1, dg1, db1 = O.activation_backward(z, dy, O.ACT_IDENTITY, O.NORM_BATCH, ones, bt, rm, one_inv,
                                          evaluation=True)
    np.testing.assert_array_equal(dz1, dy)
    _close(db1, dy.reshape(-1, 3).sum(0), 1e-14, "eval dbeta closed form")
    _close(dg1, (dy * (z - rm)).reshape(-1, 3).sum(0), 1e-13, "eval dgamma closed form")


def pin_act_backward_from_output():
    """The output form of the derivative equals the pre-activation form on y = act(z)
    (relu mask, 1 - tanh^2, sigmoid (1 - sigmoid)), and torch fp64 autograd; GELU, whose
    derivative is not a function of its output, is refused."""
    r = _rng(19)
    z = r.standard_normal((2, 5, 4, 3)) * 2
    dy = r.standard_normal(z.shape)
    for act in (O.ACT_IDENTITY, O.ACT_RELU, O.ACT_TANH, O.ACT_SIGMOID):
        y = O.apply_activation(z, act)
        _close(O.activation_backward_from_output(y, dy, act), O.activation_backward(z, dy, act)[0], 1e-14,
               f"output-form derivative act {act}")
    y = np.tanh(z)
    _close(O.activation_backward_from_output(y, dy, O.ACT_TANH), (1 - y * y) * dy, 0, "tanh closed form")
    try:
        O.activation_backward_from_output(z, dy, O.ACT_GELU)
        raise AssertionError("GELU output form accepted")
    except ValueError:
        pass


# ---------------------------------------------------------------- GELU (tanh form)
def pin_gelu_values_and_slope():
    """gelu against torch's tanh-form GELU in fp64 (values, autograd slope); closed forms
    gelu(0) = 0, gelu'(0) = 1/2; far tails: gelu(a) -> a and slope -> 1 for a >> 0,
    gelu(a) -> 0 and slope -> 0 for a << 0."""
    a = np.linspace(-7, 7, 141).reshape(1, 141, 1, 1)
    at = torch.from_numpy(a).clone().requires_grad_(True)
    ref = F.gelu(at, approximate="tanh")
    _close(O.apply_activation(a, O.ACT_GELU), ref.detach().numpy(), 1e-15, "gelu values")
    dy = _rng(60).standard_normal(a.shape)
    ref.backward(torch.from_numpy(dy))
    dz, *_ = O.activation_backward(a, dy, O.ACT_GELU)
    _close(dz, at.grad.numpy(), 1e-14, "gelu slope")
    one = np.ones((1, 1, 1, 1))
    assert O.apply_activation(0 * one, O.ACT_GELU)[0, 0, 0, 0] == 0.0
    assert abs(O.activation_backward(0 * one, one, O.ACT_GELU)[0][0, 0, 0, 0] - 0.5) < 1e-16
    big = np.array([8.0, 12.0, -8.0, -12.0]).reshape(1, 4, 1, 1)
    np.testing.assert_allclose(O.apply_activation(big, O.ACT_GELU).ravel(), [8.0, 12.0, 0.0, 0.0], atol=1e-12)
    np.testing.assert_allclose(O.activation_backward(big, np.ones_like(big), O.ACT_GELU)[0].ravel(),
                               [1.0, 1.0, 0.0, 0.0], atol=1e-12)


def pin_gelu_slope_finite_differences():
    a = np.linspace(-4, 4, 33).reshape(1, 33, 1, 1)
    h = 1e-6
    fd = (O.apply_activation(a + h, O.ACT_GELU) - O.apply_activation(a - h, O.ACT_GELU)) / (2 * h)
    dz, *_ = O.activation_backward(a, np.ones_like(a), O.ACT_GELU)
    _close(dz, fd, 1e-8, "gelu slope vs central differences")


# ---------------------------------------------------------------- layer norm / group norm
ACT_FNS = ((O.ACT_IDENTITY, lambda t: t), (O.ACT_RELU, torch.relu), (O.ACT_TANH, torch.tanh),
           (O.ACT_SIGMOID, torch.sigmoid), (O.ACT_GELU, lambda t: F.gelu(t, approximate="tanh")))


def _gn_problem(seed, shape=(3, 4, 5, 6)):
    r = _rng(seed)
    C = shape[-1]
    z = r.standard_normal(shape) * r.uniform(0.3, 3, C) + r.uniform(-1, 1, C)
    z += r.uniform(-2, 2, (shape[0], 1, 1, 1))  # per-sample offsets
    g, bt = r.uniform(0.5, 1.5, C), r.normal(0, 0.3, C)
    dy = r.standard_normal(shape)
    return z, g, bt, dy


def pin_group_stats_vs_numpy():
    """Per (sample, group) mean / biased var / inv_std against numpy on the reshaped
    tensor; layer norm (one group) over each sample's whole OH*OW*C block."""
    z, *_ = _gn_problem(61)
    N, C = z.shape[0], z.shape[-1]
    for G in (1, 2, 3, 6):
        mean, var, inv = O.group_stats(z, G, 1e-5)
        blk = z.reshape(N, -1, G, C // G).transpose(0, 2, 1, 3).reshape(N, G, -1)
        _close(mean, blk.mean(-1), 1e-13, f"group mean G={G}")
        _close(var, blk.var(-1, ddof=0), 1e-13, f"group var G={G}")
        _close(inv, 1.0 / np.sqrt(blk.var(-1) + 1e-5), 1e-13, f"group inv_std G={G}")
    mean, var, _ = O.group_stats(z, 1)
    _close(mean[:, 0], z.reshape(N, -1).mean(1), 1e-13, "layer-norm mean")
    _close(var[:, 0], z.reshape(N, -1).var(1), 1e-13, "layer-norm var")


def pin_group_stats_one_channel_groups_are_batch_stats_per_sample():
    """With one channel per group (G = C) the statistics of sample n are the batch-norm
    statistics of that sample alone (another oracle routine, pinned on its own)."""
    z, *_ = _gn_problem(62)
    C = z.shape[-1]
    mean, var, inv = O.group_stats(z, C, 1e-5)
    for n in range(z.shape[0]):
        bm, bv, bi, *_ = O.bn_stats(z[n:n + 1], 0.1, 1e-5)
        _close(mean[n], bm, 1e-13, "G=C mean")
        _close(var[n], bv, 1e-13, "G=C var")
        _close(inv[n], bi, 1e-13, "G=C inv_std")


def pin_group_norm_forward_vs_torch():
    """y against torch fp64 group_norm (per-channel affine) + activation; layer norm also
    against layer_norm over (C, H, W) with the per-channel affine applied after."""
    z, g, bt, _ = _gn_problem(63)
    zt = torch.from_numpy(z).permute(0, 3, 1, 2)
    for G in (1, 2, 6):
        mean, _, inv = O.group_stats(z, G, 1e-5)
        for act, fn in ACT_FNS:
            ref = fn(F.group_norm(zt, G, torch.from_numpy(g), torch.from_numpy(bt), eps=1e-5))
            _close(O.apply_group_norm(z, act, g, bt, mean, inv), ref.permute(0, 2, 3, 1).numpy(), 1e-12,
                   f"group norm G={G} act {act}")
    mean, _, inv = O.group_stats(z, 1, 1e-5)
    ln = F.layer_norm(zt, zt.shape[1:], eps=1e-5) * torch.from_numpy(g)[:, None, None] + \
        torch.from_numpy(bt)[:, None, None]
    _close(O.apply_group_norm(z, O.ACT_IDENTITY, g, bt, mean, inv), ln.permute(0, 2, 3, 1).numpy(), 1e-12,
           "layer norm vs torch layer_norm")


def pin_group_norm_normalises():
    """Identity activation, gamma = 1, beta = 0: each (sample, group) block has mean 0 and
    variance var/(var + eps)."""
    z, *_ = _gn_problem(64)
    N, C = z.shape[0], z.shape[-1]
    for G in (1, 3):
        mean, var, inv = O.group_stats(z, G, 1e-5)
        y = O.apply_group_norm(z, O.ACT_IDENTITY, np.ones(C), np.zeros(C), mean, inv)
        blk = y.reshape(N, -1, G, C // G).transpose(0, 2, 1, 3).reshape(N, G, -1)
        np.testing.assert_allclose(blk.mean(-1), 0.0, atol=1e-13)
        np.testing.assert_allclose(blk.var(-1), var / (var + 1e-5), rtol=1e-12)


def pin_group_norm_backward_vs_torch_autograd():
    """dz, dgamma, dbeta against torch fp64 autograd through group_norm + activation."""
    for G in (1, 2, 6):
        for act, fn in ACT_FNS:
            z, g, bt, dy = _gn_problem(70 + 7 * G + act)
            mean, _, inv = O.group_stats(z, G, 1e-5)
            dz, dg, dbt = O.group_norm_backward(z, dy, act, g, bt, mean, inv)
            zt = torch.from_numpy(z).permute(0, 3, 1, 2).clone().requires_grad_(True)
            gt = torch.from_numpy(g).clone().requires_grad_(True)
            btt = torch.from_numpy(bt).clone().requires_grad_(True)
            fn(F.group_norm(zt, G, gt, btt, eps=1e-5)).backward(torch.from_numpy(dy).permute(0, 3, 1, 2))
            _close(dz, zt.grad.permute(0, 2, 3, 1).numpy(), 1e-11, f"gn dz G={G} act {act}")
            _close(dg, gt.grad.numpy(), 1e-11, f"gn dgamma G={G} act {act}")
            _close(dbt, btt.grad.numpy(), 1e-11, f"gn dbeta G={G} act {act}")


def pin_group_norm_backward_fd_and_invariants():
    """Central differences of L(z, gamma, beta) = <act(GN(z)), dy> (statistics recomputed
    from z) match dz, dgamma, dbeta; per (sample, group) sum dz = 0."""
    act, G = O.ACT_GELU, 2
    z, g, bt, dy = _gn_problem(90, (2, 2, 3, 4))
    mean, _, inv = O.group_stats(z, G, 1e-5)
    dz, dg, dbt = O.group_norm_backward(z, dy, act, g, bt, mean, inv)
    blk = dz.reshape(2, -1, G, 2).transpose(0, 2, 1, 3).reshape(2, G, -1)
    np.testing.assert_allclose(blk.sum(-1), 0.0, atol=1e-12)

    def L(z_, g_, b_):
        m_, _, i_ = O.group_stats(z_, G, 1e-5)
        return float(np.sum(O.apply_group_norm(z_, act, g_, b_, m_, i_) * dy))

    h = 1e-6
    for idx in np.ndindex(*z.shape):
        e = np.zeros_like(z); e[idx] = h
        fd = (L(z + e, g, bt) - L(z - e, g, bt)) / (2 * h)
        assert abs(fd - dz[idx]) < 1e-7, ("gn dz", idx, fd, dz[idx])
    for c in range(4):
        e = np.zeros(4); e[c] = h
        assert abs((L(z, g + e, bt) - L(z, g - e, bt)) / (2 * h) - dg[c]) < 1e-7, ("gn dgamma", c)
        assert abs((L(z, g, bt + e) - L(z, g, bt - e)) / (2 * h) - dbt[c]) < 1e-7, ("gn dbeta", c)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
