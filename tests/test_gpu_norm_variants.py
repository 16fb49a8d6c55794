"""GPU parity of the normalisation and activation variants: GELU (tanh form), layer norm
and group norm, through the C ABI against the fp64 oracle on the same seeded inputs.

Layer norm takes per-sample statistics over OH*OW*OC values ([generic] layer-norm
branches); group norm per sample and group of consecutive channels ([doppler]
groupnorm_backward); GELU as [doppler] gelu_backward differentiates it.  Shapes cover
the three forward paths (stride-1 input-tile kernels with the statistics reduced in the
epilogue, the strided implicit GEMM, the direct kernel), one group, several groups and
one channel per group, ragged channel groups against the 16-byte vectors, fp32 and bf16.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from tests import gpu_harness as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import convolution_layer_amd  # noqa: F401


ACTN = {WL.ACT_IDENTITY: "id", WL.ACT_RELU: "relu", WL.ACT_TANH: "tanh", WL.ACT_SIGMOID: "sigm", WL.ACT_GELU: "gelu"}

GELU_CASES = [
    ((2, 15, 15, 128, 128, 3, 3, 1, 1, 1, 1), WL.BF16),  # stride-1 input-tile kernel, epilogue GELU
    ((2, 13, 11, 64, 64, 3, 3, 1, 1, 1, 1), WL.F32),
    ((2, 20, 20, 32, 64, 4, 4, 2, 2, 0, 0), WL.F32),     # strided implicit GEMM
    ((2, 10, 12, 3, 8, 3, 3, 1, 1, 1, 1), WL.F32),       # direct kernel
    ((1, 9, 7, 8, 24, 3, 3, 2, 1, 1, 0), WL.BF16),
]


def _ids(c):
    s = c[0]
    return f"{'x'.join(map(str, s[:7]))}_s{s[7]}{s[8]}_{c[1]}" + (f"_{c[2]}" if len(c) > 2 else "")


def _problem(s, dt, seed):
    shape = WL.ConvShape(*s)
    x = WL.random_tensor(shape.x_shape, dt, seed, ("normal", 0.0, 1.0))
    w = WL.random_tensor(shape.w_shape, dt, seed + 1, ("normal", 0.0, (2.0 / shape.Kdim) ** 0.5))
    b = WL.random_tensor((shape.OC,), WL.F32, seed + 2, ("uniform", -0.5, 0.5))
    dy = WL.random_tensor(shape.y_shape, dt, seed + 3, ("normal", 0.0, 1.0))
    return shape, x, w, b, dy


@pytest.mark.parametrize("case", GELU_CASES, ids=_ids)
def test_gelu_forward_and_backward(case):
    s, dt = case
    shape, x, w, b, dy = _problem(s, dt, 200)
    desc = G.shape_desc(shape, dt, WL.ACT_GELU)
    out = G.run_forward(desc, dt, G.dev(x, dt), G.dev(w, dt), G.dev(b))
    z_r = O.conv2d_forward(x, w, b, (shape.sh, shape.sw), (shape.ph, shape.pw))
    G.assert_close(G.host(out["z"]), z_r, dt, "gelu z")
    zs = WL.round_to(dt, z_r)
    G.assert_close(G.host(out["y"]), O.apply_activation(zs, WL.ACT_GELU), dt, "gelu y")
    z2 = WL.random_tensor(shape.y_shape, dt, 205, ("normal", 0.0, 2.5))
    dz, _, _ = G.run_act_bwd(desc, dt, G.dev(z2, dt), G.dev(dy, dt))
    G.assert_close(G.host(dz), O.activation_backward(z2, dy, WL.ACT_GELU)[0], dt, "gelu dz")


# (shape, dtype, groups (1 = layer norm), activation)
NORM_CASES = [
    ((2, 15, 17, 64, 72, 3, 3, 1, 1, 1, 1), WL.BF16, 1, WL.ACT_GELU),     # epilogue statistics, bf16
    ((2, 15, 17, 64, 72, 3, 3, 1, 1, 1, 1), WL.BF16, 12, WL.ACT_TANH),    # 6-channel groups over 8-wide vectors
    ((3, 30, 9, 128, 64, 3, 3, 1, 1, 1, 1), WL.BF16, 64, WL.ACT_RELU),    # one channel per group
    ((2, 13, 11, 64, 64, 3, 3, 1, 1, 1, 1), WL.F32, 1, WL.ACT_RELU),
    ((2, 13, 11, 64, 64, 3, 3, 1, 1, 1, 1), WL.F32, 8, WL.ACT_SIGMOID),
    ((2, 20, 20, 64, 130, 3, 3, 1, 1, 1, 1), WL.F32, 5, WL.ACT_IDENTITY), # 26-channel groups, two column tiles
    ((4, 20, 20, 32, 64, 4, 4, 2, 2, 0, 0), WL.F32, 4, WL.ACT_GELU),      # strided GEMM, separate statistics pass
    ((2, 11, 11, 16, 16, 3, 3, 2, 2, 1, 1), WL.BF16, 1, WL.ACT_SIGMOID),
    ((3, 9, 10, 5, 6, 3, 3, 1, 1, 1, 1), WL.F32, 3, WL.ACT_TANH),         # direct kernel, scalar vectors
]


def _norm_desc(shape, dt, groups, act, evaluation=False):
    norm = WL.NORM_LAYER if groups == 1 else WL.NORM_GROUP
    return G.shape_desc(shape, dt, act, norm, 0.1, 1e-5, evaluation=evaluation, groups=groups)


@pytest.mark.parametrize("case", NORM_CASES, ids=_ids)
def test_layer_and_group_norm_layer(case):
    """Forward (z, per-sample statistics, y) and the training backward (dz, dgamma,
    dbeta), all against the oracle; the backward on oracle-made inputs."""
    s, dt, groups, act = case
    shape, x, w, b, dy = _problem(s, dt, 210)
    r = np.random.default_rng(211)
    gamma = WL.round_to(WL.F32, r.uniform(0.5, 1.5, shape.OC))
    beta = WL.round_to(WL.F32, r.normal(0.0, 0.1, shape.OC))
    eps = 1e-5
    N, C = shape.N, shape.OC
    for evaluation in (False, True):  # no running statistics: both modes compute the same thing
        desc = _norm_desc(shape, dt, groups, act, evaluation)
        out = G.run_forward(desc, dt, G.dev(x, dt), G.dev(w, dt), G.dev(b), G.dev(gamma), G.dev(beta))
        z_r = O.conv2d_forward(x, w, b, (shape.sh, shape.sw), (shape.ph, shape.pw))
        G.assert_close(G.host(out["z"]), z_r, dt, "norm z")
        zs = WL.round_to(dt, z_r)
        mean_r, var_r, inv_r = O.group_stats(zs, groups, eps)
        # bf16: the statistics are taken over the library's own stored z (one bf16 ulp from
        # the oracle's rounded z per element); the 1e-5 bound on bf16 data is checked on
        # identical z in test_norm_statistics_exact_bf16 and on the oracle's z below.
        stat_tol = G.BN_STAT_TOL if dt == WL.F32 else G.TOL[dt]
        G.assert_bn_stats(G.host(out["save_mean"]), G.host(out["save_inv_std"]), mean_r.ravel(), var_r.ravel(),
                          inv_r.ravel(), eps, "norm fwd", stat_tol)
        y_r = O.apply_group_norm(zs, act, gamma, beta, mean_r, inv_r)
        G.assert_close(G.host(out["y"]), y_r, dt, "norm y")
    sm, si = G.run_bn_stats(desc, G.dev(zs, dt))
    G.assert_bn_stats(G.host(sm), G.host(si), mean_r.ravel(), var_r.ravel(), inv_r.ravel(), eps,
                      "norm statistics on oracle z")
    m32, i32 = WL.round_to(WL.F32, mean_r), WL.round_to(WL.F32, inv_r)
    dy = WL.round_to(dt, G.untie_relu(dy, zs, act, gamma, beta, G.expand_group_stats(m32, N, C),
                                      G.expand_group_stats(i32, N, C)))
    dz, dg, dbt = G.run_act_bwd(desc, dt, G.dev(zs, dt), G.dev(dy, dt), G.dev(gamma), G.dev(beta),
                                G.dev(m32.ravel()), G.dev(i32.ravel()))
    dz_r, dg_r, db_r = O.group_norm_backward(zs, dy, act, gamma, beta, m32, i32)
    G.assert_close(G.host(dz), dz_r, dt, "norm dz")
    G.assert_close(G.host(dg), dg_r, dt, "norm dgamma")
    G.assert_close(G.host(dbt), db_r, dt, "norm dbeta")


@pytest.mark.parametrize("groups", [1, 4])
def test_norm_statistics_exact_bf16(groups):
    """bf16 forward with layer / group norm on small-integer data (x, w in {-1, 0, 1},
    integer bias): every z is exact in fp32 and bf16, so both sides hold the same z and
    the library's statistics from its own stored z meet the 1e-5 bound."""
    shape = WL.ConvShape(3, 16, 16, 128, 64, 3, 3, 1, 1, 1, 1)
    r = np.random.default_rng(96)
    x = r.choice([-1.0, 0.0, 0.0, 0.0, 0.0, 0.0, 1.0], size=shape.x_shape)
    w = r.choice([-1.0, 0.0, 0.0, 0.0, 0.0, 0.0, 1.0], size=shape.w_shape)
    b = r.integers(-8, 9, size=shape.OC).astype(np.float64)
    gamma = WL.round_to(WL.F32, r.uniform(0.5, 1.5, shape.OC))
    beta = WL.round_to(WL.F32, r.normal(0.0, 0.1, shape.OC))
    z_r = O.conv2d_forward(x, w, b, (1, 1), (1, 1))
    assert np.max(np.abs(z_r)) < 256
    desc = _norm_desc(shape, WL.BF16, groups, WL.ACT_TANH)
    out = G.run_forward(desc, WL.BF16, G.dev(x, WL.BF16), G.dev(w, WL.BF16), G.dev(b), G.dev(gamma), G.dev(beta))
    np.testing.assert_array_equal(G.host(out["z"]), z_r)
    mean_r, var_r, inv_r = O.group_stats(z_r, groups, 1e-5)
    G.assert_bn_stats(G.host(out["save_mean"]), G.host(out["save_inv_std"]), mean_r.ravel(), var_r.ravel(),
                      inv_r.ravel(), 1e-5, f"exact bf16 norm G={groups}")


@pytest.mark.parametrize("name,groups,act", [("c3", 1, WL.ACT_GELU), ("c3", 8, WL.ACT_RELU), ("c4", 32, WL.ACT_GELU)])
def test_full_size_norm_variants(name, groups, act):
    """The c3 (fp32) and c4 (bf16) layer shapes with layer / group norm: forward and
    training backward against the oracle, every element."""
    wl = WL.WORKLOADS[name]
    s, dt = wl.shape, wl.dtype
    d = WL.make_inputs(wl)
    r = np.random.default_rng(97)
    gamma = WL.round_to(WL.F32, r.uniform(0.5, 1.5, s.OC))
    beta = WL.round_to(WL.F32, r.normal(0.0, 0.1, s.OC))
    b = d.get("b")
    desc = _norm_desc(s, dt, groups, act)
    out = G.run_forward(desc, dt, G.dev(d["x"], dt), G.dev(d["w"], dt), G.dev(b), G.dev(gamma), G.dev(beta))
    z_r = O.conv2d_forward(d["x"], d["w"], b, (s.sh, s.sw), (s.ph, s.pw))
    G.assert_close(G.host(out["z"]), z_r, dt, f"{name} norm z")
    zs = WL.round_to(dt, z_r)
    mean_r, var_r, inv_r = O.group_stats(zs, groups, 1e-5)
    stat_tol = G.BN_STAT_TOL if dt == WL.F32 else G.TOL[dt]
    G.assert_bn_stats(G.host(out["save_mean"]), G.host(out["save_inv_std"]), mean_r.ravel(), var_r.ravel(),
                      inv_r.ravel(), 1e-5, f"{name} norm fwd", stat_tol)
    G.assert_close(G.host(out["y"]), O.apply_group_norm(zs, act, gamma, beta, mean_r, inv_r), dt, f"{name} norm y")
    del out
    m32, i32 = WL.round_to(WL.F32, mean_r), WL.round_to(WL.F32, inv_r)
    dy = WL.round_to(dt, G.untie_relu(d["dy"], zs, act, gamma, beta, G.expand_group_stats(m32, s.N, s.OC),
                                      G.expand_group_stats(i32, s.N, s.OC)))
    dz, dg, dbt = G.run_act_bwd(desc, dt, G.dev(zs, dt), G.dev(dy, dt), G.dev(gamma), G.dev(beta),
                                G.dev(m32.ravel()), G.dev(i32.ravel()))
    dz_r, dg_r, db_r = O.group_norm_backward(zs, dy, act, gamma, beta, m32, i32)
    G.assert_close(G.host(dz), dz_r, dt, f"{name} norm dz")
    G.assert_close(G.host(dg), dg_r, dt, f"{name} norm dgamma")
    G.assert_close(G.host(dbt), db_r, dt, f"{name} norm dbeta")
