"""Paired-band tile plans of the stride-1 kernel, at sizes that select them: the image's
rows are cut into bands of R rows and bands of R2 rows, and every workgroup computes one
band of each kind (so every workgroup carries the same work).  Each case first asserts,
through the plan introspection call, that the paired kernel is the one that runs, then
compares full tensors with the fp64 oracle: forward z and y without normalisation, with
training batch norm (per-tile statistics from the epilogue), evaluation batch norm (the
normalisation inside the epilogue) and group norm (per-image tile statistics), and the
input gradient; 128-channel plans (two workgroups per CU) and the 64-channel one (four)."""
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


# c4's plan at 40 images (bands of 8 and 6 rows of 28-pixel half rows); 54 x 54 images
# (bands of 8 and 7 rows of 27 pixels, the last short band ragged: one row inside)
C56 = (40, 56, 56, 128, 128, 3, 3, 1, 1, 1, 1)
C54 = (40, 54, 54, 128, 128, 3, 3, 1, 1, 1, 1)
C56_37 = (37, 56, 56, 128, 128, 3, 3, 1, 1, 1, 1)
# 64 channels: 224-row blocks of 16-row fragments, four workgroups per CU (c5's plan at
# 6 images: bands of 14 and 12 rows of 16 pixels)
C224_64 = (6, 224, 224, 64, 64, 3, 3, 1, 1, 1, 1)


def _problem(s, seed):
    shape = WL.ConvShape(*s)
    dt = WL.BF16
    x = WL.random_tensor(shape.x_shape, dt, seed, ("normal", 0.0, 1.0))
    w = WL.random_tensor(shape.w_shape, dt, seed + 1, ("normal", 0.0, (2.0 / shape.Kdim) ** 0.5))
    b = WL.random_tensor((shape.OC,), WL.F32, seed + 2, ("uniform", -0.5, 0.5))
    dy = WL.random_tensor(shape.y_shape, dt, seed + 3, ("normal", 0.0, 1.0))
    r = np.random.default_rng(seed + 4)
    gamma = WL.round_to(WL.F32, r.uniform(0.5, 1.5, shape.OC))
    beta = WL.round_to(WL.F32, r.normal(0.0, 0.1, shape.OC))
    return shape, dt, x, w, b, dy, gamma, beta


def _assert_paired(desc, ops, R2):
    import convolution_layer_amd as cm
    for op in ops:
        name = cm.plan_name(desc, op)
        print(f"plan op {op}: {name}", flush=True)
        assert f" paired {R2}x" in name, name


@pytest.mark.parametrize("case", [(C56, WL.ACT_TANH, 6), (C54, WL.ACT_RELU, 7), (C224_64, WL.ACT_SIGMOID, 12)],
                         ids=["56x56_r8+6_tanh", "54x54_r8+7_ragged_relu", "224x224x64_r14+12_sigmoid"])
def test_paired_forward_and_input_gradient(case):
    s, act, R2 = case
    shape, dt, x, w, b, dy, _, _ = _problem(s, 700)
    desc = G.shape_desc(shape, dt, act)
    _assert_paired(desc, (0, 1), R2)
    out = G.run_forward(desc, dt, G.dev(x, dt), G.dev(w, dt), G.dev(b))
    z_r = O.conv2d_forward(x, w, b, (1, 1), (1, 1))
    G.assert_close(G.host(out["z"]), z_r, dt, "paired z")
    G.assert_close(G.host(out["y"]), O.apply_activation(WL.round_to(dt, z_r), act), dt, "paired y")
    del out
    dx = G.run_backward_data(desc, dt, G.dev(dy, dt), G.dev(w, dt))
    dx_r = O.conv2d_backward_data(dy, w, shape.x_shape, (1, 1), (1, 1))
    G.assert_close(G.host(dx), dx_r, dt, "paired dx")


def test_paired_batchnorm_training():
    """Per-tile statistics of both band kinds merged into the batch statistics, the
    running update and y."""
    shape, dt, x, w, b, _, gamma, beta = _problem(C56_37, 710)
    act, mom, eps = WL.ACT_RELU, 0.1, 1e-5
    r = np.random.default_rng(715)
    rm0 = WL.round_to(WL.F32, r.normal(0.0, 0.2, shape.OC))
    rv0 = WL.round_to(WL.F32, r.uniform(0.5, 2.0, shape.OC))
    desc = G.shape_desc(shape, dt, act, WL.NORM_BATCH, mom, eps)
    _assert_paired(desc, (0,), 6)
    rm_d, rv_d = G.dev(rm0), G.dev(rv0)
    out = G.run_forward(desc, dt, G.dev(x, dt), G.dev(w, dt), G.dev(b), G.dev(gamma), G.dev(beta), rm_d, rv_d)
    z_r = O.conv2d_forward(x, w, b, (1, 1), (1, 1))
    G.assert_close(G.host(out["z"]), z_r, dt, "paired bn z")
    zs = WL.round_to(dt, z_r)
    mean_r, var_r, inv_r, rm_r, rv_r = O.bn_stats(zs, mom, eps, rm0, rv0)
    # statistics of the library's own stored z (one bf16 ulp from the oracle's per element)
    G.assert_bn_stats(G.host(out["save_mean"]), G.host(out["save_inv_std"]), mean_r, var_r, inv_r, eps,
                      "paired bn fwd", G.TOL[dt])
    G.assert_close(G.host(rm_d), rm_r, dt, "paired running_mean")
    G.assert_close(G.host(rv_d), rv_r, dt, "paired running_var")
    G.assert_close(G.host(out["y"]), O.apply_activation(zs, act, WL.NORM_BATCH, gamma, beta, mean_r, inv_r), dt,
                   "paired bn y")


def test_paired_batchnorm_evaluation():
    """Normalisation with the running statistics inside both band kinds' epilogues,
    ragged last short band."""
    shape, dt, x, w, b, _, gamma, beta = _problem(C54, 720)
    act, eps = WL.ACT_SIGMOID, 1e-5
    r = np.random.default_rng(725)
    rm0 = WL.round_to(WL.F32, r.normal(0.0, 0.5, shape.OC))
    rv0 = WL.round_to(WL.F32, r.uniform(0.2, 3.0, shape.OC))
    desc = G.shape_desc(shape, dt, act, WL.NORM_BATCH, 0.1, eps, evaluation=True)
    _assert_paired(desc, (0,), 7)
    out = G.run_forward(desc, dt, G.dev(x, dt), G.dev(w, dt), G.dev(b), G.dev(gamma), G.dev(beta), G.dev(rm0),
                        G.dev(rv0))
    z_r = O.conv2d_forward(x, w, b, (1, 1), (1, 1))
    G.assert_close(G.host(out["z"]), z_r, dt, "paired eval z")
    mean_r, inv_r = O.bn_eval_stats(rm0, rv0, eps)
    m32, i32 = WL.round_to(WL.F32, mean_r), WL.round_to(WL.F32, inv_r)
    y_r = O.apply_activation(WL.round_to(dt, z_r), act, WL.NORM_BATCH, gamma, beta, m32, i32)
    G.assert_close(G.host(out["y"]), y_r, dt, "paired eval y")


def test_paired_group_norm():
    """Group statistics from per-tile partials: an image's long and short bands are
    contiguous in the tile order the per-image merge reads."""
    shape, dt, x, w, b, _, gamma, beta = _problem(C56_37, 730)
    groups, act, eps = 8, WL.ACT_GELU, 1e-5
    desc = G.shape_desc(shape, dt, act, WL.NORM_GROUP, 0.1, eps, groups=groups)
    _assert_paired(desc, (0,), 6)
    out = G.run_forward(desc, dt, G.dev(x, dt), G.dev(w, dt), G.dev(b), G.dev(gamma), G.dev(beta))
    z_r = O.conv2d_forward(x, w, b, (1, 1), (1, 1))
    G.assert_close(G.host(out["z"]), z_r, dt, "paired group z")
    zs = WL.round_to(dt, z_r)
    mean_r, var_r, inv_r = O.group_stats(zs, groups, eps)
    G.assert_bn_stats(G.host(out["save_mean"]), G.host(out["save_inv_std"]), mean_r.ravel(), var_r.ravel(),
                      inv_r.ravel(), eps, "paired group fwd", G.TOL[dt])
    G.assert_close(G.host(out["y"]), O.apply_group_norm(zs, act, gamma, beta, mean_r, inv_r), dt, "paired group y")


def test_paired_64_channel_batchnorm_training():
    """Per-tile statistics from the 64-channel paired kernel."""
    shape, dt, x, w, b, _, gamma, beta = _problem(C224_64, 740)
    act, mom, eps = WL.ACT_TANH, 0.1, 1e-5
    rm0 = np.zeros(shape.OC)
    rv0 = np.ones(shape.OC)
    desc = G.shape_desc(shape, dt, act, WL.NORM_BATCH, mom, eps)
    _assert_paired(desc, (0,), 12)
    out = G.run_forward(desc, dt, G.dev(x, dt), G.dev(w, dt), G.dev(b), G.dev(gamma), G.dev(beta), G.dev(rm0),
                        G.dev(rv0))
    z_r = O.conv2d_forward(x, w, b, (1, 1), (1, 1))
    G.assert_close(G.host(out["z"]), z_r, dt, "paired 64 bn z")
    zs = WL.round_to(dt, z_r)
    mean_r, var_r, inv_r, _, _ = O.bn_stats(zs, mom, eps, rm0, rv0)
    G.assert_bn_stats(G.host(out["save_mean"]), G.host(out["save_inv_std"]), mean_r, var_r, inv_r, eps,
                      "paired 64 bn fwd", G.TOL[dt])
    G.assert_close(G.host(out["y"]), O.apply_activation(zs, act, WL.NORM_BATCH, gamma, beta, mean_r, inv_r), dt,
                   "paired 64 bn y")
