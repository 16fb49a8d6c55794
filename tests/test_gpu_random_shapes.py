"""GPU parity on a seeded sample of random layer shapes: data type, batch, image size,
channel counts (multiples of the 16-byte vector and odd ones), kernel size, stride,
padding, activation and batch normalisation drawn at random, small enough for the oracle
to finish in well under a second each.  Every output element of the forward (z, y),
the input gradient and the weight and bias gradients is compared with the fp64 oracle;
with batch norm also the batch statistics.  The sample is fixed by its seed, so a failure
names a reproducible case (printed before it runs)."""
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


def _cases(n=40, seed=2024):
    r = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        dt = WL.BF16 if r.random() < 0.5 else WL.F32
        vec = 8 if dt == WL.BF16 else 4
        kblk = 32 if dt == WL.BF16 else 16  # input channels the MFMA paths take in whole K blocks
        def channels():
            u = r.random()
            if u < 0.15:
                return int(r.integers(1, 6))             # direct kernel, scalar channel runs
            if u < 0.4:
                return int(vec * r.integers(1, 17))      # 16-byte runs
            return int(kblk * r.integers(1, 5))          # implicit GEMM / tile kernels (dX: OC)
        IC, OC = channels(), channels()
        KH, KW = int(r.integers(1, 6)), int(r.integers(1, 6))
        sh = int(r.choice([1, 1, 1, 2, 3]))
        sw = sh if r.random() < 0.8 else int(r.choice([1, 2]))
        ph, pw = int(r.integers(0, KH)), int(r.integers(0, KW))
        N = int(r.integers(1, 4))
        H, W = int(r.integers(max(KH - 2 * ph, 1), 34)), int(r.integers(max(KW - 2 * pw, 1), 34))
        if (H + 2 * ph - KH) < 0 or (W + 2 * pw - KW) < 0:
            continue
        act = int(r.integers(0, 5))
        norm = WL.NORM_BATCH if r.random() < 0.3 else WL.NORM_NONE
        if norm == WL.NORM_BATCH and act == WL.ACT_GELU:
            act = WL.ACT_TANH
        out.append(((N, H, W, IC, OC, KH, KW, sh, sw, ph, pw), dt, act, norm))
    return out


CASES = _cases()


def _id(c):
    s, dt, act, norm = c
    return f"{'x'.join(map(str, s[:7]))}_s{s[7]}{s[8]}_p{s[9]}{s[10]}_{dt}_a{act}_n{norm}"


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_random_layer(case):
    import convolution_layer_amd as cm
    s, dt, act, norm = case
    shape = WL.ConvShape(*s)
    seed = 900 + CASES.index(case) * 10
    x = WL.random_tensor(shape.x_shape, dt, seed, ("normal", 0.0, 1.0))
    w = WL.random_tensor(shape.w_shape, dt, seed + 1, ("normal", 0.0, (2.0 / shape.Kdim) ** 0.5))
    b = WL.random_tensor((shape.OC,), WL.F32, seed + 2, ("uniform", -0.5, 0.5))
    dy = WL.random_tensor(shape.y_shape, dt, seed + 3, ("normal", 0.0, 1.0))
    r = np.random.default_rng(seed + 4)
    gamma = WL.round_to(WL.F32, r.uniform(0.5, 1.5, shape.OC))
    beta = WL.round_to(WL.F32, r.normal(0.0, 0.1, shape.OC))
    desc = G.shape_desc(shape, dt, act, norm)
    print(f"case {_id(case)}: forward plan {cm.plan_name(desc, cm.OP_FORWARD)!r}", flush=True)
    strides, pads = (shape.sh, shape.sw), (shape.ph, shape.pw)
    z_r = O.conv2d_forward(x, w, b, strides, pads)
    zs = WL.round_to(dt, z_r)
    if norm == WL.NORM_BATCH:
        rm0, rv0 = np.zeros(shape.OC), np.ones(shape.OC)
        out = G.run_forward(desc, dt, G.dev(x, dt), G.dev(w, dt), G.dev(b), G.dev(gamma), G.dev(beta), G.dev(rm0),
                            G.dev(rv0))
        mean_r, var_r, inv_r, _, _ = O.bn_stats(zs, 0.1, 1e-5, rm0, rv0)
        stat_tol = G.BN_STAT_TOL if dt == WL.F32 else G.TOL[dt]
        G.assert_bn_stats(G.host(out["save_mean"]), G.host(out["save_inv_std"]), mean_r, var_r, inv_r, 1e-5,
                          "random fwd", stat_tol)
        y_r = O.apply_activation(zs, act, WL.NORM_BATCH, gamma, beta, mean_r, inv_r)
    else:
        out = G.run_forward(desc, dt, G.dev(x, dt), G.dev(w, dt), G.dev(b))
        y_r = O.apply_activation(zs, act)
    G.assert_close(G.host(out["z"]), z_r, dt, "random z")
    G.assert_close(G.host(out["y"]), y_r, dt, "random y")
    dx = G.run_backward_data(desc, dt, G.dev(dy, dt), G.dev(w, dt))
    G.assert_close(G.host(dx), O.conv2d_backward_data(dy, w, shape.x_shape, strides, pads), dt, "random dx")
    dw, db = G.run_backward_weight(desc, G.dev(x, dt), G.dev(dy, dt))
    dw_r, db_r = O.conv2d_backward_weight(x, dy, shape.w_shape, strides, pads)
    G.assert_close(G.host(dw), dw_r, dt, "random dw")
    G.assert_close(G.host(db), db_r, dt, "random db")
