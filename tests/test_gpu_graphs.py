"""A whole training step captured once into a HIP graph and replayed three times, with
eager steps and host synchronisations between the replays: every replay reproduces the
eager step bit for bit (the library keeps no state between calls and records no
memory-set nodes).  With training-mode batch norm: forward (statistics, normalise,
activate, running statistics), activation + batch-norm backward (dgamma, dbeta), dX,
dW/db (the running statistics, which each step updates in place, are reset before each
step).  Unnormalised, in the benchmark's layout: the forward storing y only, then
backward_full from y, at sizes that take the paired-band plans (the 64-channel one with
the weight gradient forked onto the library's second stream)."""
import numpy as np
import pytest
import torch

import workloads as WL
from tests import gpu_harness as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import convolution_layer_amd  # noqa: F401


CASES = [
    # bf16 stride 1, 128 channels: statistics from the convolution's epilogue tiles
    ((2, 15, 15, 128, 128, 3, 3, 1, 1, 1, 1), WL.BF16, WL.ACT_RELU),
    # fp32 stride 1, 64 channels: the fp32 tile kernel with epilogue statistics
    ((2, 13, 11, 64, 64, 3, 3, 1, 1, 1, 1), WL.F32, WL.ACT_TANH),
    # strided implicit GEMM: standalone statistics kernels after the convolution
    ((4, 20, 20, 32, 64, 4, 4, 2, 2, 0, 0), WL.F32, WL.ACT_SIGMOID),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{'x'.join(map(str, c[0][:7]))}_{c[1]}")
def test_training_step_with_batchnorm_replays_bitwise(case):
    import convolution_layer_amd as cm
    s, dt, act = case
    shape = WL.ConvShape(*s)
    r = np.random.default_rng(440)
    tdt = G.tdtype(dt)
    x = G.dev(WL.round_to(dt, r.standard_normal(shape.x_shape)), dt)
    w = G.dev(WL.round_to(dt, r.standard_normal(shape.w_shape) * (2.0 / shape.Kdim) ** 0.5), dt)
    b = G.dev(WL.round_to(WL.F32, r.uniform(-0.5, 0.5, shape.OC)))
    gamma = G.dev(WL.round_to(WL.F32, r.uniform(0.5, 1.5, shape.OC)))
    beta = G.dev(WL.round_to(WL.F32, r.normal(0.0, 0.1, shape.OC)))
    dy = G.dev(WL.round_to(dt, r.standard_normal(shape.y_shape)), dt)
    rm0 = torch.zeros(shape.OC, dtype=torch.float32, device="cuda")
    rv0 = torch.ones(shape.OC, dtype=torch.float32, device="cuda")
    desc = G.shape_desc(shape, dt, act, WL.NORM_BATCH)
    ws = torch.empty(max(cm.workspace_size(desc, op) for op in range(5)) or 256, dtype=torch.uint8, device="cuda")

    def buffers():
        f32 = lambda n=shape.OC: torch.empty(n, dtype=torch.float32, device="cuda")
        return dict(z=torch.empty(shape.y_shape, dtype=tdt, device="cuda"),
                    y=torch.empty(shape.y_shape, dtype=tdt, device="cuda"),
                    dz=torch.empty(shape.y_shape, dtype=tdt, device="cuda"),
                    dx=torch.empty(shape.x_shape, dtype=tdt, device="cuda"),
                    dw=torch.empty(shape.w_shape, dtype=torch.float32, device="cuda"),
                    db=f32(), sm=f32(), si=f32(), dg=f32(), dbt=f32(), rm=f32(), rv=f32())

    def step(o):
        cm.conv2d_forward(desc, x, w, b, gamma, beta, o["rm"], o["rv"], o["sm"], o["si"], o["z"], o["y"], ws)
        cm.activation_backward(desc, o["z"], dy, gamma, beta, o["sm"], o["si"], o["dz"], o["dg"], o["dbt"], 0, ws)
        cm.conv2d_backward_data(desc, o["dz"], w, o["dx"], ws)
        cm.conv2d_backward_weight(desc, x, o["dz"], o["dw"], o["db"], 0, ws)

    def reset(o):
        o["rm"].copy_(rm0)
        o["rv"].copy_(rv0)

    ref = buffers()
    reset(ref)
    step(ref)
    torch.cuda.synchronize()

    g_out = buffers()
    reset(g_out)
    step(g_out)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(g_out)
    for rep in range(3):
        for k, t in g_out.items():
            if k not in ("rm", "rv"):
                t.zero_()
        reset(g_out)
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(ref[k], g_out[k]), f"replay {rep}: {k}"
        other = buffers()  # an eager step between the replays
        reset(other)
        step(other)
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(ref[k], other[k]), f"eager step after replay {rep}: {k}"
    del g


# the unnormalised training step of the benchmark layout (forward storing y only, then
# backward_full from y), at sizes that take the paired-band tile plans
FUSED_CASES = [
    ((40, 56, 56, 128, 128, 3, 3, 1, 1, 1, 1), WL.BF16, WL.ACT_TANH),
    ((6, 224, 224, 64, 64, 3, 3, 1, 1, 1, 1), WL.BF16, WL.ACT_RELU),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: f"{'x'.join(map(str, c[0][:5]))}_{c[1]}")
def test_unnormalised_step_replays_bitwise(case):
    import convolution_layer_amd as cm
    s, dt, act = case
    shape = WL.ConvShape(*s)
    desc = G.shape_desc(shape, dt, act)
    assert " paired " in cm.plan_name(desc, cm.OP_FORWARD)
    r = np.random.default_rng(450)
    tdt = G.tdtype(dt)
    x = G.dev(WL.round_to(dt, r.standard_normal(shape.x_shape)), dt)
    w = G.dev(WL.round_to(dt, r.standard_normal(shape.w_shape) * (2.0 / shape.Kdim) ** 0.5), dt)
    b = G.dev(WL.round_to(WL.F32, r.uniform(-0.5, 0.5, shape.OC)))
    dy = G.dev(WL.round_to(dt, r.standard_normal(shape.y_shape) * 0.01), dt)
    n = max(cm.workspace_size(desc, op) for op in (cm.OP_FORWARD, cm.OP_BACKWARD_FULL))
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")

    def buffers():
        return dict(y=torch.empty(shape.y_shape, dtype=tdt, device="cuda"),
                    dx=torch.empty(shape.x_shape, dtype=tdt, device="cuda"),
                    dw=torch.empty(shape.w_shape, dtype=torch.float32, device="cuda"),
                    db=torch.empty(shape.OC, dtype=torch.float32, device="cuda"))

    def step(o):
        cm.conv2d_forward(desc, x, w, b, None, None, None, None, None, None, None, o["y"], ws)
        cm.conv2d_backward_full(desc, x, w, o["y"], 1, dy, o["dx"], o["dw"], o["db"], 0, ws)

    ref = buffers()
    step(ref)
    torch.cuda.synchronize()
    g_out = buffers()
    step(g_out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(g_out)
    for rep in range(3):
        for t in g_out.values():
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(ref[k], g_out[k]), f"replay {rep}: {k}"
        other = buffers()
        step(other)
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(ref[k], other[k]), f"eager step after replay {rep}: {k}"
    del g
