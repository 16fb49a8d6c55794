"""GPU parity of the stride-1 tile kernel across its LDS layouts: the halo's 16-byte chunks
are XOR-swizzled by a key chosen for the hardware's ds_read_b128 lane passes, in one form
for 16-row fragments and another for 32-row ones, keyed on tile coordinates (row * QS +
column) in the bf16 two-wave kernels.  These shapes select 32-row plans, tile rows whose
width is not a multiple of 16 (fragments that cross a tile row), kernels 1, 2 (even: QS =
Q + 1) and 5 wide, 64 and 128 channels, bf16 and fp32; each case asserts its plan through
the introspection call, then compares the full forward (z, y) and input gradient with
the fp64 oracle."""
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


# (N, H, W, C, K, dtype, expected plan prefix)
CASES = [
    (1, 20, 30, 128, 3, WL.BF16, "halo bf16 256x128 mf32 tile 16x15"),
    (1, 12, 33, 128, 5, WL.BF16, "halo bf16 224x128 mf16 tile 11x17"),
    (1, 56, 13, 128, 2, WL.BF16, "halo bf16 256x128 mf32 tile 50x5"),
    (1, 20, 33, 64, 2, WL.BF16, "halo bf16 256x64 mf32 tile 16x12"),
    (1, 12, 56, 64, 5, WL.BF16, "halo bf16 256x64 mf32 tile 7x28"),
    (2, 20, 13, 64, 1, WL.BF16, "halo bf16 256x64 mf32 tile 15x13"),
    (1, 20, 30, 64, 3, WL.F32, "halo f32"),
    (1, 12, 33, 128, 3, WL.F32, "halo f32"),
]


def _id(c):
    return f"{c[0]}x{c[1]}x{c[2]}x{c[3]}_k{c[4]}_{c[5]}"


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_halo_layout(case):
    import convolution_layer_amd as cm
    N, H, W, C, K, dt, plan = case
    p = K // 2
    shape = WL.ConvShape(N, H, W, C, C, K, K, 1, 1, p, p)
    seed = 800 + 10 * CASES.index(case)
    x = WL.random_tensor(shape.x_shape, dt, seed, ("normal", 0.0, 1.0))
    w = WL.random_tensor(shape.w_shape, dt, seed + 1, ("normal", 0.0, (2.0 / shape.Kdim) ** 0.5))
    b = WL.random_tensor((shape.OC,), WL.F32, seed + 2, ("uniform", -0.5, 0.5))
    dy = WL.random_tensor(shape.y_shape, dt, seed + 3, ("normal", 0.0, 1.0))
    act = WL.ACT_TANH
    desc = G.shape_desc(shape, dt, act)
    for op in (cm.OP_FORWARD, cm.OP_BACKWARD_DATA):
        name = cm.plan_name(desc, op)
        print(f"case {_id(case)} op {op}: {name}", flush=True)
        assert name.startswith("halo"), name
    assert cm.plan_name(desc, cm.OP_FORWARD).startswith(plan), cm.plan_name(desc, cm.OP_FORWARD)
    out = G.run_forward(desc, dt, G.dev(x, dt), G.dev(w, dt), G.dev(b))
    z_r = O.conv2d_forward(x, w, b, (1, 1), (p, p))
    G.assert_close(G.host(out["z"]), z_r, dt, "layout z")
    G.assert_close(G.host(out["y"]), O.apply_activation(WL.round_to(dt, z_r), act), dt, "layout y")
    del out
    dx = G.run_backward_data(desc, dt, G.dev(dy, dt), G.dev(w, dt))
    G.assert_close(G.host(dx), O.conv2d_backward_data(dy, w, shape.x_shape, (1, 1), (p, p)), dt, "layout dx")
