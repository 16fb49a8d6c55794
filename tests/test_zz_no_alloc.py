"""The allocation-free forward (conv2d_forward_noalloc) against conv2d_forward with a
caller-owned workspace: two calls in a row on one GPU, the second on a smaller layer,
each compared element by element with the workspace entry point on the same inputs
(the same kernels run, so the outputs must agree bit for bit)."""
import numpy as np
import pytest
import torch

import workloads as WL
from tests import gpu_harness as G

pytestmark = pytest.mark.gpu

# (N, H, W, IC, OC, KH, KW, sh, sw, ph, pw), dtype, activation, normalization
CALLS = [
    ((8, 56, 56, 128, 128, 3, 3, 1, 1, 1, 1), WL.BF16, WL.ACT_TANH, WL.NORM_NONE),   # weight fragments in scratch
    ((4, 20, 20, 64, 64, 3, 3, 1, 1, 1, 1), WL.F32, WL.ACT_RELU, WL.NORM_BATCH),     # per-tile statistics in scratch
    ((2, 15, 17, 32, 40, 3, 3, 2, 2, 1, 1), WL.BF16, WL.ACT_SIGMOID, WL.NORM_BATCH),  # slab partials in scratch
]


def _inputs(shape, dt, seed):
    r = np.random.default_rng(seed)
    x = WL.round_to(dt, r.standard_normal(shape.x_shape))
    w = WL.round_to(dt, r.standard_normal(shape.w_shape) * (2.0 / shape.Kdim) ** 0.5)
    b = WL.round_to(WL.F32, r.uniform(-0.3, 0.3, shape.OC))
    g = WL.round_to(WL.F32, r.uniform(0.5, 1.5, shape.OC))
    bt = WL.round_to(WL.F32, r.normal(0.0, 0.1, shape.OC))
    return x, w, b, g, bt


def _run(entry, desc, dt, shape, x, w, b, g, bt, norm):
    import convolution_layer_amd as cm
    tdt = G.tdtype(dt)
    z = torch.empty(shape.y_shape, dtype=tdt, device="cuda")
    y = torch.empty(shape.y_shape, dtype=tdt, device="cuda")
    bn = norm == WL.NORM_BATCH
    f32 = lambda v: G.dev(v) if bn else None  # noqa: E731
    rm, rv = f32(np.zeros(shape.OC)), f32(np.ones(shape.OC))
    sm = torch.empty(shape.OC, dtype=torch.float32, device="cuda") if bn else None
    si = torch.empty(shape.OC, dtype=torch.float32, device="cuda") if bn else None
    args = (desc, x, w, b, f32(g), f32(bt), rm, rv, sm, si, z, y)
    if entry == "noalloc":
        cm.conv2d_forward_noalloc(*args)
    else:
        cm.conv2d_forward(*args, cm.workspace(desc, cm.OP_FORWARD))
    torch.cuda.synchronize()
    return [t for t in (z, y, sm, si, rm, rv) if t is not None]


def test_noalloc_forward_matches_workspace_forward():
    import convolution_layer_amd as cm
    sizes = []
    for i, (s, dt, act, norm) in enumerate(CALLS):
        shape = WL.ConvShape(*s)
        desc = G.shape_desc(shape, dt, act, norm)
        need = cm.workspace_size(desc, cm.OP_FORWARD)
        assert 0 < need <= cm.NOALLOC_SCRATCH_BYTES, (s, need)
        sizes.append(need)
        x, w, b, g, bt = _inputs(shape, dt, 300 + i)
        xd, wd, bd = G.dev(x, dt), G.dev(w, dt), G.dev(b)
        ref = _run("workspace", desc, dt, shape, xd, wd, bd, g, bt, norm)
        got = _run("noalloc", desc, dt, shape, xd, wd, bd, g, bt, norm)
        for r_, g_ in zip(ref, got):
            assert torch.equal(r_, g_), f"call {i} {s}: outputs differ"
    assert sizes[0] > sizes[1] > sizes[2]  # each later call is a smaller layer


def test_noalloc_rejects_layers_beyond_the_scratch():
    import convolution_layer_amd as cm
    # 4096 channels with batch norm: 16 MiB of statistics partials
    shape = WL.ConvShape(2, 32, 32, 8, 4096, 1, 1, 2, 2, 0, 0)
    desc = G.shape_desc(shape, WL.BF16, WL.ACT_RELU, WL.NORM_BATCH)
    assert cm.workspace_size(desc, cm.OP_FORWARD) > cm.NOALLOC_SCRATCH_BYTES
    bf = dict(dtype=torch.bfloat16, device="cuda")
    f32 = lambda: torch.ones(shape.OC, dtype=torch.float32, device="cuda")  # noqa: E731
    x, w = torch.zeros(shape.x_shape, **bf), torch.zeros(shape.w_shape, **bf)
    z, y = torch.empty(shape.y_shape, **bf), torch.full(shape.y_shape, 7.0, **bf)
    with pytest.raises(cm.ConvmiError) as e:
        cm.conv2d_forward_noalloc(desc, x, w, None, f32(), f32(), None, None, f32(), f32(), z, y)
    assert e.value.status == cm.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)  # nothing ran
