"""GPU parity of conv2d_backward_full (the [generic] listing's backward_full: the
activation derivative, dX and dW/db of an unnormalised layer in one call) against the
oracle's composition activation_backward -> conv2d_backward_data / _weight, with the
derivative taken from the stored z or from the stored output y (identity, relu, tanh,
sigmoid: 1, [y > 0], 1 - y^2, y(1 - y)).  Both sides get the same rounded z or y and dy;
the library keeps dz in the data type between the steps, as the pages store it."""
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


CASES = [
    ((2, 15, 15, 128, 128, 3, 3, 1, 1, 1, 1), WL.BF16, WL.ACT_TANH),
    ((1, 40, 37, 64, 64, 3, 3, 1, 1, 1, 1), WL.BF16, WL.ACT_IDENTITY),
    ((2, 13, 11, 64, 64, 3, 3, 1, 1, 1, 1), WL.F32, WL.ACT_RELU),
    ((2, 23, 23, 4, 32, 8, 8, 4, 4, 0, 0), WL.F32, WL.ACT_SIGMOID),
    ((2, 10, 12, 3, 8, 3, 3, 1, 1, 1, 1), WL.F32, WL.ACT_GELU),
    ((2, 9, 70, 128, 256, 3, 3, 1, 1, 1, 1), WL.BF16, WL.ACT_RELU),
    # the stride-1 weight-gradient kernel with a run-time k-step count, 64-channel tiles
    # (one and several segments per row)
    ((2, 12, 48, 128, 128, 3, 3, 1, 1, 1, 1), WL.BF16, WL.ACT_SIGMOID),
    ((2, 10, 32, 64, 64, 3, 3, 1, 1, 1, 1), WL.BF16, WL.ACT_TANH),
    ((1, 9, 224, 64, 128, 3, 3, 1, 1, 1, 1), WL.BF16, WL.ACT_RELU),
]


def _ids(c):
    s = c[0]
    return f"{'x'.join(map(str, s[:7]))}_s{s[7]}_{c[1]}_a{c[2]}"


def _run(desc, dt, shape, x, w, saved, from_out, dy, with_dx=True):
    import convolution_layer_amd as cm
    dx = torch.empty(shape.x_shape, dtype=G.tdtype(dt), device="cuda") if with_dx else None
    dw = torch.empty(shape.w_shape, dtype=torch.float32, device="cuda")
    db = torch.empty(shape.OC, dtype=torch.float32, device="cuda")
    cm.conv2d_backward_full(desc, G.dev(x, dt), G.dev(w, dt), G.dev(saved, dt), int(from_out), G.dev(dy, dt), dx, dw,
                            db, 0, cm.workspace(desc, cm.OP_BACKWARD_FULL))
    return dx, dw, db


def _check(shape, dt, act, x, w, z, dy, from_out, name, with_dx=True):
    st, pd = (shape.sh, shape.sw), (shape.ph, shape.pw)
    desc = G.shape_desc(shape, dt, act)
    if from_out:
        saved = WL.round_to(dt, O.apply_activation(z, act))
        dz_r = O.activation_backward_from_output(saved, dy, act)
    else:
        saved = z
        dz_r = O.activation_backward(z, dy, act)[0]
    dx, dw, db = _run(desc, dt, shape, x, w, saved, from_out, dy, with_dx)
    if with_dx:
        G.assert_close(G.host(dx), O.conv2d_backward_data(dz_r, w, shape.x_shape, st, pd), dt, f"{name} dx")
    dw_r, db_r = O.conv2d_backward_weight(x, dz_r, shape.w_shape, st, pd)
    G.assert_close(G.host(dw), dw_r, dt, f"{name} dw")
    G.assert_close(G.host(db), db_r, dt, f"{name} db")


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_backward_full_matches_composition(case):
    s, dt, act = case
    shape = WL.ConvShape(*s)
    r = np.random.default_rng(400)
    x = WL.round_to(dt, r.standard_normal(shape.x_shape))
    w = WL.round_to(dt, r.standard_normal(shape.w_shape) * (2.0 / shape.Kdim) ** 0.5)
    z = WL.round_to(dt, r.standard_normal(shape.y_shape) * 1.5)
    dy = WL.round_to(dt, r.standard_normal(shape.y_shape))
    _check(shape, dt, act, x, w, z, dy, False, "from z")
    if act != WL.ACT_GELU:
        _check(shape, dt, act, x, w, z, dy, True, "from y")
    _check(shape, dt, act, x, w, z, dy, act != WL.ACT_GELU, "no dx", with_dx=False)


@pytest.mark.parametrize("name", ["c4", "c5"])
def test_backward_full_workloads(name):
    """The bench's backward at full size, from the stored output y, every element."""
    wl = WL.WORKLOADS[name]
    s, dt = wl.shape, wl.dtype
    d = WL.make_inputs(wl)
    z = WL.round_to(dt, O.conv2d_forward(d["x"], d["w"], d.get("b"), (s.sh, s.sw), (s.ph, s.pw)))
    _check(s, dt, wl.act, d["x"], d["w"], z, d["dy"], True, f"{name} full")


@pytest.mark.parametrize("s", [(2, 15, 15, 128, 128, 3, 3, 1, 1, 1, 1), (2, 10, 32, 64, 64, 3, 3, 1, 1, 1, 1)])
def test_backward_full_relu_bitwise_equals_separate_calls(s):
    """ReLU: the output-form mask [y > 0] equals [z > 0], so backward_full must reproduce
    activation_backward -> conv2d_backward_weight / conv2d_backward_data bit for bit."""
    import convolution_layer_amd as cm
    shape, dt, act = WL.ConvShape(*s), WL.BF16, WL.ACT_RELU
    r = np.random.default_rng(410)
    x = G.dev(WL.round_to(dt, r.standard_normal(shape.x_shape)), dt)
    w = G.dev(WL.round_to(dt, r.standard_normal(shape.w_shape) * 0.05), dt)
    z = WL.round_to(dt, r.standard_normal(shape.y_shape))
    y = G.dev(np.maximum(z, 0.0), dt)
    dy = G.dev(WL.round_to(dt, r.standard_normal(shape.y_shape)), dt)
    desc = G.shape_desc(shape, dt, act)
    dx = torch.empty(shape.x_shape, dtype=torch.bfloat16, device="cuda")
    dw = torch.empty(shape.w_shape, dtype=torch.float32, device="cuda")
    db = torch.empty(shape.OC, dtype=torch.float32, device="cuda")
    cm.conv2d_backward_full(desc, x, w, y, 1, dy, dx, dw, db, 0, cm.workspace(desc, cm.OP_BACKWARD_FULL))
    dz, _, _ = G.run_act_bwd(desc, dt, G.dev(z, dt), dy)
    dw2, db2 = G.run_backward_weight(desc, x, dz)
    dx2 = G.run_backward_data(desc, dt, dz, w)
    assert torch.equal(dw, dw2) and torch.equal(db, db2) and torch.equal(dx, dx2)


def test_backward_full_refuses_normalised_layers_and_gelu_output():
    import convolution_layer_amd as cm
    shape = WL.ConvShape(1, 8, 8, 8, 8, 3, 3, 1, 1, 1, 1)
    t = torch.zeros(64, dtype=torch.float32, device="cuda")
    desc = G.shape_desc(shape, WL.F32, WL.ACT_RELU, WL.NORM_BATCH)
    with pytest.raises(cm.ConvmiError) as e:
        cm.conv2d_backward_full(desc, t, t, t, 0, t, t, t, None)
    assert e.value.status == cm.ERR_UNSUPPORTED
    desc = G.shape_desc(shape, WL.F32, WL.ACT_GELU)
    with pytest.raises(cm.ConvmiError) as e:
        cm.conv2d_backward_full(desc, t, t, t, 1, t, t, t, None)
    assert e.value.status == cm.ERR_INVALID_ARG


@pytest.mark.parametrize("s", [(2, 15, 15, 128, 128, 3, 3, 1, 1, 1, 1), (2, 10, 32, 64, 64, 3, 3, 1, 1, 1, 1),
                               (2, 13, 11, 64, 64, 3, 3, 1, 1, 1, 1)])
def test_backward_full_side_stream_in_graph_and_on_a_caller_stream(s):
    """The weight gradient runs on the library's second stream, forked from and joined into
    the caller's: eager on a non-default stream, then captured into a HIP graph and replayed
    three times (with eager calls and synchronisations between the replays), every result
    equals the call on the default stream bit for bit, and the work that follows on the
    caller's stream sees finished gradients."""
    import convolution_layer_amd as cm
    shape = WL.ConvShape(*s)
    dt = WL.BF16 if s[3] == 128 or s[1] == 10 else WL.F32
    act = WL.ACT_TANH
    r = np.random.default_rng(420)
    x = G.dev(WL.round_to(dt, r.standard_normal(shape.x_shape)), dt)
    w = G.dev(WL.round_to(dt, r.standard_normal(shape.w_shape) * 0.05), dt)
    y = G.dev(WL.round_to(dt, np.tanh(r.standard_normal(shape.y_shape))), dt)
    dy = G.dev(WL.round_to(dt, r.standard_normal(shape.y_shape)), dt)
    desc = G.shape_desc(shape, dt, act)
    ws = cm.workspace(desc, cm.OP_BACKWARD_FULL)
    tdt = G.tdtype(dt)

    def outs():
        return (torch.empty(shape.x_shape, dtype=tdt, device="cuda"),
                torch.empty(shape.w_shape, dtype=torch.float32, device="cuda"),
                torch.empty(shape.OC, dtype=torch.float32, device="cuda"))

    ref = outs()
    cm.conv2d_backward_full(desc, x, w, y, 1, dy, *ref, 0, ws)
    torch.cuda.synchronize()
    ref = tuple(t.clone() for t in ref)

    side = torch.cuda.Stream()
    got = outs()
    with torch.cuda.stream(side):
        cm.conv2d_backward_full(desc, x, w, y, 1, dy, *got, 0, ws, stream=side)
        sums = [t.double().sum() for t in got]  # ordered after the join on the same stream
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(ref, got))
    assert all(float(a) == float(t.double().sum()) for a, t in zip(sums, ref))

    g_out = outs()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        cm.conv2d_backward_full(desc, x, w, y, 1, dy, *g_out, 0, ws, stream=cap)  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cm.conv2d_backward_full(desc, x, w, y, 1, dy, *g_out, 0, ws)
    for rep in range(3):
        for t in g_out:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(ref, g_out)), f"replay {rep}"
        other = outs()
        cm.conv2d_backward_full(desc, x, w, y, 1, dy, *other, 0, ws)  # eager work between replays
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(ref, other))
    del g


def test_backward_full_two_host_threads_share_the_side_stream():
    """Two host threads, each on its own stream with its own buffers, call
    conv2d_backward_full on a layer whose weight gradient runs on the library's second
    stream (64-channel bf16 stride 1); the shared fork/join events are taken under the
    library's lock, so every result equals the single-threaded one bit for bit."""
    import threading
    import convolution_layer_amd as cm
    shape, dt, act = WL.ConvShape(2, 10, 32, 64, 64, 3, 3, 1, 1, 1, 1), WL.BF16, WL.ACT_TANH
    desc = G.shape_desc(shape, dt, act)
    r = np.random.default_rng(430)
    x = G.dev(WL.round_to(dt, r.standard_normal(shape.x_shape)), dt)
    w = G.dev(WL.round_to(dt, r.standard_normal(shape.w_shape) * 0.05), dt)
    y = G.dev(WL.round_to(dt, np.tanh(r.standard_normal(shape.y_shape))), dt)
    dy = G.dev(WL.round_to(dt, r.standard_normal(shape.y_shape)), dt)

    def outs():
        return (torch.empty(shape.x_shape, dtype=torch.bfloat16, device="cuda"),
                torch.empty(shape.w_shape, dtype=torch.float32, device="cuda"),
                torch.empty(shape.OC, dtype=torch.float32, device="cuda"))

    ref = outs()
    cm.conv2d_backward_full(desc, x, w, y, 1, dy, *ref, 0, cm.workspace(desc, cm.OP_BACKWARD_FULL))
    torch.cuda.synchronize()
    results, errors = {}, []

    def worker(k):
        try:
            torch.cuda.set_device(0)
            st = torch.cuda.Stream()
            ws = cm.workspace(desc, cm.OP_BACKWARD_FULL)
            got = []
            with torch.cuda.stream(st):
                for _ in range(12):
                    o = outs()
                    cm.conv2d_backward_full(desc, x, w, y, 1, dy, *o, 0, ws, stream=st)
                    got.append(o)
            st.synchronize()
            results[k] = got
        except Exception as e:  # reported below, on the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    assert sorted(results) == [0, 1]
    for got in results.values():
        for o in got:
            assert all(torch.equal(a, b) for a, b in zip(ref, o))
