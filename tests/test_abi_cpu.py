"""The C ABI on the CPU: the library loads, exports every symbol include/convmi.h
declares, computes output sizes and workspace sizes, and rejects bad arguments with the
documented status before any device work (no GPU needed: argument checking happens on
the host and returns before the first HIP call)."""
import ctypes as C
import os
import re
import subprocess

import pytest

import workloads as WL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "convmi.h")


@pytest.fixture(scope="module")
def cm():
    import convolution_layer_amd as cm_
    return cm_


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = header_functions()
    for n in ("conv2d_forward", "conv2d_backward_data", "conv2d_backward_weight", "bn_stats_training",
              "activation_backward"):
        assert n in names


def test_library_exports_every_declared_symbol(cm):
    names = header_functions()
    assert set(names) == set(cm.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", cm.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for n in names:
        assert n in exported, n
        assert hasattr(cm.lib, n)
    # nothing but the C ABI is exported
    assert exported == set(names), exported - set(names)


def test_version(cm):
    assert "gfx950" in cm.version()


@pytest.mark.parametrize("name", sorted(WL.WORKLOADS))
def test_output_dims_match_workloads(cm, name):
    wl = WL.WORKLOADS[name]
    s = wl.shape
    d = cm.make_desc(s.N, s.H, s.W, s.IC, s.OC, s.KH, s.KW, (s.sh, s.sw), (s.ph, s.pw), wl.act, wl.norm)
    assert cm.output_dims(d) == (s.OH, s.OW)
    for op in range(6):
        n = cm.workspace_size(d, op)
        assert n >= 0 and n % 256 == 0
    if wl.norm == WL.NORM_BATCH:
        assert cm.workspace_size(d, cm.OP_BN_STATS) > 0
        assert cm.workspace_size(d, cm.OP_ACTIVATION_BACKWARD) > 0


def _good(cm, **kw):
    base = dict(N=2, H=8, W=8, IC=16, OC=16, KH=3, KW=3, stride=(1, 1), pad=(1, 1))
    base.update(kw)
    return cm.make_desc(base["N"], base["H"], base["W"], base["IC"], base["OC"], base["KH"], base["KW"],
                        base["stride"], base["pad"], base.get("activation", 0), base.get("normalization", 0),
                        base.get("mode", 0), base.get("dtype", 0), base.get("momentum", 0.1), base.get("eps", 1e-5),
                        base.get("groups", 1))


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), 1), (dict(IC=-1), 1), (dict(KH=0), 1), (dict(stride=(0, 1)), 1), (dict(pad=(-1, 0)), 1),
    (dict(KH=11, pad=(0, 0)), 1), (dict(dtype=7), 1), (dict(activation=9), 1), (dict(activation=5), 1),
    (dict(normalization=4), 1), (dict(mode=5), 1), (dict(normalization=1, eps=0.0), 1),
    (dict(normalization=2, eps=0.0), 1), (dict(normalization=3, groups=0), 1), (dict(normalization=3, groups=5), 1),
    (dict(normalization=1, momentum=1.5), 1), (dict(N=1 << 40), 2),
])
def test_bad_descriptor(cm, kw, status):
    d = _good(cm, **kw)
    oh, ow = C.c_int64(), C.c_int64()
    st = cm.lib.convmi_output_dims(C.byref(d), C.byref(oh), C.byref(ow))
    assert st == status, cm.lib.convmi_last_error()
    assert cm.lib.convmi_last_error().decode()


def test_norm_variant_descriptors(cm):
    """GELU, layer norm and group norm (groups dividing OC) are valid descriptors; their
    statistics take N*groups entries and the calls refuse running statistics."""
    oh, ow = C.c_int64(), C.c_int64()
    for kw in (dict(activation=cm.ACT_GELU), dict(normalization=cm.NORM_LAYER), dict(normalization=cm.NORM_GROUP, groups=4),
               dict(normalization=cm.NORM_GROUP, groups=16, mode=1)):
        d = _good(cm, **kw)
        assert cm.lib.convmi_output_dims(C.byref(d), C.byref(oh), C.byref(ow)) == cm.OK
    d = _good(cm, normalization=cm.NORM_GROUP, groups=4)
    assert cm.stat_count(d) == 2 * 4
    for op in (cm.OP_FORWARD, cm.OP_BN_STATS, cm.OP_ACTIVATION_BACKWARD):
        assert cm.workspace_size(d, op) > 0
    vec = [A + 0x300000 + 0x1000 * i for i in range(6)]
    args = [C.byref(d), A, A + 0x100000, None, vec[0], vec[1], vec[2], vec[3], vec[4], vec[5], A + 0x400000,
            A + 0x200000, None, 0, None]
    assert cm.lib.conv2d_forward(*args) == cm.ERR_INVALID_ARG
    assert "running" in cm.lib.convmi_last_error().decode()
    st = cm.lib.bn_stats_training(C.byref(d), A, vec[4], vec[5], vec[2], vec[3], None, 0, None)
    assert st == cm.ERR_INVALID_ARG


def test_evaluation_mode_checks(cm):
    """Evaluation mode is a valid descriptor; with batch norm the forward needs the
    running statistics, and the training-statistics call refuses it."""
    d = _good(cm, mode=1, normalization=1)
    oh, ow = C.c_int64(), C.c_int64()
    assert cm.lib.convmi_output_dims(C.byref(d), C.byref(oh), C.byref(ow)) == cm.OK
    f = cm.lib.conv2d_forward
    vec = [A + 0x300000 + 0x1000 * i for i in range(6)]  # gamma, beta, rm, rv, save_mean, save_inv_std
    args = [C.byref(d), A, A + 0x100000, None, vec[0], vec[1], None, None, vec[4], vec[5], A + 0x400000,
            A + 0x200000, None, 0, None]
    assert f(*args) == cm.ERR_INVALID_ARG  # running statistics missing
    assert "running" in cm.lib.convmi_last_error().decode()
    st = cm.lib.bn_stats_training(C.byref(d), A, vec[4], vec[5], None, None, None, 0, None)
    assert st == cm.ERR_INVALID_ARG
    assert "evaluation" in cm.lib.convmi_last_error().decode()


def test_null_desc(cm):
    assert cm.lib.convmi_output_dims(None, None, None) == cm.ERR_INVALID_ARG


# fake device addresses: argument checks run first, so these are never dereferenced
A = 0x7F0000000000
MIS = A + 4


def test_forward_argument_checks(cm):
    d = _good(cm)
    f = cm.lib.conv2d_forward
    ok = [C.byref(d), A, A + 0x100000, None, None, None, None, None, None, None, None, A + 0x200000, None, 0, None]
    args = list(ok); args[1] = None
    assert f(*args) == cm.ERR_INVALID_ARG  # x NULL
    args = list(ok); args[2] = MIS
    assert f(*args) == cm.ERR_MISALIGNED  # w misaligned
    args = list(ok); args[11] = None
    assert f(*args) == cm.ERR_INVALID_ARG  # y NULL
    args = list(ok); args[10] = args[11]
    assert f(*args) == cm.ERR_INVALID_ARG  # z == y
    args = list(ok); args[11] = A
    assert f(*args) == cm.ERR_INVALID_ARG  # y overlaps x
    dbn = _good(cm, normalization=1)
    args = list(ok); args[0] = C.byref(dbn)
    assert f(*args) == cm.ERR_INVALID_ARG  # batch norm without z / gamma / ...
    assert "z" in cm.lib.convmi_last_error().decode()


def test_workspace_checks(cm):
    d = _good(cm, normalization=1)
    need = cm.workspace_size(d, cm.OP_BN_STATS)
    assert need > 0
    f = cm.lib.bn_stats_training
    base = [C.byref(d), A, A + 0x1000, A + 0x2000, None, None]
    assert f(*base, None, 0, None) == cm.ERR_WORKSPACE
    assert f(*base, A + 0x10000, need - 1, None) == cm.ERR_WORKSPACE
    assert f(*base, A + 0x10000 + 16, need, None) == cm.ERR_MISALIGNED
    assert f(*base[:4], A + 0x3000, None, A + 0x10000, need, None) == cm.ERR_INVALID_ARG  # running pair
    dn = _good(cm)
    assert f(C.byref(dn), A, A + 0x1000, A + 0x2000, None, None, A + 0x10000, need, None) == cm.ERR_INVALID_ARG


def test_backward_argument_checks(cm):
    d = _good(cm)
    assert cm.lib.conv2d_backward_data(C.byref(d), A, A + 0x100000, None, None, 0, None) == cm.ERR_INVALID_ARG
    assert cm.lib.conv2d_backward_data(C.byref(d), A, A + 0x100000, A, None, 0, None) == cm.ERR_INVALID_ARG
    assert cm.lib.conv2d_backward_weight(C.byref(d), A, A + 0x100000, A + 0x200000, None, 2, None, 0,
                                         None) == cm.ERR_INVALID_ARG  # accumulate must be 0/1
    assert cm.lib.conv2d_backward_weight(C.byref(d), A, MIS, A + 0x200000, None, 0, None, 0,
                                         None) == cm.ERR_MISALIGNED
    f = cm.lib.activation_backward
    assert f(C.byref(d), A, A + 0x100000, None, None, None, None, A + 0x100000 + 16, None, None, 0, None, 0,
             None) == cm.ERR_INVALID_ARG  # dz partially overlaps dy
    dbn = _good(cm, normalization=1)
    assert f(C.byref(dbn), A, A + 0x100000, None, None, None, None, A + 0x200000, None, None, 0, None, 0,
             None) == cm.ERR_INVALID_ARG  # gamma missing


def test_python_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    """The product path has no CPU fallback: a missing library is an ImportError."""
    import importlib.util
    src = os.path.join(ROOT, "convolution_layer_amd", "__init__.py")
    pkg = tmp_path / "fakepkg"
    pkg.mkdir()
    (pkg / "__init__.py").write_text(open(src).read())
    spec = importlib.util.spec_from_file_location("fakepkg", pkg / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    with pytest.raises(ImportError):
        spec.loader.exec_module(mod)


def test_noalloc_forward_rejects_layers_beyond_its_scratch(cm):
    """A layer whose forward needs more scratch than the static array: WORKSPACE status,
    returned on the host before any device call (so this runs without a GPU)."""
    d = cm.make_desc(2, 32, 32, 8, 4096, 1, 1, (2, 2), (0, 0), cm.ACT_RELU, cm.NORM_BATCH, dtype=cm.BF16)
    assert cm.workspace_size(d, cm.OP_FORWARD) > cm.NOALLOC_SCRATCH_BYTES
    p = 1 << 20  # never dereferenced: the size check comes first
    st = cm.lib.conv2d_forward_noalloc(C.byref(d), p, p, None, p, p, None, None, p, p, p, p, None)
    assert st == cm.ERR_WORKSPACE
    assert b"static limit" in cm.lib.convmi_last_error()


def test_noalloc_scratch_limit_matches_header(cm):
    m = re.search(r"#define CONVMI_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == cm.NOALLOC_SCRATCH_BYTES


# Property tests over random descriptors (host logic only: sizes and argument checks).
from hypothesis import HealthCheck, given, settings, strategies as st  # noqa: E402


@st.composite
def descriptors(draw):
    KH, KW = draw(st.integers(1, 9)), draw(st.integers(1, 9))
    sh, sw = draw(st.integers(1, 5)), draw(st.integers(1, 5))
    ph, pw = draw(st.integers(0, 4)), draw(st.integers(0, 4))
    H, W = draw(st.integers(1, 80)), draw(st.integers(1, 80))
    N = draw(st.integers(1, 16))
    IC = draw(st.sampled_from([1, 3, 4, 8, 16, 24, 32, 64, 96, 128, 256]))
    OC = draw(st.sampled_from([1, 8, 16, 30, 32, 64, 72, 128, 256]))
    norm = draw(st.integers(0, 3))
    groups = draw(st.sampled_from([g for g in (1, 2, 4, 8) if OC % g == 0])) if norm == 3 else 1
    return dict(N=N, H=H, W=W, IC=IC, OC=OC, KH=KH, KW=KW, stride=(sh, sw), pad=(ph, pw),
                activation=draw(st.integers(0, 4)), normalization=norm, dtype=draw(st.integers(0, 1)), groups=groups)


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(descriptors())
def test_random_descriptors_sizes_and_checks(cm, kw):
    """Output sizes follow the floor formula and every operation's workspace query
    succeeds on a valid descriptor; the fused backward's workspace holds dz and the two
    products' workspaces side by side; an empty output is rejected as INVALID_ARG."""
    d = _good(cm, **kw)
    oh_ref = (kw["H"] + 2 * kw["pad"][0] - kw["KH"]) // kw["stride"][0] + 1
    ow_ref = (kw["W"] + 2 * kw["pad"][1] - kw["KW"]) // kw["stride"][1] + 1
    oh, ow = C.c_int64(), C.c_int64()
    status = cm.lib.convmi_output_dims(C.byref(d), C.byref(oh), C.byref(ow))
    if oh_ref < 1 or ow_ref < 1:
        assert status == cm.ERR_INVALID_ARG
        return
    assert status == cm.OK, cm.lib.convmi_last_error()
    assert (oh.value, ow.value) == (oh_ref, ow_ref)
    sizes = [cm.workspace_size(d, op) for op in range(6)]
    assert all(n >= 0 for n in sizes)
    full = sizes[cm.OP_BACKWARD_FULL]
    if kw["normalization"] == 0:
        assert full >= sizes[cm.OP_BACKWARD_DATA] + sizes[cm.OP_BACKWARD_WEIGHT]
    if kw["normalization"] != 0:
        assert sizes[cm.OP_BN_STATS] > 0 and sizes[cm.OP_ACTIVATION_BACKWARD] > 0


@settings(max_examples=200, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(descriptors(), st.sampled_from(["stride0", "pad_neg", "groups", "eps", "kernel_big"]))
def test_random_invalid_descriptors_are_rejected(cm, kw, fault):
    """One planted fault in an otherwise valid descriptor gives INVALID_ARG from every
    host check, before any device work."""
    if fault == "stride0":
        kw["stride"] = (0, kw["stride"][1])
    elif fault == "pad_neg":
        kw["pad"] = (kw["pad"][0], -1)
    elif fault == "groups":
        kw["normalization"], kw["groups"] = 3, kw["OC"] + 1
    elif fault == "eps":
        kw["normalization"] = max(kw["normalization"], 1)
    else:
        kw["KH"], kw["pad"] = kw["H"] + 1, (0, kw["pad"][1])
    d = _good(cm, **kw)
    if fault == "eps":
        d.eps = 0.0
    oh, ow = C.c_int64(), C.c_int64()
    assert cm.lib.convmi_output_dims(C.byref(d), C.byref(oh), C.byref(ow)) == cm.ERR_INVALID_ARG
    n = C.c_size_t()
    for op in range(6):
        assert cm.lib.convmi_workspace_size(C.byref(d), op, C.byref(n)) == cm.ERR_INVALID_ARG


PLAN_RE = re.compile(r"^halo (bf16|f32) (\d+)x(\d+) mf(\d+) tile (\d+)x(\d+) hb([12])(?: paired (\d+)x(\d+) in (\d+) rows)?$")


@pytest.mark.parametrize("name", sorted(WL.WORKLOADS))
def test_plan_names_of_the_workloads(cm, name):
    """The forward and input-gradient plans each workload takes (host-side planner)."""
    wl = WL.WORKLOADS[name]
    s = wl.shape
    d = cm.make_desc(s.N, s.H, s.W, s.IC, s.OC, s.KH, s.KW, (s.sh, s.sw), (s.ph, s.pw), wl.act, wl.norm,
                     dtype=cm.BF16 if wl.dtype == WL.BF16 else cm.F32)
    expect = {"c1": "direct", "c2a": "implicit gemm", "c2b": "implicit gemm", "c2c": "implicit gemm",
              "c3": "halo f32 256x64 mf16 tile 16x16 hb1",
              "c4": "halo bf16 224x128 mf16 tile 8x28 hb2 paired 6x28 in 192 rows",
              "c5": "halo bf16 224x64 mf16 tile 14x16 hb1 paired 12x16 in 192 rows"}[name]
    assert cm.plan_name(d, cm.OP_FORWARD) == expect
    assert cm.plan_name(d, cm.OP_BACKWARD_DATA) == expect


def test_plan_name_checks(cm):
    d = _good(cm)
    buf = C.create_string_buffer(8)
    assert cm.lib.convmi_plan_name(C.byref(d), cm.OP_FORWARD, buf, 8) == cm.OK
    assert len(buf.value) == 7  # cut to the buffer, NUL-terminated
    assert cm.lib.convmi_plan_name(C.byref(d), cm.OP_FORWARD, None, 8) == cm.ERR_INVALID_ARG
    assert cm.lib.convmi_plan_name(C.byref(d), cm.OP_FORWARD, buf, 0) == cm.ERR_INVALID_ARG
    for op in (cm.OP_BACKWARD_WEIGHT, cm.OP_BN_STATS, cm.OP_ACTIVATION_BACKWARD, cm.OP_BACKWARD_FULL, 9):
        assert cm.lib.convmi_plan_name(C.byref(d), op, buf, 8) == cm.ERR_INVALID_ARG
    bad = _good(cm, N=0)
    assert cm.lib.convmi_plan_name(C.byref(bad), cm.OP_FORWARD, buf, 8) == cm.ERR_INVALID_ARG


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(st.integers(1, 96), st.integers(3, 120), st.integers(3, 120), st.sampled_from([(3, 1), (5, 2), (1, 0)]),
       st.sampled_from([64, 128]))
def test_paired_band_geometry(cm, N, H, W, kp, IC):
    """Stride-1 bf16 layers with 128 output channels: a paired plan's bands of R and R2
    rows tile the image, every band starts inside it, and the tiles fit their blocks."""
    k, p = kp
    d = cm.make_desc(N, H, W, IC, 128, k, k, (1, 1), (p, p), 0, 0, dtype=cm.BF16)
    m = PLAN_RE.match(cm.plan_name(d, cm.OP_FORWARD))
    if not m or m.group(8) is None:
        return
    bm, R, Q, R2, Q2, bm2 = (int(m.group(i)) for i in (2, 5, 6, 8, 9, 10))
    OH, OW = cm.output_dims(d)
    assert Q2 == Q and R2 < R and R * Q <= bm and R2 * Q <= bm2 < bm
    nb = -(-OH // (R + R2))
    assert nb * R + (nb - 1) * R2 < OH <= nb * (R + R2)
    assert -(-OW // Q) * Q >= OW
