"""Python binding of libconvmi.so, the gfx950 conv2d training-layer library.

Argument marshalling only: every function below passes device pointers (torch tensors'
``data_ptr()``), sizes and the current HIP stream straight to the C ABI declared in
include/convmi.h, whose entry points have the same names.  All computation happens in
the library's HIP kernels.  If the library is not built, importing this package raises
ImportError: there is no fallback path.

Tensors must be CUDA (HIP) tensors, contiguous, in the layouts of convmi.h: x/dx NHWC
[N,H,W,IC], w/dw OHWI [OC,KH,KW,IC], z/y/dy/dz NHWC [N,OH,OW,OC]; data tensors are
float32 or bfloat16 per ``desc.dtype``; bias, gamma, beta, running and saved statistics,
dw, db, dgamma, dbeta are float32.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libconvmi.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_MISALIGNED, ERR_HIP = range(6)
F32, BF16 = 0, 1
ACT_IDENTITY, ACT_RELU, ACT_TANH, ACT_SIGMOID, ACT_GELU = 0, 1, 2, 3, 4
NORM_NONE, NORM_BATCH, NORM_LAYER, NORM_GROUP = 0, 1, 2, 3
MODE_TRAIN, MODE_EVAL = 0, 1
OP_FORWARD, OP_BACKWARD_DATA, OP_BACKWARD_WEIGHT, OP_BN_STATS, OP_ACTIVATION_BACKWARD, OP_BACKWARD_FULL = range(6)

STATUS_NAMES = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "WORKSPACE", 4: "MISALIGNED", 5: "HIP"}

# Every symbol include/convmi.h declares.
EXPORTS = ("convmi_output_dims", "convmi_workspace_size", "conv2d_forward", "conv2d_forward_noalloc",
           "conv2d_backward_data",
           "conv2d_backward_weight", "bn_stats_training", "activation_backward", "conv2d_backward_full",
           "convmi_plan_name", "convmi_last_error",
           "convmi_version")


class ConvDesc(C.Structure):
    """Mirror of convmi_desc."""
    _fields_ = [("N", C.c_int64), ("H", C.c_int64), ("W", C.c_int64), ("IC", C.c_int64), ("OC", C.c_int64),
                ("KH", C.c_int64), ("KW", C.c_int64),
                ("stride_h", C.c_int32), ("stride_w", C.c_int32), ("pad_h", C.c_int32), ("pad_w", C.c_int32),
                ("activation", C.c_int32), ("normalization", C.c_int32), ("mode", C.c_int32),
                ("dtype", C.c_int32), ("momentum", C.c_float), ("eps", C.c_float), ("groups", C.c_int32)]


class ConvmiError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"convmi status {status} ({STATUS_NAMES.get(status, '?')}): {message}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(python convolution_layer_amd/build.py)")
    L = C.CDLL(LIB_PATH)
    vp, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
    dp = C.POINTER(ConvDesc)
    L.convmi_last_error.restype = C.c_char_p
    L.convmi_version.restype = C.c_char_p
    L.convmi_output_dims.argtypes = [dp, C.POINTER(C.c_int64), C.POINTER(C.c_int64)]
    L.convmi_workspace_size.argtypes = [dp, i32, C.POINTER(sz)]
    L.conv2d_forward.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.conv2d_forward_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.conv2d_backward_data.argtypes = [dp, vp, vp, vp, vp, sz, vp]
    L.conv2d_backward_weight.argtypes = [dp, vp, vp, vp, vp, i32, vp, sz, vp]
    L.bn_stats_training.argtypes = [dp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.activation_backward.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    L.conv2d_backward_full.argtypes = [dp, vp, vp, vp, i32, vp, vp, vp, vp, i32, vp, sz, vp]
    L.convmi_plan_name.argtypes = [dp, i32, C.c_char_p, sz]
    for name in EXPORTS:
        if name not in ("convmi_last_error", "convmi_version"):
            getattr(L, name).restype = C.c_int
    return L


lib = _load()


def version() -> str:
    return lib.convmi_version().decode()


def make_desc(N, H, W, IC, OC, KH, KW, stride=(1, 1), pad=(0, 0), activation=ACT_IDENTITY,
              normalization=NORM_NONE, mode=MODE_TRAIN, dtype=F32, momentum=0.1, eps=1e-5, groups=1) -> ConvDesc:
    return ConvDesc(N, H, W, IC, OC, KH, KW, stride[0], stride[1], pad[0], pad[1], activation, normalization,
                    mode, dtype, momentum, eps, groups)


def stat_count(desc: ConvDesc) -> int:
    """Entries of save_mean / save_inv_std: OC (batch norm) or N * groups (layer, group)."""
    if desc.normalization == NORM_BATCH:
        return desc.OC
    return desc.N * (desc.groups if desc.normalization == NORM_GROUP else 1)


def _check(status: int):
    if status != OK:
        raise ConvmiError(status, lib.convmi_last_error().decode())


def output_dims(desc: ConvDesc):
    oh, ow = C.c_int64(), C.c_int64()
    _check(lib.convmi_output_dims(C.byref(desc), C.byref(oh), C.byref(ow)))
    return oh.value, ow.value


def workspace_size(desc: ConvDesc, op: int) -> int:
    n = C.c_size_t()
    _check(lib.convmi_workspace_size(C.byref(desc), op, C.byref(n)))
    return n.value


def plan_name(desc: ConvDesc, op: int) -> str:
    """Kernel plan of the forward or the input gradient for this descriptor (host only)."""
    buf = C.create_string_buffer(128)
    _check(lib.convmi_plan_name(C.byref(desc), op, buf, len(buf)))
    return buf.value.decode()


def _ptr(t):
    """Device pointer of a contiguous GPU tensor, or None."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("convmi needs device (HIP) tensors")
    if not t.is_contiguous():
        raise ValueError("convmi needs contiguous tensors")
    return t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ws(workspace):
    if workspace is None:
        return None, 0
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def workspace(desc: ConvDesc, op: int, device="cuda"):
    """Allocate the caller-owned workspace one operation needs (None when 0 bytes)."""
    import torch
    n = workspace_size(desc, op)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def conv2d_forward(desc, x, w, bias, gamma, beta, running_mean, running_var, save_mean, save_inv_std, z, y,
                   workspace=None, stream=None):
    wp, wn = _ws(workspace)
    _check(lib.conv2d_forward(C.byref(desc), _ptr(x), _ptr(w), _ptr(bias), _ptr(gamma), _ptr(beta),
                              _ptr(running_mean), _ptr(running_var), _ptr(save_mean), _ptr(save_inv_std),
                              _ptr(z), _ptr(y), wp, wn, _stream(stream)))


def conv2d_forward_noalloc(desc, x, w, bias, gamma, beta, running_mean, running_var, save_mean, save_inv_std, z,
                           y, stream=None):
    _check(lib.conv2d_forward_noalloc(C.byref(desc), _ptr(x), _ptr(w), _ptr(bias), _ptr(gamma), _ptr(beta),
                                      _ptr(running_mean), _ptr(running_var), _ptr(save_mean), _ptr(save_inv_std),
                                      _ptr(z), _ptr(y), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 8 << 20  # CONVMI_NOALLOC_SCRATCH_BYTES


def conv2d_backward_data(desc, dz, w, dx, workspace=None, stream=None):
    wp, wn = _ws(workspace)
    _check(lib.conv2d_backward_data(C.byref(desc), _ptr(dz), _ptr(w), _ptr(dx), wp, wn, _stream(stream)))


def conv2d_backward_weight(desc, x, dz, dw, db, accumulate=0, workspace=None, stream=None):
    wp, wn = _ws(workspace)
    _check(lib.conv2d_backward_weight(C.byref(desc), _ptr(x), _ptr(dz), _ptr(dw), _ptr(db), int(accumulate),
                                      wp, wn, _stream(stream)))


def bn_stats_training(desc, z, save_mean, save_inv_std, running_mean=None, running_var=None, workspace=None,
                      stream=None):
    wp, wn = _ws(workspace)
    _check(lib.bn_stats_training(C.byref(desc), _ptr(z), _ptr(save_mean), _ptr(save_inv_std),
                                 _ptr(running_mean), _ptr(running_var), wp, wn, _stream(stream)))


def activation_backward(desc, z, dy, gamma, beta, save_mean, save_inv_std, dz, dgamma=None, dbeta=None,
                        accumulate=0, workspace=None, stream=None):
    wp, wn = _ws(workspace)
    _check(lib.activation_backward(C.byref(desc), _ptr(z), _ptr(dy), _ptr(gamma), _ptr(beta), _ptr(save_mean),
                                   _ptr(save_inv_std), _ptr(dz), _ptr(dgamma), _ptr(dbeta), int(accumulate),
                                   wp, wn, _stream(stream)))


def conv2d_backward_full(desc, x, w, saved, saved_is_output, dy, dx, dw, db, accumulate=0, workspace=None,
                         stream=None):
    wp, wn = _ws(workspace)
    _check(lib.conv2d_backward_full(C.byref(desc), _ptr(x), _ptr(w), _ptr(saved), int(saved_is_output), _ptr(dy),
                                    _ptr(dx), _ptr(dw), _ptr(db), int(accumulate), wp, wn, _stream(stream)))
