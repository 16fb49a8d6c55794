"""fp64 CPU oracle for the conv2d training layer (ctypes over liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg, never by the product path (convolution_layer_amd).  It shares no code
with the HIP library.  All arrays are float64, C-contiguous, in the layouts of
oracle.c (NHWC activations, OHWI weights).  Every routine is a plain definition; see
oracle.c for the page each one follows.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

ACT_IDENTITY, ACT_RELU, ACT_TANH, ACT_SIGMOID, ACT_GELU = 0, 1, 2, 3, 4
NORM_NONE, NORM_BATCH, NORM_LAYER, NORM_GROUP = 0, 1, 2, 3

_lib = None
_D = C.POINTER(C.c_double)
_L = C.POINTER(C.c_int64)
_i = C.c_int64


def lib():
    global _lib
    if _lib is None:
        _lib = _load(_build.LIB, rebuild=True)
    return _lib


def _load(path: str, rebuild: bool = False):
    if rebuild:
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
    L = C.CDLL(path)
    dims = [_i] * 11
    L.oracle_out_extent.restype = _i
    L.oracle_out_extent.argtypes = [_i, _i, _i, _i]
    L.oracle_num_threads.restype = C.c_int
    L.oracle_conv2d_forward.argtypes = [_D, _D, _D, _D] + dims
    L.oracle_conv2d_forward_at.argtypes = [_D, _D, _D, _L, _i, _D] + dims
    L.oracle_bn_stats.argtypes = [_D, _i, _i, C.c_double, C.c_double, _D, _D, _D, _D, _D]
    L.oracle_apply_activation.argtypes = [_D, _i, _i, C.c_int, C.c_int, _D, _D, _D, _D, _D]
    L.oracle_activation_backward.argtypes = [_D, _D, _i, _i, C.c_int, C.c_int, _D, _D, _D, _D,
                                             _D, _D, _D]
    L.oracle_bn_eval_stats.argtypes = [_D, _D, _i, C.c_double, _D, _D]
    L.oracle_activation_backward_eval.argtypes = [_D, _D, _i, _i, C.c_int, _D, _D, _D, _D, _D, _D, _D]
    L.oracle_conv2d_backward_data.argtypes = [_D, _D, _D] + dims
    L.oracle_conv2d_backward_data_at.argtypes = [_D, _D, _L, _i, _D] + dims
    L.oracle_conv2d_backward_weight.argtypes = [_D, _D, _D, _D] + dims
    L.oracle_conv2d_backward_weight_at.argtypes = [_D, _D, _L, _i, _D] + dims
    L.oracle_bias_grad.argtypes = [_D, _i, _i, _D]
    L.oracle_activation_backward_from_output.restype = C.c_int
    L.oracle_activation_backward_from_output.argtypes = [_D, _D, _i, C.c_int, _D]
    L.oracle_group_stats.argtypes = [_D, _i, _i, _i, _i, C.c_double, _D, _D, _D]
    L.oracle_apply_group_norm.argtypes = [_D, _i, _i, _i, _i, C.c_int, _D, _D, _D, _D, _D]
    L.oracle_group_norm_backward.argtypes = [_D, _D, _i, _i, _i, _i, C.c_int, _D, _D, _D, _D, _D, _D, _D]
    return L


class using:
    """Context manager: route this module's calls to another build of oracle.c (the
    mutation tests load deliberately broken copies to show the pins catch them)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _lib
        _lib = _load(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _p(a):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags.c_contiguous, (a.dtype, a.flags)
    return a.ctypes.data_as(_D)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def out_extent(n: int, k: int, s: int, p: int) -> int:
    return int(lib().oracle_out_extent(n, k, s, p))


def _dims(x_shape, w_shape, stride, pad):
    N, H, W, IC = x_shape
    OC, KH, KW, IC2 = w_shape
    assert IC == IC2, (x_shape, w_shape)
    sh, sw = stride
    ph, pw = pad
    OH, OW = out_extent(H, KH, sh, ph), out_extent(W, KW, sw, pw)
    return (N, H, W, IC, OC, KH, KW, sh, sw, ph, pw), (N, OH, OW, OC)


def conv2d_forward(x, w, b=None, stride=(1, 1), pad=(0, 0)):
    """z = conv(x, w) + b (cross-correlation, zero padding)."""
    x, w, b = _f64(x), _f64(w), _f64(b)
    dims, yshape = _dims(x.shape, w.shape, stride, pad)
    z = np.zeros(yshape)
    lib().oracle_conv2d_forward(_p(x), _p(w), _p(b), _p(z), *dims)
    return z


def conv2d_forward_at(x, w, b, idx, stride=(1, 1), pad=(0, 0)):
    """z at listed outputs idx[i] = (n, oh, ow, oc)."""
    x, w, b = _f64(x), _f64(w), _f64(b)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    dims, _ = _dims(x.shape, w.shape, stride, pad)
    out = np.zeros(len(idx))
    lib().oracle_conv2d_forward_at(_p(x), _p(w), _p(b), idx.ctypes.data_as(_L), len(idx), _p(out), *dims)
    return out


def bn_stats(z, momentum=0.1, eps=1e-5, running_mean=None, running_var=None):
    """Training batch-norm statistics over all but the last axis of z.

    Returns (mean, var, inv_std, new_running_mean, new_running_var); the running pair is
    None when not given."""
    z = _f64(z)
    C_ = z.shape[-1]
    M = z.size // C_
    mean, var, inv = np.zeros(C_), np.zeros(C_), np.zeros(C_)
    rm = None if running_mean is None else np.array(running_mean, dtype=np.float64)
    rv = None if running_var is None else np.array(running_var, dtype=np.float64)
    lib().oracle_bn_stats(_p(z), M, C_, momentum, eps, _p(mean), _p(var), _p(inv), _p(rm), _p(rv))
    return mean, var, inv, rm, rv


def bn_eval_stats(running_mean, running_var, eps=1e-5):
    """Evaluation-mode statistics: (mean, inv_std) from the running pair."""
    rm, rv = _f64(running_mean), _f64(running_var)
    mean, inv = np.zeros(rm.size), np.zeros(rm.size)
    lib().oracle_bn_eval_stats(_p(rm), _p(rv), rm.size, eps, _p(mean), _p(inv))
    return mean, inv


def apply_activation(z, act, norm=NORM_NONE, gamma=None, beta=None, mean=None, inv_std=None):
    z = _f64(z)
    C_ = z.shape[-1]
    y = np.zeros_like(z)
    lib().oracle_apply_activation(_p(z), z.size // C_, C_, act, norm, _p(_f64(gamma)), _p(_f64(beta)),
                                  _p(_f64(mean)), _p(_f64(inv_std)), _p(y))
    return y


def activation_backward(z, dy, act, norm=NORM_NONE, gamma=None, beta=None, mean=None, inv_std=None,
                        evaluation=False):
    """Returns (dz, dgamma, dbeta); dgamma/dbeta are None without batch norm.
    evaluation=True takes the batch-norm statistics as constants (evaluation mode)."""
    z, dy = _f64(z), _f64(dy)
    assert z.shape == dy.shape
    C_ = z.shape[-1]
    dz = np.zeros_like(z)
    dg = np.zeros(C_) if norm == NORM_BATCH else None
    dbt = np.zeros(C_) if norm == NORM_BATCH else None
    if evaluation and norm == NORM_BATCH:
        lib().oracle_activation_backward_eval(_p(z), _p(dy), z.size // C_, C_, act, _p(_f64(gamma)),
                                              _p(_f64(beta)), _p(_f64(mean)), _p(_f64(inv_std)), _p(dz),
                                              _p(dg), _p(dbt))
        return dz, dg, dbt
    lib().oracle_activation_backward(_p(z), _p(dy), z.size // C_, C_, act, norm, _p(_f64(gamma)),
                                     _p(_f64(beta)), _p(_f64(mean)), _p(_f64(inv_std)), _p(dz),
                                     _p(dg), _p(dbt))
    return dz, dg, dbt


def activation_backward_from_output(y, dy, act):
    """dz = act'(z) * dy of an unnormalised layer, with the derivative written in terms of
    the stored output y = act(z) (identity, relu, tanh, sigmoid)."""
    y, dy = _f64(y), _f64(dy)
    assert y.shape == dy.shape
    dz = np.zeros_like(y)
    if lib().oracle_activation_backward_from_output(_p(y), _p(dy), y.size, act, _p(dz)) != 0:
        raise ValueError("this activation's derivative is not a function of its output")
    return dz


def conv2d_backward_data(dz, w, x_shape, stride=(1, 1), pad=(0, 0)):
    dz, w = _f64(dz), _f64(w)
    dims, yshape = _dims(x_shape, w.shape, stride, pad)
    assert tuple(dz.shape) == yshape, (dz.shape, yshape)
    dx = np.zeros(x_shape)
    lib().oracle_conv2d_backward_data(_p(dz), _p(w), _p(dx), *dims)
    return dx


def conv2d_backward_data_at(dz, w, x_shape, idx, stride=(1, 1), pad=(0, 0)):
    """dx at listed inputs idx[i] = (n, ih, iw, ic)."""
    dz, w = _f64(dz), _f64(w)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    dims, yshape = _dims(x_shape, w.shape, stride, pad)
    assert tuple(dz.shape) == yshape
    out = np.zeros(len(idx))
    lib().oracle_conv2d_backward_data_at(_p(dz), _p(w), idx.ctypes.data_as(_L), len(idx), _p(out), *dims)
    return out


def conv2d_backward_weight(x, dz, w_shape, stride=(1, 1), pad=(0, 0)):
    """Returns (dw, db)."""
    x, dz = _f64(x), _f64(dz)
    dims, yshape = _dims(x.shape, w_shape, stride, pad)
    assert tuple(dz.shape) == yshape
    dw = np.zeros(w_shape)
    db = np.zeros(w_shape[0])
    lib().oracle_conv2d_backward_weight(_p(x), _p(dz), _p(dw), _p(db), *dims)
    return dw, db


def conv2d_backward_weight_at(x, dz, w_shape, idx, stride=(1, 1), pad=(0, 0)):
    """dw at listed weights idx[i] = (oc, kh, kw, ic)."""
    x, dz = _f64(x), _f64(dz)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    dims, yshape = _dims(x.shape, w_shape, stride, pad)
    assert tuple(dz.shape) == yshape
    out = np.zeros(len(idx))
    lib().oracle_conv2d_backward_weight_at(_p(x), _p(dz), idx.ctypes.data_as(_L), len(idx), _p(out), *dims)
    return out


def bias_grad(dz):
    dz = _f64(dz)
    C_ = dz.shape[-1]
    db = np.zeros(C_)
    lib().oracle_bias_grad(_p(dz), dz.size // C_, C_, _p(db))
    return db


# ------------------------------------------------------------ layer norm / group norm
def _nsc(z):
    """[N, OH, OW, C] -> (N, S = OH*OW, C)."""
    N, C_ = z.shape[0], z.shape[-1]
    return N, z.size // (N * C_), C_


def group_stats(z, groups=1, eps=1e-5):
    """Per-sample, per-channel-group statistics of z [N, OH, OW, C] (groups=1: layer norm).
    Returns (mean, var, inv_std), each [N, groups]."""
    z = _f64(z)
    N, S, C_ = _nsc(z)
    assert C_ % groups == 0
    mean, var, inv = np.zeros((N, groups)), np.zeros((N, groups)), np.zeros((N, groups))
    lib().oracle_group_stats(_p(z), N, S, C_, groups, eps, _p(mean), _p(var), _p(inv))
    return mean, var, inv


def apply_group_norm(z, act, gamma, beta, mean, inv_std):
    """y = act(gamma[c] * (z - mean[n, g]) * inv_std[n, g] + beta[c]); groups from mean's shape."""
    z = _f64(z)
    N, S, C_ = _nsc(z)
    mean, inv_std = _f64(mean).reshape(N, -1), _f64(inv_std).reshape(N, -1)
    y = np.zeros_like(z)
    lib().oracle_apply_group_norm(_p(z), N, S, C_, mean.shape[1], act, _p(_f64(gamma)), _p(_f64(beta)), _p(mean),
                                  _p(inv_std), _p(y))
    return y


def group_norm_backward(z, dy, act, gamma, beta, mean, inv_std):
    """Training backward through group (layer) norm + activation: (dz, dgamma, dbeta)."""
    z, dy = _f64(z), _f64(dy)
    assert z.shape == dy.shape
    N, S, C_ = _nsc(z)
    mean, inv_std = _f64(mean).reshape(N, -1), _f64(inv_std).reshape(N, -1)
    dz, dg, dbt = np.zeros_like(z), np.zeros(C_), np.zeros(C_)
    lib().oracle_group_norm_backward(_p(z), _p(dy), N, S, C_, mean.shape[1], act, _p(_f64(gamma)), _p(_f64(beta)),
                                     _p(mean), _p(inv_std), _p(dz), _p(dg), _p(dbt))
    return dz, dg, dbt
