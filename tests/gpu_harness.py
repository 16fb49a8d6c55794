"""Helpers for the GPU parity tests: move the seeded fp64 inputs onto the device in the
storage dtype, call the library through its C ABI (convolution_layer_amd), bring the
results back as fp64, and measure errors against the oracle.

Tolerances (normwise, per tensor: max|gpu - oracle| / max|oracle|): 1e-4 for fp32 data,
2e-2 for bf16 data with fp32 accumulation; batch-norm mean within 1e-5*sqrt(var+eps)
and inv_std within 1e-5 relative, per channel.
"""
from __future__ import annotations

import numpy as np
import torch

import workloads as WL

TOL = {WL.F32: 1e-4, WL.BF16: 2e-2}
BN_STAT_TOL = 1e-5

# (what, observed normwise error, tolerance) of every comparison made in this process;
# tests/conftest.py prints them at the end of the run so the headroom is visible.
OBSERVED: list = []


def tdtype(dt: str):
    return torch.bfloat16 if dt == WL.BF16 else torch.float32


def cdtype(dt: str) -> int:
    import convolution_layer_amd as cm
    return cm.BF16 if dt == WL.BF16 else cm.F32


def dev(a, dt: str | None = None):
    """fp64 numpy (already rounded to dt) -> contiguous device tensor of dt (fp32 if None)."""
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    return t.to(tdtype(dt) if dt else torch.float32).contiguous().cuda()


def host(t) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def normwise(g, r) -> float:
    g, r = np.asarray(g, dtype=np.float64), np.asarray(r, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if r.size == 0:
        return 0.0
    scale = float(np.max(np.abs(r)))
    err = float(np.max(np.abs(g - r)))
    return err / scale if scale > 0 else err


def assert_close(g, r, dt: str, what: str, tol: float | None = None):
    tol = TOL[dt] if tol is None else tol
    e = normwise(g, r)
    OBSERVED.append((what, e, tol))
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    assert e <= tol, f"{what}: normwise error {e:.3e} > {tol:.0e}"
    return e


def relu_kink_ties(z, gamma, beta, mean, inv_std):
    """Elements whose normalised activation input a = gamma*(z - mean)*inv_std + beta
    (fp64, from the same fp32 statistics both sides receive) lies within 8 fp32 roundings
    of the ReLU kink.  There the library's fp32 a and the oracle's fp64 a may fall on
    different sides of 0, flipping that element's ReLU derivative (an integer decision
    taken from a floating-point value).  The tests zero dy at these elements on BOTH
    sides, so the decision no longer matters, and check that they are few."""
    zh = (np.asarray(z, np.float64) - mean) * inv_std
    a = gamma * zh + beta
    return np.abs(a) <= 2.0 ** -21 * (np.abs(gamma * zh) + np.abs(beta))


def expand_group_stats(v, N, C):
    """Per (sample, group) statistics [N*G] -> [N, 1, 1, C], broadcastable over z."""
    v = np.asarray(v, np.float64).reshape(N, -1)
    return np.repeat(v, C // v.shape[1], axis=1).reshape(N, 1, 1, C)


def untie_relu(dy, z, act, gamma, beta, mean, inv_std):
    """dy with the ReLU-kink ties (relu_kink_ties) zeroed; other activations are smooth
    and pass through unchanged."""
    import workloads as WL_
    if act != WL_.ACT_RELU:
        return dy
    ties = relu_kink_ties(z, gamma, beta, mean, inv_std)
    n = int(ties.sum())
    assert n <= 4 + 1e-5 * ties.size, f"{n} of {ties.size} activation inputs sit at the ReLU kink"
    return np.where(ties, 0.0, dy)


def assert_bn_stats(mean_g, inv_g, mean_r, var_r, inv_r, eps, what="", tol=BN_STAT_TOL):
    """Per channel |dmean| <= tol*sqrt(var+eps) (plus one fp32 ulp of the mean, the
    resolution of the stored fp32 result) and |dinv_std| <= tol*inv_std."""
    dm = np.abs(np.asarray(mean_g) - mean_r)
    bound = tol * np.sqrt(var_r + eps) + np.abs(mean_r) * 2.0 ** -23
    di = np.abs(np.asarray(inv_g) - inv_r) / inv_r
    OBSERVED.append((f"{what} mean (of bound)", float(np.max(dm / bound)) * tol, tol))
    OBSERVED.append((f"{what} inv_std", float(np.max(di)), tol))
    assert np.all(dm <= bound), f"{what} mean: {np.max(dm / bound):.3e} of bound"
    assert np.all(di <= tol), f"{what} inv_std: {np.max(di):.3e}"


def desc_for(wl: WL.Workload):
    import convolution_layer_amd as cm
    s = wl.shape
    return cm.make_desc(s.N, s.H, s.W, s.IC, s.OC, s.KH, s.KW, (s.sh, s.sw), (s.ph, s.pw), wl.act, wl.norm,
                        cm.MODE_TRAIN, cdtype(wl.dtype), wl.momentum, wl.eps)


def shape_desc(shape: WL.ConvShape, dt: str, act=0, norm=0, momentum=0.1, eps=1e-5, evaluation=False, groups=1):
    import convolution_layer_amd as cm
    s = shape
    return cm.make_desc(s.N, s.H, s.W, s.IC, s.OC, s.KH, s.KW, (s.sh, s.sw), (s.ph, s.pw), act, norm,
                        cm.MODE_EVAL if evaluation else cm.MODE_TRAIN, cdtype(dt), momentum, eps, groups)


def sample_indices(shape4, count: int, seed: int) -> np.ndarray:
    """Random multi-indices plus the corners of every axis (border handling)."""
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.integers(0, n, size=count) for n in shape4], axis=1)
    corners = np.array(np.meshgrid(*[[0, n - 1] for n in shape4], indexing="ij")).reshape(4, -1).T
    return np.concatenate([idx, corners]).astype(np.int64)


# ------------------------------------------------------------------ library calls
def run_forward(desc, dt, x, w, b=None, gamma=None, beta=None, rmean=None, rvar=None, want_z=True):
    """Returns dict of device tensors (z, y, and BN outputs when present)."""
    import convolution_layer_amd as cm
    oh, ow = cm.output_dims(desc)
    shape = (desc.N, oh, ow, desc.OC)
    z = torch.empty(shape, dtype=tdtype(dt), device="cuda") if want_z else None
    y = torch.empty(shape, dtype=tdtype(dt), device="cuda")
    out = {"z": z, "y": y}
    sm = si = None
    if desc.normalization != cm.NORM_NONE:
        sm = torch.empty(cm.stat_count(desc), dtype=torch.float32, device="cuda")
        si = torch.empty(cm.stat_count(desc), dtype=torch.float32, device="cuda")
        out.update(save_mean=sm, save_inv_std=si, running_mean=rmean, running_var=rvar)
    ws = cm.workspace(desc, cm.OP_FORWARD)
    cm.conv2d_forward(desc, x, w, b, gamma, beta, rmean, rvar, sm, si, z, y, ws)
    return out


def run_backward_data(desc, dt, dz, w):
    import convolution_layer_amd as cm
    dx = torch.empty((desc.N, desc.H, desc.W, desc.IC), dtype=tdtype(dt), device="cuda")
    cm.conv2d_backward_data(desc, dz, w, dx, cm.workspace(desc, cm.OP_BACKWARD_DATA))
    return dx


def run_backward_weight(desc, x, dz, with_bias=True, accumulate=0, dw=None, db=None):
    import convolution_layer_amd as cm
    if dw is None:
        dw = torch.empty((desc.OC, desc.KH, desc.KW, desc.IC), dtype=torch.float32, device="cuda")
    if db is None and with_bias:
        db = torch.empty(desc.OC, dtype=torch.float32, device="cuda")
    cm.conv2d_backward_weight(desc, x, dz, dw, db if with_bias else None, accumulate,
                              cm.workspace(desc, cm.OP_BACKWARD_WEIGHT))
    return dw, db


def run_bn_stats(desc, z, rmean=None, rvar=None):
    import convolution_layer_amd as cm
    sm = torch.empty(cm.stat_count(desc), dtype=torch.float32, device="cuda")
    si = torch.empty(cm.stat_count(desc), dtype=torch.float32, device="cuda")
    cm.bn_stats_training(desc, z, sm, si, rmean, rvar, cm.workspace(desc, cm.OP_BN_STATS))
    return sm, si


def run_act_bwd(desc, dt, z, dy, gamma=None, beta=None, mean=None, inv=None, dz=None, accumulate=0,
                dgamma=None, dbeta=None):
    import convolution_layer_amd as cm
    if dz is None:
        dz = torch.empty_like(dy)
    if desc.normalization != cm.NORM_NONE:
        if dgamma is None:
            dgamma = torch.empty(desc.OC, dtype=torch.float32, device="cuda")
        if dbeta is None:
            dbeta = torch.empty(desc.OC, dtype=torch.float32, device="cuda")
    cm.activation_backward(desc, z, dy, gamma, beta, mean, inv, dz, dgamma, dbeta, accumulate,
                           cm.workspace(desc, cm.OP_ACTIVATION_BACKWARD))
    return dz, dgamma, dbeta
