"""Helpers shared by the parity tests: error metric and host<->device moves.

The error of a tensor is norm-wise: max|gpu - ref| / max|ref| over the whole
tensor, where ref is the fp64 oracle.  Element-wise relative error is
undefined near zero.
"""
import numpy as np
import torch

# tolerances on the norm-wise relative error
TOL_BF16 = 2e-2   # bf16 inputs/outputs, fp32 state
TOL_F32 = 1e-4    # fp32 inputs/outputs and state


def rel_err(gpu, ref):
    g = gpu.detach().double().cpu().numpy() if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    denom = np.abs(r).max()
    if denom == 0:
        return float(np.abs(g).max())
    return float(np.abs(g - r).max() / denom)


def rel_err_per(gpu, ref, axis):
    """The largest norm-wise error over the slices along `axis` (each V head,
    or each sequence): max over i of max|gpu_i - ref_i| / max|ref_i|.  A
    slice of small magnitude cannot hide behind the tensor-wide maximum."""
    g = gpu.detach().double().cpu().numpy() if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    g, r = np.moveaxis(g, axis, 0), np.moveaxis(r, axis, 0)
    worst = 0.0
    for gi, ri in zip(g, r):
        denom = np.abs(ri).max()
        worst = max(worst, float(np.abs(gi - ri).max() / denom) if denom > 0 else float(np.abs(gi).max()))
    return worst


def np64(t):
    return None if t is None else t.double().cpu().numpy()


def dev(t):
    return None if t is None else t.cuda()


def report(name, **errs):
    print(name, " ".join(f"{k}={v:.3e}" for k, v in errs.items()), flush=True)
