"""Shared test utilities: the error ratio and conversions (no method arithmetic)."""
import numpy as np
import torch

TOL = 0.008  # relative L2 error ratio, as in the FLA backend pull request's test plan


def ratio(x, ref):
    """||x - ref||_2 / ||ref||_2 in fp64 (||x||_2 when ref is all zero)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    nr = np.linalg.norm(ref.ravel())
    nd = np.linalg.norm((x - ref).ravel())
    if nr == 0.0:
        return float(np.linalg.norm(x.ravel()))
    return float(nd / nr)


def np64(t):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def to_dev(d, device="cuda"):
    out = {}
    for k, v in d.items():
        out[k] = v.to(device) if isinstance(v, torch.Tensor) else v
    return out
