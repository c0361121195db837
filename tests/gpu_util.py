"""Helpers shared by the GPU parity tests: the tolerance gates and host <-> device copies."""
import numpy as np
import torch

MAX_REL_TOL = 1e-4
NMSE_TOL = 1e-7


def dev():
    return torch.device("cuda:0")


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def f16_bits(t):
    return t.cpu().numpy().view(np.uint16)


def f32_bits(t):
    return t.cpu().numpy().view(np.uint32)


def errors(y, ref):
    """Normwise max relative error and NMSE (both in fp64)."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert y.shape == r.shape, (y.shape, r.shape)
    denom = np.abs(r).max()
    if denom == 0.0:
        return (0.0 if np.all(y == 0) else np.inf), (0.0 if np.all(y == 0) else np.inf)
    max_rel = np.abs(y - r).max() / denom
    nmse = ((y - r) ** 2).sum() / (r ** 2).sum()
    return max_rel, nmse


def assert_close(y, ref, what=""):
    max_rel, nmse = errors(y, ref)
    assert max_rel <= MAX_REL_TOL and nmse <= NMSE_TOL, f"{what}: max_rel {max_rel:.3e} nmse {nmse:.3e}"
    return max_rel, nmse
