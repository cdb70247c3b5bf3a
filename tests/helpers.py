"""Shared test plumbing: device upload of synthetic weights, error metrics, GPU guard."""

import numpy as np
import pytest


def have_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def require_gpu():
    if not have_gpu():
        pytest.fail("GPU test collected without a GPU: run it on an MI355X box")


def to_device(W, keys=None):
    """Upload a dict of numpy arrays (uint16 = bfloat16 bits) to CUDA tensors. Arrays that
    are the same object share one device tensor."""
    import torch
    out, seen = {}, {}
    for k, a in W.items():
        if keys is not None and k not in keys:
            continue
        if id(a) in seen:
            out[k] = seen[id(a)]
            continue
        if a.dtype == np.uint16:
            t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
        out[k] = t
        seen[id(a)] = t
    return out


def max_abs_err(got, want):
    return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))))


def norm_max_err(got, want):
    """max |got - want| / max |want| over the whole tensor (the bf16-path metric)."""
    want = np.asarray(want, np.float64)
    return float(np.max(np.abs(np.asarray(got, np.float64) - want)) / np.max(np.abs(want)))
