"""Helpers shared by the GPU parity tests (host <-> device copies, checks)."""
import sys

import numpy as np

TOL = 2e-3          # max|y - y_ref| / max|y_ref| for the matmuls


def announce(*parts):
    """Print and flush what the next GPU step is, so a dying box names it."""
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()


def dev(a, device="cuda:0"):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to(device)


def host(t):
    return t.detach().cpu().numpy()


def rel_err(y_gpu, y_ref):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    denom = np.max(np.abs(y_ref))
    return float(np.max(np.abs(y_gpu - y_ref)) / denom) if denom > 0 else float(np.max(np.abs(y_gpu)))


def guarded_empty(shape, dtype, device="cuda:0", pad=4096, fill=0x5A):
    """A tensor view followed by `pad` sentinel bytes, to catch writes past its end."""
    import torch
    n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    raw = torch.full((n + pad,), fill, dtype=torch.uint8, device=device)
    view = raw[:n].view(dtype).view(*shape)
    return view, raw, n


def sentinel_intact(raw, n, fill=0x5A):
    tail = raw[n:].cpu().numpy()
    return bool(np.all(tail == fill))
