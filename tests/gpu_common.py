"""Helpers shared by the GPU parity tests (host-side marshalling only)."""
import sys

import numpy as np
import torch

TOL = {"f32": 1e-5, "bf16": 2e-2}   # max-abs error against the fp64 oracle
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


def say(*a):
    """Name the case before a GPU step runs (flushed, so a dying box still shows it)."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def dev(x, dtype: str):
    """float32 numpy (values exact in `dtype`) -> contiguous device tensor."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(TDT[dtype]).contiguous()


def host(t) -> np.ndarray:
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def bits(t) -> np.ndarray:
    """Raw bit pattern of a device tensor (for bit-exact comparisons, NaN included)."""
    if t.dtype == torch.bfloat16:
        return t.detach().view(torch.int16).cpu().numpy()
    return t.detach().view(torch.int32).cpu().numpy()


def rows_of(out_np, rows):
    """Pick (b, h, i) rows out of a [B, H, L, d] array."""
    rows = np.asarray(rows)
    return out_np[rows[:, 0], rows[:, 1], rows[:, 2]]


def all_rows(B, H, L):
    bb, hh, ii = np.meshgrid(np.arange(B), np.arange(H), np.arange(L), indexing="ij")
    return np.stack([bb.ravel(), hh.ravel(), ii.ravel()], axis=1)


def max_err(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    assert np.isfinite(a).all(), "non-finite GPU output"
    return float(np.abs(a - b).max()) if a.size else 0.0


def guarded(shape, dtype, fill, pad=4096):
    """A device tensor of `shape` inside a buffer with `pad` canary elements
    (value `fill`) before and after; returns (buffer, view)."""
    n = 1
    for x in shape:
        n *= x
    buf = torch.full((n + 2 * pad,), fill, dtype=dtype, device="cuda")
    return buf, buf[pad:pad + n].view(*shape)


def guard_intact(buf, fill, pad=4096) -> bool:
    return bool((buf[:pad] == fill).all()) and bool((buf[-pad:] == fill).all())
