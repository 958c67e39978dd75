"""Helpers shared by the GPU parity tests: device upload of the seeded inputs,
sentinel-filled pools, layout conversion to the oracle's orientation and the
relative-error metrics.

Tolerance metric: rel = ||x - ref||_F / ||ref||_F per (sequence, head) for
outputs and per (slot, head) for states; the bar is 1e-4 for fp32 inputs and
2e-2 for bf16/fp16 inputs.
"""

import numpy as np
import torch

import workloads as wl

DEV = "cuda:0"
TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 2e-2}
SENTINEL = {"f32": -7.25, "bf16": -7.25, "f16": -7.25}   # exactly representable in all three


def i32(x):
    return torch.as_tensor(np.asarray(x, dtype=np.int32)).to(DEV)


def make_pool(n_slots, H, dk, dv, pool_dtype, fill=True):
    p = torch.empty((n_slots, H, dv, dk), dtype=wl.DTYPES[pool_dtype], device=DEV)
    if fill:
        p.fill_(SENTINEL[pool_dtype])
    return p


def to_math(pool_slot):
    """[H, d_v, d_k] pool slot -> float64 (H, d_k, d_v) oracle state."""
    return np.swapaxes(wl.exact(pool_slot.detach().cpu()), -1, -2)


def rel(x, ref):
    nr = np.linalg.norm(ref)
    if nr == 0.0:
        return 0.0 if np.linalg.norm(x) == 0.0 else np.inf
    return float(np.linalg.norm(x - ref) / nr)


def rel_per_head(x, ref, head_axis):
    """Max over heads of the per-head relative Frobenius error."""
    xs = np.moveaxis(x, head_axis, 0)
    rs = np.moveaxis(ref, head_axis, 0)
    return max(rel(a, b) for a, b in zip(xs, rs))


def untouched(pool, slots, pool_dtype):
    """True if every slot in ``slots`` still holds the sentinel bit pattern."""
    if len(slots) == 0:
        return True
    sel = pool[torch.as_tensor(list(slots), device=pool.device, dtype=torch.long)]
    return bool((sel == SENTINEL[pool_dtype]).all().item())


def rne(x32, pool_dtype):
    """One RNE cast of an fp32 tensor into the pool dtype (torch's cast is RNE)."""
    return x32.to(wl.DTYPES[pool_dtype])
