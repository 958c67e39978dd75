"""Helpers shared by the GPU parity tests: device upload of the seeded inputs,
sentinel-filled pools, layout conversion to the oracle's orientation and the
error metrics.

Two metrics, both asserted against the same bar (1e-4 for fp32 inputs, 2e-2
for bf16/fp16 inputs):
  * per (sequence, head): rel = ||x - ref||_F / ||ref||_F over all the
    tokens of one sequence and head (outputs) or one slot and head (states);
  * per row: one row is the d-vector of one (token, head) of an output, or
    one pool row (one value column of S, d_k entries) of a state; its error
    is ||x_row - ref_row|| / max(||ref_row||, ROW_FLOOR * rms), where rms is
    the root-mean-square row norm of ref over the same head.  With 16-bit
    operands the rounding error of a row scales with the operands it is
    built from (the head's state and keys), not with the row's own norm, so
    a row that cancels to a small norm (the output at the first token of a
    sequence started from a zero state is o_1 = u_1 (q_1 . k_1), small when
    q_1 . k_1 is) has a large relative error at an ordinary absolute one;
    measured on the GPU, the worst rows' absolute errors stay below 1e-2 of
    their head's rms row norm.  Rows at or above a quarter of that rms are
    held to their own norm; a row that is wrong outright has an error of
    about its own norm and fails either way.
Each check also reports max|x - ref| / max|ref| over the compared arrays.
"""

import numpy as np
import torch

import workloads as wl

DEV = "cuda:0"
TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 2e-2}
SENTINEL = {"f32": -7.25, "bf16": -7.25, "f16": -7.25}   # exactly representable in all three
ROW_FLOOR = 0.25


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


def ulp16(x, pool_dtype):
    """Spacing of the 16-bit pool format at |x| (fp16: 10 stored mantissa
    bits, subnormals from 2^-24; bf16: 7 bits): the distance between the two
    representable values around x, so a once-rounded value lies within half
    of it."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(ax)
    bits, tiny = (10, 2.0 ** -24) if pool_dtype == "f16" else (7, 2.0 ** -133)
    return np.where(ax == 0, tiny, np.maximum(np.ldexp(1.0, e - 1 - bits), tiny))


def rounding_excess(got, ref, pool_dtype, slack_rel=1e-6):
    """|got - ref| in units of (half a 16-bit ulp of ref + slack_rel of the
    largest |ref| of the state): at most 1 for a state computed in fp32 from
    exact operands and rounded once, to nearest, into the pool. The slack
    covers the fp32 arithmetic's own error, which matters only for elements
    near zero, whose 16-bit ulp is as small as that error."""
    ref = np.asarray(ref, dtype=np.float64)
    slack = slack_rel * np.abs(ref).max(axis=(-2, -1), keepdims=True)
    return np.abs(np.asarray(got, dtype=np.float64) - ref) / (0.5 * ulp16(ref, pool_dtype) + slack)


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


def row_errors(x, ref, head_axis, floor=None):
    """Row metric of ``x`` against ``ref``; rows run along the last axis and
    ``head_axis`` (not the last) names the head axis.  Returns a dict:
    ``row`` the worst floored row error, ``row_raw`` the worst unfloored
    one, ``absmax`` max|x - ref| / max|ref|."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return dict(row=0.0, row_raw=0.0, absmax=0.0)
    d = ref.shape[-1]
    xs = np.moveaxis(x, head_axis, 0).reshape(x.shape[head_axis], -1, d)
    rs = np.moveaxis(ref, head_axis, 0).reshape(ref.shape[head_axis], -1, d)
    err = np.linalg.norm(xs - rs, axis=-1)            # (heads, rows)
    nrm = np.linalg.norm(rs, axis=-1)
    rms = np.sqrt(np.mean(nrm * nrm, axis=-1, keepdims=True))
    den = np.maximum(nrm, (ROW_FLOOR if floor is None else floor) * rms)
    with np.errstate(divide="ignore", invalid="ignore"):
        floored = np.where(den > 0, err / den, np.where(err > 0, np.inf, 0.0))
        raw = np.where(nrm > 0, err / nrm, np.where(err > 0, np.inf, 0.0))
    amax = float(np.max(np.abs(rs)))
    absmax = float(np.max(np.abs(xs - rs)) / amax) if amax > 0 else (0.0 if np.all(xs == rs) else np.inf)
    # where the worst unfloored row is: its norm and its error in units of its head's rms row norm
    hw, rw = np.unravel_index(int(np.argmax(raw)), raw.shape)
    r = float(rms[hw, 0]) if rms[hw, 0] > 0 else 1.0
    return dict(row=float(np.max(floored)), row_raw=float(np.max(raw)), absmax=absmax,
                raw_at_norm=float(nrm[hw, rw]) / r, raw_at_err=float(err[hw, rw]) / r)


def state_rows(S, S_ref, floor=None):
    """Row metric of states in the oracle's (H, d_k, d_v) orientation, one
    row per pool row (value column of S)."""
    return row_errors(np.swapaxes(S, -1, -2), np.swapaxes(S_ref, -1, -2), 0, floor)


class Worst:
    """Running maxima of the metrics of a test, asserted against one bar."""

    def __init__(self, tol, floor=None):
        self.tol = tol
        self.floor = floor   # row floor in units of the head's rms row norm (ROW_FLOOR if None)
        self.m = {}

    def add(self, key, stats):
        if isinstance(stats, dict):
            if stats.get("row_raw", 0.0) >= self.m.get(f"{key}.row_raw", 0.0):
                for k in ("raw_at_norm", "raw_at_err"):
                    if k in stats:
                        self.m[f"{key}.{k}"] = stats[k]
            for k, v in stats.items():
                if k in ("raw_at_norm", "raw_at_err"):
                    continue
                name = f"{key}.{k}"
                self.m[name] = max(self.m.get(name, 0.0), v)
        else:
            self.m[key] = max(self.m.get(key, 0.0), float(stats))

    def out(self, key, x, ref, head_axis):
        """Per-head Frobenius and row metrics of an output block."""
        self.add(key, rel_per_head(x, ref, head_axis))
        self.add(key, row_errors(x, ref, head_axis, self.floor))

    def state(self, key, S, S_ref):
        """Per-head Frobenius and row metrics of (H, d_k, d_v) states."""
        self.add(key, rel_per_head(S, S_ref, 0))
        self.add(key, state_rows(S, S_ref, self.floor))

    def check(self, label=""):
        """Assert every Frobenius and floored row metric is under the bar
        (the unfloored row and absmax numbers are reported only)."""
        fl = ROW_FLOOR if self.floor is None else self.floor
        print(f"[parity] {label} tol={self.tol:g} floor={fl:g} " +
              " ".join(f"{k}={v:.3g}" for k, v in sorted(self.m.items())), flush=True)
        for k, v in self.m.items():
            if k.split(".")[-1] in ("row_raw", "absmax", "raw_at_norm", "raw_at_err"):
                continue
            assert v < self.tol, (label, k, v, self.m)
        return self.m


def untouched(pool, slots, pool_dtype):
    """True if every slot in ``slots`` still holds the sentinel bit pattern."""
    if len(slots) == 0:
        return True
    sel = pool[torch.as_tensor(list(slots), device=pool.device, dtype=torch.long)]
    return bool((sel == SENTINEL[pool_dtype]).all().item())


def rne(x32, pool_dtype):
    """One RNE cast of an fp32 tensor into the pool dtype (torch's cast is RNE)."""
    return x32.to(wl.DTYPES[pool_dtype])
