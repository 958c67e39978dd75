"""Seeded synthetic inputs for the KDA state recurrence.

This module serves both sides of every parity check (the HIP library through
its binding, and the fp64 oracle) and holds none of the method's arithmetic:
it only draws random numbers, normalises q and k, rounds values to the input
or pool dtype (round-to-nearest-even, via torch's CPU casts) and lays the
buffers out.  The oracle receives the exact rounded values as float64.

Recipe (the workload shapes of the prefill and speculative-decode paths):
  * q, k ~ N(0, 1), then L2-normalised per (token, head) over d_k in fp64;
  * v ~ N(0, 1); beta logit b ~ N(0, 1) (beta = sigmoid(b));
  * g = log alpha ~ U(-0.1, -0.001) per key channel;
  * everything rounded once to the input dtype;
  * pool states ~ N(0, 1), rounded once to the pool dtype.
Each tensor is drawn per head from its own stream
``numpy.random.default_rng([seed, tag, head])`` so that any subset of heads
can be regenerated without the rest.  Integer draws (lengths, slots,
accepted lengths, snapshot chunks) use ``default_rng([seed, tag])``.

Layouts (shared with the C ABI):
  tokens  q, k, g: [T_total, H, d_k]; v, o: [T_total, H, d_v]; b: [T_total, H]
  spec    q, k, g: [n_req, L, H, d_k]; v: [n_req, L, H, d_v]; b: [n_req, L, H]
  pool    [n_slots, H, d_v, d_k]  (the transpose of the (d_k, d_v) state)
"""

from __future__ import annotations

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

TAG_Q, TAG_K, TAG_V, TAG_B, TAG_G = 1, 2, 3, 4, 5
TAG_LEN, TAG_SLOT, TAG_POOL, TAG_ACC, TAG_TRACK = 6, 7, 8, 9, 10

G_LO, G_HI = -0.1, -0.001


def _rng(*key):
    return np.random.default_rng([int(x) for x in key])


def to_dtype(x64, dtype):
    """Round a float64 array once (RNE) into a CPU torch tensor of ``dtype``."""
    return torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float64)).to(DTYPES[dtype])


def exact(t):
    """float64 NumPy copy of a CPU torch tensor (exact: every dtype here embeds in fp64)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def token_inputs(n_tokens, H, dk, dv, in_dtype, seed, shape_prefix=None, heads=None):
    """Draw q, k, v, g, b for ``n_tokens`` token rows of H heads.

    Returns a dict of CPU torch tensors in ``in_dtype``.  ``shape_prefix``
    reshapes the leading token axis (e.g. (n_req, L) for the spec layout).
    ``heads`` draws only those heads (the head axis then follows that
    list): each head has its own streams, so the values are the same as in
    the full draw.
    """
    T = int(n_tokens)
    dt = DTYPES[in_dtype]
    hs = list(range(H)) if heads is None else [int(x) for x in heads]
    n_h = len(hs)
    q = torch.empty((T, n_h, dk), dtype=dt)
    k = torch.empty((T, n_h, dk), dtype=dt)
    v = torch.empty((T, n_h, dv), dtype=dt)
    g = torch.empty((T, n_h, dk), dtype=dt)
    b = torch.empty((T, n_h), dtype=dt)
    for j, h in enumerate(hs):
        q[:, j] = to_dtype(_unit_rows(_rng(seed, TAG_Q, h).standard_normal((T, dk))), in_dtype)
        k[:, j] = to_dtype(_unit_rows(_rng(seed, TAG_K, h).standard_normal((T, dk))), in_dtype)
        v[:, j] = to_dtype(_rng(seed, TAG_V, h).standard_normal((T, dv)), in_dtype)
        b[:, j] = to_dtype(_rng(seed, TAG_B, h).standard_normal(T), in_dtype)
        g[:, j] = to_dtype(_rng(seed, TAG_G, h).uniform(G_LO, G_HI, (T, dk)), in_dtype)
    out = {"q": q, "k": k, "v": v, "g": g, "b": b}
    if shape_prefix is not None:
        pre = tuple(int(x) for x in shape_prefix)
        out = {n: t.reshape(pre + tuple(t.shape[1:])) for n, t in out.items()}
    return out


def pool_state(slot, H, dk, dv, pool_dtype, seed):
    """Contents of one pool slot, [H, d_v, d_k], rounded to the pool dtype."""
    return to_dtype(_rng(seed, TAG_POOL, slot).standard_normal((H, dv, dk)), pool_dtype)


def distinct_slots(n, n_slots, seed, tag=TAG_SLOT, exclude=()):
    """``n`` distinct slot ids in [0, n_slots), none of them in ``exclude``."""
    free = np.setdiff1d(np.arange(n_slots), np.asarray(list(exclude), dtype=np.int64))
    if n > free.size:
        raise ValueError("not enough free slots")
    return _rng(seed, tag).permutation(free)[:n].astype(np.int32)


# --------------------------------------------------------------------------
# Workload descriptions.  A prefill case is a dict with
#   lengths, H, dk, dv, chunk, in_dtype, pool_dtype, n_slots,
#   init_slots (-1 = zero state), final_slots, tracks [(seq, c, slot)],
#   track_f32 (bool), seed
# A spec case has n_req, L, H, dk, dv, in_dtype, pool_dtype, n_slots,
#   ckpt_slots, accepted, fork_src, fork_dst, seed.
# --------------------------------------------------------------------------

def prefill_case(lengths, H, dk, dv, chunk, in_dtype, pool_dtype, n_slots,
                 init_slots, final_slots, tracks, track_f32=True, seed=0, name=""):
    return dict(name=name, lengths=[int(x) for x in lengths], H=H, dk=dk, dv=dv,
                chunk=chunk, in_dtype=in_dtype, pool_dtype=pool_dtype,
                n_slots=int(n_slots), init_slots=[int(x) for x in init_slots],
                final_slots=[int(x) for x in final_slots],
                tracks=[(int(s), int(c), int(sl)) for s, c, sl in tracks],
                track_f32=bool(track_f32), seed=int(seed))


def tiny_prefill(seed=0):
    """1 sequence, T = 64, H = 2, d_k = d_v = 16, chunk 16, fp32 throughout;
    zero initial state; final state to slot 1 and the snapshot after chunk 2
    (32 tokens) to slot 2 of a 4-slot fp32 pool, plus the fp32 snapshot."""
    return prefill_case([64], 2, 16, 16, 16, "f32", "f32", 4, [-1], [1], [(0, 2, 2)],
                        True, seed, "tiny T=64 H=2 d=16 C=16 f32")


def single_layer_prefill(seed=1):
    """1 sequence, T = 8229 (128 full chunks + a tail of 37), H = 32 heads,
    d_k = d_v = 128, chunk 64, bf16 inputs, fp32 pool, zero initial state,
    snapshot at the last full chunk boundary (c = 128)."""
    return prefill_case([8229], 32, 128, 128, 64, "bf16", "f32", 4, [-1], [0], [(0, 128, 1)],
                        True, seed, "single-layer T=8229 H=32 d=128 C=64 bf16")


def varlen_prefill(pool_dtype="f32", seed=2, n_seqs=16, H=32, lo=512, hi=16384, n_slots=1024, in_dtype="bf16"):
    """16 packed sequences with lengths ~ U[512, 16384], H = 32, d = 128,
    chunk 64, bf16 inputs (or in_dtype); initial states from 16 distinct random slots of a
    1024-slot pool; final states and one snapshot per sequence (chunk
    c_i ~ U{1..floor(T_i/64)}) to fresh slots, plus the fp32 snapshots."""
    lengths = _rng(seed, TAG_LEN).integers(lo, hi + 1, n_seqs)
    slots = distinct_slots(3 * n_seqs, n_slots, seed)
    init, final, trk = slots[:n_seqs], slots[n_seqs:2 * n_seqs], slots[2 * n_seqs:]
    cs = [int(_rng(seed, TAG_TRACK, i).integers(1, max(1, L // 64) + 1)) for i, L in enumerate(lengths)]
    tracks = [(i, cs[i], int(trk[i])) for i in range(n_seqs)]
    return prefill_case(lengths, H, 128, 128, 64, in_dtype, pool_dtype, n_slots, init, final,
                        tracks, True, seed, f"varlen {n_seqs} seqs H={H} d=128 C=64 {in_dtype} pool={pool_dtype}")


def long_prefill(seed=4, T=131072, H=32):
    """1 sequence, T = 131072, H = 32, d = 128, chunk 64, bf16, zero initial
    state, fp32 pool; snapshots every 64 chunks (c = 64 m, m = 1..T/4096)
    plus anchors c = 64 m + 4 for m in {1, 16, 31}."""
    n_blocks = T // 4096
    cs = [64 * m for m in range(1, n_blocks + 1)]
    anchors = [64 * m + 4 for m in (1, 16, 31) if 64 * m + 4 <= T // 64]
    tracks = [(0, c, 2 + i) for i, c in enumerate(cs + anchors)]
    return prefill_case([T], H, 128, 128, 64, "bf16", "f32", 2 + len(tracks), [-1], [0],
                        tracks, True, seed, f"long T={T} H={H} d=128 C=64 bf16")


def spec_case(n_req=256, L=8, H=32, d=128, in_dtype="bf16", pool_dtype="f32", n_slots=1024,
              n_fork_src=64, fanout=4, seed=3):
    """Speculative decode: n_req requests, one checkpoint slot each, L
    speculative positions, accepted length ~ U{0..L}; in-place commit; then
    a fork of n_fork_src committed checkpoints to ``fanout`` fresh children."""
    ckpt = distinct_slots(n_req, n_slots, seed)
    acc = _rng(seed, TAG_ACC).integers(0, L + 1, n_req).astype(np.int32)
    src = ckpt[_rng(seed, TAG_SLOT + 100).permutation(n_req)[:n_fork_src]]
    dst = distinct_slots(n_fork_src * fanout, n_slots, seed + 1000, exclude=ckpt)
    return dict(name=f"spec n_req={n_req} L={L} H={H} d={d} {in_dtype} pool={pool_dtype}",
                n_req=n_req, L=L, H=H, dk=d, dv=d, in_dtype=in_dtype, pool_dtype=pool_dtype,
                n_slots=n_slots, ckpt_slots=ckpt, accepted=acc,
                fork_src=np.repeat(src, fanout).astype(np.int32), fork_dst=dst, seed=seed)


def prefill_tokens(case):
    """Token tensors for a prefill case plus its cu_seqlens (int32)."""
    T = sum(case["lengths"])
    toks = token_inputs(T, case["H"], case["dk"], case["dv"], case["in_dtype"], case["seed"])
    cu = np.zeros(len(case["lengths"]) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(case["lengths"])
    return toks, cu
