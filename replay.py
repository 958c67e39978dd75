"""Kernel-level replay-consistency harness.

The state-semantics page (sec. 4, and the measurement to-do at its end) asks
whether output computed by resuming from a checkpoint matches output computed
straight through: the chunked prefill kernel and the recurrent verify kernel
reach the same tokens by different floating-point paths (and the checkpoint
itself is rounded to the pool dtype), so small differences are expected; the
page wants their size and the distribution of the first position at which
the resumed output departs from the original.  This harness measures that at
kernel level (no model, so there is no autoregressive feedback; a departure is
a position whose relative difference exceeds a tolerance):

1. one sequence of T tokens is prefilled once (chunk C), with snapshots of the
   state every ``every`` chunks written to pool slots in the pool dtype;
2. from each snapshot c, the verify kernel re-runs the next L tokens
   [c C, c C + L) -- the recurrent path resuming from the checkpoint;
3. per (checkpoint, position, head) the relative difference
   ||o_verify - o_prefill|| / ||o_prefill|| over the head's d_v outputs;
   per tolerance, the first position over it for each (checkpoint, head);
   and the fraction of output elements that are bitwise identical;
4. commit folds all L positions into a fresh slot, which is compared with the
   prefill's own snapshot L / C chunks later (same tokens, other path).

Everything runs through the library's C ABI (via the Python binding) on one
GPU; the comparisons are plain torch arithmetic on the results.

    python replay.py [--T 16384] [--heads 32] [--pool f32|bf16|f16] [--every 4] [--L 256]

prints one JSON line.
"""

from __future__ import annotations

import argparse
import json

import numpy as np
import torch

import linear_attention_state_kda_amd as kda
import workloads as wl

TAUS = (5e-3, 1e-2, 2e-2)   # the outputs are bf16: one rounding is up to 2^-9 ~ 2e-3 relative


def _i32(x, dev):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=dev)


def run(T=16384, H=32, d=128, C=64, pool_dtype="f32", every=4, L=256, seed=11, dev="cuda:0",
        taus=TAUS, keep=False):
    """Run the harness; returns a dict of statistics (and the raw tensors when
    ``keep``)."""
    if L % C or L > 256 or T < L + every * C:
        raise ValueError("need L a multiple of C, L <= 256 and T >= L + every * C")
    toks = wl.token_inputs(T, H, d, d, "bf16", seed)
    x = {n: toks[n].to(dev) for n in "qkvgb"}
    n_chunks = T // C
    ckpts = [c for c in range(every, n_chunks + 1, every) if c * C + L <= T]
    step = L // C
    # snapshots: every checkpoint, plus the chunk L / C later for the commit check
    snap = sorted(set(ckpts) | {c + step for c in ckpts})
    slot_of = {c: i for i, c in enumerate(snap)}
    final_slot = len(snap)
    commit_base = final_slot + 1
    n_slots = commit_base + len(ckpts)
    pool = torch.zeros((n_slots, H, d, d), dtype=wl.DTYPES[pool_dtype], device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    cu = _i32([0, T], dev)
    o_pre = kda.chunk_prefill(x["q"], x["k"], x["v"], x["g"], x["b"], cu, C, pool, _i32([-1], dev),
                              _i32([final_slot], dev), track_ptr=_i32([0, len(snap)], dev),
                              track_chunk=_i32(snap, dev), track_slot=_i32([slot_of[c] for c in snap], dev),
                              dev_err=err)
    # resume from each checkpoint: verify over the next L tokens
    starts = [c * C for c in ckpts]
    sp = {n: torch.stack([x[n][s:s + L] for s in starts]).contiguous() for n in "qkvgb"}
    ck = _i32([slot_of[c] for c in ckpts], dev)
    o_ver, u_rec, kg_rec = kda.recurrent_verify(sp["q"], sp["k"], sp["v"], sp["g"], sp["b"], pool, ck,
                                                dev_err=err)
    dst = _i32([commit_base + i for i in range(len(ckpts))], dev)
    kda.commit(pool, ck, _i32([L] * len(ckpts), dev), u_rec, kg_rec, dst_slot=dst, dev_err=err)
    torch.cuda.synchronize()
    if err.item() != 0:
        raise RuntimeError(f"device error flags {err.item()}")

    # per (checkpoint, position, head) relative output difference
    ref = torch.stack([o_pre[s:s + L] for s in starts]).float()            # [n_ck, L, H, d]
    diff = (o_ver.float() - ref).norm(dim=-1) / ref.norm(dim=-1).clamp_min(1e-30)   # [n_ck, L, H]
    stats = {"T": T, "H": H, "d": d, "chunk": C, "pool_dtype": pool_dtype, "in_dtype": "bf16",
             "L": L, "every_chunks": every, "checkpoints": len(ckpts), "pairs": len(ckpts) * H}
    stats["identical_fraction"] = (o_ver == torch.stack([o_pre[s:s + L] for s in starts])).float().mean().item()
    flat = diff.flatten()
    stats["rel_diff"] = {"max": flat.max().item(), "median": flat.median().item(),
                         "p99": torch.quantile(flat[:1 << 24], 0.99).item(),
                         "mean_by_position_band": {
                             f"{lo}-{hi - 1}": diff[:, lo:hi].mean().item()
                             for lo, hi in ((0, 1), (1, 8), (8, 64), (64, 256)) if hi <= L}}
    first = {}
    for tau in taus:
        over = diff > tau                                                   # [n_ck, L, H]
        pos = torch.where(over.any(dim=1), over.float().argmax(dim=1), torch.full_like(over[:, 0], L,
                          dtype=torch.float32)).flatten()                   # first t over tau, L if none
        never = (pos >= L).float().mean().item()
        hit = pos[pos < L]
        first[f"{tau:g}"] = {"never_fraction": never,
                             "first_position_quantiles": None if hit.numel() == 0 else {
                                 q: torch.quantile(hit, q).item() for q in (0.0, 0.1, 0.5, 0.9)}}
    stats["first_over_tolerance"] = first
    # commit after L positions vs the prefill's snapshot L / C chunks later
    sc = []
    for i, c in enumerate(ckpts):
        a = pool[commit_base + i].float()
        b = pool[slot_of[c + step]].float()
        sc.append(((a - b).flatten(1).norm(dim=1) / b.flatten(1).norm(dim=1)).max().item())
    stats["commit_vs_snapshot_rel"] = {"max": max(sc), "median": float(np.median(sc))}
    if keep:
        stats["_tensors"] = dict(toks=toks, o_pre=o_pre, o_ver=o_ver, pool=pool, ckpts=ckpts,
                                 slot_of=slot_of, commit_base=commit_base, diff=diff)
    return stats


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--T", type=int, default=16384)
    ap.add_argument("--heads", type=int, default=32)
    ap.add_argument("--pool", default="f32", choices=sorted(wl.DTYPES))
    ap.add_argument("--every", type=int, default=4)
    ap.add_argument("--L", type=int, default=256)
    ap.add_argument("--seed", type=int, default=11)
    a = ap.parse_args()
    s = run(T=a.T, H=a.heads, pool_dtype=a.pool, every=a.every, L=a.L, seed=a.seed)
    print(json.dumps(s), flush=True)


if __name__ == "__main__":
    main()
