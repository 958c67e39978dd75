"""Long-context prefill and replay consistency on the GPU (through the C ABI).

Workload: one sequence of T = 131072 tokens, H = 32, d = 128, chunk 64, bf16
inputs, fp32 pool, zero initial state; snapshots every 64 chunks
(c = 64 m, m = 1..32, the last one being the final state) and anchors at
c = 64 m + 4 for m in {1, 16, 31}.  For those m, the recurrent verify kernel
re-runs the 256 tokens [4096 m, 4096 m + 256) from snapshot 64 m and commit
folds all 256 positions in; that state must match anchor 64 m + 4 (the
chunked path's state 256 tokens later) and the oracle, and the verify
outputs must match the prefill outputs at those positions.  This is the
kernel-level part of the replay-consistency question (state-semantics page,
sec. 4 and the closing to-do list): the chunk kernel and the recurrent
kernel take different floating-point paths, so the test reports their
difference and bounds both against the fp64 oracle (2e-2 relative).
The oracle runs on two sampled heads over the whole sequence, and on all 32
heads over three 4096-token windows, each started from the kernel's own fp32
snapshot at the window's start and compared row by row (outputs) and with the
next snapshot.
"""

import numpy as np
import pytest
import torch

import linear_attention_state_kda_amd as kda
import workloads as wl
from oracle import kda_oracle as ko
from tests.gpu_util import DEV, Worst, i32, make_pool, rel_per_head, to_math

pytestmark = pytest.mark.gpu

HEADS = [0, 17]


def test_long_context_prefill_and_replay():
    case = wl.long_prefill()
    T, H, d, C = case["lengths"][0], case["H"], case["dk"], case["chunk"]
    toks, cu = wl.prefill_tokens(case)
    dev = {n: toks[n].to(DEV) for n in "qkvgb"}
    pool = make_pool(case["n_slots"] + 3, H, d, d, "f32")
    tracks = case["tracks"]
    n_track = len(tracks)
    track_f32 = torch.empty((n_track, H, d, d), dtype=torch.float32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    o = kda.chunk_prefill(dev["q"], dev["k"], dev["v"], dev["g"], dev["b"], i32(cu), C, pool,
                          i32([-1]), i32(case["final_slots"]), track_ptr=i32([0, n_track]),
                          track_chunk=i32([t[1] for t in tracks]),
                          track_slot=i32([t[2] for t in tracks]), track_f32=track_f32, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0

    # ---- oracle on sampled heads: outputs everywhere, every snapshot, final
    ex = {n: wl.exact(toks[n][:, HEADS]) for n in "qkvgb"}
    keep = sorted({c * C for _, c, _ in tracks})
    o_ref, _, S_T, kept = ko.run_sequence(ex["q"], ex["k"], ex["v"], ex["g"], ex["b"],
                                          np.zeros((len(HEADS), d, d)), keep_after=keep)
    hsel = torch.as_tensor(HEADS, device=DEV)
    o_gpu = wl.exact(o[:, hsel].cpu())
    assert rel_per_head(o_gpu, o_ref, 1) < 2e-2
    # per 4096-token block as well, so an error late in the sequence is not averaged away
    for lo in range(0, T, 4096):
        assert rel_per_head(o_gpu[lo:lo + 4096], o_ref[lo:lo + 4096], 1) < 2e-2
    worst_snap = 0.0
    for e, (_, c, slot) in enumerate(tracks):
        got = to_math(track_f32[e][hsel])
        worst_snap = max(worst_snap, rel_per_head(got, kept[c * C], 0))
        assert torch.equal(pool[slot], track_f32[e])        # fp32 pool: the cast is exact
    assert worst_snap < 2e-2
    assert rel_per_head(to_math(pool[case["final_slots"][0]][hsel]), S_T, 0) < 2e-2
    w = Worst(2e-2)
    w.out("o", o_gpu, o_ref, 1)
    w.state("final", to_math(pool[case["final_slots"][0]][hsel]), S_T)
    w.check("long T=131072 heads 0,17 whole sequence")

    # ---- all heads on three 4096-token windows, each from the kernel's fp32
    #      snapshot at its start: outputs row by row and the next snapshot
    e_of = {c: e for e, (_, c, _) in enumerate(tracks)}
    for m in (1, 16, 31):
        lo, hi = 4096 * m, 4096 * (m + 1)
        S_start = to_math(track_f32[e_of[64 * m]])
        exw = {n: wl.exact(toks[n][lo:hi]) for n in "qkvgb"}
        o_w, _, S_w, _ = ko.run_sequence(exw["q"], exw["k"], exw["v"], exw["g"], exw["b"], S_start)
        ww = Worst(2e-2)
        ww.out("o", wl.exact(o[lo:hi].cpu()), o_w, 1)
        ww.state("snap", to_math(track_f32[e_of[64 * (m + 1)]]), S_w)
        ww.check(f"long T=131072 all heads, tokens [{lo}, {hi}) from the fp32 snapshot c={64 * m}")

    # ---- replay: verify 256 tokens from snapshot 64 m, commit, compare with anchor 64 m + 4
    L = 256
    ms = [1, 16, 31]
    slot_of = {c: slot for _, c, slot in tracks}
    starts = [4096 * m for m in ms]
    sp = {n: torch.stack([dev[n][s:s + L] for s in starts]).contiguous() for n in "qkvgb"}
    ckpt = i32([slot_of[64 * m] for m in ms])
    vo, u_rec, kg_rec = kda.recurrent_verify(sp["q"], sp["k"], sp["v"], sp["g"], sp["b"], pool, ckpt,
                                             dev_err=err)
    dst = i32([case["n_slots"], case["n_slots"] + 1, case["n_slots"] + 2])
    kda.commit(pool, ckpt, i32([L, L, L]), u_rec, kg_rec, dst_slot=dst, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    report = []
    wr = Worst(2e-2)
    for i, m in enumerate(ms):
        s = starts[i]
        anchor = to_math(pool[slot_of[64 * m + 4]][hsel])
        committed = to_math(pool[int(dst[i])][hsel])
        oracle_state = kept[s + L]
        # recurrent (verify + commit) vs chunked (anchor) vs oracle
        assert rel_per_head(committed, oracle_state, 0) < 2e-2
        assert rel_per_head(anchor, oracle_state, 0) < 2e-2
        diff = rel_per_head(committed, anchor, 0)
        assert diff < 2e-2
        vo_h = wl.exact(vo[i][:, hsel].cpu())
        assert rel_per_head(vo_h, o_ref[s:s + L], 1) < 2e-2
        assert rel_per_head(vo_h, o_gpu[s:s + L], 1) < 2e-2
        report.append((m, diff, rel_per_head(committed, oracle_state, 0), rel_per_head(anchor, oracle_state, 0)))
        wr.state("committed", committed, oracle_state)
        wr.state("anchor", anchor, oracle_state)
        wr.out("verify_o", vo_h, o_ref[s:s + L], 1)
    wr.check("long T=131072 replay: verify+commit of 256 tokens vs oracle, heads 0,17")
    print("replay (m, |recurrent-chunked|, recurrent vs oracle, chunked vs oracle):", report)
