"""GPU parity of kda_chunk_prefill through the C ABI against the fp64 oracle.

Cases: the tiny fp32 workload (T = 64, H = 2, d = 16, chunk 16); small
multi-sequence bf16/fp16 runs at d = 128, chunk 64 that span several chunks,
ragged tails, an empty and a one-token sequence, pool and zero initial
states, and snapshots at c = 0, interior chunks and c = floor(T_i / C), with
16-, 32- and 64-column scan tiles (by the number of (sequence, head) pairs); the
single-layer workload (T = 8229, H = 32) in full; the varlen workload (16
sequences, lengths 512..16384) on sampled heads with fp32, fp16 and bf16
pools; and device-side error reporting.

Checks: outputs, final states and snapshots within the bar (1e-4 relative for
fp32 inputs, 2e-2 for 16-bit inputs); every pool write is one RNE cast of the
fp32 value (pool slot == cast(track_f32) bitwise); the fp32 snapshot is
strictly closer to the oracle than its bf16 rounding; untouched pool slots
keep their sentinel bits; two runs are bitwise identical.
"""

import numpy as np
import pytest
import torch

import linear_attention_state_kda_amd as kda
import workloads as wl
from oracle import kda_oracle as ko
from tests.gpu_util import DEV, TOL, Worst, i32, make_pool, rne, to_math, untouched

pytestmark = pytest.mark.gpu


_TOKENS = {}


def tokens(case):
    """Seeded token tensors of a case, cached across parametrisations."""
    key = (tuple(case["lengths"]), case["H"], case["dk"], case["dv"], case["in_dtype"], case["seed"])
    if key not in _TOKENS:
        _TOKENS.clear()
        _TOKENS[key] = wl.prefill_tokens(case)
    return _TOKENS[key]


def csr_tracks(case):
    """Sort the (seq, c, slot) requests by sequence into the CSR arrays."""
    n = len(case["lengths"])
    order = sorted(range(len(case["tracks"])), key=lambda e: case["tracks"][e][0])
    tr = [case["tracks"][e] for e in order]
    ptr = np.zeros(n + 1, dtype=np.int32)
    for s, _, _ in tr:
        ptr[s + 1] += 1
    return np.cumsum(ptr).astype(np.int32), tr


def run_gpu(case, toks, cu, pool=None, repeat=1):
    H, dk, dv, C = case["H"], case["dk"], case["dv"], case["chunk"]
    pdt = case["pool_dtype"]
    if pool is None:
        pool = make_pool(case["n_slots"], H, dk, dv, pdt)
        for s in case["init_slots"]:
            if s >= 0:
                pool[s] = wl.pool_state(s, H, dk, dv, pdt, case["seed"]).to(DEV)
    ptr, tr = csr_tracks(case)
    n_track = len(tr)
    track_f32 = torch.full((max(n_track, 1), H, dv, dk), float("nan"), device=DEV) if case["track_f32"] else None
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    dev = {n: toks[n].to(DEV) for n in "qkvgb"}
    outs = []
    for _ in range(repeat):
        o = kda.chunk_prefill(dev["q"], dev["k"], dev["v"], dev["g"], dev["b"], i32(cu), C, pool,
                              i32(case["init_slots"]), i32(case["final_slots"]),
                              track_ptr=i32(ptr), track_chunk=i32([t[1] for t in tr]),
                              track_slot=i32([t[2] for t in tr]), track_f32=track_f32, dev_err=err)
        outs.append(o)
    torch.cuda.synchronize()
    return dict(o=outs[-1], outs=outs, pool=pool, track_f32=track_f32, err=int(err.item()), tr=tr)


def oracle(case, toks, cu, heads, seqs=None):
    """Oracle outputs, final states and snapshots on ``heads`` for the
    sequences ``seqs`` (all by default); o is returned for those sequences'
    token ranges (zeros elsewhere) and snaps for their tracks (None elsewhere)."""
    H, dk, dv, C = case["H"], case["dk"], case["dv"], case["chunk"]
    n = len(case["lengths"])
    seqs = list(range(n)) if seqs is None else list(seqs)
    _, tr = csr_tracks(case)
    T = int(cu[-1])
    o = np.zeros((T, len(heads), dv))
    finals = [None] * n
    snaps = [None] * len(tr)
    for i in seqs:
        lo, hi = int(cu[i]), int(cu[i + 1])
        ex = {x: wl.exact(toks[x][lo:hi])[:, heads] for x in "qkvgb"}
        S0 = np.zeros((1, len(heads), dk, dv))
        s = case["init_slots"][i]
        if s >= 0:
            S0[0] = np.swapaxes(wl.exact(wl.pool_state(s, H, dk, dv, case["pool_dtype"], case["seed"])),
                                -1, -2)[heads]
        mine = [e for e, t in enumerate(tr) if t[0] == i]
        o_i, fin_i, snaps_i = ko.prefill_ref(ex["q"], ex["k"], ex["v"], ex["g"], ex["b"], [0, hi - lo], S0, C,
                                             [(0, tr[e][1]) for e in mine])
        o[lo:hi] = o_i
        finals[i] = fin_i[0]
        for e, sn in zip(mine, snaps_i):
            snaps[e] = sn
    return o, finals, snaps


def check_case(case, toks, cu, g, heads, check_untouched=True, seqs=None, label=""):
    """Compare a GPU run with the oracle on ``heads`` (and the sequences
    ``seqs``, all by default) and run the rounding checks."""
    n = len(case["lengths"])
    seqs = list(range(n)) if seqs is None else list(seqs)
    w = Worst(TOL[case["in_dtype"]])
    assert g["err"] == 0, f"device error bits {g['err']}"
    o_ref, fin_ref, snaps = oracle(case, toks, cu, heads, seqs)
    hsel = torch.as_tensor(heads, device=DEV)
    o = wl.exact(g["o"][:, hsel].cpu())
    for i in seqs:
        lo, hi = int(cu[i]), int(cu[i + 1])
        if hi > lo:
            w.out("o", o[lo:hi], o_ref[lo:hi], 1)
        fs = case["final_slots"][i]
        if fs >= 0:
            w.state("final", to_math(g["pool"][fs][hsel]), fin_ref[i])
    pdt = case["pool_dtype"]
    for e, (s, c, slot) in enumerate(g["tr"]):
        if s not in seqs:
            continue
        ref = snaps[e]
        if g["track_f32"] is not None:
            snap32 = g["track_f32"][e]
            got = to_math(snap32[hsel])
            w.state("snap", got, ref)
            if c == 0:
                # before the first chunk the snapshot is the initial state itself
                assert np.array_equal(got, ref)
            else:
                # fp32 snapshot strictly closer than its bf16 rounding
                via_bf16 = to_math(snap32.to(torch.bfloat16)[hsel])
                assert np.linalg.norm(got - ref) < np.linalg.norm(via_bf16 - ref)
            if slot >= 0:
                # exactly one RNE cast from the fp32 accumulator into the pool
                assert torch.equal(g["pool"][slot], rne(snap32, pdt))
        elif slot >= 0:
            w.state("snap", to_math(g["pool"][slot][hsel]), ref)
    worst = w.check(label or case.get("name", ""))
    if check_untouched:
        written = set(case["init_slots"]) | set(case["final_slots"]) | {t[2] for t in case["tracks"]}
        others = sorted(set(range(case["n_slots"])) - written)
        assert untouched(g["pool"], others, pdt)
    return worst


# ---------------------------------------------------------------- tiny fp32

def test_tiny_fp32():
    case = wl.tiny_prefill()
    toks, cu = tokens(case)
    g = run_gpu(case, toks, cu)
    w = check_case(case, toks, cu, g, list(range(case["H"])))
    print("tiny fp32 worst rel", w)


def test_tiny_fp32_varlen_and_init():
    case = wl.prefill_case([37, 0, 16, 1, 64, 50], 2, 16, 16, 16, "f32", "f32", 16,
                           init_slots=[3, -1, 4, 5, -1, 6], final_slots=[7, 8, 9, 10, 11, 12],
                           tracks=[(0, 0, 13), (0, 2, 14), (4, 4, 15), (2, 1, -1), (5, 3, -1), (1, 0, -1)],
                           track_f32=True, seed=7)
    toks, cu = tokens(case)
    g = run_gpu(case, toks, cu)
    check_case(case, toks, cu, g, [0, 1])


# ---------------------------------------------------------------- d = 128, chunk 64

SMALL_LENS = [300, 64, 1, 0, 130, 37, 128]


@pytest.mark.parametrize("in_dtype,pool_dtype", [("bf16", "f32"), ("bf16", "bf16"), ("bf16", "f16"),
                                                  ("f16", "f32")])
def test_small_multi_sequence(in_dtype, pool_dtype):
    n = len(SMALL_LENS)
    init = [20, -1, 21, 22, -1, 23, -1]
    final = [0, 1, 2, 3, 4, 5, 6]
    tracks = [(0, 0, 7), (0, 2, 8), (0, 4, 9), (1, 1, 10), (4, 1, 11), (4, 2, 12), (5, 0, 13),
              (6, 2, 14), (6, 1, -1), (3, 0, 15)]
    case = wl.prefill_case(SMALL_LENS, 3, 128, 128, 64, in_dtype, pool_dtype, 24, init, final,
                           tracks, True, seed=11)
    toks, cu = tokens(case)
    g = run_gpu(case, toks, cu)
    w = check_case(case, toks, cu, g, [0, 1, 2])
    print(in_dtype, pool_dtype, "worst rel", w)


@pytest.mark.parametrize("H,in_dtype,pool_dtype", [(8, "bf16", "f32"), (12, "bf16", "bf16"),
                                                     (12, "bf16", "f32"), (12, "f16", "f16")])
def test_wide_column_tiles(H, in_dtype, pool_dtype):
    """Enough (sequence, head) pairs that the scan takes wider column tiles:
    7 x 8 = 56 pairs (32-column tiles), 7 x 12 = 84 pairs (64-column tiles);
    every head checked against the oracle."""
    init = [20, -1, 21, 22, -1, 23, -1]
    final = [0, 1, 2, 3, 4, 5, 6]
    tracks = [(0, 0, 7), (0, 2, 8), (0, 4, 9), (1, 1, 10), (4, 1, 11), (4, 2, 12), (5, 0, 13),
              (6, 2, 14), (6, 1, -1), (3, 0, 15)]
    case = wl.prefill_case(SMALL_LENS, H, 128, 128, 64, in_dtype, pool_dtype, 24, init, final,
                           tracks, True, seed=16)
    toks, cu = tokens(case)
    g = run_gpu(case, toks, cu)
    w = check_case(case, toks, cu, g, list(range(H)))
    print("wide tiles H", H, in_dtype, pool_dtype, "worst rel", w)


@pytest.mark.parametrize("H", [2, 12, 16])
def test_leading_empty_sequences(H):
    """Empty sequences first (chunk offset 0 on head 0): nothing of theirs is
    read from the workspace; their final state is the initial state cast
    once; the sequences after them are unaffected.  H = 12 and 16 take the
    32- and 64-column tiles."""
    lens = [0, 0, 70, 0, 64]
    case = wl.prefill_case(lens, H, 128, 128, 64, "bf16", "f32", 12, [5, -1, 6, 7, -1],
                           [0, 1, 2, 3, 4], [(0, 0, 8), (2, 1, 9)], True, seed=17)
    toks, cu = tokens(case)
    g = run_gpu(case, toks, cu)
    check_case(case, toks, cu, g, list(range(H)))


def test_final_over_own_init_slot():
    case = wl.prefill_case([200, 77], 2, 128, 128, 64, "bf16", "f32", 4, [0, 1], [0, 1],
                           [(0, 3, 2)], True, seed=12)
    toks, cu = tokens(case)
    g = run_gpu(case, toks, cu)
    check_case(case, toks, cu, g, [0, 1])


def test_single_sequence_inside_the_buffer():
    """One sequence that starts past the buffer's first token and ends before
    its last (cu_seqlens = [100, 330] over 400 tokens: three full chunks and
    a 38-token tail): a single sequence gets no chunk map, so its records
    take chunk slots from 0 while its tokens start at row 100."""
    case = wl.prefill_case([400], 4, 128, 128, 64, "bf16", "f32", 4, [1], [2], [(0, 2, 3)], True, seed=17)
    toks, _ = tokens(case)
    cu = np.array([100, 330], dtype=np.int32)
    g = run_gpu(case, toks, cu)
    check_case(case, toks, cu, g, list(range(4)))


@pytest.mark.parametrize("length", [0, 1, 64, 65])
def test_single_sequence_edge_lengths(length):
    """One sequence, so no chunk map: empty (a zero-token buffer: the final
    state and the chunk-0 snapshot are the initial state cast once), one
    token, exactly one chunk (its end snapshot is the final state), one
    chunk and one token."""
    tracks = [(0, 0, 2)] + ([(0, length // 64, 3)] if length >= 64 else [])
    case = wl.prefill_case([length], 2, 128, 128, 64, "bf16", "f32", 6, [4], [1], tracks, True,
                           seed=18 + length)
    toks, cu = tokens(case)
    g = run_gpu(case, toks, cu)
    check_case(case, toks, cu, g, [0, 1])


def test_bitwise_deterministic():
    case = wl.prefill_case([500, 70], 4, 128, 128, 64, "bf16", "f32", 4, [-1, -1], [0, 1],
                           [(0, 5, 2)], True, seed=13)
    toks, cu = tokens(case)
    g = run_gpu(case, toks, cu, repeat=2)
    assert torch.equal(g["outs"][0], g["outs"][1])


def test_device_errors_are_flagged():
    # track chunk beyond floor(T/C), track slot and final slot out of range
    case = wl.prefill_case([100], 2, 128, 128, 64, "bf16", "f32", 4, [-1], [9],
                           [(0, 2, 1), (0, 1, 77)], True, seed=14)
    toks, cu = tokens(case)
    g = run_gpu(case, toks, cu)
    assert g["err"] & kda.DEV_ERR_TRACK
    assert g["err"] & kda.DEV_ERR_SLOT
    assert untouched(g["pool"], [0, 1, 2, 3], "f32")
    # malformed cu_seqlens: the bad sequence is skipped and flagged
    case2 = wl.prefill_case([64, 64], 2, 128, 128, 64, "bf16", "f32", 4, [-1, -1], [0, 1], [], False, seed=15)
    toks2, _ = tokens(case2)
    bad_cu = np.array([0, 100, 90], dtype=np.int32)
    g2 = run_gpu(case2, toks2, bad_cu)
    assert g2["err"] & kda.DEV_ERR_SEQLEN
    # a single sequence has no chunk map: its scan flags the pair itself and
    # writes nothing (beyond the 64 tokens, negative start, decreasing)
    case3 = wl.prefill_case([64], 2, 128, 128, 64, "bf16", "f32", 4, [-1], [0], [], False, seed=16)
    toks3, _ = tokens(case3)
    for bad in ([0, 100], [-1, 10], [40, 20]):
        g3 = run_gpu(case3, toks3, np.array(bad, dtype=np.int32))
        assert g3["err"] & kda.DEV_ERR_SEQLEN, bad
        assert untouched(g3["pool"], [0, 1, 2, 3], "f32"), bad


# ---------------------------------------------------------------- full-size workloads

def test_single_layer_full():
    """T = 8229, H = 32, d = 128, chunk 64, bf16, fp32 pool, snapshot at
    c = 128: every head against the oracle."""
    case = wl.single_layer_prefill()
    toks, cu = tokens(case)
    g = run_gpu(case, toks, cu)
    w = check_case(case, toks, cu, g, list(range(32)))
    print("single-layer worst rel", w)


def test_single_layer_fp16_sampled_heads():
    """The single-layer shape (T = 8229: 128 chunks and a 37-token tail,
    H = 32) with fp16 inputs and an fp16 pool from a pool initial state:
    heads 0, 13 and 31 against the oracle over the whole sequence, and the
    snapshot at c = 128 rounded once into the pool."""
    case = wl.prefill_case([8229], 32, 128, 128, 64, "f16", "f16", 4, [2], [0], [(0, 128, 1)], True, seed=19,
                           name="single-layer fp16")
    toks, cu = tokens(case)
    g = run_gpu(case, toks, cu)
    w = check_case(case, toks, cu, g, [0, 13, 31])
    print("single-layer fp16 worst", w)


@pytest.mark.parametrize("pool_dtype", ["f32", "f16", "bf16"])
def test_varlen_sampled_heads(pool_dtype):
    """16 sequences (lengths 512..16384), H = 32, per-sequence snapshots,
    random initial slots of a 1024-slot pool, one run at full shape (64-column
    scan tiles, 512 (sequence, head) pairs): the oracle on heads 0 and 21 of
    every sequence, and on all 32 heads of the four shortest sequences
    (outputs, final states and snapshots of every head)."""
    case = wl.varlen_prefill(pool_dtype=pool_dtype)
    toks, cu = tokens(case)
    g = run_gpu(case, toks, cu)
    w = check_case(case, toks, cu, g, [0, 21], label=f"varlen pool={pool_dtype} heads 0,21")
    shortest = sorted(range(len(case["lengths"])), key=lambda i: case["lengths"][i])[:4]
    w_all = check_case(case, toks, cu, g, list(range(case["H"])), check_untouched=False, seqs=shortest,
                       label=f"varlen pool={pool_dtype} all heads of seqs {shortest} "
                             f"(lengths {[case['lengths'][i] for i in shortest]})")
    print("varlen", pool_dtype, "worst", w, w_all)


def test_varlen_fp16_inputs():
    """The varlen batch at full shape with fp16 inputs and an fp16 pool (the
    64-column fp16 scan tiles): the oracle on heads 0 and 21 of every
    sequence and on all 32 heads of the two shortest sequences, including
    each snapshot's single rounding into the pool."""
    case = wl.varlen_prefill(pool_dtype="f16", in_dtype="f16", seed=5)
    toks, cu = tokens(case)
    g = run_gpu(case, toks, cu)
    w = check_case(case, toks, cu, g, [0, 21], label="varlen fp16 heads 0,21")
    shortest = sorted(range(len(case["lengths"])), key=lambda i: case["lengths"][i])[:2]
    w_all = check_case(case, toks, cu, g, list(range(case["H"])), check_untouched=False, seqs=shortest,
                       label=f"varlen fp16 all heads of seqs {shortest}")
    print("varlen fp16 worst", w, w_all)
