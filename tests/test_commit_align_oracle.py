"""Pins for the align-mode commit oracle (kda_oracle.commit_align_ref), on
the CPU.

Which slot receives which state is fixed here by literal cases worked from
the block definition (token t, 1-based, belongs to block (t - 1) //
block_size; a block's slot ends up holding the state at its last token),
and every written state is compared with a token-by-token replay of the
original inputs from the checkpoint (``replay_ref``), not with the commit
formula the oracle itself uses.
"""

import numpy as np
import pytest

import workloads as wl
from oracle import kda_oracle as ko

H, D, L, BS = 2, 8, 4, 5


def case(n_req, seed):
    toks = wl.token_inputs(n_req * L, H, D, D, "f32", seed, shape_prefix=(n_req, L))
    ex = {n: wl.exact(toks[n]) for n in "qkvgb"}
    rng = np.random.default_rng(seed)
    S0 = rng.standard_normal((n_req, H, D, D))
    _, u_rec, kg_rec, _ = ko.verify_ref(ex["q"], ex["k"], ex["v"], ex["g"], ex["b"], S0)
    return ex, S0, kg_rec[..., :D], kg_rec[..., D:], u_rec


# (p, n) -> {table position of the written slot: accepted tokens replayed}
CASES = [
    ((2, 2), {0: 2}),            # tokens 3, 4 stay in block 0
    ((3, 4), {0: 2, 1: 4}),      # tokens 4, 5 close block 0; 6, 7 open block 1
    ((5, 3), {1: 3}),            # p = 5 is block 0's last token: block 0 keeps S_5
    ((4, 1), {0: 1}),            # token 5 closes block 0 exactly: no new block yet
    ((7, 0), {}),                # nothing accepted
    ((9, 4), {1: 1, 2: 4}),      # token 10 closes block 1
]


def test_slot_selection_and_states():
    n_req = len(CASES)
    ex, S0, k_rec, g_rec, u_rec = case(n_req, 31)
    table = np.array([[10 * r + b for b in range(4)] for r in range(n_req)])
    p = [c[0][0] for c in CASES]
    n = [c[0][1] for c in CASES]
    slots = {}
    for r in range(n_req):
        b0 = (p[r] - 1) // BS
        for b in range(4):
            slots[int(table[r][b])] = S0[r] if b == b0 else np.full((H, D, D), np.nan)
    writes, err = ko.commit_align_ref(slots, table, p, n, BS, k_rec, g_rec, u_rec)
    assert err == 0
    want = {int(table[r][pos]): (r, cnt) for r, (_, w) in enumerate(CASES) for pos, cnt in w.items()}
    assert set(writes) == set(want)
    for slot, (r, cnt) in want.items():
        rep = ko.replay_ref(*(ex[x][r] for x in "qkvgb"), S0[r], cnt)
        assert np.allclose(writes[slot], rep, rtol=1e-12, atol=1e-12)


def test_errors_skip_the_request():
    ex, S0, k_rec, g_rec, u_rec = case(3, 32)
    table = np.array([[0, 1], [2, 3], [4, 5]])
    slots = {s: S0[s // 2] for s in range(6)}
    # request 0: n > L; request 1: p = 0; request 2: p = 9, n = 2 needs block 2, beyond its row
    writes, err = ko.commit_align_ref(slots, table, [3, 0, 9], [L + 1, 1, 2], BS, k_rec, g_rec, u_rec)
    assert err == ko.ERR_ACCEPT | ko.ERR_SLOT
    assert writes == {}


@pytest.mark.parametrize("p", range(1, 16))
def test_matches_replay_for_every_offset(p):
    ex, S0, k_rec, g_rec, u_rec = case(1, 40 + p)
    table = np.array([[100, 101, 102, 103, 104]])
    slots = {s: np.full((H, D, D), np.nan) for s in table[0]}
    slots[100 + (p - 1) // BS] = S0[0]
    for n in range(L + 1):
        writes, err = ko.commit_align_ref(slots, table, [p], [n], BS, k_rec, g_rec, u_rec)
        assert err == 0
        # the state after p + n tokens sits in the block of token p + n
        if n:
            run = ko.replay_ref(*(ex[x][0] for x in "qkvgb"), S0[0], n)
            assert np.allclose(writes[100 + (p + n - 1) // BS], run, rtol=1e-12, atol=1e-12)
        else:
            assert writes == {}


# (p, n) with BS = 5 -> (tokens, running block) worked from the block definition
NEXT = [((2, 2), (4, 0)), ((3, 4), (7, 1)), ((5, 3), (8, 1)), ((4, 1), (5, 0)), ((7, 0), (7, 1)),
        ((9, 4), (13, 2)), ((1, 0), (1, 0)), ((10, 0), (10, 1)), ((10, 1), (11, 2))]


def test_next_step_literal_cases():
    n_req = len(NEXT)
    table = np.array([[10 * r + b + 1 for b in range(4)] for r in range(n_req)])
    p = [c[0][0] for c in NEXT]
    n = [c[0][1] for c in NEXT]
    tokens, block, ckpt, bias = ko.align_next_ref(table, p, n, BS, L, n_slots=1000)
    for r, (_, (t, b)) in enumerate(NEXT):
        assert (tokens[r], block[r], ckpt[r], bias[r]) == (t, b, table[r][b], 0), r


def test_next_step_errors():
    table = np.array([[0, 1], [2, 3], [4, 5], [6, 99]])
    # n > L; p = 0; a block beyond the row; a slot outside the pool (n_slots = 8)
    tokens, block, ckpt, bias = ko.align_next_ref(table, [3, 0, 9, 7], [L + 1, 1, 2, 1], BS, L, n_slots=8)
    assert list(tokens) == [3, 0, 9, 7]
    assert list(block) == [-1] * 4 and list(ckpt) == [-1] * 4 and list(bias) == [0] * 4


def test_next_step_chains_to_replay():
    """Two align steps, the second from the first's running block: the state
    the second writes at its running block is the replay of both windows."""
    ex, S0, k_rec, g_rec, u_rec = case(1, 50)
    table = np.array([[200, 201, 202, 203]])
    p, n1 = 3, 4                                     # tokens 4..7: closes block 0, opens block 1
    slots = {s: np.full((H, D, D), np.nan) for s in table[0]}
    slots[200] = S0[0]
    w1, err = ko.commit_align_ref(slots, table, [p], [n1], BS, k_rec, g_rec, u_rec)
    assert err == 0
    t1, b1, c1, _ = ko.align_next_ref(table, [p], [n1], BS, L, n_slots=1000)
    assert (t1[0], b1[0], c1[0]) == (7, 1, 201)
    slots.update(w1)
    # second window: the next tokens of the same stream, verified from slot c1
    toks2 = wl.token_inputs(L, H, D, D, "f32", 51, shape_prefix=(1, L))
    ex2 = {x: wl.exact(toks2[x]) for x in "qkvgb"}
    _, u2, kg2, _ = ko.verify_ref(ex2["q"], ex2["k"], ex2["v"], ex2["g"], ex2["b"], slots[int(c1[0])][None])
    n2 = 4                                           # tokens 8..11: closes block 1 at 10, opens block 2
    w2, err = ko.commit_align_ref(slots, table, [int(t1[0])], [n2], BS, kg2[..., :D], kg2[..., D:], u2)
    assert err == 0
    t2, b2, c2, _ = ko.align_next_ref(table, [int(t1[0])], [n2], BS, L, n_slots=1000)
    assert (t2[0], b2[0], c2[0]) == (11, 2, 202)
    whole = {x: np.concatenate([ex[x][0][:n1], ex2[x][0][:n2]]) for x in "qkvgb"}
    rep = ko.replay_ref(*(whole[x] for x in "qkvgb"), S0[0], n1 + n2)
    assert np.allclose(w2[int(c2[0])], rep, rtol=1e-12, atol=1e-12)
    rep10 = ko.replay_ref(*(whole[x] for x in "qkvgb"), S0[0], 10 - p)   # block 1 ends at token 10
    assert np.allclose(w2[201], rep10, rtol=1e-12, atol=1e-12)
