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
