"""GPU parity of kda_commit_align (through the C ABI) against the oracle's
align-mode commit, and against token-by-token replays: block-aligned state
slots, with windows that stay inside a block, close it exactly, start at a
block end, or cross into the next block."""

import numpy as np
import pytest
import torch

import linear_attention_state_kda_amd as kda
import workloads as wl
from oracle import kda_oracle as ko
from tests.gpu_util import DEV, Worst, i32, make_pool, to_math

pytestmark = pytest.mark.gpu


def run_case(pool_dtype, block_size, p, n, H=4, L=8, blocks=4, seed=61):
    d = 128
    n_req = len(p)
    toks = wl.token_inputs(n_req * L, H, d, d, "bf16", seed, shape_prefix=(n_req, L))
    table = np.arange(n_req * blocks, dtype=np.int32).reshape(n_req, blocks)[:, ::-1].copy() + 3
    pool = make_pool(n_req * blocks + 3, H, d, d, pool_dtype)
    slots = {}
    S0 = []
    for r in range(n_req):
        b0 = (max(p[r], 1) - 1) // block_size
        s0 = int(table[r][b0])
        st = wl.pool_state(s0, H, d, d, pool_dtype, seed)
        pool[s0] = st.to(DEV)
        S0.append(np.swapaxes(wl.exact(st), -1, -2))
    dev = {x: toks[x].to(DEV) for x in "qkvgb"}
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    # records from the verify kernel, each request from its running slot
    ck = [int(table[r][(max(p[r], 1) - 1) // block_size]) for r in range(n_req)]
    _, u_rec, kg_rec = kda.recurrent_verify(dev["q"], dev["k"], dev["v"], dev["g"], dev["b"], pool, i32(ck),
                                            dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    before = pool.clone()
    kda.commit_align(pool, i32(table), i32(p), i32(n), block_size, u_rec, kg_rec, dev_err=err)
    torch.cuda.synchronize()
    for r in range(n_req):
        for b in range(blocks):
            slots.setdefault(int(table[r][b]), np.full((H, d, d), np.nan))
        slots[ck[r]] = S0[r]
    kg64 = wl.exact(kg_rec.cpu())
    writes, want_err = ko.commit_align_ref(slots, table, p, n, block_size, kg64[..., :d], kg64[..., d:],
                                           u_rec.cpu().double().numpy())
    return dict(pool=pool, before=before, writes=writes, err=err.item(), want_err=want_err, toks=toks, S0=S0,
                table=table, ck=ck)


@pytest.mark.parametrize("pool_dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("block_size", [9, 12, 64])
def test_commit_align_matches_oracle(pool_dtype, block_size):
    bs = block_size
    # positions around the block ends of blocks 0 and 1, and every accepted length
    p = [1, bs - 3, bs - 1, bs, bs + 1, 2 * bs - 2, 2 * bs, 5, bs - 8, 2 * bs - 1]
    n = [8, 5, 1, 3, 0, 8, 8, 2, 8, 6]
    r = run_case(pool_dtype, bs, p, n)
    assert r["err"] == 0 and r["want_err"] == 0
    w = Worst(1e-4 if pool_dtype == "f32" else 2e-2)
    written = set(r["writes"])
    for slot in range(r["pool"].shape[0]):
        if slot in written:
            w.state("state", to_math(r["pool"][slot]), r["writes"][slot])
        else:
            assert torch.equal(r["pool"][slot], r["before"][slot]), slot
    w.check(f"commit_align pool={pool_dtype} block={bs}")


def test_commit_align_states_are_replays():
    """The states written equal token-by-token replays of the accepted
    positions from the checkpoint (fp32 pool)."""
    bs = 9
    p, n = [7, 9, 3], [5, 4, 6]
    r = run_case("f32", bs, p, n, seed=62)
    ex = {x: wl.exact(r["toks"][x]) for x in "qkvgb"}
    w = Worst(1e-4)
    for i in range(len(p)):
        for j in range(1, n[i] + 1):
            t = p[i] + j                                   # 1-based token index
            last_of_block = t % bs == 0 or j == n[i]
            if not last_of_block:
                continue
            slot = int(r["table"][i][(t - 1) // bs])
            rep = ko.replay_ref(*(ex[x][i] for x in "qkvgb"), r["S0"][i], j)
            w.state("replay", to_math(r["pool"][slot]), rep)
    w.check("commit_align vs replays")


def test_commit_align_errors():
    bs = 9
    # n > L; p = 0; p + n runs past the table (4 blocks of 9 = 36 tokens); one valid request
    p, n = [5, 0, 33, 10], [9, 1, 8, 3]
    r = run_case("f32", bs, p, n, seed=63)
    assert r["err"] == kda.DEV_ERR_ACCEPT | kda.DEV_ERR_SLOT == r["want_err"]
    written = set(r["writes"])
    assert written == {int(r["table"][3][1])}
    for slot in range(r["pool"].shape[0]):
        if slot not in written:
            assert torch.equal(r["pool"][slot], r["before"][slot]), slot


def test_commit_align_short_window():
    """L = 3, block size 4 (the smallest allowed): every request crosses or
    touches a block end."""
    bs, L = 4, 3
    p = [1, 2, 3, 4, 5, 6, 7, 8]
    n = [3, 3, 2, 1, 3, 0, 2, 3]
    r = run_case("f32", bs, p, n, L=L, seed=64)
    assert r["err"] == 0 and r["want_err"] == 0
    written = set(r["writes"])
    w = Worst(1e-4)
    for slot in range(r["pool"].shape[0]):
        if slot in written:
            w.state("state", to_math(r["pool"][slot]), r["writes"][slot])
        else:
            assert torch.equal(r["pool"][slot], r["before"][slot]), slot
    w.check("commit_align L=3 block 4")
