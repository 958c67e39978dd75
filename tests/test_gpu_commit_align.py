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
from tests.gpu_util import DEV, Worst, i32, make_pool, rounding_excess, to_math

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
    nxt = [torch.full((n_req,), 12345, dtype=torch.int32, device=DEV) for _ in range(4)]
    kda.commit_align(pool, i32(table), i32(p), i32(n), block_size, u_rec, kg_rec, dev_err=err,
                     next_tokens=nxt[0], next_block=nxt[1], next_ckpt=nxt[2], copy_bias=nxt[3])
    torch.cuda.synchronize()
    # the next step's values: bitwise what the oracle's post-processing gives
    want_next = ko.align_next_ref(table, p, n, block_size, L, pool.shape[0])
    for got, want in zip(nxt, want_next):
        assert np.array_equal(got.cpu().numpy(), want), (got, want)
    for r in range(n_req):
        for b in range(blocks):
            slots.setdefault(int(table[r][b]), np.full((H, d, d), np.nan))
        slots[ck[r]] = S0[r]
    kg64 = wl.exact(kg_rec.cpu())
    writes, want_err = ko.commit_align_ref(slots, table, p, n, block_size, kg64[..., :d], kg64[..., d:],
                                           u_rec.cpu().double().numpy())
    return dict(pool=pool, before=before, writes=writes, err=err.item(), want_err=want_err, toks=toks, S0=S0,
                table=table, ck=ck, next=[t.cpu().numpy() for t in nxt])


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
    worst_ulp = 0.0
    for slot in range(r["pool"].shape[0]):
        if slot in written:
            got = to_math(r["pool"][slot])
            w.state("state", got, r["writes"][slot])
            if pool_dtype != "f32":   # rounded once from fp32 on exact records: within half a 16-bit ulp (+ fp32 error)
                ex = float(rounding_excess(got, r["writes"][slot], pool_dtype).max())
                worst_ulp = max(worst_ulp, ex)
                assert ex <= 1.0, (slot, ex)
        else:
            assert torch.equal(r["pool"][slot], r["before"][slot]), slot
    w.check(f"commit_align pool={pool_dtype} block={bs}")
    if pool_dtype != "f32":
        print(f"[parity] commit_align pool={pool_dtype} block={bs}: worst {worst_ulp:.3f} of (half a 16-bit ulp + fp32 slack)")


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
    assert list(r["next"][1]) == [-1, -1, -1, 1] and list(r["next"][2][:3]) == [-1, -1, -1]
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


@pytest.mark.parametrize("pool_dtype", ["f32", "bf16"])
def test_commit_align_chain_from_running_block(pool_dtype):
    """Three speculative steps on the device alone: each verify reads the
    checkpoint slot the previous align commit wrote to ``next_ckpt``, and
    each align commit takes ``next_tokens`` as its token count, with no
    host arithmetic in between; every written state then equals a replay of
    the accepted tokens of all steps so far, and the slots of finished
    blocks hold the state at their last token."""
    H, d, L, bs, n_req, blocks = 4, 128, 8, 12, 5, 5
    seed = 71
    p0 = np.array([1, 5, 11, 12, 20], dtype=np.int32)
    table = (np.arange(n_req * blocks, dtype=np.int32).reshape(n_req, blocks) * 3 + 2).astype(np.int32)
    pool = make_pool(int(table.max()) + 1, H, d, d, pool_dtype)
    S0 = []
    for r in range(n_req):
        s0 = int(table[r][(p0[r] - 1) // bs])
        st = wl.pool_state(s0, H, d, d, pool_dtype, seed)
        pool[s0] = st.to(DEV)
        S0.append(np.swapaxes(wl.exact(st), -1, -2))
    accepted = np.random.default_rng([seed, 1]).integers(0, L + 1, (3, n_req)).astype(np.int32)
    accepted[0, 2] = L                              # request 2 closes its first block in step 0
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    tok = i32(p0)
    ck = i32([int(table[r][(p0[r] - 1) // bs]) for r in range(n_req)])
    tbl = i32(table)
    steps = []
    for step in range(3):
        toks = wl.token_inputs(n_req * L, H, d, d, "bf16", seed + 10 + step, shape_prefix=(n_req, L))
        steps.append(toks)
        dev = {x: toks[x].to(DEV) for x in "qkvgb"}
        _, u_rec, kg_rec = kda.recurrent_verify(dev["q"], dev["k"], dev["v"], dev["g"], dev["b"], pool, ck,
                                                dev_err=err)
        nt, nb, nc, bias = (torch.empty(n_req, dtype=torch.int32, device=DEV) for _ in range(4))
        kda.commit_align(pool, tbl, tok, i32(accepted[step]), bs, u_rec, kg_rec, dev_err=err,
                         next_tokens=nt, next_block=nb, next_ckpt=nc, copy_bias=bias)
        tok, ck = nt, nc
    torch.cuda.synchronize()
    assert err.item() == 0
    assert np.array_equal(tok.cpu().numpy(), p0 + accepted.sum(axis=0))
    assert not bias.cpu().numpy().any()
    w = Worst(1e-4 if pool_dtype == "f32" else 2e-2)
    for r in range(n_req):
        ex = {x: np.concatenate([wl.exact(steps[s][x][r])[:accepted[s, r]] for s in range(3)]) for x in "qkvgb"}
        total = int(accepted[:, r].sum())
        p_end = int(p0[r]) + total
        # the running block's slot: the state after all accepted tokens
        rep = ko.replay_ref(*(ex[x] for x in "qkvgb"), S0[r], total)
        assert int(ck[r].item()) == int(table[r][(p_end - 1) // bs])
        w.state("current", to_math(pool[int(ck[r].item())]), rep)
        # every block finished along the way: the state at its last token
        for b in range((int(p0[r]) - 1) // bs, (p_end - 1) // bs):
            last = (b + 1) * bs
            rep_b = ko.replay_ref(*(ex[x] for x in "qkvgb"), S0[r], last - int(p0[r]))
            w.state("block_end", to_math(pool[int(table[r][b])]), rep_b)
    w.check(f"commit_align three-step chain pool={pool_dtype}")
