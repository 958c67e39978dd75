"""GPU parity of the state paths through the C ABI: kda_state_copy,
kda_recurrent_verify and kda_commit against the fp64 oracle.

Copy is bit-exact.  Verify and commit compute in fp32 from exactly the
values the oracle receives; the bar is 1e-4 relative for fp32 inputs and
2e-2 for bf16/fp16 inputs (per (request, head) Frobenius), with the
records checked bitwise (kg_rec is a copy of the inputs).
"""

import numpy as np
import pytest
import torch

import linear_attention_state_kda_amd as kda
import workloads as wl
from oracle import kda_oracle as ko
from tests.gpu_util import DEV, TOL, Worst, i32, make_pool, rel_per_head, rounding_excess, to_math, untouched

pytestmark = pytest.mark.gpu


def fill_slots(pool, slots, pool_dtype, seed):
    H, dv, dk = pool.shape[1:]
    host = {}
    for s in slots:
        st = wl.pool_state(int(s), H, dk, dv, pool_dtype, seed)
        pool[int(s)] = st.to(DEV)
        host[int(s)] = st
    return host


# ---------------------------------------------------------------- copy

@pytest.mark.parametrize("pool_dtype", ["f32", "bf16", "f16"])
def test_copy_fork_matches_oracle_bitwise(pool_dtype):
    case = wl.spec_case(n_req=256, L=8, H=32, d=128, pool_dtype=pool_dtype, seed=3)
    n_slots = case["n_slots"]
    pool = make_pool(n_slots, 32, 128, 128, pool_dtype)
    srcs = sorted(set(case["fork_src"].tolist()))
    host = fill_slots(pool, srcs, pool_dtype, 3)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    kda.state_copy(pool, i32(case["fork_src"]), i32(case["fork_dst"]), dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    # oracle over the involved slots only (remapped to a compact host pool of raw bits)
    itype = torch.int32 if pool_dtype == "f32" else torch.int16
    involved = srcs + sorted(case["fork_dst"].tolist())
    idx = {s: i for i, s in enumerate(involved)}
    sentinel_bits = make_pool(1, 32, 128, 128, pool_dtype)[0].cpu().view(itype).numpy()
    cpu_pool = np.stack([host[s].view(itype).numpy() if s in host else sentinel_bits for s in involved])
    ref = ko.copy_ref(cpu_pool, [idx[s] for s in case["fork_src"].tolist()],
                      [idx[d] for d in case["fork_dst"].tolist()])
    got = pool[torch.as_tensor(involved, device=DEV)].cpu().view(itype).numpy()
    assert np.array_equal(got, ref)
    others = sorted(set(range(n_slots)) - set(involved))
    assert untouched(pool, others, pool_dtype)


def test_copy_edge_cases():
    pool = make_pool(8, 2, 128, 128, "f32")
    host = fill_slots(pool, [0, 1], "f32", 5)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    # src == dst is a no-op; an out-of-range pair is skipped and flagged
    kda.state_copy(pool, i32([1, 0, 9]), i32([1, 3, 4]), dev_err=err)
    torch.cuda.synchronize()
    assert err.item() & kda.DEV_ERR_SLOT
    assert torch.equal(pool[1].cpu(), host[1])
    assert torch.equal(pool[3].cpu(), host[0])
    assert untouched(pool, [2, 4, 5, 6, 7], "f32")
    # zero pairs launches nothing
    kda.state_copy(pool, i32([]), i32([]))
    torch.cuda.synchronize()


def test_copy_groups_sharing_a_source():
    """Pairs that share a source are written by the group's first valid
    pair: interleaved groups, a no-op pair (dst == src) leading its group,
    an invalid destination inside a group and an invalid source (both
    flagged and skipped), and one source forked to 300 children, whose
    pairs span two windows of 256 pairs, the first pair of the second
    window having an invalid destination."""
    n_slots = 420
    pool = make_pool(n_slots, 2, 128, 128, "f32")
    host = fill_slots(pool, [3, 5, 7, 20], "f32", 9)
    src = [5, 7, 5, 5, 430, 7, 5, 3, 3] + [20] * 300
    dst = [10, 11, 5, 12, 13, 14, 999, 15, 16] + list(range(100, 400))
    assert dst[256] == 347
    dst[256] = 1000
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    kda.state_copy(pool, i32(src), i32(dst), dev_err=err)
    torch.cuda.synchronize()
    assert err.item() & kda.DEV_ERR_SLOT
    expect = {10: 5, 12: 5, 11: 7, 14: 7, 15: 3, 16: 3, **{d: 20 for d in range(100, 400) if d != 347}}
    for d, s_ in expect.items():
        assert torch.equal(pool[d].cpu(), host[s_]), (d, s_)
    for s_ in (3, 5, 7, 20):
        assert torch.equal(pool[s_].cpu(), host[s_])
    written = set(expect) | {3, 5, 7, 20}
    assert untouched(pool, sorted(set(range(n_slots)) - written), "f32")


def test_copy_groups_across_windows():
    """1,100 pairs over 37 sources, each source's children spread over all
    five windows of 256 pairs (and over several places inside each): every
    destination receives its source's bits and the sources stay unchanged."""
    n_src, n_pairs = 37, 1100
    n_slots = n_src + n_pairs
    pool = make_pool(n_slots, 2, 128, 128, "bf16")
    host = fill_slots(pool, list(range(n_src)), "bf16", 11)
    src = [i % n_src for i in range(n_pairs)]
    dst = [n_src + (i * 7) % n_pairs for i in range(n_pairs)]   # a permutation of the child slots
    assert len(set(dst)) == n_pairs
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    kda.state_copy(pool, i32(src), i32(dst), dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    out = pool.cpu()
    for s_, d in zip(src, dst):
        assert torch.equal(out[d], host[s_]), (s_, d)
    for s_ in range(n_src):
        assert torch.equal(out[s_], host[s_])


# ---------------------------------------------------------------- verify

def run_verify_case(n_req, L, H, in_dtype, pool_dtype, seed):
    d = 128
    toks = wl.token_inputs(n_req * L, H, d, d, in_dtype, seed, shape_prefix=(n_req, L))
    n_slots = n_req + 3
    ckpt = wl.distinct_slots(n_req, n_slots, seed)
    pool = make_pool(n_slots, H, d, d, pool_dtype)
    host = fill_slots(pool, ckpt, pool_dtype, seed)
    before = pool.clone()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    dev = {n: toks[n].to(DEV) for n in "qkvgb"}
    o, u_rec, kg_rec = kda.recurrent_verify(dev["q"], dev["k"], dev["v"], dev["g"], dev["b"], pool,
                                            i32(ckpt), dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    assert torch.equal(pool, before)                      # checkpoints are read only
    ex = {n: wl.exact(toks[n]) for n in "qkvgb"}
    S0 = np.stack([np.swapaxes(wl.exact(host[int(s)]), -1, -2) for s in ckpt])
    o_ref, u_ref, kg_ref, S_L = ko.verify_ref(ex["q"], ex["k"], ex["v"], ex["g"], ex["b"], S0)
    return dict(o=wl.exact(o.cpu()), u=u_rec.cpu().double().numpy(), kg=kg_rec.cpu(),
                o_ref=o_ref, u_ref=u_ref, kg_ref=kg_ref, toks=toks, ckpt=ckpt, pool=pool,
                host=host, S0=S0, S_L=S_L, dev=dev, u_rec=u_rec, kg_rec=kg_rec, ex=ex)


def check_verify(r, in_dtype, label, reqs=None):
    """Every request's outputs (per (request, head) and per (position, head)
    row) at the input dtype's bar and its u records at the fp32 bar (u is
    fp32 arithmetic on exact inputs); the key / raw-gate records bitwise.
    With 16-bit inputs each output element is an fp32 result rounded once
    into the input dtype, so it must also lie within half a 16-bit ulp of
    the fp64 oracle plus the fp32 arithmetic's error (1e-5 of the position's
    largest output: 128-term fp32 dot products, ~sqrt(128) x 2^-24 of the
    sum of their terms' magnitudes, which matters only near zero)."""
    n_req = r["o"].shape[0]
    wo, wu = Worst(TOL[in_dtype]), Worst(1e-4)
    worst_ulp = 0.0
    for i in (range(n_req) if reqs is None else reqs):
        wo.out("o", r["o"][i], r["o_ref"][i], 1)
        wu.out("u", r["u"][i], r["u_ref"][i], 0)
        if in_dtype != "f32":   # [L, H, dv] -> per position: max over (H, dv)
            ex = float(rounding_excess(np.swapaxes(r["o"][i], 0, 1), np.swapaxes(r["o_ref"][i], 0, 1),
                                       in_dtype, slack_rel=1e-5).max())
            worst_ulp = max(worst_ulp, ex)
            assert ex <= 1.0, (i, ex)
    wo.check(label + " o")
    wu.check(label + " u")
    if in_dtype != "f32":
        print(f"[parity] {label} o per element: worst {worst_ulp:.3f} of (half a 16-bit ulp + fp32 slack)")
    # key / raw-gate records are lossless copies of the inputs
    assert np.array_equal(wl.exact(r["kg"]), r["kg_ref"])


@pytest.mark.parametrize("in_dtype,pool_dtype", [("bf16", "f32"), ("f32", "f32"), ("bf16", "bf16"),
                                                  ("f16", "f16"), ("f32", "bf16")])
def test_verify_matches_oracle(in_dtype, pool_dtype):
    r = run_verify_case(n_req=12, L=8, H=3, in_dtype=in_dtype, pool_dtype=pool_dtype, seed=21)
    check_verify(r, in_dtype, f"verify {in_dtype} pool={pool_dtype}")


def test_verify_full_spec_shape():
    """256 requests x 32 heads x L = 8, bf16 inputs, fp32 pool (the
    speculative-decode workload)."""
    r = run_verify_case(n_req=256, L=8, H=32, in_dtype="bf16", pool_dtype="f32", seed=3)
    check_verify(r, "bf16", "verify 256 req x 32 heads L=8")


def test_verify_long_window():
    """L = 256, the largest built window."""
    r = run_verify_case(n_req=2, L=256, H=2, in_dtype="bf16", pool_dtype="f32", seed=22)
    check_verify(r, "bf16", "verify L=256")


@pytest.mark.parametrize("L", [1, 3, 9, 13])
def test_verify_window_lengths(L):
    """One-block and multi-block windows (ragged last block) with more
    (request, head) items than workgroups resident at once, so every
    workgroup steps through several items."""
    n_req = 40
    r = run_verify_case(n_req=n_req, L=L, H=32, in_dtype="bf16", pool_dtype="f32", seed=40 + L)
    check_verify(r, "bf16", f"verify L={L}")


@pytest.mark.parametrize("L", [8, 11])
def test_verify_bad_slot_skips_request(L):
    """A request whose checkpoint slot is out of range is flagged and its
    outputs are left as they were; the other requests are unaffected."""
    n_req, H, d, seed = 40, 32, 128, 51
    toks = wl.token_inputs(n_req * L, H, d, d, "bf16", seed, shape_prefix=(n_req, L))
    n_slots = n_req + 3
    ckpt = wl.distinct_slots(n_req, n_slots, seed).copy()
    pool = make_pool(n_slots, H, d, d, "f32")
    host = fill_slots(pool, ckpt, "f32", seed)
    bad = {7: -1, 23: n_slots}
    ck_dev = ckpt.copy()
    for i, s in bad.items():
        ck_dev[i] = s
    dev = {n: toks[n].to(DEV) for n in "qkvgb"}
    o = torch.full((n_req, L, H, d), 7.0, dtype=torch.bfloat16, device=DEV)
    u_rec = torch.full((n_req, H, L, d), 7.0, dtype=torch.float32, device=DEV)
    kg_rec = torch.full((n_req, H, L, 2 * d), 7.0, dtype=torch.bfloat16, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    kda.recurrent_verify(dev["q"], dev["k"], dev["v"], dev["g"], dev["b"], pool, i32(ck_dev),
                         o=o, u_rec=u_rec, kg_rec=kg_rec, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() & kda.DEV_ERR_SLOT
    for i in bad:
        assert bool((o[i] == 7.0).all()) and bool((u_rec[i] == 7.0).all()) and bool((kg_rec[i] == 7.0).all())
    good = [i for i in range(n_req) if i not in bad]
    ex = {n: wl.exact(toks[n])[good] for n in "qkvgb"}
    S0 = np.stack([np.swapaxes(wl.exact(host[int(ckpt[i])]), -1, -2) for i in good])
    o_ref, u_ref, kg_ref, _ = ko.verify_ref(ex["q"], ex["k"], ex["v"], ex["g"], ex["b"], S0)
    o_got, u_got = wl.exact(o.cpu())[good], u_rec.cpu().double().numpy()[good]
    check_verify(dict(o=o_got, o_ref=o_ref, u=u_got, u_ref=u_ref, kg=kg_rec.cpu()[good], kg_ref=kg_ref),
                 "bf16", f"verify L={L} with bad slots")


# ---------------------------------------------------------------- commit

@pytest.mark.parametrize("pool_dtype,in_dtype", [("f32", "bf16"), ("bf16", "bf16"), ("f16", "bf16"),
                                                  ("f32", "f32")])
def test_commit_matches_oracle(pool_dtype, in_dtype):
    n_req, L, H, d = 24, 8, 2, 128
    r = run_verify_case(n_req=n_req, L=L, H=H, in_dtype=in_dtype, pool_dtype=pool_dtype, seed=31)
    acc = np.arange(n_req, dtype=np.int32) % (L + 1)     # every length 0..L, n = 0 included
    pool = r["pool"]
    ckpt = r["ckpt"]
    before = pool.clone()
    # oracle records = exactly the values handed to the kernel
    u_in = r["u_rec"]
    kg_in = r["kg_rec"]
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    kda.commit(pool, i32(ckpt), i32(acc), u_in, kg_in, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    u64 = u_in.cpu().double().numpy()
    kg64 = wl.exact(kg_in.cpu())
    tol = 1e-4 if pool_dtype == "f32" else 2e-2
    wc, wr = Worst(tol), Worst(tol)
    for i in range(n_req):
        s = int(ckpt[i])
        got = to_math(pool[s])
        ref = ko.commit_ref(r["S0"][i], kg64[i, :, :, :d], kg64[i, :, :, d:], u64[i], int(acc[i]))
        if acc[i] == 0:
            assert torch.equal(pool[s], before[s])       # in place, nothing accepted: untouched
        else:
            wc.state("commit", got, ref)
            if pool_dtype != "f32":   # rounded once from fp32 on exact records: within half a 16-bit ulp (+ fp32 error)
                ex = float(rounding_excess(got, ref, pool_dtype).max())
                assert ex <= 1.0, (i, ex)
            # and the rebuilt state equals a replay of the accepted positions
            # (the records hold exactly the replay's inputs and its fp32 u)
            rep = ko.replay_ref(*(r["ex"][n][i] for n in "qkvgb"), r["S0"][i], int(acc[i]))
            wr.state("replay", got, rep)
    wc.check(f"commit pool={pool_dtype} in={in_dtype} vs closed form")
    wr.check(f"commit pool={pool_dtype} in={in_dtype} vs replay")


def test_verify_commit_full_shape_fp16():
    """The speculative-decode shape (256 requests x 32 heads, L = 8) with fp16
    inputs and an fp16 pool: verify's outputs at the fp16 bar, then every
    committed state element within half an fp16 ulp of the fp64 closed form plus
    the fp32 arithmetic's own error (the commit accumulates at most L = 8
    terms of the state's magnitude in fp32, ~2^-24 relative each, then rounds
    once, to nearest even, into the pool: 1e-6 of the head's largest element
    covers the fp32 part, which matters only for elements near zero, whose
    fp16 ulp is as small as that error)."""
    n_req, L, H, d = 256, 8, 32, 128
    r = run_verify_case(n_req=n_req, L=L, H=H, in_dtype="f16", pool_dtype="f16", seed=8)
    check_verify(r, "f16", "verify fp16 256 req x 32 heads L=8")
    acc = wl.spec_case(seed=8)["accepted"]
    pool, ckpt = r["pool"], r["ckpt"]
    before = pool.clone()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    kda.commit(pool, i32(ckpt), i32(acc), r["u_rec"], r["kg_rec"], dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    u64 = r["u_rec"].cpu().double().numpy()
    kg64 = wl.exact(r["kg_rec"].cpu())
    worst = 0.0
    for i in range(n_req):
        s_ = int(ckpt[i])
        if acc[i] == 0:
            assert torch.equal(pool[s_], before[s_])
            continue
        ref = ko.commit_ref(r["S0"][i], kg64[i, :, :, :d], kg64[i, :, :, d:], u64[i], int(acc[i]))
        got = to_math(pool[s_])
        excess = rounding_excess(got, ref, "f16")
        worst = max(worst, float(excess.max()))
        assert excess.max() <= 1.0, (i, float(excess.max()))
    print(f"[parity] commit fp16 pool 256 req x 32 heads: worst |got - ref| = {worst:.3f} of (half an fp16 ulp + fp32 slack)")


def test_commit_to_other_slot_and_errors():
    n_req, L, H, d = 4, 8, 2, 128
    r = run_verify_case(n_req=n_req, L=L, H=H, in_dtype="bf16", pool_dtype="f32", seed=41)
    pool = r["pool"]
    n_slots = pool.shape[0]
    ckpt = r["ckpt"]
    free = sorted(set(range(n_slots)) - set(ckpt.tolist()))
    dst = np.array([free[0], free[1], ckpt[2], ckpt[3]], dtype=np.int32)
    acc = np.array([0, 5, 3, 9], dtype=np.int32)          # request 3 asks for more than L
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    before = pool.clone()
    kda.commit(pool, i32(ckpt), i32(acc), r["u_rec"], r["kg_rec"], dst_slot=i32(dst), dev_err=err)
    torch.cuda.synchronize()
    assert err.item() & kda.DEV_ERR_ACCEPT
    assert torch.equal(pool[int(dst[0])], before[int(ckpt[0])])   # n = 0 to another slot = copy
    assert torch.equal(pool[int(ckpt[3])], before[int(ckpt[3])])  # rejected request untouched
    u64 = r["u_rec"].cpu().double().numpy()
    kg64 = wl.exact(r["kg_rec"].cpu())
    ref = ko.commit_ref(r["S0"][1], kg64[1, :, :, :d], kg64[1, :, :, d:], u64[1], 5)
    w = Worst(1e-4)
    w.state("commit", to_math(pool[int(dst[1])]), ref)
    w.check("commit to another slot")
    assert torch.equal(pool[int(ckpt[1])], before[int(ckpt[1])])  # source kept


def test_verify_commit_full_spec_shape():
    """The full speculative-decode step: 256 requests, H = 32, L = 8,
    accepted ~ U{0..8}, in-place commit of every request checked against a
    replay of its accepted positions, then the fork of 64 committed
    checkpoints to 4 children each checked bitwise."""
    case = wl.spec_case(seed=3)
    r = run_verify_case(n_req=256, L=8, H=32, in_dtype="bf16", pool_dtype="f32", seed=3)
    pool, ckpt = r["pool"], r["ckpt"]
    acc = case["accepted"]
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    before = pool.clone()
    kda.commit(pool, i32(ckpt), i32(acc), r["u_rec"], r["kg_rec"], dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    w = Worst(1e-4)
    for i in range(256):                                            # every request
        s = int(ckpt[i])
        if acc[i] == 0:
            assert torch.equal(pool[s], before[s])
            continue
        rep = ko.replay_ref(*(r["ex"][n][i] for n in "qkvgb"), r["S0"][i], int(acc[i]))
        w.state("commit", to_math(pool[s]), rep)
    w.check("commit 256 req x 32 heads vs replay")
    # fork: the spec case's sources are slots of the same checkpoint draw
    # (distinct_slots with the same seed), its children fresh slots
    n_slots = pool.shape[0]
    src = np.array([int(x) for x in case["fork_src"]], dtype=np.int32)
    src = np.array([ckpt[list(case["ckpt_slots"]).index(x)] for x in src], dtype=np.int32)
    free = sorted(set(range(n_slots)) - set(int(x) for x in ckpt))
    dst = np.array(free[:len(src)], dtype=np.int32) if len(free) >= len(src) else None
    if dst is None:                                                 # pool too small for 256 children
        big = make_pool(n_slots + len(src), 32, 128, 128, "f32")
        big[:n_slots] = pool
        pool = big
        dst = np.arange(n_slots, n_slots + len(src), dtype=np.int32)
    committed = pool.clone()
    kda.state_copy(pool, i32(src), i32(dst), dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    for s_, d_ in zip(src, dst):
        assert torch.equal(pool[int(d_)], committed[int(s_)])
    others = sorted(set(range(pool.shape[0])) - set(int(x) for x in dst))
    assert torch.equal(pool[torch.as_tensor(others, device=DEV)], committed[torch.as_tensor(others, device=DEV)])
