"""GPU parity of the fused q/k L2 normalisation (flags = KDA_QK_L2NORM).

The workloads specify q and k "L2-normalised per head"; with the flag the
prefill and verify kernels take q and k unnormalised and normalise each
(token, head) row over d_k themselves, rounding the result once to the input
dtype.  The oracle side is the same two steps on the CPU: ``l2norm_rows`` in
fp64, one rounding to the input dtype, then the unchanged recurrence.

Inputs: the seeded token rows of ``workloads.token_inputs`` with every q and
k row scaled by its own factor in [0.3, 4] before rounding, so no row
arrives normalised.
"""

import numpy as np
import pytest
import torch

import linear_attention_state_kda_amd as kda
import workloads as wl
from oracle import kda_oracle as ko
from tests.gpu_util import DEV, TOL, Worst, i32, make_pool, rel_per_head, to_math

pytestmark = pytest.mark.gpu


def raw_tokens(n_tokens, H, d, in_dtype, seed, shape_prefix=None):
    toks = wl.token_inputs(n_tokens, H, d, d, in_dtype, seed, shape_prefix=shape_prefix)
    rng = np.random.default_rng([seed, 99])
    for n in "qk":
        x = wl.exact(toks[n])
        scale = rng.uniform(0.3, 4.0, size=x.shape[:-1] + (1,))
        toks[n] = wl.to_dtype(x * scale, in_dtype)
    return toks


def normalised(toks, in_dtype):
    """The oracle's view: q and k normalised in fp64, rounded once to in_dtype."""
    ex = {n: wl.exact(toks[n]) for n in "qkvgb"}
    for n in "qk":
        ex[n] = wl.exact(wl.to_dtype(ko.l2norm_rows(ex[n]), in_dtype))
    return ex


@pytest.mark.parametrize("H,in_dtype", [(3, "bf16"), (12, "bf16"), (3, "f16")])
def test_prefill_normalises_q_k(H, in_dtype):
    lens = [300, 64, 1, 0, 130, 37]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, d, C = int(cu[-1]), 128, 64
    toks = raw_tokens(T, H, d, in_dtype, seed=31)
    n = len(lens)
    pool = make_pool(2 * n, H, d, d, "f32")
    init = [-1, 7, -1, 8, -1, 9]
    S0 = np.zeros((n, H, d, d))
    for i, s in enumerate(init):
        if s >= 0:
            pool[s] = wl.pool_state(s, H, d, d, "f32", 31).to(DEV)
            S0[i] = to_math(pool[s])
    tracks = [(0, 2, 10), (4, 1, 11)]
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    dev = {x: toks[x].to(DEV) for x in "qkvgb"}
    o = kda.chunk_prefill(dev["q"], dev["k"], dev["v"], dev["g"], dev["b"], i32(cu), C, pool,
                          i32(init), i32(list(range(n))), track_ptr=i32([0, 1, 1, 1, 1, 2, 2]),
                          track_chunk=i32([2, 1]), track_slot=i32([10, 11]), dev_err=err,
                          qk_l2norm=True)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ex = normalised(toks, in_dtype)
    o_ref, fin_ref, snaps = ko.prefill_ref(ex["q"], ex["k"], ex["v"], ex["g"], ex["b"], cu, S0, C,
                                           [(s, c) for s, c, _ in tracks])
    w = Worst(TOL[in_dtype])
    og = wl.exact(o.cpu())
    for i in range(n):
        lo, hi = int(cu[i]), int(cu[i + 1])
        if hi > lo:
            w.out("o", og[lo:hi], o_ref[lo:hi], 1)
        w.state("final", to_math(pool[i]), fin_ref[i])
    for e, (_, _, slot) in enumerate(tracks):
        w.state("snap", to_math(pool[slot]), snaps[e])
    w.check(f"prefill l2norm H={H} {in_dtype}")


def test_prefill_fp32_normalises_q_k():
    """The fp32 configuration (d = 16, chunk 16): normalisation in fp32 is
    held to the fp32 bar."""
    lens = [64, 37, 16, 5]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H, d, C = int(cu[-1]), 2, 16, 16
    toks = raw_tokens(T, H, d, "f32", seed=34)
    n = len(lens)
    pool = make_pool(n, H, d, d, "f32")
    dev = {x: toks[x].to(DEV) for x in "qkvgb"}
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    o = kda.chunk_prefill(dev["q"], dev["k"], dev["v"], dev["g"], dev["b"], i32(cu), C, pool,
                          i32([-1] * n), i32(list(range(n))), dev_err=err, qk_l2norm=True)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ex = normalised(toks, "f32")
    o_ref, fin_ref, _ = ko.prefill_ref(ex["q"], ex["k"], ex["v"], ex["g"], ex["b"], cu,
                                       np.zeros((n, H, d, d)), C)
    og = wl.exact(o.cpu())
    w = Worst(1e-4)
    for i in range(n):
        lo, hi = int(cu[i]), int(cu[i + 1])
        w.out("o", og[lo:hi], o_ref[lo:hi], 1)
        w.state("final", to_math(pool[i]), fin_ref[i])
    w.check("prefill l2norm fp32 d=16")


def test_prefill_flag_on_normalised_input_changes_little():
    """Inputs already normalised (the workloads' own draw): the flag only
    re-rounds, so outputs stay within the 16-bit bar of the flag-off run."""
    case = wl.prefill_case([200, 77], 2, 128, 128, 64, "bf16", "f32", 4, [-1, -1], [0, 1], [], False,
                           seed=32)
    toks, cu = wl.prefill_tokens(case)
    dev = {x: toks[x].to(DEV) for x in "qkvgb"}
    outs = []
    for flag in (False, True):
        pool = make_pool(4, 2, 128, 128, "f32")
        o = kda.chunk_prefill(dev["q"], dev["k"], dev["v"], dev["g"], dev["b"], i32(cu), 64, pool,
                              i32([-1, -1]), i32([0, 1]), qk_l2norm=flag)
        torch.cuda.synchronize()
        outs.append(wl.exact(o.cpu()))
    assert rel_per_head(outs[1], outs[0], 1) < 1e-2


@pytest.mark.parametrize("L,in_dtype", [(8, "bf16"), (13, "bf16"), (8, "f16"), (8, "f32")])
def test_verify_and_commit_normalise_q_k(L, in_dtype):
    n_req, H, d = 6, 3, 128
    toks = raw_tokens(n_req * L, H, d, in_dtype, seed=33, shape_prefix=(n_req, L))
    ckpt = wl.distinct_slots(n_req, n_req + 2, 33)
    pool = make_pool(n_req + 2, H, d, d, "f32")
    for s in ckpt:
        pool[int(s)] = wl.pool_state(int(s), H, d, d, "f32", 33).to(DEV)
    S0 = np.stack([to_math(pool[int(s)]) for s in ckpt])
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    dev = {x: toks[x].to(DEV) for x in "qkvgb"}
    o, u_rec, kg_rec = kda.recurrent_verify(dev["q"], dev["k"], dev["v"], dev["g"], dev["b"], pool,
                                            i32(ckpt), dev_err=err, qk_l2norm=True)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ex = normalised(toks, in_dtype)
    kg = wl.exact(kg_rec.cpu())
    # the key record holds the normalised key: equal to the oracle's rounding
    # except where fp32 and fp64 normalisation round to neighbours (one ulp)
    key = kg[..., :d]
    key_ref = np.transpose(ex["k"], (0, 2, 1, 3))
    mant = {"bf16": 7, "f16": 10, "f32": 23}[in_dtype]
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(key_ref), 1e-30))) - mant)
    if in_dtype == "f16":
        ulp = np.maximum(ulp, 2.0 ** -24)
    if in_dtype == "f32":
        # fp32 normalisation (hardware reciprocal square root) against fp64:
        # a few ulp, never a different rounding region
        assert np.all(np.abs(key - key_ref) <= 8 * ulp)
    else:
        assert np.all(np.abs(key - key_ref) <= ulp)
        assert np.mean(key == key_ref) > 0.99
    assert np.array_equal(kg[..., d:], np.transpose(ex["g"], (0, 2, 1, 3)))   # the raw gate as is
    # Where a 16-bit key rounds to the neighbouring value the recurrence is
    # that of the kernel's key, so the oracle takes the key from the record
    # (checked just above against l2norm_rows); u and the commit are then
    # fp32 arithmetic on exact inputs and are held to the fp32 bar.  (With
    # fp32 inputs the two keys differ by a few fp32 ulp only.)
    ex["k"] = np.transpose(key, (0, 2, 1, 3))
    o_ref, u_ref, kg_ref, _ = ko.verify_ref(ex["q"], ex["k"], ex["v"], ex["g"], ex["b"], S0)
    og, ug = wl.exact(o.cpu()), u_rec.cpu().double().numpy()
    wo, wu = Worst(TOL[in_dtype]), Worst(1e-4)
    for i in range(n_req):
        wo.out("o", og[i], o_ref[i], 1)
        wu.out("u", ug[i], u_ref[i], 0)
    wo.check(f"verify l2norm {in_dtype} L={L} o")
    wu.check(f"verify l2norm {in_dtype} L={L} u")
    # commit from those records = replay of the normalised tokens
    acc = np.random.default_rng([33, 5]).integers(0, L + 1, n_req)
    kda.commit(pool, i32(ckpt), i32(acc), u_rec, kg_rec, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    wc = Worst(1e-4)
    for i, s in enumerate(ckpt):
        n = int(acc[i])
        ref = ko.replay_ref(ex["q"][i], ex["k"][i], ex["v"][i], ex["g"][i], ex["b"][i], S0[i], n)
        wc.state("commit", to_math(pool[int(s)]), ref)
    wc.check(f"commit l2norm {in_dtype} L={L}")
