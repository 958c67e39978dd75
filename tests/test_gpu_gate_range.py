"""Strong gates on the GPU (through the C ABI): the supported gate range of
the chunked prefill and of verify.

The prefill scales keys by e^-Gamma inside a chunk (Gamma the cumulative log
decay since the chunk start), which must stay finite in the operand type.
Inside the documented range (chunk decay above about -11 for fp16 inputs,
about -88 for bf16) the results meet the 16-bit bar against the fp64
oracle, at decays far stronger than the workloads' (g per channel down to
-0.165 for fp16, -1.3 for bf16, against -0.1); beyond it the call sets
KDA_DEV_ERR_GATE.  With gates this strong the state forgets within a token
or two, so an output row is about u_t (q_t . k_t) and its norm follows
|q_t . k_t| down to near zero, while its rounding error follows the sizes
of q_t and k_t: rows are measured against the larger of their own norm and
their head's rms row norm (the bar on the absolute error of a row) rather
than the usual quarter of it.  verify does the same over its blocks of 8 positions in
fp32 (range about -88 per block)."""

import numpy as np
import pytest
import torch

import linear_attention_state_kda_amd as kda
import workloads as wl
from oracle import kda_oracle as ko
from tests.gpu_util import DEV, TOL, Worst, i32, make_pool, to_math

pytestmark = pytest.mark.gpu


def strong_tokens(n_tokens, H, d, in_dtype, g_lo, g_hi, seed, shape_prefix=None):
    toks = wl.token_inputs(n_tokens, H, d, d, in_dtype, seed, shape_prefix=shape_prefix)
    rng = np.random.default_rng([seed, 77])
    toks["g"] = wl.to_dtype(rng.uniform(g_lo, g_hi, tuple(toks["g"].shape)), in_dtype)
    return toks


def prefill(toks, lens, in_dtype, H, d=128, C=64):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    n = len(lens)
    pool = make_pool(n + 1, H, d, d, "f32")
    pool[n] = wl.pool_state(n, H, d, d, "f32", 5).to(DEV)
    init = [n] + [-1] * (n - 1)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    dev = {x: toks[x].to(DEV) for x in "qkvgb"}
    o = kda.chunk_prefill(dev["q"], dev["k"], dev["v"], dev["g"], dev["b"], i32(cu), C, pool, i32(init),
                          i32(list(range(n))), dev_err=err)
    torch.cuda.synchronize()
    S0 = np.zeros((n, H, d, d))
    S0[0] = to_math(pool[n])
    return cu, o, pool, int(err.item()), S0


@pytest.mark.parametrize("in_dtype,g_lo,g_hi", [("f16", -0.165, -0.1), ("bf16", -1.3, -1.0)])
def test_prefill_strong_gates_inside_range(in_dtype, g_lo, g_hi):
    H, lens = 4, [300, 64, 37]
    toks = strong_tokens(sum(lens), H, 128, in_dtype, g_lo, g_hi, seed=81)
    cu, o, pool, err, S0 = prefill(toks, lens, in_dtype, H)
    assert err == 0
    ex = {x: wl.exact(toks[x]) for x in "qkvgb"}
    assert ex["g"].reshape(-1, 128)[:64].sum(axis=0).min() < {"f16": -6.4, "bf16": -64.0}[in_dtype]
    o_ref, fin_ref, _ = ko.prefill_ref(ex["q"], ex["k"], ex["v"], ex["g"], ex["b"], cu, S0, 64)
    w = Worst(TOL[in_dtype], floor=1.0)
    og = wl.exact(o.cpu())
    for i in range(len(lens)):
        lo, hi = int(cu[i]), int(cu[i + 1])
        w.out("o", og[lo:hi], o_ref[lo:hi], 1)
        w.state("final", to_math(pool[i]), fin_ref[i])
    w.check(f"prefill {in_dtype} gates U({g_lo}, {g_hi})")


@pytest.mark.parametrize("in_dtype,g_lo,g_hi", [("f16", -0.4, -0.3), ("bf16", -2.0, -1.6)])
def test_prefill_gates_beyond_range_are_flagged(in_dtype, g_lo, g_hi):
    H, lens = 2, [130]
    toks = strong_tokens(sum(lens), H, 128, in_dtype, g_lo, g_hi, seed=82)
    _, _, _, err, _ = prefill(toks, lens, in_dtype, H)
    assert err & kda.DEV_ERR_GATE


def test_prefill_fp32_gates_beyond_range_are_flagged():
    H, lens = 2, [40]
    toks = strong_tokens(sum(lens), H, 16, "f32", -7.0, -6.0, seed=83)   # 16-token chunk decay below -96
    _, _, _, err, _ = prefill(toks, lens, "f32", H, d=16, C=16)
    assert err & kda.DEV_ERR_GATE


def run_verify(toks, n_req, L, H, d=128):
    ckpt = wl.distinct_slots(n_req, n_req + 1, 9)
    pool = make_pool(n_req + 1, H, d, d, "f32")
    for s in ckpt:
        pool[int(s)] = wl.pool_state(int(s), H, d, d, "f32", 9).to(DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    dev = {x: toks[x].to(DEV) for x in "qkvgb"}
    o, u_rec, _ = kda.recurrent_verify(dev["q"], dev["k"], dev["v"], dev["g"], dev["b"], pool, i32(ckpt),
                                       dev_err=err)
    torch.cuda.synchronize()
    S0 = np.stack([to_math(pool[int(s)]) for s in ckpt])
    return o, u_rec, int(err.item()), S0


def test_verify_strong_gates():
    n_req, L, H = 4, 11, 2
    toks = strong_tokens(n_req * L, H, 128, "bf16", -10.0, -8.0, seed=84, shape_prefix=(n_req, L))
    o, u_rec, err, S0 = run_verify(toks, n_req, L, H)
    assert err == 0                       # 8 positions x at most -10: above -88
    ex = {x: wl.exact(toks[x]) for x in "qkvgb"}
    o_ref, u_ref, _, _ = ko.verify_ref(ex["q"], ex["k"], ex["v"], ex["g"], ex["b"], S0)
    wo, wu = Worst(2e-2, floor=1.0), Worst(1e-4)
    og, ug = wl.exact(o.cpu()), u_rec.cpu().double().numpy()
    for i in range(n_req):
        wo.out("o", og[i], o_ref[i], 1)
        wu.out("u", ug[i], u_ref[i], 0)
    wo.check("verify gates U(-10, -8) o")
    wu.check("verify gates U(-10, -8) u")
    toks = strong_tokens(n_req * L, H, 128, "bf16", -13.0, -12.0, seed=85, shape_prefix=(n_req, L))
    _, _, err, _ = run_verify(toks, n_req, L, H)
    assert err & kda.DEV_ERR_GATE          # 8 positions x -12: below -88
