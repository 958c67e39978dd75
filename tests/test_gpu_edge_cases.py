"""Edge cases of the prefill on the GPU (through the C ABI) against the
fp64 oracle.

* Many short sequences: 700 sequences of 0..90 tokens (several empty, many
  shorter than one chunk), H = 2, so the one-block chunk map runs three
  passes of its prefix and the scan sees 1,400 (sequence, head) pairs
  (64-column tiles); initial states from pool slots and zeros, a snapshot
  per sequence that has a full chunk.
* Batches of 128 and 129 sequences: the two sides of the chunk map's
  longest-first ranking limit.
* Degenerate gates, the special cases the recurrence reduces to:
  g = 0 with b = -30 (beta = sigmoid(-30) ~ 9e-14): no decay and no write,
  so the state stays the initial state and o_t = S0^T q_t;
  g = 0 with b = +30 (beta = 1 in fp32): the delta rule without decay,
  S_t = (I - k_t k_t^T) S_{t-1} + k_t v_t^T.
"""

import numpy as np
import pytest
import torch

import linear_attention_state_kda_amd as kda
import workloads as wl
from oracle import kda_oracle as ko
from tests.gpu_util import DEV, Worst, i32, make_pool, to_math
from tests.test_gpu_prefill import check_case, run_gpu

pytestmark = pytest.mark.gpu


def test_many_short_sequences():
    n = 700
    lens = np.random.default_rng([95, 1]).integers(0, 91, n)
    lens[[0, 5, 6, 350, 699]] = 0
    init = [(700 + i) if i % 3 == 0 else -1 for i in range(n)]
    final = list(range(n))
    tracks = [(i, 1, 1400 + i) for i in range(n) if lens[i] >= 64] + [(3, 0, -1)]
    case = wl.prefill_case(lens, 2, 128, 128, 64, "bf16", "f32", 1400 + n, init, final, tracks, True, seed=95,
                           name="700 short sequences H=2")
    toks, cu = wl.prefill_tokens(case)
    g = run_gpu(case, toks, cu)
    check_case(case, toks, cu, g, [0, 1])


@pytest.mark.parametrize("n", [128, 129])
def test_batch_at_the_ordering_limit(n):
    """Up to 128 sequences the chunk map ranks them longest first for the
    scan (ties by index); 129 take the batch order.  Lengths 0..300 with many
    equal chunk counts, H = 2 (64-column scan tiles): every sequence against
    the oracle in both regimes."""
    lens = np.random.default_rng([97, n]).integers(0, 301, n)
    lens[[0, 7, n - 1]] = [0, 300, 64]
    init = [(n + i) if i % 4 == 0 else -1 for i in range(n)]
    final = list(range(n))
    tracks = [(i, 1, 2 * n + i) for i in range(n) if lens[i] >= 64]
    case = wl.prefill_case(lens, 2, 128, 128, 64, "bf16", "f32", 3 * n, init, final, tracks, True, seed=97,
                           name=f"{n} sequences H=2")
    toks, cu = wl.prefill_tokens(case)
    g = run_gpu(case, toks, cu)
    check_case(case, toks, cu, g, [0, 1])


@pytest.mark.parametrize("b_logit", [-30.0, 30.0])
def test_degenerate_gates(b_logit):
    lens, H, d = [200, 77], 2, 128
    T = sum(lens)
    cu = np.array([0, 200, 277], dtype=np.int32)
    toks = wl.token_inputs(T, H, d, d, "bf16", 96)
    toks["g"] = torch.zeros_like(toks["g"])
    toks["b"] = torch.full_like(toks["b"], b_logit)
    pool = make_pool(6, H, d, d, "f32")
    for s in (4, 5):
        pool[s] = wl.pool_state(s, H, d, d, "f32", 96).to(DEV)
    S0 = np.stack([to_math(pool[4]), to_math(pool[5])])
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    dev = {x: toks[x].to(DEV) for x in "qkvgb"}
    o = kda.chunk_prefill(dev["q"], dev["k"], dev["v"], dev["g"], dev["b"], i32(cu), 64, pool, i32([4, 5]),
                          i32([0, 1]), dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    ex = {x: wl.exact(toks[x]) for x in "qkvgb"}
    o_ref, fin_ref, _ = ko.prefill_ref(ex["q"], ex["k"], ex["v"], ex["g"], ex["b"], cu, S0, 64)
    og = wl.exact(o.cpu())
    w = Worst(2e-2)
    for i in range(2):
        lo, hi = int(cu[i]), int(cu[i + 1])
        w.out("o", og[lo:hi], o_ref[lo:hi], 1)
        w.state("final", to_math(pool[i]), fin_ref[i])
    w.check(f"degenerate gates g=0 b={b_logit}")
    if b_logit < 0:
        # beta ~ 9e-14: the state is untouched up to that size
        for i in range(2):
            assert np.max(np.abs(to_math(pool[i]) - S0[i])) <= 1e-6 * np.max(np.abs(S0[i]))
            # and each output is the initial state read by the query (bf16 output rounding)
            lo, hi = int(cu[i]), int(cu[i + 1])
            direct = np.einsum("thk,hkv->thv", ex["q"][lo:hi], S0[i])
            assert np.max(np.abs(og[lo:hi] - direct)) <= 1e-2 * np.max(np.abs(direct))
    else:
        # beta = 1, alpha = 1: the textbook delta rule, brute force on one head
        o_b, S_b = ko.brute_ref(ex["q"][:64, :1], ex["k"][:64, :1], ex["v"][:64, :1], ex["g"][:64, :1],
                                ex["b"][:64, :1], S0[0][:1])
        o_t, _, S_t, _ = ko.run_sequence(ex["q"][:64, :1], ex["k"][:64, :1], ex["v"][:64, :1], ex["g"][:64, :1],
                                         ex["b"][:64, :1], S0[0][:1])
        assert np.allclose(o_b, o_t, rtol=1e-10, atol=1e-10) and np.allclose(S_b, S_t, rtol=1e-10, atol=1e-10)
