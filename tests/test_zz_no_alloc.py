"""The allocation-free prefill entry point (kda_chunk_prefill_noalloc,
through the C ABI) against kda_chunk_prefill with a caller-allocated
workspace: two calls in a row, the single-layer workload (T = 8229, H = 32,
230 MB of records in the library's 256 MiB static scratch) and then a
smaller multi-sequence batch, each bit for bit equal to the workspace
call's outputs, final states, snapshots and fp32 snapshots (the two share
every kernel, and the kernels are deterministic).  A batch whose workspace
would exceed the scratch is refused before any launch."""

import numpy as np
import pytest
import torch

import linear_attention_state_kda_amd as kda
import workloads as wl
from tests.gpu_util import DEV, i32, make_pool

pytestmark = pytest.mark.gpu


def both(case):
    toks, cu = wl.prefill_tokens(case)
    H, d, C = case["H"], case["dk"], case["chunk"]
    dev = {n: toks[n].to(DEV) for n in "qkvgb"}
    tr = sorted(case["tracks"], key=lambda t: t[0])
    ptr = np.zeros(len(case["lengths"]) + 1, dtype=np.int32)
    for s, _, _ in tr:
        ptr[s + 1:] += 1
    out = []
    for fn in (kda.chunk_prefill, kda.chunk_prefill_noalloc):
        pool = make_pool(case["n_slots"], H, d, d, case["pool_dtype"])
        for s in case["init_slots"]:
            if s >= 0:
                pool[s] = wl.pool_state(s, H, d, d, case["pool_dtype"], case["seed"]).to(DEV)
        tf = torch.full((max(len(tr), 1), H, d, d), float("nan"), device=DEV)
        o = torch.full((int(cu[-1]), H, d), 3.0, dtype=wl.DTYPES[case["in_dtype"]], device=DEV)
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        print(f"[no_alloc] {fn.__name__} on {case['name'] or case['lengths']}", flush=True)
        fn(dev["q"], dev["k"], dev["v"], dev["g"], dev["b"], i32(cu), C, pool, i32(case["init_slots"]),
           i32(case["final_slots"]), track_ptr=i32(ptr), track_chunk=i32([t[1] for t in tr]),
           track_slot=i32([t[2] for t in tr]), track_f32=tf, o=o, dev_err=err)
        torch.cuda.synchronize()
        assert err.item() == 0
        out.append((o, pool, tf))
    return out


def test_noalloc_matches_workspace_call_twice():
    big = wl.single_layer_prefill()
    small = wl.prefill_case([300, 64, 1, 0, 130, 37], 4, 128, 128, 64, "bf16", "f32", 16,
                            [10, -1, 11, -1, 12, -1], [0, 1, 2, 3, 4, 5], [(0, 2, 6), (4, 1, 7), (3, 0, 8)],
                            True, seed=91)
    need = kda.prefill_workspace_bytes(1, 8229, 32, 128, 128, 64, torch.bfloat16)
    assert need <= kda.NOALLOC_SCRATCH_BYTES
    for case in (big, small):          # the second call is the smaller input
        (o_ws, pool_ws, tf_ws), (o_na, pool_na, tf_na) = both(case)
        assert torch.equal(o_na, o_ws)
        assert torch.equal(pool_na, pool_ws)
        assert torch.equal(tf_na.nan_to_num(7.0), tf_ws.nan_to_num(7.0))


def test_noalloc_refuses_more_than_the_scratch():
    H, d = 32, 128
    T = 2 * 8229
    q = torch.zeros((T, H, d), dtype=torch.bfloat16, device=DEV)
    pool = make_pool(2, H, d, d, "f32")
    with pytest.raises(kda.KdaError) as e:
        kda.chunk_prefill_noalloc(q, q, q, q, q[:, :, 0].contiguous(), i32([0, 8229, T]), 64, pool,
                                  i32([-1, -1]), i32([0, 1]))
    assert e.value.status == 3        # KDA_ERR_WORKSPACE, before any launch
    assert bool((pool == -7.25).all())
