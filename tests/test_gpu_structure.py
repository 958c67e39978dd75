"""Structural properties of the GPU path that hold bitwise (through the C ABI).

* Packing independence: a sequence prefilled inside a packed batch gives the
  same outputs, snapshots and final state, bit for bit, as the sequence
  prefilled alone (every (chunk, head) record and every (sequence, head)
  chain depends only on that sequence's tokens).
* Split invariance: prefilling T1 = 4 full chunks, then the rest of the
  sequence from the final state left in an fp32 pool slot, reproduces the
  one-shot run bit for bit (the same chunks meet the same fp32 state).
* Concurrent calls on three streams (two prefills with their own
  workspaces and a verify) equal the same calls one after the other.
* Graph capture: prefill, verify, commit, align commit (with its next-step
  outputs), copy and the conv-state update captured once in a HIP graph and
  replayed three times, with eager work and synchronisations in between,
  reproduce the eager results bit for bit each time.
"""

import numpy as np
import pytest
import torch

import linear_attention_state_kda_amd as kda
import workloads as wl
from tests.gpu_util import DEV, i32, make_pool

pytestmark = pytest.mark.gpu

H, D, C = 2, 128, 64


def run_prefill(toks, lens, pool, init, final, tracks=(), track_f32=None):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    dev = {n: toks[n].to(DEV) for n in "qkvgb"}
    ptr = np.zeros(len(lens) + 1, dtype=np.int32)
    for s, _, _ in tracks:
        ptr[s + 1:] += 1
    o = kda.chunk_prefill(dev["q"], dev["k"], dev["v"], dev["g"], dev["b"], i32(cu), C, pool,
                          i32(init), i32(final), track_ptr=i32(ptr),
                          track_chunk=i32([c for _, c, _ in tracks]),
                          track_slot=i32([sl for _, _, sl in tracks]), track_f32=track_f32)
    torch.cuda.synchronize()
    return o


def test_prefill_packing_independence():
    lens = [300, 130, 77]
    toks = wl.token_inputs(sum(lens), H, D, D, "bf16", 41)
    cu = np.concatenate([[0], np.cumsum(lens)])
    packed_pool = make_pool(8, H, D, D, "f32")
    packed_pool[6] = wl.pool_state(6, H, D, D, "f32", 41).to(DEV)
    tf_packed = torch.zeros((2, H, D, D), device=DEV)
    o_packed = run_prefill(toks, lens, packed_pool, [-1, 6, -1], [0, 1, 2], [(0, 2, 3), (1, 1, 4)], tf_packed)
    for i, L in enumerate(lens):
        part = {n: toks[n][cu[i]:cu[i + 1]] for n in "qkvgb"}
        pool = make_pool(8, H, D, D, "f32")
        pool[6] = packed_pool[6]
        tracks = {0: [(0, 2, 3)], 1: [(0, 1, 4)]}.get(i, [])
        tf = torch.zeros((max(len(tracks), 1), H, D, D), device=DEV)
        o = run_prefill(part, [L], pool, [[-1, 6, -1][i]], [i], tracks, tf)
        assert torch.equal(o, o_packed[cu[i]:cu[i + 1]])
        assert torch.equal(pool[i], packed_pool[i])
        for e, (_, _, sl) in enumerate(tracks):
            assert torch.equal(pool[sl], packed_pool[sl])
            assert torch.equal(tf[e], tf_packed[sl - 3])


def test_prefill_split_invariance():
    T, T1 = 4 * C + 101, 4 * C
    toks = wl.token_inputs(T, H, D, D, "bf16", 42)
    pool = make_pool(6, H, D, D, "f32")
    pool[5] = wl.pool_state(5, H, D, D, "f32", 42).to(DEV)
    o_one = run_prefill(toks, [T], pool, [5], [0], [(0, 4, 1)], torch.zeros((1, H, D, D), device=DEV))
    first = {n: toks[n][:T1] for n in "qkvgb"}
    rest = {n: toks[n][T1:] for n in "qkvgb"}
    o_a = run_prefill(first, [T1], pool, [5], [2])
    o_b = run_prefill(rest, [T - T1], pool, [2], [3])
    assert torch.equal(pool[2], pool[1])                 # state after 4 chunks = snapshot c = 4
    assert torch.equal(torch.cat([o_a, o_b]), o_one)
    assert torch.equal(pool[3], pool[0])                 # final states


def test_concurrent_calls_on_streams():
    """Two prefills (each with its own workspace) and a verify issued on
    three streams at once give, bit for bit, what they give one after the
    other: the library keeps no state between calls beyond the caller's
    buffers."""
    def setup(seed, lens):
        toks = wl.token_inputs(sum(lens), H, D, D, "bf16", seed)
        cu = i32(np.concatenate([[0], np.cumsum(lens)]))
        dev = {n: toks[n].to(DEV) for n in "qkvgb"}
        pool = make_pool(4, H, D, D, "f32")
        ws = torch.empty(kda.prefill_workspace_bytes(len(lens), sum(lens), H, D, D, C, torch.bfloat16),
                         dtype=torch.uint8, device=DEV)
        return dev, cu, pool, ws, len(lens)
    calls = [setup(51, [700, 333]), setup(52, [1030])]
    vt = {n: x.to(DEV) for n, x in wl.token_inputs(16 * 8, H, D, D, "bf16", 53, shape_prefix=(16, 8)).items()}
    vpool = make_pool(16, H, D, D, "f32")
    for s_ in range(16):
        vpool[s_] = wl.pool_state(s_, H, D, D, "f32", 53).to(DEV)
    ck = i32(list(range(16)))

    def run_all(streams):
        outs = []
        for _, _, pool, _, _ in calls:
            pool.fill_(0.0)
        torch.cuda.synchronize()   # the pools are clear before any stream starts
        for (dev, cu, pool, ws, n), st in zip(calls, streams[:2]):
            with torch.cuda.stream(st):
                o = kda.chunk_prefill(dev["q"], dev["k"], dev["v"], dev["g"], dev["b"], cu, C, pool,
                                      i32([-1] * n), i32(list(range(n))), workspace=ws)
            outs.append((o, pool))
        with torch.cuda.stream(streams[2]):
            vo = kda.recurrent_verify(vt["q"], vt["k"], vt["v"], vt["g"], vt["b"], vpool, ck)
        torch.cuda.synchronize()
        return [(o.clone(), p.clone()) for o, p in outs], [x.clone() for x in vo]

    cur = torch.cuda.current_stream()
    serial = run_all([cur, cur, cur])
    side = [torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for _ in range(3):
        conc = run_all(side)
        for (o1, p1), (o2, p2) in zip(serial[0], conc[0]):
            assert torch.equal(o1, o2) and torch.equal(p1, p2)
        for a, b in zip(serial[1], conc[1]):
            assert torch.equal(a, b)


def test_graph_capture_replay():
    # prefill (two sequences), then verify / commit / copy on four requests
    lens = [150, 64]
    ptoks = {n: t.to(DEV) for n, t in wl.token_inputs(sum(lens), H, D, D, "bf16", 43).items()}
    cu = i32(np.concatenate([[0], np.cumsum(lens)]))
    n_req, L = 4, 8
    stoks = {n: t.to(DEV) for n, t in
             wl.token_inputs(n_req * L, H, D, D, "bf16", 44, shape_prefix=(n_req, L)).items()}
    pool0 = make_pool(16, H, D, D, "f32")
    for s in range(4):
        pool0[s] = wl.pool_state(s, H, D, D, "f32", 43).to(DEV)
    pool = pool0.clone()
    o_p = torch.empty((sum(lens), H, D), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(kda.prefill_workspace_bytes(2, sum(lens), H, D, D, C, torch.bfloat16),
                     dtype=torch.uint8, device=DEV)
    track_f32 = torch.empty((1, H, D, D), device=DEV)
    o_v = torch.empty((n_req, L, H, D), dtype=torch.bfloat16, device=DEV)
    u_rec = torch.empty((n_req, H, L, D), device=DEV)
    kg_rec = torch.empty((n_req, H, L, 2 * D), dtype=torch.bfloat16, device=DEV)
    args = dict(init=i32([0, -1]), final=i32([4, 5]), ptr=i32([0, 1, 1]), tc=i32([2]), ts=i32([6]),
                ckpt=i32([0, 1, 2, 3]), acc=i32([8, 0, 3, 5]), src=i32([0, 2]), dst=i32([7, 8]))
    # align commit on a pool of its own: tables of 2 blocks of 12 tokens per request
    apool0 = make_pool(12, H, D, D, "f32")
    for s in range(4):
        apool0[s] = wl.pool_state(20 + s, H, D, D, "f32", 43).to(DEV)
    apool = apool0.clone()
    a_table = i32([[0, 4], [1, 5], [2, 6], [3, 7]])
    a_tok, a_acc = i32([5, 10, 12, 1]), i32([8, 3, 4, 0])
    a_next = [torch.zeros(n_req, dtype=torch.int32, device=DEV) for _ in range(4)]
    # conv windows: two tensors, a fork copy, an in-place compaction and a clear
    conv0 = [(torch.arange(8 * 11 * 256, device=DEV, dtype=torch.float32).reshape(8, 11, 256) % 977).to(torch.bfloat16),
             torch.arange(8 * 6 * 64, device=DEV, dtype=torch.float32).reshape(8, 6, 64) * 0.5]
    conv = [t.clone() for t in conv0]
    c_dst, c_src, c_shift = i32([1, 2, 3]), i32([0, 2, -1]), i32([0, 2, 0])

    def calls():
        kda.chunk_prefill(ptoks["q"], ptoks["k"], ptoks["v"], ptoks["g"], ptoks["b"], cu, C, pool,
                          args["init"], args["final"], track_ptr=args["ptr"], track_chunk=args["tc"],
                          track_slot=args["ts"], track_f32=track_f32, o=o_p, workspace=ws)
        kda.recurrent_verify(stoks["q"], stoks["k"], stoks["v"], stoks["g"], stoks["b"], pool,
                             args["ckpt"], o=o_v, u_rec=u_rec, kg_rec=kg_rec)
        kda.commit(pool, args["ckpt"], args["acc"], u_rec, kg_rec)
        kda.commit_align(apool, a_table, a_tok, a_acc, 12, u_rec, kg_rec, next_tokens=a_next[0],
                         next_block=a_next[1], next_ckpt=a_next[2], copy_bias=a_next[3])
        kda.state_copy(pool, args["src"], args["dst"])
        kda.conv_state_update(conv, [3, 2], c_dst, c_src, c_shift)

    outs = (o_p, track_f32, o_v, u_rec, kg_rec, *a_next, pool, apool, *conv)
    calls()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pool.copy_(pool0)
        apool.copy_(apool0)
        for t, t0 in zip(conv, conv0):
            t.copy_(t0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        pool.copy_(pool0)                 # eager work between replays
        apool.copy_(apool0)
        for t, t0 in zip(conv, conv0):
            t.copy_(t0)
        for t in outs[:9]:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, eager):
            assert torch.equal(got, want), rep
