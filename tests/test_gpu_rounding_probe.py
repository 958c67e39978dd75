"""The single-rounding probe run through the kernels that write 16-bit pools.

The SGLang PR #34820 summary (key files: the track-state dtype test; review
comments) names a probe showing that an fp16 state pool must be written by
one rounding of the fp32 state, not by a detour through bf16.  The value
x = 1 + 2^-8 (golden fixture `double_round_probe.json`) separates the two:
one RNE rounding to fp16 keeps it (bits 0x3C04), rounding through bf16 first
gives 1.0 (0x3C00); one rounding to bf16 gives 1.0 (0x3F80).

Construction: zero initial state, g = 0 (no decay), b = 30 (sigmoid(30) is
exactly 1 in fp32), a one-hot key e_i on the first token and zero keys after
it, every value channel of the first token equal to x.  The recurrence then
leaves S[i][:] = x exactly and every other entry 0, in any summation order,
so each kernel that casts the state into a pool (prefill final state,
prefill snapshot, commit) must store the fixture's bits.
"""

import json
import os

import numpy as np
import pytest
import torch

import linear_attention_state_kda_amd as kda
from tests.gpu_util import DEV, i32

pytestmark = pytest.mark.gpu

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "double_round_probe.json")))
X = GOLDEN["x"]
BITS = {"f16": GOLDEN["fp16_direct_bits"], "bf16": GOLDEN["bf16_bits"]}
TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
KEY = 3   # the one-hot key channel


def probe_tokens(T, H, d, in_dtype, shape_prefix=()):
    q = torch.zeros(shape_prefix + (T, H, d))
    k = torch.zeros_like(q)
    v = torch.zeros_like(q)
    k[..., 0, :, KEY] = 1.0
    q[..., :, :, KEY] = 1.0
    v[..., 0, :, :] = X
    g = torch.zeros_like(q)
    b = torch.full(shape_prefix + (T, H), 30.0)
    return [t.to(TD[in_dtype]).to(DEV) for t in (q, k, v, g, b)]


def expect_row_bits(slot, pool_dtype):
    """Pool slot [H, d_v, d_k]: column KEY holds x's bits, everything else is 0."""
    bits = slot.view(torch.int16).to(torch.int32) & 0xFFFF
    want = torch.zeros_like(bits)
    want[:, :, KEY] = BITS[pool_dtype]
    assert torch.equal(bits, want), (pool_dtype, torch.unique(bits).tolist())


@pytest.mark.parametrize("pool_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("in_dtype,d,C", [("f32", 16, 16), ("f16", 128, 64)])
def test_prefill_final_and_snapshot_round_once(in_dtype, d, C, pool_dtype):
    T, H = 2 * C + 5, 2
    q, k, v, g, b = probe_tokens(T, H, d, in_dtype)
    pool = torch.full((3, H, d, d), -7.25, dtype=TD[pool_dtype], device=DEV)
    track_f32 = torch.full((1, H, d, d), float("nan"), device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    kda.chunk_prefill(q, k, v, g, b, i32([0, T]), C, pool, i32([-1]), i32([0]),
                      track_ptr=i32([0, 1]), track_chunk=i32([2]), track_slot=i32([1]),
                      track_f32=track_f32, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    want32 = torch.zeros_like(track_f32)
    want32[..., KEY] = X
    assert torch.equal(track_f32, want32)        # the fp32 snapshot holds x exactly
    expect_row_bits(pool[0], pool_dtype)          # final state
    expect_row_bits(pool[1], pool_dtype)          # snapshot at c = 2
    assert bool((pool[2] == -7.25).all())         # untouched slot


@pytest.mark.parametrize("pool_dtype", ["f16", "bf16"])
def test_commit_rounds_once(pool_dtype):
    n_req, L, H, d = 2, 4, 2, 128
    q, k, v, g, b = probe_tokens(L, H, d, "f16", shape_prefix=(n_req,))
    pool = torch.zeros((3, H, d, d), dtype=TD[pool_dtype], device=DEV)
    pool[2] = -7.25
    ckpt = i32([0, 1])
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    _, u_rec, kg_rec = kda.recurrent_verify(q, k, v, g, b, pool, ckpt, dev_err=err)
    kda.commit(pool, ckpt, i32([1, L]), u_rec, kg_rec, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    # the fp32 correction of the first position is x itself
    assert bool((u_rec[:, :, 0, :] == X).all())
    expect_row_bits(pool[0], pool_dtype)          # committed after one position
    expect_row_bits(pool[1], pool_dtype)          # after all L (zero keys change nothing)
    assert bool((pool[2] == -7.25).all())
