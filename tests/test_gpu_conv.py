"""GPU parity of kda_conv_state_update (through the C ABI) against the
conv-state oracle: bit-exact on every tensor, including slots and rows the
call must leave alone."""

import numpy as np
import pytest
import torch

import linear_attention_state_kda_amd as kda
import workloads as wl
from oracle import conv_oracle as co
from tests.gpu_util import DEV, i32

pytestmark = pytest.mark.gpu

INT_OF = {torch.bfloat16: torch.int16, torch.float16: torch.int16, torch.float32: torch.int32}
NP_OF = {torch.int16: np.uint16, torch.int32: np.uint32}


def rand_bits(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    it = INT_OF[dtype]
    hi = 1 << (16 if it == torch.int16 else 31)
    return torch.randint(0, hi, shape, dtype=torch.int64, generator=g).to(it).view(dtype).to(DEV)


def bits(t):
    it = INT_OF[t.dtype]
    return t.view(it).cpu().numpy().view(NP_OF[it])


def run_and_check(tensors, keep, dst, src, shift):
    before = [bits(t) for t in tensors]
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    kda.conv_state_update(tensors, keep, i32(dst), i32(src), i32(shift), dev_err=err)
    torch.cuda.synchronize()
    want, want_err = co.conv_update_ref(before, keep, dst, src, shift)
    for t, w in zip(tensors, want):
        assert np.array_equal(bits(t), w)
    assert err.item() == want_err
    return want_err


def test_conv_update_matches_oracle():
    a = rand_bits((16, 11, 4096), torch.bfloat16, 1)
    b = rand_bits((16, 6, 64), torch.float32, 2)
    big = rand_bits((16, 14, 512), torch.bfloat16, 3)
    c = big[:, :9, :]                                     # slot stride of 14 rows, 9 rows used
    pad_before = bits(big)[:, 9:]
    keep = [3, 2, 4]                                      # shifts up to min(11-3, 6-2, 9-4) = 4
    ops = [(0, -1, 0),                                    # clear
           (1, 5, 0),                                     # fork copy of the history
           (6, 6, 1), (7, 7, 2), (8, 8, 0), (9, 9, 4),    # in-place compactions (one no-op)
           (10, 11, 3),                                   # shift into another slot
           (16, 2, 0), (12, 17, 0), (13, 3, 5), (14, -2, 0),   # bad dst, bad src, bad shift, bad src
           (15, -1, 7)]                                   # clear (shift ignored)
    dst, src, shift = (list(x) for x in zip(*ops))
    e = run_and_check([a, b, c], keep, dst, src, shift)
    assert e == kda.DEV_ERR_SLOT | kda.DEV_ERR_SHIFT
    assert np.array_equal(bits(big)[:, 9:], pad_before)  # rows beyond the window untouched


@pytest.mark.parametrize("shift_max", [0, 8])
def test_conv_single_tensor_every_shift(shift_max):
    t = rand_bits((12, 11, 256), torch.float16, 4)
    ops = [(s, s, min(s, shift_max)) for s in range(9)]   # in place, shifts 0..8
    dst, src, shift = (list(x) for x in zip(*ops))
    assert run_and_check([t], [3], dst, src, shift) == 0


def test_conv_speculative_decode_shape():
    """The decode step's conv half at the speculative-decode workload: three
    conv tensors (q, k, v; 32 heads x 128 = 4096 channels, width 4 so 3
    history rows, plus 8 speculative rows), 1024 slots; compaction of the
    256 requests in place at their accepted lengths, then the fork of 64
    committed requests to 4 fresh children each."""
    case = wl.spec_case(seed=3)
    ts = [rand_bits((case["n_slots"], 11, 4096), torch.bfloat16, 10 + j) for j in range(3)]
    keep = [3, 3, 3]
    ck = case["ckpt_slots"].tolist()
    assert run_and_check(ts, keep, ck, ck, case["accepted"].tolist()) == 0
    n = len(case["fork_src"])
    assert run_and_check(ts, keep, case["fork_dst"].tolist(), case["fork_src"].tolist(), [0] * n) == 0


def test_conv_whole_slot_copy():
    """keep == rows: a copy moves the whole window; no shift is valid."""
    t = rand_bits((6, 4, 128), torch.bfloat16, 6)
    u = rand_bits((6, 4, 32), torch.float32, 7)
    dst, src, shift = [1, 2, 3, 4], [0, -1, 5, 5], [0, 0, 1, 0]
    e = run_and_check([t, u], [4, 4], dst, src, shift)
    assert e == kda.DEV_ERR_SHIFT


def test_conv_no_ops():
    t = rand_bits((4, 5, 64), torch.bfloat16, 5)
    before = bits(t)
    e = torch.empty(0, dtype=torch.int32, device=DEV)
    kda.conv_state_update([t], [2], e, e, e)
    torch.cuda.synchronize()
    assert np.array_equal(bits(t), before)
