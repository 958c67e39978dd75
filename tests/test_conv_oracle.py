"""Pins for the conv-state oracle (oracle/conv_oracle.py), on the CPU.

Each test fixes the behaviour from the operation's meaning rather than from
the oracle's own indexing: the compaction is checked against the direct
definition of a short convolution's history window after n accepted
positions (state-semantics page sec. 2; RecoverSSM summary step 4), and the
clear / copy / error cases against literal expectations.
"""

import numpy as np
import pytest

from oracle import conv_oracle as co


def _bits(rng, n_slots, rows, dim, dtype=np.uint16):
    return rng.integers(0, np.iinfo(dtype).max, size=(n_slots, rows, dim), dtype=dtype)


def test_literal_shift_example():
    # one channel, a window of 5 rows, history of 2: sliding by 2 puts rows
    # 2 and 3 first and leaves rows 2.. as they were
    t = np.array([[[10], [11], [12], [13], [14]]], dtype=np.uint16)
    (out,), err = co.conv_update_ref([t], [2], dst=[0], src=[0], shift=[2])
    assert err == 0
    assert out[0, :, 0].tolist() == [12, 13, 12, 13, 14]


def test_clear_zeroes_every_row_of_dst_only():
    rng = np.random.default_rng(1)
    a, b = _bits(rng, 6, 7, 16), _bits(rng, 6, 4, 8, np.uint32)
    (oa, ob), err = co.conv_update_ref([a, b], [3, 2], dst=[2], src=[-1], shift=[0])
    assert err == 0
    assert not oa[2].any() and not ob[2].any()
    for o, t in ((oa, a), (ob, b)):
        keep_slots = [s for s in range(6) if s != 2]
        assert np.array_equal(o[keep_slots], t[keep_slots])


def test_copy_writes_history_rows_only():
    rng = np.random.default_rng(2)
    a = _bits(rng, 5, 9, 24)
    (o,), err = co.conv_update_ref([a], [3], dst=[4], src=[1], shift=[0])
    assert err == 0
    assert np.array_equal(o[4, :3], a[1, :3])
    assert np.array_equal(o[4, 3:], a[4, 3:])        # speculative rows of dst unchanged
    assert np.array_equal(o[:4], a[:4])


@pytest.mark.parametrize("keep,L", [(3, 8), (1, 4), (5, 2)])
def test_compaction_is_the_window_after_accept(keep, L):
    rng = np.random.default_rng(3 + keep)
    dim, T = 12, 64
    stream = rng.integers(0, 60000, size=(T, dim), dtype=np.uint16)
    t = 20                                             # last position already in the history
    window = np.concatenate([stream[t - keep + 1:t + 1], stream[t + 1:t + 1 + L]])   # history + L speculative
    for n in range(L + 1):
        slots = _bits(rng, 3, keep + L, dim)
        slots[1] = window
        (o,), err = co.conv_update_ref([slots], [keep], dst=[1], src=[1], shift=[n])
        assert err == 0
        assert np.array_equal(o[1, :keep], co.window_after_accept(stream, t, keep, n))
        assert np.array_equal(o[[0, 2]], slots[[0, 2]])


def test_window_definition_itself():
    stream = np.arange(40, dtype=np.uint16)[:, None] * np.ones((1, 3), dtype=np.uint16)
    w = co.window_after_accept(stream, 10, 3, 2)
    assert w[:, 0].tolist() == [10, 11, 12]


def test_errors_flag_and_skip_the_whole_op():
    rng = np.random.default_rng(4)
    a, b = _bits(rng, 4, 6, 8), _bits(rng, 4, 10, 8)
    # ops: bad dst; bad src; shift too large for tensor a (rows - keep = 4) though fine for b;
    # src below -1; then one valid copy that must still happen
    dst, src, shift = [4, 1, 2, 3, 0], [0, 7, 1, -2, 3], [0, 0, 5, 0, 1]
    (oa, ob), err = co.conv_update_ref([a, b], [2, 2], dst, src, shift)
    assert err == co.ERR_SLOT | co.ERR_SHIFT
    assert np.array_equal(oa[1:], a[1:]) and np.array_equal(ob[1:], b[1:])
    assert np.array_equal(oa[0, :2], a[3, 1:3]) and np.array_equal(ob[0, :2], b[3, 1:3])
    assert np.array_equal(oa[0, 2:], a[0, 2:])

