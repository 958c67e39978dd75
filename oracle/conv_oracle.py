"""Plain CPU oracle for the conv-state half of the KDA state tuple.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously correct
definition that the library's conv-state call is checked against.  Only
``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import it; the library never does, and this module imports nothing
from the library.  It works on raw bits (unsigned integer arrays), because
the operation moves bits and never converts them.

Sources (cited by page title and section):

* [P1] "State semantics deep water: rollback, fork, replay consistency, TP
  state", sec. 2: the state tuple of a KDA layer has a short-convolution
  window part besides the recurrent matrix.  SGLang clears or copies the
  conv-state pool slots of many tensors (one pointer, stride and feature
  length per tensor) in one launch instead of one launch per tensor; vLLM's
  speculative-decode context treats the conv state as a sliding window that
  is moved with an offset copy, and the recurrent state as a whole block.
* [P3] prhub summary of vLLM PR #51855 (Kimi-K3 RecoverSSM), "Implementation
  breakdown" steps 2 and 4: decode under speculation keeps an extended conv
  window (history plus the speculative positions), and after sampling the
  commit compacts the conv history to the accepted length.

Layout and semantics (the readings adopted here; the pages give the
operations, not a layout):

* A conv tensor holds, per slot, a window of ``rows`` positions by ``dim``
  channels, position-major: element (slot, row, channel).  Its first
  ``keep`` rows are the history carried from step to step (the short
  convolution's width minus one); the rows after them hold the extended
  window's speculative positions.
* One op (dst, src, shift) is applied to every tensor of the call:
    src == -1          every row of slot dst becomes 0 (a fresh request);
    src >= 0           rows [0, keep) of dst become rows [shift, shift + keep)
                       of src, rows >= keep of dst unchanged.  shift = 0 is the
                       fork / copy-on-write copy of the history; src == dst
                       with shift = n is the compaction after n accepted
                       positions (the window slides by n).
  An op whose slots lie outside [0, n_slots) of any tensor, or whose shift
  lies outside [0, rows - keep] of any tensor, is flagged and skipped as a
  whole.
* The ops of one call are independent: distinct dst slots, and no op reads a
  slot that another op writes.  The oracle applies them in order, each
  reading the slots as they were before the call.
"""

from __future__ import annotations

import numpy as np

ERR_SLOT = 1    # a slot index out of range
ERR_SHIFT = 16  # a shift outside [0, rows - keep]


def conv_update_ref(tensors, keep, dst, src, shift):
    """Apply the ops to copies of ``tensors``.

    tensors: list of integer arrays [n_slots, rows, dim] (the raw bits of each
    conv tensor); keep: list of history lengths, one per tensor; dst, src,
    shift: equal-length integer sequences (the ops).  Returns (new tensors,
    error bits)."""
    before = [np.array(t, copy=True) for t in tensors]
    out = [np.array(t, copy=True) for t in tensors]
    err = 0
    for d, s, n in zip(dst, src, shift):
        d, s, n = int(d), int(s), int(n)
        bad_slot = any(not (0 <= d < t.shape[0]) or not (-1 <= s < t.shape[0]) for t in before)
        if bad_slot:
            err |= ERR_SLOT
            continue
        if s >= 0 and any(not (0 <= n <= t.shape[1] - kp) for t, kp in zip(before, keep)):
            err |= ERR_SHIFT
            continue
        for j, t in enumerate(before):
            if s < 0:
                out[j][d] = 0
            else:
                for r in range(keep[j]):
                    out[j][d, r] = t[s, r + n]
    return out, err


def window_after_accept(stream, t, keep, n):
    """History window of a short convolution after the first ``n`` of the
    speculative positions that follow position ``t`` of ``stream`` are
    accepted: the last ``keep`` inputs up to position t + n, oldest first.
    (A direct definition, independent of any slot layout, used to pin the
    compaction op.)"""
    return np.stack([stream[t + n - keep + 1 + i] for i in range(keep)])
