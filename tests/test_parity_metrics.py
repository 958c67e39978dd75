"""The row-level parity metric of the GPU tests (tests/gpu_util.py), on the
CPU: one wrong (token, head) row among thousands passes the per-(sequence,
head) Frobenius bar but fails the row bar; rounding-sized noise passes both;
the floor keeps a row far below its head's size from dominating; max|d| /
max|ref| is reported as defined."""

import numpy as np

import workloads as wl
from oracle import kda_oracle as ko
from tests.gpu_util import ROW_FLOOR, Worst, rel_per_head, row_errors, state_rows


def oracle_outputs(T=8229, H=2, d=16, seed=5):
    toks = wl.token_inputs(T, H, d, d, "f32", seed)
    ex = {n: wl.exact(toks[n]) for n in "qkvgb"}
    o, _, S, _ = ko.run_sequence(ex["q"], ex["k"], ex["v"], ex["g"], ex["b"], np.zeros((H, d, d)))
    return o, S


def test_one_wrong_row_fails_row_bar_only():
    o, _ = oracle_outputs()
    rng = np.random.default_rng(1)
    noisy = o * (1 + 2e-3 * rng.standard_normal(o.shape))
    bad = noisy.copy()
    bad[2500, 1] = 0.0                                 # one (token, head) row lost
    assert rel_per_head(bad, o, 1) < 2e-2              # averaged away per head ...
    assert row_errors(bad, o, 1)["row"] > 0.5          # ... but not per row
    assert row_errors(noisy, o, 1)["row"] < 2e-2
    w = Worst(2e-2)
    w.out("o", bad, o, 1)
    try:
        w.check("planted row")
    except AssertionError:
        pass
    else:
        raise AssertionError("the planted row passed the row bar")


def test_wrong_state_row_fails():
    _, S = oracle_outputs()
    bad = S.copy()
    bad[0, :, 3] *= 1.5                                # one pool row (value column) off by 50 %
    assert state_rows(bad, S)["row"] > 0.4
    assert state_rows(S, S)["row"] == 0.0


def test_floor_and_absmax():
    ref = np.ones((10, 1, 4))
    ref[0, 0] = 1e-6                                   # a row far below the head's typical size
    x = ref.copy()
    x[0, 0] += 1e-4
    r = row_errors(x, ref, 1)
    rms = np.sqrt(np.mean(np.sum(ref[:, 0] ** 2, axis=-1)))
    assert r["row_raw"] > 10                            # unfloored: dominated by the tiny row
    assert np.isclose(r["row"], 2e-4 / (ROW_FLOOR * rms))
    assert np.isclose(r["absmax"], 1e-4)
