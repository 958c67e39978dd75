"""Replay-consistency harness (replay.py) on a small case, with both paths
pinned to the fp64 oracle on sampled heads.

The harness compares the chunked prefill's outputs with the recurrent verify
kernel's outputs when it resumes from the prefill's own snapshots (the
measurement the state-semantics page lists as still to be done, sec. 4).
Both paths are first held to the oracle (2e-2 relative per (checkpoint,
head), the bf16-input bar); their mutual difference per (checkpoint, head)
is then at most the sum of the two, 4e-2, and the statistics the harness
reports must be consistent with the raw differences.
"""

import numpy as np
import pytest
import torch

import replay
import workloads as wl
from oracle import kda_oracle as ko
from tests.gpu_util import DEV, Worst

pytestmark = pytest.mark.gpu

HEADS = [0, 3]


@pytest.mark.parametrize("pool_dtype", ["f32", "bf16"])
def test_replay_harness_small(pool_dtype):
    T, H, C, L, every = 2048, 4, 64, 256, 4
    s = replay.run(T=T, H=H, C=C, pool_dtype=pool_dtype, every=every, L=L, seed=13, dev=DEV, keep=True)
    t = s.pop("_tensors")
    ckpts, slot_of = t["ckpts"], t["slot_of"]
    assert s["checkpoints"] == len(ckpts) == (T - L) // (every * C)

    # the prefill's outputs against the oracle on sampled heads
    toks = t["toks"]
    ex = {n: wl.exact(toks[n][:, HEADS]) for n in "qkvgb"}
    o_ref, _, _, _ = ko.run_sequence(ex["q"], ex["k"], ex["v"], ex["g"], ex["b"], np.zeros((len(HEADS), 128, 128)))
    hsel = torch.as_tensor(HEADS, device=DEV)
    o_pre = wl.exact(t["o_pre"][:, hsel].cpu())
    w = Worst(2e-2)
    w.out("prefill_o", o_pre, o_ref, 1)

    # the resumed outputs against the oracle run from the stored snapshot
    o_ver = wl.exact(t["o_ver"][:, :, hsel].cpu())                          # [n_ck, L, 2, d]
    wv = Worst(2e-2)
    for i, c in enumerate(ckpts):
        s0 = np.swapaxes(wl.exact(t["pool"][slot_of[c]][hsel].cpu()), -1, -2)   # [2, d_k, d_v]
        win = slice(c * C, c * C + L)
        ov_ref, _, _, _ = ko.verify_ref(*(ex[n][win][None] for n in "qkvgb"), s0[None])
        wv.out("verify_o", o_ver[i], ov_ref[0], 1)
    w.check(f"replay harness pool={pool_dtype} prefill")
    wv.check(f"replay harness pool={pool_dtype} resumed verify")

    # mutual difference and the harness's statistics
    diff = t["diff"]
    assert diff.shape == (len(ckpts), L, H)
    assert s["rel_diff"]["max"] == pytest.approx(diff.max().item())
    for i, c in enumerate(ckpts):
        a = t["o_ver"][i].float()
        b = t["o_pre"][c * C:c * C + L].float()
        per_head = (a - b).norm(dim=(0, 2)) / b.norm(dim=(0, 2))
        assert per_head.max().item() < 4e-2
    for tau, f in s["first_over_tolerance"].items():
        over = (diff > float(tau)).cpu().numpy()
        first = np.where(over.any(axis=1), over.argmax(axis=1), L)
        assert f["never_fraction"] == pytest.approx(float((first >= L).mean()))
    # commit of all L positions lands on the prefill's later snapshot
    assert s["commit_vs_snapshot_rel"]["max"] < 2e-2
