"""Host checks of the seeded synthetic input generators (no GPU)."""

import numpy as np
import torch

import workloads as wl


def test_token_inputs_are_seeded_and_follow_the_recipe():
    a = wl.token_inputs(50, 3, 16, 8, "bf16", seed=5)
    b = wl.token_inputs(50, 3, 16, 8, "bf16", seed=5)
    c = wl.token_inputs(50, 3, 16, 8, "bf16", seed=6)
    for n in a:
        assert torch.equal(a[n], b[n])
        assert a[n].dtype == torch.bfloat16
    assert not torch.equal(a["q"], c["q"])
    q = wl.exact(a["q"])
    assert np.allclose(np.linalg.norm(q, axis=-1), 1.0, atol=1e-2)
    g = wl.exact(a["g"])
    assert g.max() <= -0.0009 and g.min() >= -0.1005
    assert a["v"].shape == (50, 3, 8) and a["b"].shape == (50, 3)


def test_heads_are_independent_streams():
    # regenerating with fewer heads reproduces the first heads exactly
    a = wl.token_inputs(20, 4, 8, 8, "f32", seed=1)
    b = wl.token_inputs(20, 2, 8, 8, "f32", seed=1)
    for n in a:
        assert torch.equal(a[n][:, :2], b[n])


def test_spec_layout_and_slots():
    case = wl.spec_case(n_req=16, L=4, H=2, d=16, n_slots=64, n_fork_src=4, fanout=3, seed=2)
    assert len(set(case["ckpt_slots"].tolist())) == 16
    assert len(set(case["fork_dst"].tolist())) == 12
    assert not set(case["fork_dst"].tolist()) & set(case["ckpt_slots"].tolist())
    assert set(case["fork_src"].tolist()) <= set(case["ckpt_slots"].tolist())
    assert case["accepted"].min() >= 0 and case["accepted"].max() <= 4
    toks = wl.token_inputs(16 * 4, 2, 16, 16, "bf16", 2, shape_prefix=(16, 4))
    assert toks["q"].shape == (16, 4, 2, 16) and toks["b"].shape == (16, 4, 2)


def test_varlen_case_is_valid():
    case = wl.varlen_prefill(seed=2)
    assert len(case["lengths"]) == 16
    assert all(512 <= L <= 16384 for L in case["lengths"])
    slots = case["init_slots"] + case["final_slots"] + [t[2] for t in case["tracks"]]
    assert len(set(slots)) == len(slots)
    for s, c, _ in case["tracks"]:
        assert 1 <= c <= case["lengths"][s] // 64


def test_rounding_is_single_rne():
    x = np.array([1.0 + 2.0 ** -8])
    assert wl.to_dtype(x, "f16").view(torch.int16).item() == 0x3C04
    assert wl.to_dtype(x, "bf16").view(torch.int16).item() == 0x3F80
