"""The Python binding's argument checks, on the CPU.  The C ABI sees raw
pointers only, so every buffer's shape (and device) is checked in the
binding before any call: each mis-shaped argument below must raise
ValueError naming it, and a call whose shapes are all right gets as far as
the device check (the tensors here are host tensors, so no library call is
ever made)."""

import pytest
import torch

import linear_attention_state_kda_amd as kda

T, H, DK, DV, N = 100, 2, 128, 128, 3


def prefill_args():
    f = lambda *s: torch.zeros(s, dtype=torch.bfloat16)
    i = lambda *s: torch.zeros(s, dtype=torch.int32)
    return dict(q=f(T, H, DK), k=f(T, H, DK), v=f(T, H, DV), g=f(T, H, DK), b=f(T, H),
                cu_seqlens=i(N + 1), chunk=64, pool=torch.zeros((8, H, DV, DK)), init_slot=i(N),
                final_slot=i(N), track_ptr=i(N + 1), track_chunk=i(2), track_slot=i(2),
                track_f32=torch.zeros((2, H, DV, DK)), o=f(T, H, DV), dev_err=i(1))


def verify_args(n_req=4, L=8):
    f = lambda *s: torch.zeros(s, dtype=torch.bfloat16)
    return dict(q=f(n_req, L, H, DK), k=f(n_req, L, H, DK), v=f(n_req, L, H, DV), g=f(n_req, L, H, DK),
                b=f(n_req, L, H), pool=torch.zeros((8, H, DV, DK)),
                ckpt_slot=torch.zeros(n_req, dtype=torch.int32), o=f(n_req, L, H, DV),
                u_rec=torch.zeros((n_req, H, L, DV)), kg_rec=f(n_req, H, L, 2 * DK),
                dev_err=torch.zeros(1, dtype=torch.int32))


PREFILL_BAD = [("k", (T, H, DK - 1)), ("g", (T - 1, H, DK)), ("v", (T, H + 1, DV)), ("b", (T,)),
               ("o", (T - 1, H, DV)), ("init_slot", (N - 1,)), ("final_slot", (N + 1,)),
               ("track_ptr", (N,)), ("track_slot", (1,)), ("track_f32", (1, H, DV, DK)),
               ("track_f32", (2, H, DK, DV + 1)), ("pool", (8, H + 1, DV, DK)), ("dev_err", (0,))]


@pytest.mark.parametrize("name,shape", PREFILL_BAD)
def test_prefill_rejects_mis_shaped(name, shape):
    a = prefill_args()
    a[name] = torch.zeros(shape, dtype=a[name].dtype)
    with pytest.raises(ValueError, match=name.split("_")[0]):
        kda.chunk_prefill(**a)


def test_prefill_shapes_ok_reaches_device_check():
    with pytest.raises(ValueError, match="device tensor"):
        kda.chunk_prefill(**prefill_args())


VERIFY_BAD = [("k", (4, 8, H, DK - 8)), ("v", (4, 7, H, DV)), ("g", (4, 8, H, DK + 1)), ("b", (4, 8)),
              ("o", (4, 8, H, DV - 1)), ("u_rec", (4, 8, H, DV)), ("kg_rec", (4, H, 8, DK)),
              ("ckpt_slot", (3,)), ("pool", (8, H, DV, DK // 2))]


@pytest.mark.parametrize("name,shape", VERIFY_BAD)
def test_verify_rejects_mis_shaped(name, shape):
    a = verify_args()
    a[name] = torch.zeros(shape, dtype=a[name].dtype)
    with pytest.raises(ValueError, match=name.split("_")[0]):
        kda.recurrent_verify(**a)


def test_verify_shapes_ok_reaches_device_check():
    with pytest.raises(ValueError, match="device tensor"):
        kda.recurrent_verify(**verify_args())


def commit_args(n_req=4, L=8):
    i = lambda *s: torch.zeros(s, dtype=torch.int32)
    return dict(pool=torch.zeros((8, H, DV, DK)), ckpt_slot=i(n_req), accepted_len=i(n_req),
                u_rec=torch.zeros((n_req, H, L, DV)), kg_rec=torch.zeros((n_req, H, L, 2 * DK), dtype=torch.bfloat16),
                dst_slot=i(n_req), dev_err=i(1))


@pytest.mark.parametrize("name,shape", [("ckpt_slot", (3,)), ("accepted_len", (5,)), ("dst_slot", (2,)),
                                        ("kg_rec", (4, H, 7, 2 * DK)), ("kg_rec", (4, H, 8, 2 * DK - 1)),
                                        ("pool", (8, H, DV + 1, DK)), ("u_rec", (4, H, 8))])
def test_commit_rejects_mis_shaped(name, shape):
    a = commit_args()
    a[name] = torch.zeros(shape, dtype=a[name].dtype)
    with pytest.raises(ValueError):
        kda.commit(**a)


def test_commit_align_rejects_mis_shaped():
    a = commit_args()
    base = dict(pool=a["pool"], block_table=torch.zeros((4, 3), dtype=torch.int32),
                num_tokens=torch.zeros(4, dtype=torch.int32), accepted_len=torch.zeros(4, dtype=torch.int32),
                block_size=16, u_rec=a["u_rec"], kg_rec=a["kg_rec"])
    for name, shape in (("block_table", (3, 3)), ("block_table", (12,)), ("num_tokens", (3,)),
                        ("accepted_len", (5,))):
        bad = dict(base)
        bad[name] = torch.zeros(shape, dtype=torch.int32)
        with pytest.raises(ValueError, match=name.split("_")[0]):
            kda.commit_align(**bad)
    with pytest.raises(ValueError, match="device tensor"):
        kda.commit_align(**base)


def test_copy_rejects_mismatched_lengths():
    pool = torch.zeros((8, H, DV, DK))
    with pytest.raises(ValueError, match="one length"):
        kda.state_copy(pool, torch.zeros(3, dtype=torch.int32), torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError, match="device tensor"):
        kda.state_copy(pool, torch.zeros(3, dtype=torch.int32), torch.zeros(3, dtype=torch.int32))
