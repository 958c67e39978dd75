"""Thin Python binding of libkda.so, the MI355X KDA state-recurrence library.

Argument marshalling only: every step of the recurrence runs in the HIP
kernels behind the C ABI declared in ``include/kda.h``.  PyTorch provides
device memory and the current stream.  The functions carry the C names
without the ``kda_`` prefix and raise ``KdaError`` on a non-zero status.
There is no fallback: if the library is not built, loading it raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "KdaError", "lib", "DTYPE_CODES", "DEV_ERR_SLOT", "DEV_ERR_TRACK", "DEV_ERR_ACCEPT",
    "DEV_ERR_SEQLEN", "DEV_ERR_SHIFT", "DEV_ERR_GATE", "QK_L2NORM", "prefill_workspace_bytes", "chunk_prefill", "recurrent_verify",
    "commit", "commit_align", "state_copy", "conv_state_update", "chunk_prefill_noalloc",
    "NOALLOC_SCRATCH_BYTES", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

DTYPE_CODES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
STATUS = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARG", 2: "KDA_ERR_UNSUPPORTED",
          3: "KDA_ERR_WORKSPACE", 4: "KDA_ERR_LAUNCH"}
DEV_ERR_SLOT, DEV_ERR_TRACK, DEV_ERR_ACCEPT, DEV_ERR_SEQLEN, DEV_ERR_SHIFT, DEV_ERR_GATE = 1, 2, 4, 8, 16, 32
QK_L2NORM = 1   # flags bit of kda_chunk_prefill / kda_recurrent_verify
NOALLOC_SCRATCH_BYTES = 256 << 20   # KDA_NOALLOC_SCRATCH_BYTES


class KdaError(RuntimeError):
    def __init__(self, status, where):
        self.status = int(status)
        super().__init__(f"{where}: {STATUS.get(self.status, self.status)}")


class KdaPool(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("n_slots", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("H", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32)]


class KdaAlignNext(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_void_p), ("block", ctypes.c_void_p), ("ckpt_slot", ctypes.c_void_p),
                ("copy_bias", ctypes.c_void_p)]


class KdaConvTensor(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("slot_stride", ctypes.c_int64), ("n_slots", ctypes.c_int64),
                ("rows", ctypes.c_int32), ("keep", ctypes.c_int32), ("dim", ctypes.c_int32),
                ("elem_bytes", ctypes.c_int32)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_U32 = ctypes.c_uint32
_SZ = ctypes.c_size_t

_SIGS = {
    "kda_chunk_prefill_workspace": [_I32, _I64, _I32, _I32, _I32, _I32, _I32, ctypes.POINTER(_SZ)],
    "kda_chunk_prefill": [_P, _P, _P, _P, _P, _I32, _P, _P, _I32, _I64, _I32, _I32, _I32, _I32,
                          KdaPool, _P, _P, _P, _P, _P, _I32, _P, _U32, _P, _P, _SZ, _P],
    "kda_chunk_prefill_noalloc": [_P, _P, _P, _P, _P, _I32, _P, _P, _I32, _I64, _I32, _I32, _I32, _I32,
                                  KdaPool, _P, _P, _P, _P, _P, _I32, _P, _U32, _P, _P],
    "kda_recurrent_verify": [_P, _P, _P, _P, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32, KdaPool,
                             _P, _P, _P, _U32, _P, _P],
    "kda_commit": [KdaPool, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P],
    "kda_commit_align": [KdaPool, _P, _I32, _P, _P, _I32, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                         KdaAlignNext, _P, _P],
    "kda_state_copy": [KdaPool, _P, _P, _I32, _P, _P],
    "kda_conv_state_update": [ctypes.POINTER(KdaConvTensor), _I32, _P, _P, _P, _I32, _P, _P],
    "kda_status_string": [_I32],
}

_lib = None


def lib():
    """Load libkda.so (built in-tree by ``linear_attention_state_kda_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise KdaError(-1, f"libkda.so not built at {LIB_PATH}; run linear_attention_state_kda_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_char_p if name == "kda_status_string" else ctypes.c_int
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else t.data_ptr()   # ctypes passes the int as a c_void_p argument


def _shape(t, name, shape):
    """Raise ValueError unless tensor ``t`` (if given) has exactly ``shape``.
    The C ABI sees raw pointers only, so every buffer size is checked here,
    before any call: an undersized output would be written out of bounds."""
    if t is not None and t.shape != shape:   # torch.Size compares as a tuple
        raise ValueError(f"{name} must have shape {tuple(int(x) for x in shape)}, got {tuple(t.shape)}")


def _same_device(ref, tensors):
    want = ref.get_device()
    for name, t in tensors:
        if t is not None and t.get_device() != want:
            raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


def _dev(t, name, dtype=None, ndim=None):
    if t is None:
        return
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _pool(pool):
    _dev(pool, "pool", ndim=4)
    if pool.dtype not in DTYPE_CODES:
        raise ValueError("pool dtype must be float32, float16 or bfloat16")
    n, H, dv, dk = pool.shape
    return KdaPool(pool.data_ptr(), n, DTYPE_CODES[pool.dtype], H, dk, dv)


def _check(status, where):
    if status != 0:
        raise KdaError(status, where)


def prefill_workspace_bytes(n_seqs, total_tokens, H, d_k, d_v, chunk, in_dtype):
    out = _SZ(0)
    _check(lib().kda_chunk_prefill_workspace(n_seqs, total_tokens, H, d_k, d_v, chunk,
                                             DTYPE_CODES[in_dtype], ctypes.byref(out)),
           "kda_chunk_prefill_workspace")
    return int(out.value)


def _prefill_marshal(q, k, v, g, b, cu_seqlens, chunk, pool, init_slot, final_slot, track_ptr, track_chunk,
                     track_slot, track_f32, o, dev_err, workspace, qk_l2norm):
    """Checks of a prefill call; returns (o, the C arguments before the
    workspace).  ``workspace`` False means the call takes none."""
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q and v must be [T, H, d]")
    T, H, dk = q.shape
    dv = v.shape[2]
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-d tensor [n_seqs + 1]")
    n_seqs = cu_seqlens.numel() - 1
    if (track_chunk is None) != (track_slot is None) or (track_chunk is not None and track_ptr is None):
        raise ValueError("track_ptr, track_chunk and track_slot go together")
    n_track = 0 if track_chunk is None else track_chunk.numel()
    _shape(k, "k", (T, H, dk))
    _shape(g, "g", (T, H, dk))
    _shape(v, "v", (T, H, dv))
    _shape(b, "b", (T, H))
    _shape(o, "o", (T, H, dv))
    _shape(init_slot, "init_slot", (n_seqs,))
    _shape(final_slot, "final_slot", (n_seqs,))
    _shape(track_ptr, "track_ptr", (n_seqs + 1,))
    _shape(track_chunk, "track_chunk", (n_track,))
    _shape(track_slot, "track_slot", (n_track,))
    if track_f32 is not None and (track_f32.dim() != 4 or tuple(track_f32.shape[1:]) != (H, dv, dk)
                                  or track_f32.shape[0] < n_track):
        raise ValueError(f"track_f32 must be [>= {n_track}, {H}, {dv}, {dk}], got {tuple(track_f32.shape)}")
    if dev_err is not None and dev_err.numel() < 1:
        raise ValueError("dev_err needs one element")
    _shape(pool, "pool", (pool.shape[0], H, dv, dk))
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("b", b)):
        _dev(t, name, dtype=q.dtype)
    for name, t in (("cu_seqlens", cu_seqlens), ("init_slot", init_slot), ("final_slot", final_slot),
                    ("track_ptr", track_ptr), ("track_chunk", track_chunk), ("track_slot", track_slot),
                    ("dev_err", dev_err)):
        _dev(t, name, dtype=torch.int32)
    _dev(track_f32, "track_f32", dtype=torch.float32)
    _same_device(q, (("k", k), ("v", v), ("g", g), ("b", b), ("o", o), ("pool", pool),
                     ("cu_seqlens", cu_seqlens), ("init_slot", init_slot), ("final_slot", final_slot),
                     ("track_ptr", track_ptr), ("track_chunk", track_chunk), ("track_slot", track_slot),
                     ("track_f32", track_f32), ("dev_err", dev_err),
                     ("workspace", workspace if workspace is not False else None)))
    if o is None:
        o = torch.empty((T, H, dv), dtype=q.dtype, device=q.device)
    _dev(o, "o", dtype=q.dtype)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), DTYPE_CODES[q.dtype], _ptr(o),
            _ptr(cu_seqlens), n_seqs, T, H, dk, dv, chunk, _pool(pool), _ptr(init_slot),
            _ptr(final_slot), _ptr(track_ptr), _ptr(track_chunk), _ptr(track_slot), n_track,
            _ptr(track_f32), QK_L2NORM if qk_l2norm else 0, _ptr(dev_err))
    return o, args


def chunk_prefill(q, k, v, g, b, cu_seqlens, chunk, pool, init_slot, final_slot,
                  track_ptr=None, track_chunk=None, track_slot=None, track_f32=None,
                  o=None, dev_err=None, workspace=None, qk_l2norm=False):
    """kda_chunk_prefill on packed token tensors q, k, g [T, H, d_k], v [T, H, d_v],
    b [T, H]; returns o [T, H, d_v] (allocated when not given).  qk_l2norm sets
    KDA_QK_L2NORM (q and k normalised inside the kernel)."""
    o, args = _prefill_marshal(q, k, v, g, b, cu_seqlens, chunk, pool, init_slot, final_slot, track_ptr,
                               track_chunk, track_slot, track_f32, o, dev_err, workspace, qk_l2norm)
    T, H, dk = q.shape
    need = prefill_workspace_bytes(cu_seqlens.numel() - 1, T, H, dk, v.shape[2], chunk, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace", dtype=torch.uint8)
    st = lib().kda_chunk_prefill(*args, _ptr(workspace), workspace.numel(), _stream())
    _check(st, "kda_chunk_prefill")
    return o


def chunk_prefill_noalloc(q, k, v, g, b, cu_seqlens, chunk, pool, init_slot, final_slot,
                          track_ptr=None, track_chunk=None, track_slot=None, track_f32=None,
                          o=None, dev_err=None, qk_l2norm=False):
    """kda_chunk_prefill_noalloc: chunk_prefill without a workspace (the
    library's static scratch of NOALLOC_SCRATCH_BYTES per GPU holds the chunk
    records).  With ``o`` given, nothing is allocated."""
    o, args = _prefill_marshal(q, k, v, g, b, cu_seqlens, chunk, pool, init_slot, final_slot, track_ptr,
                               track_chunk, track_slot, track_f32, o, dev_err, False, qk_l2norm)
    st = lib().kda_chunk_prefill_noalloc(*args, _stream())
    _check(st, "kda_chunk_prefill_noalloc")
    return o


def recurrent_verify(q, k, v, g, b, pool, ckpt_slot, o=None, u_rec=None, kg_rec=None, dev_err=None,
                     qk_l2norm=False):
    """kda_recurrent_verify on q, k, g [n_req, L, H, d_k], v [n_req, L, H, d_v],
    b [n_req, L, H]; returns (o, u_rec, kg_rec).  qk_l2norm as in chunk_prefill."""
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q and v must be [n_req, L, H, d]")
    n_req, L, H, dk = q.shape
    dv = v.shape[3]
    _shape(k, "k", (n_req, L, H, dk))
    _shape(g, "g", (n_req, L, H, dk))
    _shape(v, "v", (n_req, L, H, dv))
    _shape(b, "b", (n_req, L, H))
    _shape(o, "o", (n_req, L, H, dv))
    _shape(u_rec, "u_rec", (n_req, H, L, dv))
    _shape(kg_rec, "kg_rec", (n_req, H, L, 2 * dk))
    _shape(ckpt_slot, "ckpt_slot", (n_req,))
    _shape(pool, "pool", (pool.shape[0], H, dv, dk))
    if dev_err is not None and dev_err.numel() < 1:
        raise ValueError("dev_err needs one element")
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("b", b)):
        _dev(t, name, dtype=q.dtype)
    _dev(ckpt_slot, "ckpt_slot", dtype=torch.int32)
    _dev(dev_err, "dev_err", dtype=torch.int32)
    _same_device(q, (("k", k), ("v", v), ("g", g), ("b", b), ("o", o), ("pool", pool),
                     ("ckpt_slot", ckpt_slot), ("u_rec", u_rec), ("kg_rec", kg_rec), ("dev_err", dev_err)))
    if o is None:
        o = torch.empty((n_req, L, H, dv), dtype=q.dtype, device=q.device)
    if u_rec is None:
        u_rec = torch.empty((n_req, H, L, dv), dtype=torch.float32, device=q.device)
    if kg_rec is None:
        kg_rec = torch.empty((n_req, H, L, 2 * dk), dtype=q.dtype, device=q.device)
    _dev(o, "o", dtype=q.dtype)
    _dev(u_rec, "u_rec", dtype=torch.float32)
    _dev(kg_rec, "kg_rec", dtype=q.dtype)
    st = lib().kda_recurrent_verify(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), DTYPE_CODES[q.dtype], _ptr(o), n_req, L, H,
        dk, dv, _pool(pool), _ptr(ckpt_slot), _ptr(u_rec), _ptr(kg_rec), QK_L2NORM if qk_l2norm else 0,
        _ptr(dev_err), _stream())
    _check(st, "kda_recurrent_verify")
    return o, u_rec, kg_rec


def _records(u_rec, kg_rec, pool):
    """Sizes (n_req, H, L, d_k, d_v) of a verify call's records, checked
    against each other and the pool."""
    if u_rec.dim() != 4 or kg_rec.dim() != 4:
        raise ValueError("u_rec and kg_rec must be 4-d [n_req, H, L, .]")
    n_req, H, L, dv = u_rec.shape
    if kg_rec.shape[3] % 2:
        raise ValueError("kg_rec's last axis holds key then gate: 2 * d_k")
    dk = kg_rec.shape[3] // 2
    _shape(kg_rec, "kg_rec", (n_req, H, L, 2 * dk))
    _shape(pool, "pool", (pool.shape[0], H, dv, dk))
    return n_req, H, L, dk, dv


def commit(pool, ckpt_slot, accepted_len, u_rec, kg_rec, dst_slot=None, dev_err=None):
    """kda_commit: rebuild each request's state at its accepted length."""
    n_req, H, L, dk, dv = _records(u_rec, kg_rec, pool)
    _shape(ckpt_slot, "ckpt_slot", (n_req,))
    _shape(accepted_len, "accepted_len", (n_req,))
    _shape(dst_slot, "dst_slot", (n_req,))
    if dev_err is not None and dev_err.numel() < 1:
        raise ValueError("dev_err needs one element")
    for name, t in (("ckpt_slot", ckpt_slot), ("accepted_len", accepted_len), ("dst_slot", dst_slot),
                    ("dev_err", dev_err)):
        _dev(t, name, dtype=torch.int32)
    _dev(u_rec, "u_rec", dtype=torch.float32)
    _dev(kg_rec, "kg_rec")
    _same_device(pool, (("ckpt_slot", ckpt_slot), ("accepted_len", accepted_len), ("dst_slot", dst_slot),
                        ("u_rec", u_rec), ("kg_rec", kg_rec), ("dev_err", dev_err)))
    st = lib().kda_commit(_pool(pool), _ptr(ckpt_slot), _ptr(dst_slot), _ptr(accepted_len),
                          _ptr(u_rec), _ptr(kg_rec), DTYPE_CODES[kg_rec.dtype], n_req, L, H, dk,
                          dv, _ptr(dev_err), _stream())
    _check(st, "kda_commit")


def commit_align(pool, block_table, num_tokens, accepted_len, block_size, u_rec, kg_rec, dev_err=None,
                 next_tokens=None, next_block=None, next_ckpt=None, copy_bias=None):
    """kda_commit_align: block-aligned commit; block_table is [n_req, blocks_per_req] int32.
    The optional int32 [n_req] outputs receive the next step's values (tokens
    held, running block, its slot as the next checkpoint, a neutral copy
    bias), written by the same launch."""
    n_req, H, L, dk, dv = _records(u_rec, kg_rec, pool)
    if block_table.dim() != 2 or block_table.shape[0] != n_req:
        raise ValueError(f"block_table must be [{n_req}, blocks_per_req], got {tuple(block_table.shape)}")
    _shape(num_tokens, "num_tokens", (n_req,))
    _shape(accepted_len, "accepted_len", (n_req,))
    outs = (("next_tokens", next_tokens), ("next_block", next_block), ("next_ckpt", next_ckpt),
            ("copy_bias", copy_bias))
    for name, t in outs:
        _shape(t, name, (n_req,))
    if dev_err is not None and dev_err.numel() < 1:
        raise ValueError("dev_err needs one element")
    _dev(block_table, "block_table", dtype=torch.int32, ndim=2)
    for name, t in (("num_tokens", num_tokens), ("accepted_len", accepted_len), ("dev_err", dev_err)) + outs:
        _dev(t, name, dtype=torch.int32)
    _dev(u_rec, "u_rec", dtype=torch.float32)
    _dev(kg_rec, "kg_rec")
    _same_device(pool, (("block_table", block_table), ("num_tokens", num_tokens),
                        ("accepted_len", accepted_len), ("u_rec", u_rec), ("kg_rec", kg_rec),
                        ("dev_err", dev_err)) + outs)
    for name, t in outs:   # the next-step arrays are written while the inputs are read
        if t is not None and any(t.data_ptr() == x.data_ptr() for x in (num_tokens, accepted_len, block_table)):
            raise ValueError(f"{name} must not alias an input")
    nxt = KdaAlignNext(*(None if t is None else t.data_ptr() for _, t in outs))
    st = lib().kda_commit_align(_pool(pool), _ptr(block_table), block_table.shape[1], _ptr(num_tokens),
                                _ptr(accepted_len), int(block_size), _ptr(u_rec), _ptr(kg_rec),
                                DTYPE_CODES[kg_rec.dtype], n_req, L, H, dk, dv, nxt, _ptr(dev_err), _stream())
    _check(st, "kda_commit_align")


def state_copy(pool, src_slot, dst_slot, dev_err=None):
    """kda_state_copy: pool[dst_slot[i]] <- pool[src_slot[i]] bitwise."""
    if src_slot.dim() != 1 or dst_slot.dim() != 1 or src_slot.numel() != dst_slot.numel():
        raise ValueError("src_slot and dst_slot must be 1-d tensors of one length")
    if dev_err is not None and dev_err.numel() < 1:
        raise ValueError("dev_err needs one element")
    _dev(src_slot, "src_slot", dtype=torch.int32)
    _dev(dst_slot, "dst_slot", dtype=torch.int32)
    _dev(dev_err, "dev_err", dtype=torch.int32)
    _same_device(pool, (("src_slot", src_slot), ("dst_slot", dst_slot), ("dev_err", dev_err)))
    st = lib().kda_state_copy(_pool(pool), _ptr(src_slot), _ptr(dst_slot), src_slot.numel(),
                              _ptr(dev_err), _stream())
    _check(st, "kda_state_copy")


def conv_state_update(tensors, keep, dst_slot, src_slot, shift, dev_err=None):
    """kda_conv_state_update on conv tensors, each [n_slots, rows, dim] with
    rows and channels contiguous (the slot stride may be larger); ``keep``
    gives each tensor's history rows.  Op i: src_slot[i] == -1 clears slot
    dst_slot[i]; otherwise rows [0, keep) of dst_slot[i] <- rows
    [shift[i], shift[i] + keep) of src_slot[i]."""
    if len(tensors) != len(keep):
        raise ValueError("one keep value per tensor")
    descs = (KdaConvTensor * max(1, len(tensors)))()
    for i, (t, kp) in enumerate(zip(tensors, keep)):
        if not t.is_cuda or t.dim() != 3:
            raise ValueError("conv tensors must be 3-d device tensors [n_slots, rows, dim]")
        n_slots, rows, dim = t.shape
        if t.stride(2) != 1 or t.stride(1) != dim:
            raise ValueError("rows and channels of a conv tensor must be contiguous")
        descs[i] = KdaConvTensor(t.data_ptr(), t.stride(0) * t.element_size(), n_slots, rows, int(kp), dim,
                                 t.element_size())
    n = dst_slot.numel()
    if src_slot.numel() != n or shift.numel() != n:
        raise ValueError("dst_slot, src_slot and shift differ in length")
    if dev_err is not None and dev_err.numel() < 1:
        raise ValueError("dev_err needs one element")
    for name, x in (("dst_slot", dst_slot), ("src_slot", src_slot), ("shift", shift), ("dev_err", dev_err)):
        _dev(x, name, dtype=torch.int32)
    if tensors:
        _same_device(tensors[0], [(f"tensors[{i}]", t) for i, t in enumerate(tensors[1:], 1)] +
                     [("dst_slot", dst_slot), ("src_slot", src_slot), ("shift", shift), ("dev_err", dev_err)])
    st = lib().kda_conv_state_update(descs, len(tensors), _ptr(dst_slot), _ptr(src_slot), _ptr(shift), n,
                                     _ptr(dev_err), _stream())
    _check(st, "kda_conv_state_update")
