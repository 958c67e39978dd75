"""Host-side checks of libkda.so (no GPU needed, no kernel launched).

* the library loads and exports exactly the functions include/kda.h declares;
* status strings;
* every host-checkable error returns its status before any launch: the
  pointers passed here are fake addresses that would fault if touched.
"""

import ctypes
import os
import re
import subprocess

import pytest

import linear_attention_state_kda_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

FAKE = ctypes.c_void_p(0x1000)       # 256-byte aligned, never dereferenced
FAKE_WS = ctypes.c_void_p(0x100000)


def declared():
    text = open(HEADER).read()
    return set(re.findall(r"^(?:kda_status|const char\*)\s+(kda_\w+)\s*\(", text, re.M))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(kda.LIB_PATH):
        from linear_attention_state_kda_amd import build
        build.build()
    return kda.lib()


def test_exports_match_header(L):
    out = subprocess.run(["nm", "-D", "--defined-only", kda.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s+(kda_\w+)$", out, re.M))
    assert declared() == exported, (declared(), exported)
    for name in declared():
        assert getattr(L, name) is not None


def test_status_strings(L):
    names = [L.kda_status_string(i).decode() for i in range(5)]
    assert names == ["KDA_OK", "KDA_ERR_INVALID_ARG", "KDA_ERR_UNSUPPORTED",
                     "KDA_ERR_WORKSPACE", "KDA_ERR_LAUNCH"]


def pool(H=2, dk=128, dv=128, dtype=0, n_slots=8, base=FAKE):
    return kda.KdaPool(base.value if base is not None else None, n_slots, dtype, H, dk, dv)


def prefill(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, in_dtype=2, o=FAKE, cu=FAKE, n_seqs=1,
             T=100, H=2, dk=128, dv=128, C=64, pool=pool(), init=FAKE, final=FAKE, tptr=None,
             tchunk=None, tslot=None, n_track=0, tf32=None, flags=0, err=None, ws=FAKE_WS,
             ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return L.kda_chunk_prefill(a["q"], a["k"], a["v"], a["g"], a["b"], a["in_dtype"], a["o"],
                               a["cu"], a["n_seqs"], a["T"], a["H"], a["dk"], a["dv"], a["C"],
                               a["pool"], a["init"], a["final"], a["tptr"], a["tchunk"], a["tslot"],
                               a["n_track"], a["tf32"], a["flags"], a["err"], a["ws"], a["ws_bytes"],
                               a["stream"])


def test_prefill_host_errors(L):
    assert prefill(L, q=None) == 1
    assert prefill(L, cu=None) == 1
    assert prefill(L, n_seqs=-1) == 1
    assert prefill(L, H=0) == 1
    assert prefill(L, dk=64, dv=64) == 2
    assert prefill(L, C=32) == 2
    assert prefill(L, in_dtype=0) == 2          # fp32 inputs are built for (16, 16, 16) only
    assert prefill(L, in_dtype=7) == 2
    assert prefill(L, pool=pool(dtype=9)) == 2
    assert prefill(L, pool=pool(H=3)) == 1      # pool shape disagrees with the call
    assert prefill(L, pool=pool(base=None)) == 1
    assert prefill(L, n_track=2) == 1           # track arrays missing
    assert prefill(L, ws_bytes=16) == 3
    assert prefill(L, ws=None) == 3
    assert prefill(L, ws=ctypes.c_void_p(0x100010)) == 3   # misaligned workspace
    for name in ("q", "k", "v", "g", "o", "tf32"):   # every vector-accessed buffer must be 16-byte aligned
        assert prefill(L, **{name: ctypes.c_void_p(0x1008)}) == 1, name
    assert prefill(L, T=1 << 33) == 2
    # launch grids beyond the work-item limit (more in test_launch_grid_limits)
    assert prefill(L, T=(1 << 31) - 1, H=129, pool=pool(H=129)) == 2
    assert prefill(L, n_seqs=1 << 20, H=256, pool=pool(H=256)) == 2
    assert prefill(L, flags=2) == 1             # unknown flag bit
    # nothing to do: returns before touching anything
    assert prefill(L, n_seqs=0, q=None, cu=None) == 0


def test_workspace_query(L):
    out = ctypes.c_size_t(0)
    assert L.kda_chunk_prefill_workspace(16, 135168, 32, 128, 128, 64, 2, ctypes.byref(out)) == 0
    rec = 55808                               # bytes per (chunk, head) record at d=128, C=64, bf16
    assert out.value == 256 + (135168 // 64 + 16) * 32 * rec
    assert kda.prefill_workspace_bytes(1, 64, 2, 16, 16, 16, __import__("torch").float32) > 0
    assert L.kda_chunk_prefill_workspace(1, 64, 2, 32, 32, 16, 2, ctypes.byref(out)) == 2
    assert L.kda_chunk_prefill_workspace(1, 64, 2, 128, 128, 64, 2, None) == 1
    assert L.kda_chunk_prefill_workspace(1, (1 << 31) - 1, 129, 128, 128, 64, 2, ctypes.byref(out)) == 2
    assert L.kda_chunk_prefill_workspace(1 << 20, 64, 256, 128, 128, 64, 2, ctypes.byref(out)) == 2


def test_verify_commit_copy_host_errors(L):
    P = pool()
    # verify: q, k, v, g, b, in_dtype, o, n_req, L, H, dk, dv, pool, ckpt, u, kg, flags, err, stream
    v = lambda **kw: L.kda_recurrent_verify(*[kw.get(n, d) for n, d in [
        ("q", FAKE), ("k", FAKE), ("v", FAKE), ("g", FAKE), ("b", FAKE), ("dt", 2), ("o", FAKE),
        ("n", 4), ("L", 8), ("H", 2), ("dk", 128), ("dv", 128), ("pool", P), ("ck", FAKE),
        ("u", FAKE), ("kg", FAKE), ("fl", 0), ("err", None), ("st", None)]])
    assert v(L=0) == 1
    assert v(fl=4) == 1
    assert v(L=257) == 2
    assert v(dk=64, dv=64) == 2
    assert v(o=None) == 1
    assert v(n=-1) == 1
    assert v(pool=pool(H=4)) == 1
    for name in ("q", "k", "v", "g", "o", "u", "kg"):   # every streamed buffer must be 16-byte aligned
        assert v(**{name: ctypes.c_void_p(FAKE.value + 8)}) == 1
    assert v(n=0) == 0
    c = lambda **kw: L.kda_commit(*[kw.get(n, d) for n, d in [
        ("pool", P), ("ck", FAKE), ("dst", None), ("acc", FAKE), ("u", FAKE), ("kg", FAKE),
        ("rdt", 2), ("n", 4), ("L", 8), ("H", 2), ("dk", 128), ("dv", 128), ("err", None),
        ("st", None)]])
    assert c(acc=None) == 1
    assert c(rdt=5) == 2
    assert c(L=300) == 2
    assert c(n=0) == 0
    s = lambda **kw: L.kda_state_copy(kw.get("pool", P), kw.get("src", FAKE), kw.get("dst", FAKE),
                                      kw.get("n", 3), None, None)
    assert s(n=-1) == 1
    assert s(src=None) == 1
    assert s(pool=pool(base=None)) == 1
    assert s(pool=pool(dtype=1, H=1, dk=3, dv=1)) == 2   # 6-byte slots cannot be copied in 16-byte units
    assert s(n=0) == 0


def test_commit_align_host_errors(L):
    P = pool()
    ca = lambda **kw: L.kda_commit_align(*[kw.get(n, d) for n, d in [
        ("pool", P), ("bt", FAKE), ("bpr", 4), ("nt", FAKE), ("acc", FAKE), ("bs", 64), ("u", FAKE),
        ("kg", FAKE), ("rdt", 2), ("n", 4), ("L", 8), ("H", 2), ("dk", 128), ("dv", 128),
        ("nx", kda.KdaAlignNext(None, None, None, None)), ("err", None), ("st", None)]])
    assert ca(bs=8) == 1            # a window of 8 could close two blocks of 8
    assert ca(bs=9, n=0) == 0
    assert ca(bpr=0) == 1
    assert ca(bt=None) == 1
    assert ca(nt=None) == 1
    assert ca(acc=None) == 1
    assert ca(L=300, bs=400) == 2
    assert ca(rdt=7) == 2
    assert ca(dk=64, dv=64) == 2
    assert ca(pool=pool(H=4)) == 1
    assert ca(n=0) == 0


def conv_tensor(base=FAKE, stride=11 * 4096 * 2, n_slots=8, rows=11, keep=3, dim=4096, eb=2):
    return kda.KdaConvTensor(base.value if base is not None else None, stride, n_slots, rows, keep, dim, eb)


def test_conv_state_update_host_errors(L):
    def call(ts, n=3, dst=FAKE, src=FAKE, sh=FAKE, n_t=None):
        arr = (kda.KdaConvTensor * max(1, len(ts)))(*ts)
        return L.kda_conv_state_update(arr, len(ts) if n_t is None else n_t, dst, src, sh, n, None, None)
    good = conv_tensor()
    assert call([good], n=0) == 0                        # nothing to do, nothing launched
    assert call([good, conv_tensor(eb=4, dim=64, stride=11 * 64 * 4)], n=0) == 0
    assert call([good], n=-1) == 1
    assert call([], n=0, n_t=0) == 1
    assert call([good] * 9, n=0) == 1                    # more than KDA_MAX_CONV_TENSORS
    assert call([conv_tensor(base=None)], n=0) == 1
    assert call([conv_tensor(base=ctypes.c_void_p(FAKE.value + 8))], n=0) == 1
    assert call([conv_tensor(keep=0)], n=0) == 1
    assert call([conv_tensor(keep=12)], n=0) == 1
    assert call([conv_tensor(stride=11 * 4096 * 2 - 16)], n=0) == 1   # slots would overlap
    assert call([conv_tensor(stride=11 * 4096 * 2 + 8)], n=0) == 1    # stride not a multiple of 16
    assert call([conv_tensor(eb=8)], n=0) == 2
    assert call([conv_tensor(dim=4100, stride=11 * 4100 * 2 + 8)], n=0) == 2   # row not 16-byte units
    assert call([good], dst=None) == 1
    assert call([good], sh=None) == 1


def test_launch_grid_limits(L):
    """A dispatch holds at most 2^32 - 1 work-items: each call rejects, on the
    host, sizes whose grid would not fit (KDA_ERR_UNSUPPORTED), at the bounds
    include/kda.h states.  A prefill just inside its bounds passes the grid
    check and stops at the workspace check instead (nothing is launched; the
    other calls have no later host check, so only their far side is run)."""
    lim = 0xFFFFFFFF
    # prefill prep: (T / 64 + n_seqs) * H workgroups of 256
    inside = 64 * (lim // 256 // 2 - 1)
    assert (inside // 64 + 1) * 2 * 256 <= lim < (inside // 64 + 2) * 2 * 256
    assert prefill(L, T=inside, ws_bytes=16) == 3
    assert prefill(L, T=inside + 64, ws_bytes=16) == 2
    # prefill scan: n_seqs * H, rounded up to 8, times 2,048
    n_in = (lim // 2048) // 8 * 8 // 2
    assert prefill(L, n_seqs=n_in, ws_bytes=16) == 3
    assert prefill(L, n_seqs=n_in + 1, ws_bytes=16) == 2
    assert L.kda_chunk_prefill_workspace(n_in + 1, 100, 2, 128, 128, 64, 2, ctypes.byref(ctypes.c_size_t())) == 2
    P = pool()
    # verify: 512 work-items per (request, head), rounded up to 8 items
    assert L.kda_recurrent_verify(FAKE, FAKE, FAKE, FAKE, FAKE, 2, FAKE, lim // 512 // 2 + 1, 8, 2, 128,
                                  128, P, FAKE, FAKE, FAKE, 0, None, None) == 2
    # commit and align commit: 256 per (request, head)
    n_c = lim // 256 // 2 + 1
    assert L.kda_commit(P, FAKE, None, FAKE, FAKE, FAKE, 2, n_c, 8, 2, 128, 128, None, None) == 2
    assert L.kda_commit_align(P, FAKE, 4, FAKE, FAKE, 64, FAKE, FAKE, 2, n_c, 8, 2, 128, 128,
                              kda.KdaAlignNext(None, None, None, None), None, None) == 2
    # copy: 256 per 16 KiB of a slot per pair (fp32 slots of 2 x 128 x 128: 8 blocks per pair)
    assert L.kda_state_copy(P, FAKE, FAKE, lim // 256 // 8 + 1, None, None) == 2
    # conv update: 256 per (op, tensor)
    arr = (kda.KdaConvTensor * 2)(conv_tensor(), conv_tensor())
    assert L.kda_conv_state_update(arr, 2, FAKE, FAKE, FAKE, lim // 256 // 2 + 1, None, None) == 2


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(kda, "_lib", None)
    monkeypatch.setattr(kda, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(kda.KdaError):
        kda.lib()


def test_prefill_noalloc_host_errors(L):
    """The allocation-free prefill: the same host checks as kda_chunk_prefill,
    and a call whose workspace would exceed the static scratch is rejected
    before any launch (so no device is touched here)."""
    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, in_dtype=2, o=FAKE, cu=FAKE, n_seqs=1,
                 T=100, H=2, dk=128, dv=128, C=64, pool=pool(), init=FAKE, final=FAKE, tptr=None,
                 tchunk=None, tslot=None, n_track=0, tf32=None, flags=0, err=None, stream=None)
        a.update(kw)
        return L.kda_chunk_prefill_noalloc(*a.values())
    assert call(q=None) == 1
    assert call(C=32) == 2
    assert call(v=ctypes.c_void_p(0x1008)) == 1
    assert call(n_seqs=0, q=None, cu=None) == 0
    out = ctypes.c_size_t(0)
    # 2 x 8229 tokens at 32 heads need about 460 MB of records: more than the 256 MiB scratch
    assert L.kda_chunk_prefill_workspace(2, 2 * 8229, 32, 128, 128, 64, 2, ctypes.byref(out)) == 0
    assert out.value > kda.NOALLOC_SCRATCH_BYTES
    assert call(n_seqs=2, T=2 * 8229, H=32, pool=pool(H=32)) == 3
    # the single-layer workload fits
    assert L.kda_chunk_prefill_workspace(1, 8229, 32, 128, 128, 64, 2, ctypes.byref(out)) == 0
    assert out.value <= kda.NOALLOC_SCRATCH_BYTES
