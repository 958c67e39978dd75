"""Plain fp64 CPU oracle for the Kimi Delta Attention (KDA) state recurrence.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously correct
definition that the HIP library is checked against.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the library itself never does, and this module imports nothing
from the library.  It shares no code with the GPU path: inputs arrive as
float64 NumPy arrays holding exactly the values the GPU receives.

Sources (cited by page title and section; the pages hold no code and no
equations, only structure):

* [P1] "State semantics deep water: rollback, fork, replay consistency, TP
  state" (forceinjection.github.io, linear-attention series, part 3).
  Sec. 1: the state is a fixed-size per-head d_k x d_v matrix that is either
  wholly present or absent.  Sec. 2: rollback of rejected speculation is an
  exact block copy of the state saved at the verify point.  Sec. 3: a
  continued candidate updates its state in place, S_t = f(S_{t-1}); a fork
  is a whole-state copy (128 x 128 per head).  Sec. 4: the beta gate goes
  through a sigmoid.
* [P2] prhub summary of SGLang PR #34820 (fp32 "track" snapshot for the
  prefix cache).  "Implementation breakdown" item 2 and the kda_prefill.py
  excerpt: at the requested chunk index the fp32 accumulator itself is the
  snapshot, taken at the point of the 64-token tile loop where the per-chunk
  state row is written; the hybrid_linear_attn_backend.py excerpt: one
  indexed cast from the fp32 buffer into the pool dtype.
* [P3] prhub summary of vLLM PR #51855 (Kimi-K3 RecoverSSM).
  "Implementation breakdown" steps 1, 3 and 4: verify reads one checkpoint,
  steps the speculative positions, and records the fp32 correction u plus
  the key and raw gate per position; commit rebuilds the state at the
  accepted length in one reverse-order, non-recursive pass.

The recurrence (the gated delta rule with a per-key-channel decay, which is
what a u/key/gate record set is sufficient to rebuild -- [P3] step 3 names u
as the state-dependent correction, so beta and v are folded into u):

    alpha_t = exp(g_t)              g_t = log alpha_t, one value per key channel
    beta_t  = sigmoid(b_t)          b_t = beta logit, one value per head
    S_dec   = Diag(alpha_t) S_{t-1}
    u_t     = beta_t (v_t - S_dec^T k_t)
    S_t     = S_dec + k_t u_t^T
    o_t     = S_t^T q_t

S has shape (d_k, d_v) per head ("math orientation", key index first).  The
GPU pool stores the transpose, [d_v][d_k] per head; converting between the
two is the caller's job and is not part of the method.

Readings where the pages are silent:
  * the gate input is g = log alpha and alpha = exp(g) with no further
    activation; the beta input is a logit and every call applies the same
    sigmoid;
  * no query scale and no q/k normalisation inside the recurrence; where a
    call normalises q and k itself (an optional flag), that is a
    preprocessing step in front of it: ``l2norm_rows`` below, then one
    rounding to the input dtype;
  * the snapshot at chunk index c is the state after c full chunks, i.e.
    after c*C tokens of that sequence, valid for 0 <= c <= floor(T_i / C);
  * accepted length n in [0, L] is the number of verified positions folded
    into the committed state; n = 0 leaves the checkpoint unchanged.

Every function below is pinned by ``tests/test_oracle_pins.py`` against
closed forms, invariants and brute force (see that file's header).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "sigmoid",
    "l2norm_rows",
    "kda_step",
    "run_sequence",
    "prefill_ref",
    "chunked_ref",
    "brute_ref",
    "verify_ref",
    "replay_ref",
    "commit_ref",
    "commit_align_ref",
    "align_next_ref",
    "copy_ref",
]


def sigmoid(x):
    """beta = 1 / (1 + exp(-x)) in float64, evaluated without overflow.

    [P1] Sec. 4: the beta gate is a sigmoid of a logit.
    """
    x = np.asarray(x, dtype=np.float64)
    z = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + z), z / (1.0 + z))


def l2norm_rows(x, eps=1e-6):
    """x / sqrt(sum x^2 + eps) over the last axis, in float64.

    The workloads normalise q and k per (token, head) over d_k ("q, k
    L2-normalised per head"); the pages fix no epsilon, so eps = 1e-6 inside
    the square root is a reading that only matters for rows of norm near
    1e-3 or below (a zero row stays zero).
    """
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def kda_step(S, q_t, k_t, v_t, g_t, b_t):
    """One token of the recurrence for every head at once.

    S: (H, d_k, d_v); q_t, k_t, g_t: (H, d_k); v_t: (H, d_v); b_t: (H,).
    Returns (S_t, o_t, u_t) with o_t, u_t of shape (H, d_v).
    """
    alpha = np.exp(g_t)
    beta = sigmoid(b_t)
    S_dec = alpha[:, :, None] * S                        # Diag(alpha) S
    pred = np.matmul(k_t[:, None, :], S_dec)[:, 0, :]    # S_dec^T k
    u = beta[:, None] * (v_t - pred)
    S_new = S_dec + k_t[:, :, None] * u[:, None, :]      # + k u^T
    o = np.matmul(q_t[:, None, :], S_new)[:, 0, :]       # S_t^T q
    return S_new, o, u


def run_sequence(q, k, v, g, b, S0, keep_after=()):
    """Token-by-token run of one sequence from the state S0.

    q, k, g: (T, H, d_k); v: (T, H, d_v); b: (T, H); S0: (H, d_k, d_v).
    keep_after: token counts t at which to keep a copy of the state S_t
    (t = 0 keeps S0).  Returns (o (T, H, d_v), u (T, H, d_v), S_T, kept)
    where kept maps t -> S_t.
    """
    T = q.shape[0]
    S = np.array(S0, dtype=np.float64, copy=True)
    keep = set(int(t) for t in keep_after)
    kept = {}
    if 0 in keep:
        kept[0] = S.copy()
    o = np.zeros((T,) + (S.shape[0], S.shape[2]))
    u = np.zeros_like(o)
    for t in range(T):
        S, o[t], u[t] = kda_step(S, q[t], k[t], v[t], g[t], b[t])
        if t + 1 in keep:
            kept[t + 1] = S.copy()
    return o, u, S, kept


def prefill_ref(q, k, v, g, b, cu_seqlens, S0, chunk, tracks=()):
    """Varlen prefill over packed sequences ([P2] Implementation breakdown).

    q, k, g: (T_total, H, d_k); v: (T_total, H, d_v); b: (T_total, H);
    cu_seqlens: (n+1,) token offsets of the packed sequences;
    S0: (n, H, d_k, d_v) initial state of each sequence;
    tracks: iterable of (seq, c) pairs asking for the state after c full
    chunks of sequence ``seq`` (0 <= c <= floor(T_seq / chunk)).
    Returns (o (T_total, H, d_v), finals (n, H, d_k, d_v), snaps list in
    the order of ``tracks``).
    """
    cu = [int(x) for x in cu_seqlens]
    n = len(cu) - 1
    tracks = [(int(s), int(c)) for s, c in tracks]
    o = np.zeros(q.shape[:2] + (v.shape[2],))
    finals = np.zeros((n,) + tuple(S0.shape[1:]))
    want = {i: [] for i in range(n)}
    for s, c in tracks:
        T_s = cu[s + 1] - cu[s]
        if not 0 <= c <= T_s // chunk:
            raise ValueError(f"track chunk {c} out of range for sequence {s}")
        want[s].append(c * chunk)
    kept_all = {}
    for i in range(n):
        lo, hi = cu[i], cu[i + 1]
        o_i, _, S_T, kept = run_sequence(q[lo:hi], k[lo:hi], v[lo:hi],
                                         g[lo:hi], b[lo:hi], S0[i], want[i])
        o[lo:hi] = o_i
        finals[i] = S_T
        for t, S_t in kept.items():
            kept_all[(i, t)] = S_t
    snaps = [kept_all[(s, c * chunk)] for s, c in tracks]
    return o, finals, snaps


def chunked_ref(q, k, v, g, b, S0, chunk):
    """Second, independent form: the chunked (WY) evaluation of one sequence.

    Within a chunk of n tokens starting from state S, with the in-chunk
    cumulative log-decay Gamma_r = sum_{s<=r} g_s:
        Kt = K*e^Gamma, Kh = K*e^-Gamma, Qt = Q*e^Gamma, Kb = K*e^(Gamma_n-Gamma)
        M  = strict_tril(Kt Kh^T),  P = tril(Qt Kh^T)
        (I + Diag(beta) M) U = Diag(beta) (V - Kt S)      (rows of U are u_t)
        O  = Qt S + P U
        S' = Diag(e^Gamma_n) S + Kb^T U
    Used only to pin ``run_sequence``; it is the algebra a chunked kernel
    evaluates ([P2] Implementation breakdown item 2: 64-token tiles).
    Returns (o (T, H, d_v), u (T, H, d_v), S_T).
    """
    T, H, dk = q.shape
    dv = v.shape[2]
    S = np.array(S0, dtype=np.float64, copy=True)
    o = np.zeros((T, H, dv))
    u = np.zeros((T, H, dv))
    for lo in range(0, T, chunk):
        hi = min(lo + chunk, T)
        n = hi - lo
        for h in range(H):
            Q, K, V = q[lo:hi, h], k[lo:hi, h], v[lo:hi, h]
            beta = sigmoid(b[lo:hi, h])
            Gam = np.cumsum(g[lo:hi, h], axis=0)           # (n, dk)
            Kt, Kh = K * np.exp(Gam), K * np.exp(-Gam)
            Qt = Q * np.exp(Gam)
            Kb = K * np.exp(Gam[-1][None, :] - Gam)
            M = np.tril(Kt @ Kh.T, -1)
            P = np.tril(Qt @ Kh.T)
            A = np.eye(n) + beta[:, None] * M
            U = np.linalg.solve(A, beta[:, None] * (V - Kt @ S[h]))
            o[lo:hi, h] = Qt @ S[h] + P @ U
            u[lo:hi, h] = U
            S[h] = np.exp(Gam[-1])[:, None] * S[h] + Kb.T @ U
    return o, u, S


def brute_ref(q, k, v, g, b, S0):
    """Third form: explicit d_k x d_k transition matrices, tiny inputs only.

        S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
    Returns (o (T, H, d_v), S_T).
    """
    T, H, dk = q.shape
    S = np.array(S0, dtype=np.float64, copy=True)
    o = np.zeros((T, H, v.shape[2]))
    eye = np.eye(dk)
    for t in range(T):
        for h in range(H):
            kk = k[t, h][:, None]
            beta = float(sigmoid(b[t, h]))
            A = (eye - beta * (kk @ kk.T)) @ np.diag(np.exp(g[t, h]))
            S[h] = A @ S[h] + beta * kk @ v[t, h][None, :]
            o[t, h] = S[h].T @ q[t, h]
    return o, S


def verify_ref(q, k, v, g, b, S0):
    """RecoverSSM verify ([P3] Implementation breakdown step 3).

    q, k, g: (n_req, L, H, d_k); v: (n_req, L, H, d_v); b: (n_req, L, H);
    S0: (n_req, H, d_k, d_v) checkpoints, read only.
    Returns (o (n_req, L, H, d_v), u_rec (n_req, H, L, d_v),
    kg_rec (n_req, H, L, 2 d_k) holding key then raw gate, S_L per request).
    """
    n_req, L, H, dk = q.shape
    dv = v.shape[3]
    o = np.zeros((n_req, L, H, dv))
    u_rec = np.zeros((n_req, H, L, dv))
    kg_rec = np.zeros((n_req, H, L, 2 * dk))
    S_L = np.zeros((n_req, H, dk, dv))
    for r in range(n_req):
        o_r, u_r, S_r, _ = run_sequence(q[r], k[r], v[r], g[r], b[r], S0[r])
        o[r] = o_r
        u_rec[r] = np.transpose(u_r, (1, 0, 2))
        kg_rec[r, :, :, :dk] = np.transpose(k[r], (1, 0, 2))
        kg_rec[r, :, :, dk:] = np.transpose(g[r], (1, 0, 2))
        S_L[r] = S_r
    return o, u_rec, kg_rec, S_L


def replay_ref(q, k, v, g, b, S0, n):
    """State after re-running the first n verified positions from S0."""
    _, _, S_n, _ = run_sequence(q[:n], k[:n], v[:n], g[:n], b[:n], S0)
    return S_n


def commit_ref(S0, k_rec, g_rec, u_rec, n):
    """RecoverSSM commit ([P3] Implementation breakdown step 4).

    Rebuild the state after n accepted positions without re-running the
    recurrence:
        S_n = Diag(e^{sum_{t<=n} g_t}) S0
              + sum_{t=1..n} Diag(e^{sum_{s=t+1..n} g_s}) k_t u_t^T,
    accumulated in reverse order t = n..1 with a running decay.
    S0: (H, d_k, d_v); k_rec, g_rec: (H, L, d_k); u_rec: (H, L, d_v).
    """
    S0 = np.asarray(S0, dtype=np.float64)
    H, dk, dv = S0.shape
    decay = np.ones((H, dk))
    acc = np.zeros((H, dk, dv))
    for t in range(n - 1, -1, -1):
        acc += (decay * k_rec[:, t])[:, :, None] * u_rec[:, t][:, None, :]
        decay = decay * np.exp(g_rec[:, t])
    return decay[:, :, None] * S0 + acc


ERR_SLOT, ERR_ACCEPT = 1, 4


def commit_align_ref(slots, block_table, num_tokens, accepted, block_size, k_rec, g_rec, u_rec):
    """Align-mode RecoverSSM commit ([P3] Implementation breakdown steps 4-5
    and the review's block-size check; the reading is this library's, the
    pages give the commit plan only in outline).

    The state is kept per block of ``block_size`` tokens: the state after p
    tokens lives in the slot of the block holding token p (1-based), that is
    block_table[r][(p - 1) // block_size]; a block's slot ends up holding the
    state at its last token.  For request r with p = num_tokens[r] >= 1 and
    n = accepted[r] accepted positions (p' = p + n), with b0 the block of
    token p and b1 the block of token p' (block_size > n, so b1 <= b0 + 1):
      b1 == b0: S_{p'} -> slot of b0 (nothing for n = 0);
      b1 == b0 + 1: the state after the last accepted token still in b0
        (m of them, possibly 0) -> slot of b0 (nothing for m = 0), and
        S_{p'} -> slot of b1.
    Every state is rebuilt from the checkpoint slots[slot of b0] with
    ``commit_ref``.  slots: dict slot -> (H, d_k, d_v) state; block_table:
    (n_req, blocks) ints; k_rec, g_rec: (n_req, H, L, d_k); u_rec:
    (n_req, H, L, d_v).  Returns (dict slot -> new state, error bits); a
    request with n outside [0, L] (ERR_ACCEPT), or p < 1, a block beyond its
    table row or a slot not in ``slots`` (ERR_SLOT) is skipped.
    """
    L = u_rec.shape[2]
    writes, err = {}, 0
    for r in range(len(num_tokens)):
        p, n = int(num_tokens[r]), int(accepted[r])
        if not 0 <= n <= L:
            err |= ERR_ACCEPT
            continue
        if p < 1:
            err |= ERR_SLOT
            continue
        b0 = (p - 1) // block_size
        # the accepted tokens p+1 .. p+n and the block each one falls in
        blocks = [(p + j - 1) // block_size for j in range(1, n + 1)]
        b1 = blocks[-1] if blocks else b0
        if b1 >= len(block_table[r]) or int(block_table[r][b0]) not in slots or int(block_table[r][b1]) not in slots:
            err |= ERR_SLOT
            continue
        s0, s1 = int(block_table[r][b0]), int(block_table[r][b1])
        S0 = slots[s0]
        rec = (k_rec[r], g_rec[r], u_rec[r])
        if b1 == b0:
            if n > 0:
                writes[s0] = commit_ref(S0, *rec, n)
        else:
            m = sum(1 for b in blocks if b == b0)   # accepted tokens that close block b0
            if m > 0:
                writes[s0] = commit_ref(S0, *rec, m)
            writes[s1] = commit_ref(S0, *rec, n)
    return writes, err


def align_next_ref(block_table, num_tokens, accepted, block_size, L, n_slots):
    """What the align-mode commit hands to the next step ([P3] Implementation
    breakdown step 4: after the commit, the align post-processing moves each
    request's running block index on and resets the next step's copy bias to
    its neutral value).  Reading: per request r with p = num_tokens[r] and
    n = accepted[r],
      tokens  = p + n, the tokens the request holds after the commit;
      block   = (p + n - 1) // block_size, the block of its last token,
                whose slot now holds its current state;
      ckpt    = block_table[r][block], the slot the next verify reads;
      bias    = 0 (neutral: the state sits at the running block itself,
                so the next step copies from no offset).
    A request the commit skips (n outside [0, L]; p < 1; a block beyond its
    table row; a slot outside [0, n_slots)) gets (p, -1, -1, 0).
    Returns four int arrays (tokens, block, ckpt, bias).
    """
    n_req = len(num_tokens)
    out = [np.zeros(n_req, dtype=np.int64) for _ in range(4)]
    for r in range(n_req):
        p, n = int(num_tokens[r]), int(accepted[r])
        row = [int(x) for x in block_table[r]]
        ok = 0 <= n <= L and p >= 1
        if ok:
            b0, b1 = (p - 1) // block_size, (p + n - 1) // block_size
            ok = b1 < len(row) and all(0 <= row[b] < n_slots for b in (b0, b1))
        if ok:
            vals = (p + n, b1, row[b1], 0)
        else:
            vals = (p, -1, -1, 0)
        for a, x in zip(out, vals):
            a[r] = x
    return tuple(out)


def copy_ref(pool, src, dst):
    """Rollback / fork as whole-state copies ([P1] Sec. 2 and Sec. 3).

    pool: array indexed by slot; returns a new pool with pool[dst[i]] set to
    the bits of pool[src[i]].  Destinations are distinct and disjoint from
    the sources, so the copies do not depend on their order.
    """
    out = np.array(pool, copy=True)
    for s, d in zip(src, dst):
        out[int(d)] = pool[int(s)]
    return out
