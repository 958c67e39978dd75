"""Pins for the fp64 oracle, checked on the CPU (-m "not gpu").

The oracle is trusted only because it agrees with things other than itself:
  * a hand-worked two-token example in exact dyadic arithmetic (golden file);
  * a brute-force form with explicit d_k x d_k transition matrices;
  * the chunked (WY) form, for several chunk sizes with ragged tails;
  * closed forms: beta = 0 is pure per-channel decay; with alpha = 1,
    beta = 1 a unit key makes S^T k = v exactly and leaves directions
    orthogonal to k unchanged; writing a full orthonormal key basis
    overwrites any initial state with sum_t k_t v_t^T;
  * a one-hot query reads one row of the state (fixes the orientation);
  * linearity of (S0, V) -> (S_T, O) for fixed q, k, g, b;
  * sigmoid against scipy's expit;
  * commit(n) = replay of the first n positions (commit(0) = S0 bitwise);
  * snapshot = the state of the run truncated to c*C tokens;
  * prefill split invariance.
Shapes use d_k != d_v wherever possible so that a transposed operand fails
loudly.  ``test_pins_catch_planted_mistakes`` plants plausible mistakes in a
copy of the token step and checks that the pins reject every one of them.
"""

import json
import os

import numpy as np
import pytest
import scipy.special

import oracle.kda_oracle as ko

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(T, H, dk, dv, seed, gscale=(-0.3, -0.001)):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = rng.uniform(gscale[0], gscale[1], (T, H, dk))
    b = rng.standard_normal((T, H))
    S0 = rng.standard_normal((H, dk, dv))
    return q, k, v, g, b, S0


def rel(x, ref):
    return np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300)


# ---------------------------------------------------------------- golden example

def golden_two_token():
    with open(os.path.join(GOLDEN, "two_token_example.json")) as f:
        return json.load(f)


def check_two_token_example():
    ex = golden_two_token()
    S = np.array(ex["S0"], dtype=np.float64)[None]
    for tok in ex["tokens"]:
        g = np.array(tok["g_value"])[None]
        b = np.array([tok.get("b_value", tok["b"])], dtype=np.float64)
        q = np.array(tok["q"], dtype=np.float64)[None]
        k = np.array(tok["k"], dtype=np.float64)[None]
        v = np.array(tok["v"], dtype=np.float64)[None]
        S, o, u = ko.kda_step(S, q, k, v, g, b)
        if not (np.allclose(u[0], tok["u"], rtol=0, atol=1e-14)
                and np.allclose(S[0], tok["S"], rtol=0, atol=1e-14)
                and np.allclose(o[0], tok["o"], rtol=0, atol=1e-14)):
            return False
    return True


def test_two_token_golden_example():
    assert check_two_token_example()


# ---------------------------------------------------------------- brute force / chunked

def check_brute(seed=0):
    q, k, v, g, b, S0 = rand_case(24, 2, 5, 3, seed)
    o, _, S, _ = ko.run_sequence(q, k, v, g, b, S0)
    o_b, S_b = ko.brute_ref(q, k, v, g, b, S0)
    return np.max(np.abs(o - o_b)) < 1e-12 and np.max(np.abs(S - S_b)) < 1e-12


def test_brute_force_equals_token_recurrence():
    for seed in range(3):
        assert check_brute(seed)


@pytest.mark.parametrize("chunk,T", [(1, 9), (3, 70), (16, 70), (16, 64), (64, 130), (64, 37)])
def test_chunked_equals_token_recurrence(chunk, T):
    q, k, v, g, b, S0 = rand_case(T, 2, 16, 8, 100 + chunk + T)
    o, u, S, _ = ko.run_sequence(q, k, v, g, b, S0)
    o_c, u_c, S_c = ko.chunked_ref(q, k, v, g, b, S0, chunk)
    assert rel(o_c, o) < 1e-12
    assert rel(u_c, u) < 1e-12
    assert rel(S_c, S) < 1e-12


def test_chunked_equals_token_recurrence_full_width():
    q, k, v, g, b, S0 = rand_case(150, 1, 128, 128, 7, gscale=(-0.1, -0.001))
    o, u, S, _ = ko.run_sequence(q, k, v, g, b, S0)
    o_c, u_c, S_c = ko.chunked_ref(q, k, v, g, b, S0, 64)
    assert rel(o_c, o) < 1e-11 and rel(S_c, S) < 1e-11 and rel(u_c, u) < 1e-11


# ---------------------------------------------------------------- closed forms

def check_beta_zero_pure_decay(seed=1):
    q, k, v, g, b, S0 = rand_case(30, 2, 6, 4, seed)
    b = np.full_like(b, -800.0)          # sigmoid(-800) underflows to exactly 0
    o, u, S, _ = ko.run_sequence(q, k, v, g, b, S0)
    G = np.cumsum(g, axis=0)             # (T, H, dk)
    S_closed = np.exp(G[-1])[:, :, None] * S0
    o_closed = np.einsum("thk,hkv->thv", q * np.exp(G), S0)
    return (np.max(np.abs(u)) == 0.0 and rel(S, S_closed) < 1e-13
            and rel(o, o_closed) < 1e-13)


def test_beta_zero_is_pure_decay():
    assert check_beta_zero_pure_decay()


def check_write_invariant(seed=2):
    rng = np.random.default_rng(seed)
    H, dk, dv = 2, 6, 4
    S = rng.standard_normal((H, dk, dv))
    for _ in range(5):
        k = rng.standard_normal((H, dk))
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        v = rng.standard_normal((H, dv))
        q = rng.standard_normal((H, dk))
        w = rng.standard_normal((H, dk))
        w -= np.sum(w * k, axis=-1, keepdims=True) * k       # w orthogonal to k
        S_new, _, _ = ko.kda_step(S, q, k, v, np.zeros((H, dk)), np.full(H, 40.0))
        read_k = np.einsum("hkv,hk->hv", S_new, k)
        keep_w = np.einsum("hkv,hk->hv", S_new, w) - np.einsum("hkv,hk->hv", S, w)
        if np.max(np.abs(read_k - v)) > 1e-13 or np.max(np.abs(keep_w)) > 1e-13:
            return False
        S = S_new
    return True


def test_unit_key_write_invariant():
    # alpha = 1 (g = 0) and beta = sigmoid(40) = 1.0 exactly in fp64
    assert float(ko.sigmoid(40.0)) == 1.0
    assert check_write_invariant()


def check_orthonormal_overwrite(seed=3):
    rng = np.random.default_rng(seed)
    H, dk, dv = 2, 5, 3
    Qm = np.stack([np.linalg.qr(rng.standard_normal((dk, dk)))[0] for _ in range(H)])
    k = np.transpose(Qm, (2, 0, 1))                     # token t uses column t
    v = rng.standard_normal((dk, H, dv))
    q = rng.standard_normal((dk, H, dk))
    g = np.zeros((dk, H, dk))
    b = np.full((dk, H), 40.0)
    S0 = rng.standard_normal((H, dk, dv))
    _, _, S, _ = ko.run_sequence(q, k, v, g, b, S0)
    expect = np.einsum("thk,thv->hkv", k, v)
    return np.max(np.abs(S - expect)) < 1e-12


def test_orthonormal_basis_overwrites_state():
    assert check_orthonormal_overwrite()


def check_onehot_query(seed=4):
    q, k, v, g, b, S0 = rand_case(12, 2, 5, 3, seed)
    i = 3
    q = np.zeros_like(q)
    q[:, :, i] = 1.0
    o, _, _, kept = ko.run_sequence(q, k, v, g, b, S0, keep_after=range(1, 13))
    return all(np.max(np.abs(o[t - 1] - kept[t][:, i, :])) == 0.0 for t in range(1, 13))


def test_onehot_query_reads_state_row():
    assert check_onehot_query()


def test_linearity_in_state_and_values():
    q, k, v, g, b, S0 = rand_case(40, 2, 6, 5, 5)
    rng = np.random.default_rng(55)
    v2 = rng.standard_normal(v.shape)
    S02 = rng.standard_normal(S0.shape)
    a1, a2 = 0.7, -1.3
    o1, _, S1, _ = ko.run_sequence(q, k, v, g, b, S0)
    o2, _, S2, _ = ko.run_sequence(q, k, v2, g, b, S02)
    o3, _, S3, _ = ko.run_sequence(q, k, a1 * v + a2 * v2, g, b, a1 * S0 + a2 * S02)
    assert rel(o3, a1 * o1 + a2 * o2) < 1e-12
    assert rel(S3, a1 * S1 + a2 * S2) < 1e-12


def test_sigmoid_matches_library():
    x = np.concatenate([np.linspace(-60, 60, 1001), [-800.0, 800.0, 0.0]])
    ref = scipy.special.expit(x)
    assert np.all(np.abs(ko.sigmoid(x) - ref) <= 4e-16 * np.abs(ref))
    assert float(ko.sigmoid(0.0)) == 0.5
    assert float(ko.sigmoid(-800.0)) == 0.0


# ---------------------------------------------------------------- verify / commit

def test_commit_equals_replay():
    rng = np.random.default_rng(6)
    n_req, L, H, dk, dv = 3, 8, 2, 6, 5
    q = rng.standard_normal((n_req, L, H, dk))
    k = rng.standard_normal((n_req, L, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((n_req, L, H, dv))
    g = rng.uniform(-0.1, -0.001, (n_req, L, H, dk))
    b = rng.standard_normal((n_req, L, H))
    S0 = rng.standard_normal((n_req, H, dk, dv))
    o, u_rec, kg_rec, S_L = ko.verify_ref(q, k, v, g, b, S0)
    for r in range(n_req):
        assert np.array_equal(kg_rec[r, :, :, :dk], np.transpose(k[r], (1, 0, 2)))
        assert np.array_equal(kg_rec[r, :, :, dk:], np.transpose(g[r], (1, 0, 2)))
        for n in range(L + 1):
            S_c = ko.commit_ref(S0[r], kg_rec[r, :, :, :dk], kg_rec[r, :, :, dk:], u_rec[r], n)
            S_r = ko.replay_ref(q[r], k[r], v[r], g[r], b[r], S0[r], n)
            assert rel(S_c, S_r) < 1e-13
            if n == 0:
                assert np.array_equal(S_c, S0[r])
            if n == L:
                assert rel(S_c, S_L[r]) < 1e-13
        # verify outputs are those of a plain run from the checkpoint
        o_r, _, _, _ = ko.run_sequence(q[r], k[r], v[r], g[r], b[r], S0[r])
        assert np.array_equal(o[r], o_r)


def test_copy_is_bitwise():
    rng = np.random.default_rng(8)
    pool = rng.standard_normal((10, 2, 3, 4)).astype(np.float32)
    out = ko.copy_ref(pool, [1, 1, 4], [6, 7, 8])
    assert np.array_equal(out[6], pool[1]) and np.array_equal(out[8], pool[4])
    for s in (0, 1, 2, 3, 4, 5, 9):
        assert np.array_equal(out[s], pool[s])


# ---------------------------------------------------------------- prefill bookkeeping

def test_snapshot_equals_truncated_run_and_split():
    C = 16
    lens = [70, 0, 32, 5]
    T = sum(lens)
    q, k, v, g, b, _ = rand_case(T, 2, 8, 6, 9)
    rng = np.random.default_rng(99)
    S0 = rng.standard_normal((len(lens), 2, 8, 6))
    cu = np.concatenate([[0], np.cumsum(lens)])
    tracks = [(0, 0), (0, 2), (0, 4), (2, 2), (3, 0), (1, 0)]
    o, finals, snaps = ko.prefill_ref(q, k, v, g, b, cu, S0, C, tracks)
    for (s, c), snap in zip(tracks, snaps):
        lo = cu[s]
        _, _, S_t, _ = ko.run_sequence(q[lo:lo + c * C], k[lo:lo + c * C], v[lo:lo + c * C],
                                       g[lo:lo + c * C], b[lo:lo + c * C], S0[s])
        assert np.array_equal(snap, S_t)
    # empty sequence: final = initial
    assert np.array_equal(finals[1], S0[1])
    # split invariance: run 0..T1 then T1..T from the carried state
    lo, hi = cu[0], cu[1]
    T1 = 23
    o_a, _, S_a, _ = ko.run_sequence(q[lo:lo + T1], k[lo:lo + T1], v[lo:lo + T1], g[lo:lo + T1], b[lo:lo + T1], S0[0])
    o_b, _, S_b, _ = ko.run_sequence(q[lo + T1:hi], k[lo + T1:hi], v[lo + T1:hi], g[lo + T1:hi], b[lo + T1:hi], S_a)
    assert rel(np.concatenate([o_a, o_b]), o[lo:hi]) < 1e-14
    assert rel(S_b, finals[0]) < 1e-14
    with pytest.raises(ValueError):
        ko.prefill_ref(q, k, v, g, b, cu, S0, C, [(3, 1)])


# ---------------------------------------------------------------- planted mistakes

def _mutants():
    sig = ko.sigmoid

    def undecayed_correction(S, q, k, v, g, b):
        a = np.exp(g); bt = sig(b)
        u = bt[:, None] * (v - np.einsum("hkv,hk->hv", S, k))
        S1 = a[:, :, None] * S + k[:, :, None] * u[:, None, :]
        return S1, np.einsum("hkv,hk->hv", S1, q), u

    def output_before_update(S, q, k, v, g, b):
        a = np.exp(g); bt = sig(b)
        Sd = a[:, :, None] * S
        u = bt[:, None] * (v - np.einsum("hkv,hk->hv", Sd, k))
        return Sd + k[:, :, None] * u[:, None, :], np.einsum("hkv,hk->hv", Sd, q), u

    def wrong_sign(S, q, k, v, g, b):
        a = np.exp(g); bt = sig(b)
        Sd = a[:, :, None] * S
        u = bt[:, None] * (v + np.einsum("hkv,hk->hv", Sd, k))
        S1 = Sd + k[:, :, None] * u[:, None, :]
        return S1, np.einsum("hkv,hk->hv", S1, q), u

    def beta_on_value_only(S, q, k, v, g, b):
        a = np.exp(g); bt = sig(b)
        Sd = a[:, :, None] * S
        u = bt[:, None] * v - np.einsum("hkv,hk->hv", Sd, k)
        S1 = Sd + k[:, :, None] * u[:, None, :]
        return S1, np.einsum("hkv,hk->hv", S1, q), u

    def decay_after_write(S, q, k, v, g, b):
        a = np.exp(g); bt = sig(b)
        u = bt[:, None] * (v - np.einsum("hkv,hk->hv", S, k))
        S1 = a[:, :, None] * (S + k[:, :, None] * u[:, None, :])
        return S1, np.einsum("hkv,hk->hv", S1, q), u

    def sigmoid_of_negative(S, q, k, v, g, b):
        a = np.exp(g); bt = sig(-b)
        Sd = a[:, :, None] * S
        u = bt[:, None] * (v - np.einsum("hkv,hk->hv", Sd, k))
        S1 = Sd + k[:, :, None] * u[:, None, :]
        return S1, np.einsum("hkv,hk->hv", S1, q), u

    def decay_by_gate_not_exp(S, q, k, v, g, b):
        a = 1.0 + g; bt = sig(b)
        Sd = a[:, :, None] * S
        u = bt[:, None] * (v - np.einsum("hkv,hk->hv", Sd, k))
        S1 = Sd + k[:, :, None] * u[:, None, :]
        return S1, np.einsum("hkv,hk->hv", S1, q), u

    return [undecayed_correction, output_before_update, wrong_sign, beta_on_value_only,
            decay_after_write, sigmoid_of_negative, decay_by_gate_not_exp]


def test_pins_catch_planted_mistakes(monkeypatch):
    checks = [check_two_token_example, check_brute, check_beta_zero_pure_decay,
              check_write_invariant, check_orthonormal_overwrite, check_onehot_query]
    assert all(c() for c in checks)
    for mutant in _mutants():
        monkeypatch.setattr(ko, "kda_step", mutant)
        failed = [c.__name__ for c in checks if not c()]
        monkeypatch.undo()
        assert failed, f"planted mistake {mutant.__name__} passed every pin"


def test_commit_pin_catches_forward_order_decay():
    # A commit that applies the decay in forward order (the usual slip) must
    # disagree with replay; the correct reverse-order rebuild agrees.
    rng = np.random.default_rng(12)
    L, H, dk, dv = 6, 1, 4, 3
    q = rng.standard_normal((L, H, dk)); k = rng.standard_normal((L, H, dk))
    v = rng.standard_normal((L, H, dv)); g = rng.uniform(-0.3, -0.01, (L, H, dk))
    b = rng.standard_normal((L, H)); S0 = rng.standard_normal((H, dk, dv))
    _, u, _, _ = ko.run_sequence(q, k, v, g, b, S0)
    kr, gr, ur = (np.transpose(x, (1, 0, 2)) for x in (k, g, u))
    n = L
    decay = np.ones((H, dk)); acc = np.zeros((H, dk, dv))
    for t in range(n):                          # forward-order slip
        acc += (decay * kr[:, t])[:, :, None] * ur[:, t][:, None, :]
        decay = decay * np.exp(gr[:, t])
    wrong = decay[:, :, None] * S0 + acc
    right = ko.commit_ref(S0, kr, gr, ur, n)
    replay = ko.replay_ref(q, k, v, g, b, S0, n)
    assert rel(right, replay) < 1e-13
    assert rel(wrong, replay) > 1e-3


def test_l2norm_rows():
    """q/k normalisation per (token, head) over d_k: a 3-4-5 row, unit norms,
    the library norm, direction, scale invariance, a zero row."""
    row = np.zeros(16)
    row[:2] = (3.0, 4.0)
    got = ko.l2norm_rows(row)
    assert np.allclose(got[:2], (0.6, 0.8), rtol=3e-8, atol=0) and not got[2:].any()
    x = np.random.default_rng(21).standard_normal((5, 3, 128)) * 4.0
    y = ko.l2norm_rows(x)
    assert np.allclose(np.sqrt((y * y).sum(-1)), 1.0, rtol=1e-9, atol=0)   # over d_k, per (token, head)
    assert np.allclose(y, x / np.linalg.norm(x, axis=-1, keepdims=True), rtol=1e-9, atol=0)
    assert np.allclose(y * np.linalg.norm(x, axis=-1, keepdims=True), x, rtol=1e-8, atol=0)
    assert np.allclose(ko.l2norm_rows(7.5 * x), y, rtol=1e-9, atol=0)
    z = ko.l2norm_rows(np.zeros((2, 128)))
    assert np.array_equal(z, np.zeros((2, 128)))
