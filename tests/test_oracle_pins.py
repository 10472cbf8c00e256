"""Pins for the CPU oracle: closed forms, invariants, library routines and
hand-worked examples that a plausible mistake in the oracle would break.

None of these compares the oracle with itself re-typed; each checks it
against something the mathematics or a library fixes independently.
"""
import json
import math
import os
from types import SimpleNamespace

import numpy as np
import pytest

from oracle import gdn_oracle as O
import gdn_synth as syn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def dims(h_k=1, h_v=1, d_k=4, d_v=4, conv_k=4):
    return SimpleNamespace(h_k=h_k, h_v=h_v, d_k=d_k, d_v=d_v, conv_k=conv_k)


def rand_core(rng, H, dv, dk):
    k = rng.standard_normal((H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = rng.standard_normal((H, dk))
    v = rng.standard_normal((H, dv))
    a = np.exp(-np.logaddexp(0, rng.standard_normal(H)))
    b = 1 / (1 + np.exp(-rng.standard_normal(H)))
    return q, k, v, a, b


# --------------------------------------------------------------------- golden

def test_hand_worked_delta_rule_d2():
    g = json.load(open(os.path.join(GOLDEN, "hand_delta_rule_d2.json")))
    for form in ("matrix", "rank1"):
        S = np.zeros((1, 2, 2))
        for st in g["steps"]:
            S, o = O.delta_rule_step(S, np.array([st["q"]]), np.array([st["k"]]),
                                     np.array([st["v"]]), np.array([st["a"]]),
                                     np.array([st["b"]]), form)
            np.testing.assert_allclose(S[0], np.array(st["S"]), atol=1e-14)
            np.testing.assert_allclose(o[0], np.array(st["o"]), atol=1e-14)


def test_hand_worked_conv_k3():
    g = json.load(open(os.path.join(GOLDEN, "hand_conv_k3.json")))
    y, win = O.conv_silu_token(np.array(g["window"]), np.array(g["x"]), np.array(g["w"]))
    z = np.array(g["z"])
    np.testing.assert_allclose(y, [zz / (1 + math.exp(-zz)) for zz in z], rtol=1e-15)
    np.testing.assert_array_equal(win, np.array(g["new_window"]))


# ---------------------------------------------------------- recurrence core

def test_matrix_form_equals_rank1_form():
    rng = np.random.default_rng(0)
    H, d = 3, 16
    S = rng.standard_normal((H, d, d))
    S1, S2 = S.copy(), S.copy()
    for _ in range(20):
        q, k, v, a, b = rand_core(rng, H, d, d)
        S1, o1 = O.delta_rule_step(S1, q, k, v, a, b, "matrix")
        S2, o2 = O.delta_rule_step(S2, q, k, v, a, b, "rank1")
        np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(S1, S2, atol=1e-13)


@pytest.mark.parametrize("form", ["matrix", "rank1"])
def test_b_zero_is_pure_decay(form):
    """b = 0: S_T = (prod a) S0 and o_t = (prod_{s<=t} a_s) S0 q_t."""
    rng = np.random.default_rng(1)
    H, d, T = 2, 8, 12
    S0 = rng.standard_normal((H, d, d))
    S = S0.copy()
    cum = np.ones(H)
    for _ in range(T):
        q, k, v, a, _ = rand_core(rng, H, d, d)
        S, o = O.delta_rule_step(S, q, k, v, a, np.zeros(H), form)
        cum = cum * a
        np.testing.assert_allclose(o, cum[:, None] * np.einsum("hij,hj->hi", S0, q),
                                   rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S, cum[:, None, None] * S0, rtol=1e-12)


@pytest.mark.parametrize("form", ["matrix", "rank1"])
def test_b_one_stores_v_at_k(form):
    """b = 1 and unit k: S' k = v for any decay a (a = 1 included)."""
    rng = np.random.default_rng(2)
    H, d = 4, 16
    S = rng.standard_normal((H, d, d))
    for a_val in (1.0, 0.3):
        q, k, v, _, _ = rand_core(rng, H, d, d)
        S, _ = O.delta_rule_step(S, q, k, v, np.full(H, a_val), np.ones(H), form)
        np.testing.assert_allclose(np.einsum("hij,hj->hi", S, k), v, atol=1e-12)


@pytest.mark.parametrize("form", ["matrix", "rank1"])
def test_orthonormal_keys_closed_form(form):
    """Distinct orthonormal keys e_pi(t), S0 = 0:
    S_T e_pi(i) = b_i (prod_{s>i} a_s) v_i, and o_t = S_t q_t."""
    rng = np.random.default_rng(3)
    d, T = 8, 8
    perm = rng.permutation(d)
    vs = rng.standard_normal((T, d))
    a = rng.uniform(0.2, 1.0, T)
    b = rng.uniform(0.0, 1.0, T)
    S = np.zeros((1, d, d))
    for t in range(T):
        k = np.zeros((1, d)); k[0, perm[t]] = 1.0
        q = rng.standard_normal((1, d))
        S, o = O.delta_rule_step(S, q, k, vs[t:t + 1], a[t:t + 1], b[t:t + 1], form)
    for i in range(T):
        want = b[i] * np.prod(a[i + 1:]) * vs[i]
        np.testing.assert_allclose(S[0][:, perm[i]], want, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("form", ["matrix", "rank1"])
def test_scalar_state_closed_form(form):
    """d_k = d_v = 1, k = +-1: s_t = a_t (1 - b_t) s_{t-1} + b_t v_t k_t."""
    rng = np.random.default_rng(4)
    T = 30
    s_ref = 0.7
    S = np.full((1, 1, 1), s_ref)
    for _ in range(T):
        k = rng.choice([-1.0, 1.0])
        v, q = rng.standard_normal(2)
        a, b = rng.uniform(0.1, 1.0), rng.uniform(0, 1)
        S, o = O.delta_rule_step(S, np.array([[q]]), np.array([[k]]), np.array([[v]]),
                                 np.array([a]), np.array([b]), form)
        s_ref = a * (1 - b) * s_ref + b * v * k
        assert abs(S[0, 0, 0] - s_ref) <= 1e-14 * max(1, abs(s_ref))
        assert abs(o[0, 0] - s_ref * q) <= 1e-14 * max(1, abs(s_ref * q))


@pytest.mark.parametrize("form", ["matrix", "rank1"])
def test_homogeneity_in_state_and_values(form):
    """Scaling (S0, v) by 2^m scales (S, o) by 2^m exactly (bitwise)."""
    rng = np.random.default_rng(5)
    H, d = 2, 8
    S = rng.standard_normal((H, d, d))
    Sx = S * 2.0 ** 7
    for _ in range(10):
        q, k, v, a, b = rand_core(rng, H, d, d)
        S, o = O.delta_rule_step(S, q, k, v, a, b, form)
        Sx, ox = O.delta_rule_step(Sx, q, k, v * 2.0 ** 7, a, b, form)
        np.testing.assert_array_equal(ox, o * 2.0 ** 7)
    np.testing.assert_array_equal(Sx, S * 2.0 ** 7)


# ---------------------------------------------------------------- front end

def test_conv_matches_torch_conv1d():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(6)
    C, K, T = 24, 4, 17
    w = rng.standard_normal((C, K))
    win = rng.standard_normal((K - 1, C))
    xs = rng.standard_normal((T, C))
    ys = []
    X = win
    for t in range(T):
        y, X = O.conv_silu_token(X, xs[t], w)
        ys.append(y)
    full = np.concatenate([win, xs], axis=0).T[None]  # [1, C, K-1+T]
    z = torch.nn.functional.conv1d(torch.from_numpy(full), torch.from_numpy(w)[:, None, :],
                                   groups=C)[0].numpy().T
    np.testing.assert_allclose(np.array(ys), torch.nn.functional.silu(torch.from_numpy(z)).numpy(),
                               rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(X, xs[-(K - 1):])


def test_front_end_normalises_q_and_k():
    rng = np.random.default_rng(7)
    dd = dims(h_k=2, h_v=4, d_k=16, d_v=8)
    C = 2 * 2 * 16 + 4 * 8
    w = rng.standard_normal((C, 4))
    q, k, v, _ = O.front_end(rng.standard_normal((3, C)), rng.standard_normal((2, 16)),
                             rng.standard_normal((2, 16)), rng.standard_normal((4, 8)),
                             w, dd, 0.25, 0.0)
    np.testing.assert_allclose(np.linalg.norm(k, axis=-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(np.linalg.norm(q, axis=-1), 0.25, rtol=1e-14)


def test_group_mapping_value_head_uses_its_group():
    """Changing q/k head g alters exactly value heads g*G .. g*G+G-1."""
    rng = np.random.default_rng(8)
    dd = dims(h_k=2, h_v=4, d_k=8, d_v=8)
    C = 2 * 2 * 8 + 4 * 8
    w = rng.standard_normal((C, 4))
    tok = dict(q=rng.standard_normal((1, 2, 8)), k=rng.standard_normal((1, 2, 8)),
               v=rng.standard_normal((1, 4, 8)), a=np.full((1, 4), 0.9), b=np.full((1, 4), 0.5))
    outs = []
    for bump in (0.0, 1.0):
        p = O.OraclePool(1, 1, dd)
        p.S[:] = rng.standard_normal(p.S.shape) if not outs else S0
        S0 = p.S.copy()
        q = tok["q"].copy(); q[0, 1] += bump
        k = tok["k"].copy(); k[0, 1] += bump
        outs.append(p.decode(0, [0], q, k, tok["v"], tok["a"], tok["b"], w)[0])
    np.testing.assert_array_equal(outs[0][:2], outs[1][:2])
    assert np.all(np.abs(outs[0][2:] - outs[1][2:]).max(axis=-1) > 0)


# ------------------------------------------------------------- chunked form

def test_unit_lower_inverse_matches_scipy():
    scipy_linalg = pytest.importorskip("scipy.linalg")
    rng = np.random.default_rng(9)
    for n in (1, 5, 16, 64):
        A = np.tril(rng.standard_normal((n, n)) * 0.3, -1)
        T = O.unit_lower_inverse(A)
        ref = scipy_linalg.solve_triangular(np.eye(n) + A, np.eye(n), lower=True,
                                            unit_diagonal=True)
        np.testing.assert_allclose(T, ref, rtol=1e-12, atol=1e-12)


def _token_loop(dd, S0, win0, tok, w):
    p = O.OraclePool(1, 1, dd, form="rank1")
    p.S[0, 0] = S0
    p.X[0, 0] = win0
    T = tok["q"].shape[0]
    out = p.prefill(0, [0, T], [0], tok["q"], tok["k"], tok["v"], tok["a"], tok["b"], w)
    return out, p.S[0, 0], p.X[0, 0]


@pytest.mark.parametrize("chunk,T,h_k,h_v,d", [(16, 64, 2, 2, 32), (13, 64, 1, 2, 16),
                                               (64, 200, 1, 2, 32), (16, 5, 2, 4, 8)])
def test_chunked_form_equals_token_loop(chunk, T, h_k, h_v, d):
    rng = np.random.default_rng(10 + chunk + T)
    dd = dims(h_k=h_k, h_v=h_v, d_k=d, d_v=d)
    s = syn.Shapes(h_k, h_v, d, d, 4)
    w = syn.draw_conv_weights(rng, s).astype(np.float64)
    tok = syn.draw_tokens(rng, s, (T,), "f32")
    S0 = rng.standard_normal((h_v, d, d))
    win0 = rng.standard_normal((3, s.c_conv))
    o1, S1, X1 = _token_loop(dd, S0, win0, tok, w)
    o2, S2, X2 = O.chunked_sequence(S0, win0, tok["q"], tok["k"], tok["v"], tok["a"], tok["b"],
                                    w, dd, chunk)
    rms = np.sqrt(np.mean(o1 ** 2))
    assert np.abs(o1 - o2).max() / rms < 1e-12
    assert np.abs(S1 - S2).max() / np.sqrt(np.mean(S1 ** 2)) < 1e-12
    np.testing.assert_array_equal(X1, X2)


# ------------------------------------------------------ pool bookkeeping

def _small_pool_case(seed=11, n_slots=6, T=9):
    rng = np.random.default_rng(seed)
    s = syn.Shapes(1, 2, 8, 8, 4)
    dd = dims(1, 2, 8, 8, 4)
    w = syn.draw_conv_weights(rng, s)
    tok = syn.draw_tokens(rng, s, (T,), "bf16")
    return rng, s, dd, w, tok


def test_split_prefill_is_bitwise_equal_to_one_pass():
    rng, s, dd, w, tok = _small_pool_case()
    T = tok["q"].shape[0]
    p1 = O.OraclePool(1, 1, dd)
    o1 = p1.prefill(0, [0, T], [0], tok["q"], tok["k"], tok["v"], tok["a"], tok["b"], w)
    for m in (1, 2, 5):
        p2 = O.OraclePool(1, 1, dd)
        sl = lambda x, a_, b_: x[a_:b_]
        oa = p2.prefill(0, [0, m], [0], *(sl(tok[n], 0, m) for n in "qkvab"), w)
        ob = p2.prefill(0, [0, T - m], [0], *(sl(tok[n], m, T) for n in "qkvab"), w)
        np.testing.assert_array_equal(np.concatenate([oa, ob]), o1)
        np.testing.assert_array_equal(p2.S, p1.S)
        np.testing.assert_array_equal(p2.X, p1.X)


def test_batched_decode_equals_single_slot_runs_and_leaves_others():
    rng, s, dd, w, _ = _small_pool_case()
    n_slots = 6
    pool = O.OraclePool(n_slots, 2, dd)
    pool.S[:] = rng.standard_normal(pool.S.shape)
    pool.X[:] = rng.standard_normal(pool.X.shape)
    ref = O.OraclePool(n_slots, 2, dd)
    ref.S[:] = pool.S; ref.X[:] = pool.X
    before_S, before_X = pool.S.copy(), pool.X.copy()
    ids = np.array([4, -1, 1, 3])
    tok = syn.draw_tokens(rng, s, (4,), "bf16")
    out = pool.decode(1, ids, tok["q"], tok["k"], tok["v"], tok["a"], tok["b"], w)
    for i, sl in enumerate(ids):
        if sl < 0:
            assert np.isnan(out[i]).all()
            continue
        o = ref.decode(1, [sl], *(tok[n][i:i + 1] for n in "qkvab"), w)
        np.testing.assert_array_equal(out[i], o[0])
    np.testing.assert_array_equal(pool.S, ref.S)
    untouched = [0, 2, 5]
    np.testing.assert_array_equal(pool.S[untouched], before_S[untouched])
    np.testing.assert_array_equal(pool.X[untouched], before_X[untouched])
    np.testing.assert_array_equal(pool.S[ids[ids >= 0], 0], before_S[ids[ids >= 0], 0])


def test_reset_slot_starts_from_zero():
    rng, s, dd, w, tok = _small_pool_case()
    pool = O.OraclePool(3, 1, dd)
    pool.S[:] = rng.standard_normal(pool.S.shape)
    pool.X[:] = rng.standard_normal(pool.X.shape)
    keep = pool.S[0].copy()
    pool.reset([2, 1])
    assert not pool.S[1:].any() and not pool.X[1:].any()
    np.testing.assert_array_equal(pool.S[0], keep)
    fresh = O.OraclePool(1, 1, dd)
    T = tok["q"].shape[0]
    o1 = pool.prefill(0, [0, T], [1], tok["q"], tok["k"], tok["v"], tok["a"], tok["b"], w)
    o2 = fresh.prefill(0, [0, T], [0], tok["q"], tok["k"], tok["v"], tok["a"], tok["b"], w)
    np.testing.assert_array_equal(o1, o2)


def test_window_holds_last_raw_inputs():
    rng, s, dd, w, tok = _small_pool_case(T=2)
    pool = O.OraclePool(1, 1, dd)
    old = rng.standard_normal(pool.X[0, 0].shape)
    pool.X[0, 0] = old
    pool.prefill(0, [0, 2], [0], tok["q"], tok["k"], tok["v"], tok["a"], tok["b"], w)
    raw = np.concatenate([tok["q"].reshape(2, -1), tok["k"].reshape(2, -1),
                          tok["v"].reshape(2, -1)], axis=1)
    np.testing.assert_array_equal(pool.X[0, 0], np.concatenate([old[2:], raw]))


@pytest.mark.parametrize("acc", [0, 1, 3, 4])
def test_verify_equals_sequential_decode(acc):
    rng, s, dd, w, _ = _small_pool_case()
    n_tok = 4
    pool = O.OraclePool(2, 1, dd)
    pool.S[:] = rng.standard_normal(pool.S.shape)
    pool.X[:] = rng.standard_normal(pool.X.shape)
    seq = O.OraclePool(2, 1, dd)
    seq.S[:] = pool.S; seq.X[:] = pool.X
    tok = syn.draw_tokens(rng, s, (1, n_tok), "bf16")
    out = pool.verify(0, [1], n_tok, tok["q"], tok["k"], tok["v"], tok["a"], tok["b"], w,
                      np.array([acc]))
    snap = None
    for t in range(n_tok):
        if t == acc:
            snap = (seq.S.copy(), seq.X.copy())
        o = seq.decode(0, [1], *(tok[n][:, t] for n in "qkvab"), w)
        np.testing.assert_array_equal(out[0, t], o[0])
    if snap is None:
        snap = (seq.S.copy(), seq.X.copy())
    np.testing.assert_array_equal(pool.S, snap[0])
    np.testing.assert_array_equal(pool.X, snap[1])


# ------------------------------------------------------- input projection

def test_in_projection_brute_force_tiny():
    """Every output of the projection recomputed with plain Python loops from
    the definitions (dot products; softplus as log(1 + e^y); the logistic)."""
    rng = np.random.default_rng(40)
    dm = dims(h_k=1, h_v=2, d_k=2, d_v=2)
    hidden, T = 5, 3
    C = 2 * 2 + 2 * 2 + 2 * 2
    x = rng.standard_normal((T, hidden))
    W = rng.standard_normal((C, hidden))
    q, k, v, a, b = O.in_projection(x, W, dm)
    flat = [[sum(x[t][i] * W[c][i] for i in range(hidden)) for c in range(C)] for t in range(T)]
    for t in range(T):
        y = flat[t]
        assert np.allclose(q[t].ravel(), y[0:2], rtol=0, atol=1e-14)
        assert np.allclose(k[t].ravel(), y[2:4], rtol=0, atol=1e-14)
        assert np.allclose(v[t].ravel(), y[4:8], rtol=0, atol=1e-14)
        for h in range(2):
            assert math.isclose(a[t][h], math.exp(-math.log(1.0 + math.exp(y[8 + h]))), rel_tol=1e-13)
            assert math.isclose(b[t][h], 1.0 / (1.0 + math.exp(-y[10 + h])), rel_tol=1e-13)


def test_in_projection_one_hot_rows_select_inputs():
    """W rows that are unit vectors pick input features: the raw q, k, v are
    exact copies of permuted inputs, and a = 1 / (1 + e^x) exactly."""
    rng = np.random.default_rng(41)
    dm = dims(h_k=2, h_v=4, d_k=4, d_v=4)
    C = 2 * 2 * 4 + 4 * 4 + 2 * 4
    hidden = C
    perm = rng.permutation(hidden)
    W = np.eye(hidden)[perm]                      # row c = e_perm[c]
    x = rng.standard_normal((7, hidden))
    q, k, v, a, b = O.in_projection(x, W, dm)
    y = x[:, perm]
    np.testing.assert_array_equal(q.reshape(7, -1), y[:, :8])
    np.testing.assert_array_equal(k.reshape(7, -1), y[:, 8:16])
    np.testing.assert_array_equal(v.reshape(7, -1), y[:, 16:32])
    np.testing.assert_allclose(a, 1.0 / (1.0 + np.exp(y[:, 32:36])), rtol=1e-15)
    np.testing.assert_allclose(b, 1.0 / (1.0 + np.exp(-y[:, 36:40])), rtol=1e-15)


def test_in_projection_gate_symmetry_and_limits():
    """exp(-softplus(-y)) and sigmoid(y) are the same function: with the a
    rows the negated b rows, a == b; large logits saturate a -> 0, b -> 1."""
    rng = np.random.default_rng(42)
    dm = dims(h_k=1, h_v=3, d_k=2, d_v=2)
    hidden = 6
    Wb = rng.standard_normal((3, hidden))
    W = np.concatenate([rng.standard_normal((2 + 2 + 6, hidden)), -Wb, Wb])
    x = rng.standard_normal((5, hidden))
    _, _, _, a, b = O.in_projection(x, W, dm)
    np.testing.assert_allclose(a, b, rtol=1e-14)
    _, _, _, a, b = O.in_projection(np.full((1, hidden), 100.0), np.concatenate(
        [np.zeros((10, hidden)), np.ones((6, hidden))]), dm)
    assert np.all(a < 1e-200) and np.all(b == 1.0)


def test_fp32_timing_variant_tracks_fp64_oracle():
    """The fp32 variant (used only to time the CPU baseline) runs the same
    steps: on the tiny layer, after a 64-token prefill, decode and verify, its
    outputs and states agree with the fp64 oracle to fp32 rounding."""
    case = syn.tiny_layer_case()
    s, w = case["shapes"], case["conv_w"]
    pre, dec = case["prefill"], case["decode"]
    res = {}
    for dt in (np.float64, np.float32):
        op = O.OraclePool(2, 1, s, form="rank1", dtype=dt)
        o1 = op.prefill(0, [0, 64], [1], *(pre[n] for n in "qkvab"), w)
        o2 = op.decode(0, [1], *(dec[n][:1] for n in "qkvab"), w)
        o3 = op.verify(0, [1], 4, *(dec[n][1:5][None] for n in "qkvab"), w, np.array([3]))
        res[dt] = (o1, o2, o3, op.S.astype(np.float64))
        assert op.S.dtype == dt
    for a, b in zip(res[np.float32], res[np.float64]):
        a, b = np.nan_to_num(a), np.nan_to_num(b)
        assert np.abs(a - b).max() <= 1e-4 * np.sqrt(np.mean(b * b)), np.abs(a - b).max()
