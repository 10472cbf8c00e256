"""GPU checks at the extremes of the gates, where the delta rule reduces to
something with a closed form (the gated delta rule of "Plan
(research-based): Qwen3.6-35B-A3B -- parity fix + path to >150 tok/s",
section "What the research found"):

  * b = 0: no write, the state only decays.  S' = a S exactly (fp32
    products, a zero's sign aside) in the decode and verify kernels (their
    update is fma(a, s, 0)); in the chunked
    prefill S_T = (prod a) S_0 and o_t = (prod_{s<=t} a_s) S_0 q_t.
  * b = 1, a = 1 and unit k (eps negligible): the update stores v at k, so
    S k = v right after the token.
  * a -> 0: the state forgets.  Decay factors down to 1e-30 and below the
    kernels' clamp of log a at -87 (a = 1e-45, an fp32 denormal), inside
    prefill chunks, in decode/verify and in the verify ring, against the
    oracle (which takes a as given).
"""
import numpy as np
import pytest

import gdn_synth as syn
from gpu_util import (check_f32, check_out, dev, host, load_slots, make_pool, oracle_pool, say,
                      scramble_pool, tokens_to_dev)
from oracle import gdn_oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

QN = syn.QWEN3_NEXT


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_state_layer_amd import binding
    binding.load_library()


def _exactly(got, expect):
    """Equal fp32 values, element by element (exact, no tolerance; a zero's
    sign may differ: fma(a, -0, +0) is +0)."""
    got = np.asarray(got, np.float32)
    expect = np.asarray(expect, np.float32)
    return got.shape == expect.shape and bool(np.all(got == expect))


def _decode_case(n, seed, s=QN, io="bf16", n_slots=256):
    rng = np.random.default_rng(seed)
    w = syn.draw_conv_weights(rng, s)
    ids = rng.permutation(n_slots)[:n].astype(np.int32)
    tok = syn.draw_tokens(rng, s, (n,), io)
    contents = syn.draw_pool_contents(seed, ids, s, io)
    return w, ids, tok, contents


@pytest.mark.parametrize("n", [4, 64])
def test_decode_b0_state_is_bitwise_decay(n):
    """b = 0 at decode (n = 4 runs the row-split kernel, 64 the one-workgroup
    kernel): every listed slot's state becomes fp32(a) * S exactly (a zero's
    sign aside), outputs
    match the oracle, other slots are untouched."""
    s, io, n_slots = QN, "bf16", 256
    w_np, ids, tok, contents = _decode_case(n, 900 + n)
    tok["b"][:] = 0.0
    say(f"decode b=0, {n} of {n_slots} slots")
    pool = make_pool(s, n_slots, io)
    scramble_pool(pool, 901)
    load_slots(pool, contents)
    st0, wn0 = pool.state.clone(), pool.window.clone()
    out = torch.empty((n, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda")
    td = tokens_to_dev(tok, io)
    pool.decode(0, dev(ids, torch.int32), td["q"], td["k"], td["v"], td["a"], td["b"], dev(w_np), out)
    torch.cuda.synchronize()
    assert pool.error() == 0
    got = pool.state[torch.from_numpy(ids.astype(np.int64)).cuda()].cpu().numpy()
    for i, sl in enumerate(ids):
        expect = np.float32(tok["a"][i])[:, None, None] * contents[int(sl)][0][0]
        bad = got[i, 0] != expect
        if bad.any():
            h, r, c = np.nonzero(bad)
            say(f"  slot {sl} (entry {i}): {bad.sum()} elements differ, heads {np.unique(h)[:8]}, "
                f"rows {np.unique(r)[:8]}, cols {np.unique(c)[:8]}; first: got {got[i, 0][h[0], r[0], c[0]]!r} "
                f"expected {expect[h[0], r[0], c[0]]!r}, before {contents[int(sl)][0][0][h[0], r[0], c[0]]!r}, "
                f"a {tok['a'][i][h[0]]!r}")
        assert not bad.any(), f"slot {sl}: not a*S"
    op = oracle_pool(s, contents, ids, form="rank1")
    ref = op.decode(0, np.arange(n), tok["q"], tok["k"], tok["v"], tok["a"], tok["b"], w_np)
    check_out("outputs", host(out), ref, io)
    assert np.array_equal(host(pool.window[torch.from_numpy(ids.astype(np.int64)).cuda()]), op.X)
    mask = torch.ones(n_slots, dtype=torch.bool, device="cuda")
    mask[torch.from_numpy(ids.astype(np.int64)).cuda()] = False
    assert torch.equal(pool.state[mask], st0[mask]) and torch.equal(pool.window[mask], wn0[mask])


def test_verify_b0_commit_is_bitwise_decay_chain():
    """b = 0 at verify (16 slots x 4 tokens, accept_len 0..4): the committed
    state is the fp32 product chain a_n * (... * (a_1 * S)), exactly."""
    s, io, n, n_tok = QN, "bf16", 16, 4
    rng = np.random.default_rng(910)
    w_np = syn.draw_conv_weights(rng, s)
    ids = rng.permutation(64)[:n].astype(np.int32)
    acc = np.array([0, 1, 2, 3, 4] * 3 + [4], np.int32)
    tok = syn.draw_tokens(rng, s, (n, n_tok), io)
    tok["b"][:] = 0.0
    contents = syn.draw_pool_contents(911, ids, s, io)
    say("verify b=0, 16 slots x 4 tokens")
    pool = make_pool(s, 64, io)
    load_slots(pool, contents)
    out = torch.empty((n, n_tok, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda")
    td = tokens_to_dev(tok, io)
    pool.verify(0, dev(ids, torch.int32), n_tok, td["q"], td["k"], td["v"], td["a"], td["b"],
                dev(w_np), dev(acc, torch.int32), out)
    torch.cuda.synchronize()
    got = pool.state[torch.from_numpy(ids.astype(np.int64)).cuda()].cpu().numpy()
    for i, sl in enumerate(ids):
        S = contents[int(sl)][0][0].astype(np.float32)
        for t in range(acc[i]):
            S = np.float32(tok["a"][i, t])[:, None, None] * S
        assert _exactly(got[i, 0], S), f"slot {sl}: not the decay chain"
    op = oracle_pool(s, contents, ids, form="rank1")
    ref = op.verify(0, np.arange(n), n_tok, tok["q"], tok["k"], tok["v"], tok["a"], tok["b"], w_np, acc)
    check_out("outputs", host(out), ref, io)


def _front_end(s, window, tok_i, w_np, eps):
    """The oracle's conv + SiLU + normalisation for one token of one slot."""
    q, k, v, _ = O.front_end(window, tok_i["q"], tok_i["k"], tok_i["v"], np.asarray(w_np, np.float64),
                             s, s.d_k ** -0.5, eps)
    return O.expand_groups(k, s.h_v), v


@pytest.mark.parametrize("n", [4, 64])
def test_decode_b1_a1_stores_v_at_k(n):
    """b = 1, a = 1, eps = 1e-30 (so k^ is unit to fp32 rounding): after the
    token, S k^ = v^ for every value head of every entry."""
    s, io, eps = QN, "bf16", 1e-30
    w_np, ids, tok, contents = _decode_case(n, 920 + n)
    tok["a"][:] = 1.0
    tok["b"][:] = 1.0
    say(f"decode b=1 a=1, {n} slots")
    pool = make_pool(s, 256, io, eps=eps)
    load_slots(pool, contents)
    out = torch.empty((n, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda")
    td = tokens_to_dev(tok, io)
    pool.decode(0, dev(ids, torch.int32), td["q"], td["k"], td["v"], td["a"], td["b"], dev(w_np), out)
    torch.cuda.synchronize()
    got = host(pool.state[torch.from_numpy(ids.astype(np.int64)).cuda()])[:, 0]
    worst = 0.0
    for i, sl in enumerate(ids):
        k_hat, v_hat = _front_end(s, contents[int(sl)][1][0], {m: tok[m][i] for m in "qkv"}, w_np, eps)
        Sk = np.einsum("hij,hj->hi", got[i], k_hat)
        worst = max(worst, float(np.abs(Sk - v_hat).max() / np.sqrt(np.mean(v_hat ** 2))))
    say(f"  max |S k^ - v^| / rms(v^) = {worst:.3e}")
    assert worst <= 1e-4


def _prefill(pool, cu, ids, tok, w, chunk, io):
    s = pool.desc
    T = int(cu[-1])
    td = tokens_to_dev(tok, io)
    out = torch.full((T, s.h_v, s.d_v), float("nan"), dtype=pool.io_torch, device="cuda")
    ws = torch.empty(max(pool.prefill_workspace_bytes(len(ids), T, chunk), 256), dtype=torch.uint8,
                     device="cuda")
    pool.prefill(0, dev(cu, torch.int32), dev(ids, torch.int32), T, chunk, td["q"], td["k"], td["v"],
                 td["a"], td["b"], w, out, ws)
    torch.cuda.synchronize()
    return out


PREFILL_EDGE = syn.Shapes(2, 4, 128, 128, 4)


def test_prefill_b0_is_pure_decay():
    """b = 0 in the chunked prefill, from non-zero states: S_T = (prod a) S_0
    per value head and o_t = (prod_{s<=t} a_s) S_0 q^_t (closed form), and
    the oracle."""
    s, io, chunk = PREFILL_EDGE, "bf16", 64
    rng = np.random.default_rng(930)
    lens = np.array([200, 64, 1, 130])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ids = np.array([3, 0, 2, 5], np.int32)
    w_np = syn.draw_conv_weights(rng, s)
    tok = syn.draw_tokens(rng, s, (int(cu[-1]),), io)
    tok["b"][:] = 0.0
    contents = syn.draw_pool_contents(931, ids, s, io)
    say("prefill b=0 (pure decay)")
    pool = make_pool(s, 6, io)
    load_slots(pool, contents)
    out = _prefill(pool, cu, ids, tok, dev(w_np), chunk, io)
    assert pool.error() == 0
    op = oracle_pool(s, contents, ids, form="rank1")
    ref = op.prefill(0, cu, np.arange(len(ids)), tok["q"], tok["k"], tok["v"], tok["a"], tok["b"], w_np)
    check_out("outputs vs oracle", host(out), ref, io)
    closed_o = np.zeros_like(ref)
    closed_S = np.zeros((len(ids), s.h_v, s.d_v, s.d_k))
    for j, sl in enumerate(ids):
        S0 = contents[int(sl)][0][0].astype(np.float64)
        X = contents[int(sl)][1][0].astype(np.float64)
        decay = np.ones(s.h_v)
        for t in range(cu[j], cu[j + 1]):
            q, _, _, X = O.front_end(X, tok["q"][t], tok["k"][t], tok["v"][t],
                                     np.asarray(w_np, np.float64), s, s.d_k ** -0.5, 1e-6)
            decay = decay * tok["a"][t].astype(np.float64)
            closed_o[t] = decay[:, None] * np.einsum("hij,hj->hi", S0, O.expand_groups(q, s.h_v))
        closed_S[j] = decay[:, None, None] * S0
    check_out("outputs vs closed form", host(out), closed_o, io)
    check_f32("states vs closed form", host(pool.state[torch.from_numpy(ids.astype(np.int64)).cuda()])[:, 0],
              closed_S)


def test_prefill_b1_a1_stores_last_v_at_last_k():
    """b = 1, a = 1, eps = 1e-30 in the chunked prefill: after each sequence
    the state maps its last k^ to its last v^ (to the chunked form's
    precision), and outputs and states match the oracle."""
    s, io, chunk, eps = PREFILL_EDGE, "bf16", 64, 1e-30
    rng = np.random.default_rng(940)
    lens = np.array([300, 64, 2, 77])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ids = np.array([1, 4, 0, 2], np.int32)
    w_np = syn.draw_conv_weights(rng, s)
    tok = syn.draw_tokens(rng, s, (int(cu[-1]),), io)
    tok["a"][:] = 1.0
    tok["b"][:] = 1.0
    contents = syn.draw_pool_contents(941, ids, s, io)
    say("prefill b=1 a=1")
    pool = make_pool(s, 6, io, eps=eps)
    load_slots(pool, contents)
    out = _prefill(pool, cu, ids, tok, dev(w_np), chunk, io)
    assert pool.error() == 0
    op = oracle_pool(s, contents, ids, form="rank1", eps=eps)
    ref = op.prefill(0, cu, np.arange(len(ids)), tok["q"], tok["k"], tok["v"], tok["a"], tok["b"], w_np)
    check_out("outputs vs oracle", host(out), ref, io)
    got = host(pool.state[torch.from_numpy(ids.astype(np.int64)).cuda()])[:, 0]
    check_f32("states vs oracle", got, op.S[:, 0])
    worst = 0.0
    for j, sl in enumerate(ids):
        t = cu[j + 1] - 1
        k_hat, v_hat = _front_end(s, op_window_before(contents[int(sl)][1][0], tok, cu[j], t, s),
                                  {m: tok[m][t] for m in "qkv"}, w_np, eps)
        Sk = np.einsum("hij,hj->hi", got[j], k_hat)
        worst = max(worst, float(np.abs(Sk - v_hat).max() / np.sqrt(np.mean(v_hat ** 2))))
    say(f"  max |S k^_T - v^_T| / rms(v^_T) = {worst:.3e}")
    assert worst <= 2e-3


def op_window_before(window0, tok, t0, t, s):
    """Raw conv window in front of token t of a sequence starting at t0 with
    window0 (the last conv_k-1 raw inputs before t)."""
    rows = [np.concatenate([tok["q"][u].ravel(), tok["k"][u].ravel(), tok["v"][u].ravel()])
            for u in range(t0, t)]
    X = np.concatenate([np.asarray(window0, np.float64)] + [np.asarray(r, np.float64)[None] for r in rows])
    return X[-(s.conv_k - 1):]


def _vanishing_a(tok, rng):
    """a in {1e-30, 1e-45} on a sprinkling of tokens (the rest keep their
    draws), and a = 1 on another sprinkling."""
    a = tok["a"]
    u = rng.random(a.shape)
    a[u < 0.04] = np.float32(1e-30)
    a[(u >= 0.04) & (u < 0.08)] = np.float32(1e-45)
    a[(u >= 0.08) & (u < 0.20)] = 1.0


@pytest.mark.parametrize("chunk,io", [(64, "bf16"), (16, "f32")])
def test_prefill_vanishing_decay_vs_oracle(chunk, io):
    """Decays of 1e-30 and 1e-45 (below the clamp of log a at -87) and of 1
    inside chunks, continuing slots: the chunked prefill forgets like the
    oracle's token loop."""
    s = PREFILL_EDGE
    rng = np.random.default_rng(950 + chunk)
    lens = np.array([257, 64, 5, 190])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ids = np.array([2, 0, 5, 1], np.int32)
    w_np = syn.draw_conv_weights(rng, s)
    tok = syn.draw_tokens(rng, s, (int(cu[-1]),), io)
    _vanishing_a(tok, rng)
    contents = syn.draw_pool_contents(951, ids, s, io)
    say(f"prefill vanishing decay, chunk {chunk}, {io}")
    pool = make_pool(s, 6, io)
    load_slots(pool, contents)
    out = _prefill(pool, cu, ids, tok, dev(w_np), chunk, io)
    assert pool.error() == 0
    op = oracle_pool(s, contents, ids, form="rank1")
    ref = op.prefill(0, cu, np.arange(len(ids)), tok["q"], tok["k"], tok["v"], tok["a"], tok["b"], w_np)
    check_out("outputs", host(out), ref, io)
    check_f32("states", host(pool.state[torch.from_numpy(ids.astype(np.int64)).cuda()]), op.S)


def test_decode_and_verify_vanishing_decay_vs_oracle():
    """The same gates at decode (one token) and verify (4 tokens, commit 1..4)."""
    s, io, n, n_tok = QN, "bf16", 8, 4
    rng = np.random.default_rng(960)
    w_np = syn.draw_conv_weights(rng, s)
    ids = rng.permutation(32)[:n].astype(np.int32)
    contents = syn.draw_pool_contents(961, ids, s, io)
    pool = make_pool(s, 32, io)
    load_slots(pool, contents)
    op = oracle_pool(s, contents, ids, form="rank1")
    w = dev(w_np)
    did = dev(ids, torch.int32)
    say("decode/verify vanishing decay")
    d1 = syn.draw_tokens(rng, s, (n,), io)
    _vanishing_a(d1, rng)
    d1["a"][0] = np.float32(1e-45)      # whole entries that forget
    d1["a"][1] = np.float32(1e-30)
    o = torch.empty((n, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda")
    t1 = tokens_to_dev(d1, io)
    pool.decode(0, did, t1["q"], t1["k"], t1["v"], t1["a"], t1["b"], w, o)
    r1 = op.decode(0, np.arange(n), d1["q"], d1["k"], d1["v"], d1["a"], d1["b"], w_np)
    check_out("decode outputs", host(o), r1, io)
    v4 = syn.draw_tokens(rng, s, (n, n_tok), io)
    _vanishing_a(v4, rng)
    acc = rng.integers(1, n_tok + 1, size=n).astype(np.int32)
    ov = torch.empty((n, n_tok, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda")
    t4 = tokens_to_dev(v4, io)
    pool.verify(0, did, n_tok, t4["q"], t4["k"], t4["v"], t4["a"], t4["b"], w, dev(acc, torch.int32), ov)
    r4 = op.verify(0, np.arange(n), n_tok, v4["q"], v4["k"], v4["v"], v4["a"], v4["b"], w_np, acc)
    torch.cuda.synchronize()
    assert pool.error() == 0
    check_out("verify outputs", host(ov), r4, io)
    check_f32("states", host(pool.state[torch.from_numpy(ids.astype(np.int64)).cuda()]), op.S)
