"""GPU parity of the verify ring (gdn_ring_verify / gdn_ring_commit /
gdn_ring_flush) against the fp64 oracle: draft outputs equal the oracle's
verify outputs on the slot's logical state, commits advance the logical
state by the accepted tokens, and after a flush the state tile is the
oracle's state.  Bookkeeping is checked bit for bit: ring counts, windows,
untouched slots, a verify that writes nothing, reset and copy."""
import numpy as np
import pytest

import gdn_synth as syn
from gpu_util import (check_f32, check_out, dev, host, load_slots, make_pool, oracle_pool, say,
                      scramble_pool, tokens_to_dev)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from oracle import gdn_oracle as O  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_state_layer_amd import binding
    binding.load_library()


def _ring_verify(pool, ids, n_tok, td, w):
    s = pool.desc
    out = torch.full((ids.numel(), n_tok, s.h_v, s.d_v), float("nan"), dtype=pool.io_torch,
                     device="cuda")
    pool.ring_verify(0, ids, n_tok, td["q"], td["k"], td["v"], td["a"], td["b"], w, out)
    return out


def _snapshot(pool):
    return (pool.state.clone(), pool.window.clone(), pool.ring_count.clone(),
            pool.ring_records.clone())


def _same(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


def _run_cycles(s, io, ring_len, n_tok, n_cycles, n_slots, ids_np, seed, acc_fn=None,
                tok_fn=None):
    """Verify -> compare with the oracle -> commit, n_cycles times, then flush.
    tok_fn(tok, rng), if given, edits each cycle's drawn tokens in place."""
    rng = np.random.default_rng(seed)
    n = len(ids_np)
    w_np = syn.draw_conv_weights(rng, s)
    w = dev(w_np)
    live = ids_np[ids_np >= 0]
    contents = syn.draw_pool_contents(seed + 1, live, s, io)
    pool = make_pool(s, n_slots, io, ring_len=ring_len)
    scramble_pool(pool, seed + 2)
    pool.ring_count.zero_()
    load_slots(pool, contents)
    order = np.where(ids_np >= 0, ids_np, live[0])       # oracle slot j <-> entry j
    op = oracle_pool(s, contents, order)
    ids = dev(ids_np, torch.int32)
    live_idx = torch.from_numpy(live.astype(np.int64)).cuda()
    mask = torch.ones(n_slots, dtype=torch.bool, device="cuda")
    mask[live_idx] = False
    untouched = [x[mask] for x in _snapshot(pool)]
    count = np.zeros(n, np.int64)
    ent = ids_np >= 0
    outs, refs = [], []
    folds = 0
    for cyc in range(n_cycles):
        tok = syn.draw_tokens(rng, s, (n, n_tok), io)
        if tok_fn is not None:
            tok_fn(tok, rng)
        td = tokens_to_dev(tok, io)
        acc = (acc_fn(rng, cyc, n) if acc_fn else rng.integers(0, n_tok + 1, size=n)).astype(np.int32)
        before = _snapshot(pool)
        out = _ring_verify(pool, ids, n_tok, td, w)
        torch.cuda.synchronize()
        assert _same(before, _snapshot(pool)), "ring_verify wrote to the pool"
        ref = op.verify(0, np.where(ent, np.arange(n), -1), n_tok, tok["q"], tok["k"], tok["v"],
                        tok["a"], tok["b"], w_np, np.zeros(n, np.int32))
        outs.append(host(out)[ent])
        refs.append(ref[ent])
        pool.ring_commit(0, ids, n_tok, td["q"], td["k"], td["v"], td["a"], td["b"], w,
                         dev(acc, torch.int32))
        op.verify(0, np.where(ent, np.arange(n), -1), n_tok, tok["q"], tok["k"], tok["v"],
                  tok["a"], tok["b"], w_np, acc)
        for i in range(n):
            if acc[i] > 0:
                if count[i] + acc[i] > ring_len:
                    count[i] = 0
                    folds += ent[i]
                else:
                    count[i] += acc[i]
        torch.cuda.synchronize()
        got = pool.ring_count[torch.from_numpy(ids_np[ent].astype(np.int64)).cuda(), 0].cpu().numpy()
        assert np.array_equal(got, count[ent]), f"cycle {cyc}: ring counts {got} != {count[ent]}"
        assert np.array_equal(host(pool.window[live_idx]), op.X[ent]), f"cycle {cyc}: windows"
    say(f"  {n_cycles} cycles, {folds} folds, final counts {count[ent].tolist()}")
    check_out("draft outputs (all cycles)", np.array(outs), np.array(refs), io)
    pool.ring_flush(0, ids)
    torch.cuda.synchronize()
    assert int(pool.ring_count[live_idx].abs().sum()) == 0, "flush left tokens in a ring"
    check_f32("states after flush", host(pool.state[live_idx]), op.S[ent])
    assert np.array_equal(host(pool.window[live_idx]), op.X[ent])
    assert _same(untouched, [x[mask] for x in _snapshot(pool)]), "an untouched slot changed"
    assert pool.error() == 0
    return folds


def _vanishing_decay(tok, rng):
    """a = 1e-30 or 1e-45 (below the kernels' clamp of log a at -87) on a
    fifth of the tokens, a = 1 on another fifth."""
    u = rng.random(tok["a"].shape)
    tok["a"][u < 0.1] = np.float32(1e-30)
    tok["a"][(u >= 0.1) & (u < 0.2)] = np.float32(1e-45)
    tok["a"][(u >= 0.2) & (u < 0.4)] = 1.0


@pytest.mark.parametrize("io,ring_len,n_tok", [("bf16", 8, 4), ("f32", 24, 8)])
def test_ring_cycles_vanishing_decay_vs_oracle(io, ring_len, n_tok):
    """Ring verify/commit/flush with decays that make the state forget
    (down to below the clamp) and with no decay, against the oracle."""
    s = syn.Shapes(2, 4, 128, 128, 4)
    say(f"ring cycles, vanishing decay: io={io} L={ring_len} n_tok={n_tok}")
    ids_np = np.array([2, 6, 0, 3], np.int32)
    folds = _run_cycles(s, io, ring_len, n_tok, 10, 8, ids_np, 700 + ring_len,
                        tok_fn=_vanishing_decay)
    assert folds > 0, "no cycle reached a fold"


@pytest.mark.parametrize("h_k,h_v,d,io,ring_len,n_tok", [
    (2, 2, 32, "f32", 4, 2),        # one token tile
    (2, 4, 64, "bf16", 8, 4),       # one token tile
    (2, 4, 128, "bf16", 24, 8),     # two token tiles (24 + 8 = 32)
    (1, 2, 32, "bf16", 16, 3),      # two token tiles, ragged
])
def test_ring_cycles_vs_oracle(h_k, h_v, d, io, ring_len, n_tok):
    s = syn.Shapes(h_k, h_v, d, d, 4)
    say(f"ring cycles: {s} io={io} L={ring_len} n_tok={n_tok}")
    ids_np = np.array([5, 1, -1, 6, 3], np.int32)
    folds = _run_cycles(s, io, ring_len, n_tok, 12, 8, ids_np, 300 + d + ring_len)
    assert folds > 0, "no cycle reached a fold"


def test_ring_cycles_qwen3_next_shapes():
    """Qwen3-Next shapes, ring of 8 (twice the 4-token speculation), accepted
    lengths uniform on 1..4 as in the verify workload."""
    s, io = syn.QWEN3_NEXT, "bf16"
    say(f"ring cycles: Qwen3-Next {s}")
    ids_np = np.array([9, 2, 14, 0, 7, 11], np.int32)
    folds = _run_cycles(s, io, 8, 4, 6, 16, ids_np, 410,
                        acc_fn=lambda rng, c, n: rng.integers(1, 5, size=n))
    assert folds > 0


@pytest.mark.parametrize("h_k,h_v,d,n,n_slots", [(8, 16, 64, 96, 128), (16, 32, 128, 32, 40)])
def test_ring_cycles_many_entries_vs_oracle(h_k, h_v, d, n, n_slots):
    """More (entry, value head) commit items than one round of workgroups
    (1536 and 1024), so the commit walks them persistently, folding entries
    first; a padding entry among them; ring of 8, accepted lengths uniform on
    1..4, against the oracle."""
    s, io = syn.Shapes(h_k, h_v, d, d, 4), "bf16"
    say(f"ring cycles, {n} entries: {s}")
    ids_np = np.random.default_rng(97 + n).permutation(n_slots)[:n].astype(np.int32)
    ids_np[5] = -1
    folds = _run_cycles(s, io, 8, 4, 6, n_slots, ids_np, 520 + n,
                        acc_fn=lambda rng, c, m: rng.integers(1, 5, size=m))
    assert folds > 0


def test_ring_conv_k_2_and_8():
    for K in (2, 8):
        s = syn.Shapes(2, 4, 64, 64, K)
        say(f"ring cycles: conv_k={K}")
        _run_cycles(s, "bf16", 6, 3, 8, 6, np.array([4, 0, 2], np.int32), 520 + K)


def test_flush_of_empty_ring_and_zero_acceptance_change_nothing():
    s, io = syn.Shapes(2, 4, 64, 64, 4), "bf16"
    rng = np.random.default_rng(600)
    pool = make_pool(s, 6, io, ring_len=8)
    scramble_pool(pool, 601)
    pool.ring_count.zero_()
    ids = dev(np.array([1, 4], np.int32), torch.int32)
    before = _snapshot(pool)
    pool.ring_flush(0, ids)
    tok = tokens_to_dev(syn.draw_tokens(rng, s, (2, 4), io), io)
    w = dev(syn.draw_conv_weights(rng, s))
    pool.ring_commit(0, ids, 4, tok["q"], tok["k"], tok["v"], tok["a"], tok["b"], w,
                     dev(np.zeros(2, np.int32), torch.int32))
    torch.cuda.synchronize()
    assert _same(before, _snapshot(pool))


def test_reset_empties_and_copy_carries_the_ring():
    """Copy a slot with a part-filled ring: both copies then verify and
    commit identically (bitwise); reset empties a ring and zeroes the slot."""
    s, io, n_tok = syn.Shapes(2, 4, 64, 64, 4), "bf16", 3
    say("ring reset / copy")
    rng = np.random.default_rng(700)
    w = dev(syn.draw_conv_weights(rng, s))
    pool = make_pool(s, 6, io, ring_len=10)
    load_slots(pool, syn.draw_pool_contents(701, [2], s, io))
    src = dev(np.array([2], np.int32), torch.int32)
    for _ in range(2):
        td = tokens_to_dev(syn.draw_tokens(rng, s, (1, n_tok), io), io)
        pool.ring_commit(0, src, n_tok, td["q"], td["k"], td["v"], td["a"], td["b"], w,
                         dev(np.array([2], np.int32), torch.int32))
    torch.cuda.synchronize()
    assert int(pool.ring_count[2, 0]) == 4
    pool.copy(src, dev(np.array([5], np.int32), torch.int32))
    torch.cuda.synchronize()
    assert int(pool.ring_count[5, 0]) == 4
    both = dev(np.array([2, 5], np.int32), torch.int32)
    tok = syn.draw_tokens(rng, s, (1, n_tok), io)
    tok2 = {k_: np.concatenate([v_, v_]) for k_, v_ in tok.items()}
    td = tokens_to_dev(tok2, io)
    out = _ring_verify(pool, both, n_tok, td, w)
    torch.cuda.synchronize()
    assert torch.equal(out[0], out[1])
    pool.ring_commit(0, both, n_tok, td["q"], td["k"], td["v"], td["a"], td["b"], w,
                     dev(np.array([3, 3], np.int32), torch.int32))
    pool.ring_flush(0, both)
    torch.cuda.synchronize()
    assert torch.equal(pool.state[2], pool.state[5]) and torch.equal(pool.window[2], pool.window[5])
    pool.reset(src)
    torch.cuda.synchronize()
    assert int(pool.ring_count[2, 0]) == 0
    assert int(pool.state[2].abs().sum()) == 0 and int(pool.window[2].float().abs().sum()) == 0
    assert pool.error() == 0


def test_one_call_path_requires_a_flushed_ring():
    """GDN_VALIDATE: decode, verify and prefill refuse a slot whose ring holds
    tokens (GDN_ERR_RING) without touching memory; after a flush they run.
    A pool without a ring refuses the ring calls."""
    import gated_deltanet_state_layer_amd as G
    s, io = syn.Shapes(2, 4, 64, 64, 4), "bf16"
    rng = np.random.default_rng(800)
    w = dev(syn.draw_conv_weights(rng, s))
    pool = make_pool(s, 4, io, flags=G.GDN_VALIDATE, ring_len=8)
    ids = dev(np.array([1], np.int32), torch.int32)
    td = tokens_to_dev(syn.draw_tokens(rng, s, (1, 2), io), io)
    pool.ring_commit(0, ids, 2, td["q"], td["k"], td["v"], td["a"], td["b"], w,
                     dev(np.array([2], np.int32), torch.int32))
    torch.cuda.synchronize()
    snap = _snapshot(pool)
    d1 = tokens_to_dev(syn.draw_tokens(rng, s, (1,), io), io)
    out = torch.zeros((1, s.h_v, s.d_v), dtype=pool.io_torch, device="cuda")
    with pytest.raises(G.GdnError) as ei:
        pool.decode(0, ids, d1["q"], d1["k"], d1["v"], d1["a"], d1["b"], w, out)
    assert ei.value.status == -6
    cu = dev(np.array([0, 1], np.int32), torch.int32)
    with pytest.raises(G.GdnError) as ei:
        pool.prefill(0, cu, ids, 1, 16, d1["q"], d1["k"], d1["v"], d1["a"], d1["b"], w, out,
                     torch.empty(pool.prefill_workspace_bytes(1, 1, 16), dtype=torch.uint8,
                                 device="cuda"))
    assert ei.value.status == -6
    torch.cuda.synchronize()
    assert _same(snap, _snapshot(pool))
    pool.ring_flush(0, ids)
    pool.decode(0, ids, d1["q"], d1["k"], d1["v"], d1["a"], d1["b"], w, out)
    torch.cuda.synchronize()
    assert pool.error() == 0
    plain = make_pool(s, 4, io)
    with pytest.raises(G.GdnError) as ei:
        plain.ring_flush(0, ids)
    assert ei.value.status == -2


def test_ring_layers_are_independent_and_accept_len_is_clamped():
    """Two layers: ring calls on layer 1 leave layer 0 bitwise unchanged, ring
    counts are per layer, and accept_len outside 0..n_tok is clamped (9 acts
    as n_tok, -3 as 0), as the oracle's verify clamps nothing but is given
    the clamped values."""
    s, io, n_tok = syn.Shapes(2, 4, 64, 64, 4), "bf16", 3
    say("ring: two layers, clamped accept_len")
    rng = np.random.default_rng(900)
    n_slots, ids_np = 6, np.array([4, 1], np.int32)
    contents = syn.draw_pool_contents(901, ids_np, s, io, n_layers=2)
    pool = make_pool(s, n_slots, io, n_layers=2, ring_len=8)
    load_slots(pool, contents)
    l0 = (pool.state[:, 0].clone(), pool.window[:, 0].clone(), pool.ring_count[:, 0].clone())
    w_np = syn.draw_conv_weights(rng, s)
    w = dev(w_np)
    ids = dev(ids_np, torch.int32)
    op = O.OraclePool(2, 1, s)
    for j, sl in enumerate(ids_np):
        op.S[j, 0], op.X[j, 0] = contents[int(sl)][0][1], contents[int(sl)][1][1]
    outs, refs = [], []
    for acc_raw in ([9, -3], [2, 9], [1, 1]):
        tok = syn.draw_tokens(rng, s, (2, n_tok), io)
        td = tokens_to_dev(tok, io)
        out = torch.full((2, n_tok, s.h_v, s.d_v), float("nan"), dtype=pool.io_torch, device="cuda")
        pool.ring_verify(1, ids, n_tok, td["q"], td["k"], td["v"], td["a"], td["b"], w, out)
        refs.append(op.verify(0, np.arange(2), n_tok, tok["q"], tok["k"], tok["v"], tok["a"],
                              tok["b"], w_np, np.zeros(2, np.int32)))
        outs.append(host(out))
        pool.ring_commit(1, ids, n_tok, td["q"], td["k"], td["v"], td["a"], td["b"], w,
                         dev(np.array(acc_raw, np.int32), torch.int32))
        op.verify(0, np.arange(2), n_tok, tok["q"], tok["k"], tok["v"], tok["a"], tok["b"], w_np,
                  np.clip(np.array(acc_raw), 0, n_tok).astype(np.int32))
    torch.cuda.synchronize()
    # counts: 3 then 0 (slot 4: 3, then 3+2=5, then 6); slot 1: 0, then 3, then 4
    assert pool.ring_count[4, 1].item() == 6 and pool.ring_count[1, 1].item() == 4
    assert torch.equal(pool.ring_count[:, 0], l0[2]), "layer 0 ring counts changed"
    check_out("draft outputs", np.array(outs), np.array(refs), io)
    pool.ring_flush(1, ids)
    torch.cuda.synchronize()
    idx = torch.from_numpy(ids_np.astype(np.int64)).cuda()
    check_f32("layer-1 states after flush", host(pool.state[idx, 1]), op.S[:, 0])
    assert np.array_equal(host(pool.window[idx, 1]), op.X[:, 0])
    assert torch.equal(pool.state[:, 0], l0[0]) and torch.equal(pool.window[:, 0], l0[1]), \
        "layer 0 changed"
    assert pool.error() == 0


@pytest.mark.parametrize("i", range(30))
def test_ring_cycles_random_configuration_vs_oracle(i):
    """Verify -> commit cycles then a flush on 30 seeded random
    configurations (q/k heads 1-2, 1-4 value heads per group, d 32/64/128,
    conv widths 2-8, bf16 and fp32 io, rings of 1-24 tokens, 1-8 drafts,
    accepted lengths 0..n_tok, up to 40 entries with padding), against the
    oracle: every cycle's draft outputs, ring counts and windows, the states
    after the flush, and every slot the calls do not name."""
    rng = np.random.default_rng(4242 + 65537 * i)
    h_k = int(rng.integers(1, 3))
    h_v = h_k * int(rng.choice([1, 2, 3, 4]))
    d = int(rng.choice([32, 64, 128]))
    s = syn.Shapes(h_k, h_v, d, d, int(rng.choice([2, 3, 4, 4, 6, 8])))
    io = str(rng.choice(["bf16", "f32"]))
    n_tok = int(rng.integers(1, 9))
    ring_len = int(rng.integers(1, 25))
    n = int(rng.choice([1, 3, 8, 17, 40]))
    n_slots = n + int(rng.integers(1, 9))
    ids_np = rng.permutation(n_slots)[:n].astype(np.int32)
    if n > 1:
        ids_np[rng.random(n) < 0.1] = -1
    if (ids_np < 0).all():
        ids_np[0] = n_slots - 1 if n_slots - 1 not in ids_np else 0
    say(f"ring sweep {i}: {s} io={io} L={ring_len} n_tok={n_tok} entries={n} of {n_slots}")
    _run_cycles(s, io, ring_len, n_tok, int(rng.integers(4, 9)), n_slots, ids_np,
                int(rng.integers(1 << 20)))
