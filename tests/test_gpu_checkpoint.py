"""GPU parity: slot copy and prefill state checkpoints (prefix caching: a
cache hit is only possible where a state checkpoint was stored, and a state
is copied whole), against the fp64 oracle."""
from __future__ import annotations

import numpy as np
import pytest

import gdn_synth as syn
from gpu_util import (check_f32, check_out, check_state, dev, host, load_slots, make_pool, oracle_pool,
                      say, scramble_pool, tokens_to_dev)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_state_layer_amd import binding
    binding.load_library()


def _i32(x):
    return dev(np.asarray(x, np.int32), torch.int32)


def test_slot_copy_is_bitwise_and_touches_only_destinations():
    s, io = syn.Shapes(2, 4, 64, 64, 4), "bf16"
    say("slot copy")
    pool = make_pool(s, 9, io, n_layers=2)
    scramble_pool(pool, 5)
    st0, wn0 = pool.state.clone(), pool.window.clone()
    pool.copy(_i32([3, 5, -1, 2]), _i32([0, 7, 4, -1]))
    torch.cuda.synchronize()
    assert pool.error() == 0
    assert torch.equal(pool.state[0], st0[3]) and torch.equal(pool.window[0], wn0[3])
    assert torch.equal(pool.state[7], st0[5]) and torch.equal(pool.window[7], wn0[5])
    keep = [1, 2, 3, 4, 5, 6, 8]
    assert torch.equal(pool.state[keep], st0[keep]) and torch.equal(pool.window[keep], wn0[keep])
    # out of range: flagged, nothing written
    pool.copy(_i32([1]), _i32([9]))
    torch.cuda.synchronize()
    assert pool.error() == 1
    assert torch.equal(pool.state[keep], st0[keep])


def _oracle_checkpoints(s, contents, ids_np, cu, tok, w, every):
    """Oracle slot contents after every `every` tokens of each sequence:
    {(j, m): (state, window)} for checkpoint m of sequence j, plus the
    per-token outputs and the final oracle pool."""
    op = oracle_pool(s, contents, ids_np)
    T = int(cu[-1])
    out = np.full((T, s.h_v, s.d_v), np.nan)
    snaps = {}
    for j in range(len(ids_np)):
        s0, s1 = int(cu[j]), int(cu[j + 1])
        m = 0
        for p0 in range(s0, s1, every):
            p1 = min(p0 + every, s1)
            part = {n: tok[n][p0:p1] for n in tok}
            seg = op.prefill(0, [0, p1 - p0], [j], part["q"], part["k"], part["v"], part["a"],
                             part["b"], w)
            out[p0:p1] = seg
            if p1 - p0 == every:
                snaps[(j, m)] = (op.S[j].copy(), op.X[j].copy())
                m += 1
    return out, snaps, op


@pytest.mark.parametrize("h_k,h_v,d,chunk,every,io", [(1, 2, 64, 64, 128, "bf16"),
                                                      (1, 2, 32, 16, 48, "f32"),
                                                      (16, 32, 32, 16, 160, "f32")])
def test_prefill_checkpoints_vs_oracle(h_k, h_v, d, chunk, every, io):
    """Two sequences (one continuing from a non-zero slot), checkpoints every
    `every` tokens into listed slots: each checkpoint slot holds the state
    and window after that many tokens; a checkpoint row past the sequence's
    end and a negative checkpoint slot leave their slots untouched.  The last
    case has more than 512 (chunk, q/k head) work items, so the factor stages
    q and k in two passes."""
    s = syn.Shapes(h_k, h_v, d, d, 4)
    say(f"checkpoints: {s} chunk={chunk} every={every} io={io}")
    rng = np.random.default_rng(500 + d)
    lens = [4 * every + 8, 2 * every + every // 2]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    tok = syn.draw_tokens(rng, s, (T,), io)
    w = syn.draw_conv_weights(rng, s)
    ids_np = np.array([1, 6], np.int32)
    # seq 0: rows for checkpoints 0..3 (slots 2, 3, -1, 4); seq 1: rows 0..2 (5, 7, 8), the
    # third beyond its length
    off_np = np.array([0, 4, 7], np.int32)
    ck_np = np.array([2, 3, -1, 4, 5, 7, 8], np.int32)
    pool = make_pool(s, 10, io)
    scramble_pool(pool, 8)
    contents = syn.draw_pool_contents(12, np.array([6]), s, io)   # slot 6 continues
    load_slots(pool, contents)
    pool.reset(_i32([1]))
    st0, wn0 = pool.state.clone(), pool.window.clone()
    td = tokens_to_dev(tok, io)
    out = torch.full((T, s.h_v, s.d_v), float("nan"), dtype=td["v"].dtype, device="cuda")
    ws = torch.empty(pool.prefill_workspace_bytes(2, T, chunk), dtype=torch.uint8, device="cuda")
    pool.prefill_ckpt(0, _i32(cu), _i32(ids_np), T, chunk, td["q"], td["k"], td["v"], td["a"],
                      td["b"], dev(w), out, every, _i32(off_np), _i32(ck_np), ws)
    torch.cuda.synchronize()
    assert pool.error() == 0
    ref, snaps, op = _oracle_checkpoints(s, {6: contents[6]}, ids_np, cu, tok, w, every)
    check_out("outputs", host(out), ref, io)
    check_f32("final states", host(pool.state[ids_np.astype(np.int64)]), op.S)
    where = {(0, 0): 2, (0, 1): 3, (0, 3): 4, (1, 0): 5, (1, 1): 7}
    assert set(snaps) == {(0, 0), (0, 1), (0, 2), (0, 3), (1, 0), (1, 1)}
    for key, slot in where.items():
        st, wn = snaps[key]
        check_f32(f"checkpoint {key} state", host(pool.state[slot]), st)
        assert np.array_equal(host(pool.window[slot]), wn), f"checkpoint {key} window"
    for slot in (0, 8, 9):   # unused checkpoint row (8), never listed (0, 9)
        assert torch.equal(pool.state[slot], st0[slot]) and torch.equal(pool.window[slot], wn0[slot])


def test_resume_from_a_copied_checkpoint_matches_one_pass():
    """Prefix caching end to end: checkpoint a 640-token prefill at 256 and
    512 tokens, copy the 512-token checkpoint into a fresh slot, prefill the
    remaining 128 tokens there: outputs and final state match the one-pass
    prefill (within tolerance) and the oracle."""
    s, io, chunk, every = syn.QWEN3_NEXT, "bf16", 64, 256
    say("resume from checkpoint")
    rng = np.random.default_rng(77)
    T = 640
    tok = syn.draw_tokens(rng, s, (T,), io)
    w = dev(syn.draw_conv_weights(rng, s))
    td = tokens_to_dev(tok, io)
    pool = make_pool(s, 6, io)
    out = torch.empty((T, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(pool.prefill_workspace_bytes(1, T, chunk), dtype=torch.uint8, device="cuda")
    pool.prefill_ckpt(0, _i32([0, T]), _i32([0]), T, chunk, td["q"], td["k"], td["v"], td["a"],
                      td["b"], w, out, every, _i32([0, 2]), _i32([2, 3]), ws)
    pool.copy(_i32([3]), _i32([5]))
    rest = {n: td[n][512:].contiguous() for n in td}
    out2 = torch.empty((T - 512, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda")
    pool.prefill(0, _i32([0, T - 512]), _i32([5]), T - 512, chunk, rest["q"], rest["k"],
                 rest["v"], rest["a"], rest["b"], w, out2, ws)
    torch.cuda.synchronize()
    assert pool.error() == 0
    check_out("resumed outputs vs one pass", host(out2), host(out[512:]), io)
    check_f32("resumed state vs one pass", host(pool.state[5]), host(pool.state[0]))
    assert torch.equal(pool.window[5], pool.window[0])


def test_validate_mode_rejects_overlapping_checkpoint_slots():
    import gated_deltanet_state_layer_amd as G
    s, io = syn.Shapes(1, 2, 32, 32, 4), "f32"
    pool = make_pool(s, 6, io, flags=G.GDN_VALIDATE)
    scramble_pool(pool, 3)
    st0 = pool.state.clone()
    T = 64
    tok = tokens_to_dev(syn.draw_tokens(np.random.default_rng(1), s, (T,), io), io)
    w = dev(syn.draw_conv_weights(np.random.default_rng(2), s))
    out = torch.empty((T, s.h_v, s.d_v), device="cuda")
    ws = torch.empty(pool.prefill_workspace_bytes(1, T, 16), dtype=torch.uint8, device="cuda")
    args = (0, _i32([0, T]), _i32([1]), T, 16, tok["q"], tok["k"], tok["v"], tok["a"], tok["b"], w,
            out)
    for every, ck, status in ((32, [1], -3), (32, [2, 2], -3), (24, [2], -1), (32, [6], -3)):
        with pytest.raises(G.GdnError) as e:
            pool.prefill_ckpt(*args, every, _i32([0, len(ck)]), _i32(ck), ws)
        assert e.value.status == status
    # more checkpoint rows than any call can fill (64 / 32 + 1 = 3): rejected
    # before the row list is sized from the device value or read
    for last in (4, 1 << 30):
        with pytest.raises(G.GdnError) as e:
            pool.prefill_ckpt(*args, 32, _i32([0, last]), _i32([2]), ws)
        assert e.value.status == -3
    with pytest.raises(G.GdnError) as e:
        pool.copy(_i32([1, 2]), _i32([2, 3]))   # destination 2 is also a source
    assert e.value.status == -3
    torch.cuda.synchronize()
    assert torch.equal(pool.state, st0)


@pytest.mark.parametrize("i", range(20))
def test_prefill_checkpoints_random_configuration_vs_oracle(i):
    """20 seeded random configurations of prefill with checkpoints (q/k heads
    1-2, 1-4 value heads per group, d 32/64/128, chunk 16/32/64, interval of
    1-4 chunks, conv widths 2-8, bf16 and fp32 io, 1-5 sequences, fresh and
    continuing slots, checkpoint rows past a sequence's end and negative
    checkpoint slots), against the oracle: outputs, final states and
    windows, every stored checkpoint, and every slot nothing was written to."""
    rng = np.random.default_rng(9001 + 6007 * i)
    h_k = int(rng.integers(1, 3))
    d = int(rng.choice([32, 64, 128]))
    s = syn.Shapes(h_k, h_k * int(rng.choice([1, 2, 3, 4])), d, d, int(rng.choice([2, 3, 4, 4, 6, 8])))
    chunk = int(rng.choice([16, 32, 64]))
    every = chunk * int(rng.integers(1, 5))
    io = str(rng.choice(["bf16", "f32"]))
    n_seq = int(rng.integers(1, 6))
    lens = rng.integers(1, 5 * every + 1, n_seq)
    rows = [int(lens[j] // every + rng.integers(0, 2)) for j in range(n_seq)]   # maybe one past the end
    n_rows = sum(rows)
    n_slots = n_seq + n_rows + 2
    perm = rng.permutation(n_slots).astype(np.int32)
    ids_np = perm[:n_seq]
    ck_np = perm[n_seq:n_seq + n_rows].copy()
    ck_np[rng.random(n_rows) < 0.15] = -1
    off_np = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    say(f"checkpoint sweep {i}: {s} chunk={chunk} every={every} io={io} lens={lens.tolist()} "
        f"rows={rows}")
    tok = syn.draw_tokens(rng, s, (T,), io)
    w = syn.draw_conv_weights(rng, s)
    pool = make_pool(s, n_slots, io)
    scramble_pool(pool, int(rng.integers(1 << 30)))
    cont = [int(x) for x in ids_np if rng.random() < 0.4]
    contents = syn.draw_pool_contents(int(rng.integers(1 << 30)), np.array(cont, np.int64), s, io) \
        if cont else {}
    if contents:
        load_slots(pool, contents)
    fresh = [int(x) for x in ids_np if int(x) not in cont]
    if fresh:
        pool.reset(_i32(fresh))
    st0, wn0 = pool.state.clone(), pool.window.clone()
    td = tokens_to_dev(tok, io)
    out = torch.full((T, s.h_v, s.d_v), float("nan"), dtype=td["v"].dtype, device="cuda")
    ws = torch.empty(max(pool.prefill_workspace_bytes(n_seq, T, chunk), 256), dtype=torch.uint8,
                     device="cuda")
    pool.prefill_ckpt(0, _i32(cu), _i32(ids_np), T, chunk, td["q"], td["k"], td["v"], td["a"],
                      td["b"], dev(w), out, every, _i32(off_np), _i32(ck_np), ws)
    torch.cuda.synchronize()
    assert pool.error() == 0
    ref, snaps, op = _oracle_checkpoints(s, {k: contents[k] for k in cont}, ids_np, cu, tok, w, every)
    check_out("outputs", host(out), ref, io)
    written = set()
    for j, sl in enumerate(ids_np):
        check_state(f"final state of slot {sl}", host(pool.state[int(sl)]), op.S[j])
        assert np.array_equal(host(pool.window[int(sl)]), op.X[j]), f"final window of slot {sl}"
        written.add(int(sl))
        for m in range(rows[j]):
            ck = int(ck_np[off_np[j] + m])
            if ck < 0 or (j, m) not in snaps:   # a negative slot, or a row past the end
                continue
            st, wn = snaps[(j, m)]
            check_state(f"checkpoint {m} of sequence {j} (slot {ck})", host(pool.state[ck]), st)
            assert np.array_equal(host(pool.window[ck]), wn), f"checkpoint window {(j, m)}"
            written.add(ck)
    for sl in range(n_slots):
        if sl not in written:
            assert torch.equal(pool.state[sl], st0[sl]) and torch.equal(pool.window[sl], wn0[sl]), \
                f"slot {sl} changed"
