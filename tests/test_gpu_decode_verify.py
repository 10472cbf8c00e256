"""GPU parity: multi-slot decode and speculative verify through the C ABI,
element by element against the fp64 oracle on the same seeded inputs, plus
the bitwise bookkeeping guarantees (untouched slots, windows, reset, batch
invariance, verify == sequential decode)."""
import numpy as np
import pytest

import gated_deltanet_state_layer_amd as G
import gdn_synth as syn
from gpu_util import (check_f32, check_out, dev, host, load_slots, make_pool, oracle_pool, say,
                      scramble_pool, tokens_to_dev)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_state_layer_amd import binding
    binding.load_library()


def _decode(pool, layer, ids, td, w, io):
    n = ids.numel()
    s = pool.desc
    out = torch.full((n, s.h_v, s.d_v), float("nan"), dtype=pool.io_torch, device="cuda")
    pool.decode(layer, ids, td["q"], td["k"], td["v"], td["a"], td["b"], w, out)
    return out


@pytest.mark.parametrize("n_active", [1, 4, 16, 64, 256])
def test_decode_qwen3_next_shapes_vs_oracle(n_active):
    """N of 256 slots (256: every slot of the pool, the largest batch a pool
    of that size takes); the oracle uses the literal matrix form up to 64
    slots and the equal rank-1 form beyond, to stay within seconds."""
    case = syn.decode_case(n_active)
    s, io = case["shapes"], case["io"]
    say(f"decode: N={n_active} of {case['n_slots']} slots, {s}")
    pool = make_pool(s, case["n_slots"], io)
    scramble_pool(pool, 7 + n_active)
    ids_np = case["slot_ids"]
    contents = syn.draw_pool_contents(case["pool_seed"], ids_np, s, io)
    load_slots(pool, contents)
    st0, wn0 = pool.state.clone(), pool.window.clone()
    td = tokens_to_dev(case["tokens"], io)
    w = dev(case["conv_w"])
    ids = dev(ids_np, torch.int32)
    out = _decode(pool, 0, ids, td, w, io)
    torch.cuda.synchronize()
    assert pool.error() == 0

    op = oracle_pool(s, contents, ids_np, form="matrix" if n_active <= 64 else "rank1")
    tok = case["tokens"]
    ref = op.decode(0, np.arange(n_active), tok["q"], tok["k"], tok["v"], tok["a"], tok["b"],
                    case["conv_w"])
    check_out("outputs", host(out), ref, io)
    idx = torch.from_numpy(ids_np.astype(np.int64)).cuda()
    check_f32("final states", host(pool.state[idx]), op.S)
    assert np.array_equal(host(pool.window[idx]), op.X), "windows are not the raw inputs"
    mask = torch.ones(case["n_slots"], dtype=torch.bool, device="cuda")
    mask[idx] = False
    assert torch.equal(pool.state[mask], st0[mask]), "an untouched slot's state changed"
    assert torch.equal(pool.window[mask], wn0[mask]), "an untouched slot's window changed"


@pytest.mark.parametrize("h_k,h_v,d,io", [(2, 2, 32, "f32"), (2, 8, 64, "bf16"),
                                          (1, 1, 128, "f32"), (3, 6, 128, "bf16")])
def test_decode_many_steps_other_shapes(h_k, h_v, d, io):
    """Token-by-token decode from zero state over 40 steps on several shapes."""
    s = syn.Shapes(h_k, h_v, d, d, 4)
    say(f"decode steps: {s} io={io}")
    rng = np.random.default_rng(17 + d + h_v)
    w = syn.draw_conv_weights(rng, s)
    n_slots, ids_np = 5, np.array([3, 0], dtype=np.int32)
    T = 40
    tok = syn.draw_tokens(rng, s, (T, 2), io)
    pool = make_pool(s, n_slots, io)
    op = oracle_pool(s, None, ids_np)
    ids, wd = dev(ids_np, torch.int32), dev(w)
    outs, refs = [], []
    for t in range(T):
        tt = {n: tok[n][t] for n in tok}
        outs.append(host(_decode(pool, 0, ids, tokens_to_dev(tt, io), wd, io)))
        refs.append(op.decode(0, [0, 1], tt["q"], tt["k"], tt["v"], tt["a"], tt["b"], w))
    check_out("outputs", np.array(outs), np.array(refs), io)
    check_f32("final states", host(pool.state[ids.long()]), op.S)
    assert not host(pool.state[[1, 2, 4]]).any()


def test_batched_decode_is_bitwise_batch_invariant():
    case = syn.decode_case(16, seed=2001)
    s, io = case["shapes"], case["io"]
    say("batch invariance, 16 slots")
    ids_np = case["slot_ids"]
    contents = syn.draw_pool_contents(case["pool_seed"], ids_np, s, io)
    td = tokens_to_dev(case["tokens"], io)
    w = dev(case["conv_w"])
    pa = make_pool(s, case["n_slots"], io)
    load_slots(pa, contents)
    pb = make_pool(s, case["n_slots"], io)
    load_slots(pb, contents)
    out_a = _decode(pa, 0, dev(ids_np, torch.int32), td, w, io)
    outs_b = []
    for i in range(len(ids_np)):
        one = {n: td[n][i:i + 1] for n in td}
        outs_b.append(_decode(pb, 0, dev(ids_np[i:i + 1], torch.int32), one, w, io))
    torch.cuda.synchronize()
    assert torch.equal(out_a, torch.cat(outs_b))
    assert torch.equal(pa.state, pb.state) and torch.equal(pa.window, pb.window)


@pytest.mark.parametrize("h_k,h_v,d,io,n", [(16, 32, 128, "bf16", 1), (16, 32, 128, "bf16", 4),
                                            (16, 32, 128, "f32", 16), (4, 4, 128, "f32", 1),
                                            (2, 4, 64, "bf16", 3)])
def test_row_split_decode_is_bitwise_one_workgroup_decode(h_k, h_v, d, io, n):
    """Few entries: decode spreads each head's rows over several workgroups
    (the q/k window rolled by the last of them).  Three consecutive steps,
    with a padding entry, equal the one-workgroup-per-group kernel (a pool
    with GDN_GROUP_KERNEL; verify with one token, accept_len 1) bitwise, and
    every roll counter is back to zero."""
    s = syn.Shapes(h_k, h_v, d, d, 4)
    say(f"row-split decode: {s} io={io} n={n}")
    rng = np.random.default_rng(300 + n + d)
    n_slots = 3 * n + 2
    ids_np = rng.permutation(n_slots)[:n].astype(np.int32)
    ids_pad = np.concatenate([ids_np, [-1]]).astype(np.int32)
    w = dev(syn.draw_conv_weights(rng, s))
    contents = syn.draw_pool_contents(55, ids_np, s, io)
    pa = make_pool(s, n_slots, io)
    load_slots(pa, contents)
    pb = make_pool(s, n_slots, io, flags=G.GDN_GROUP_KERNEL)
    load_slots(pb, contents)
    ids = dev(ids_pad, torch.int32)
    one = dev(np.ones(n + 1, np.int32), torch.int32)
    for step in range(3):
        tok = syn.draw_tokens(rng, s, (n + 1,), io)
        td = tokens_to_dev(tok, io)
        oa = _decode(pa, 0, ids, td, w, io)
        tv = tokens_to_dev({m: tok[m][:, None] for m in tok}, io)
        ob = _verify(pb, 0, ids, 1, tv, w, one)[:, 0]
        torch.cuda.synchronize()
        assert torch.equal(oa[:n], ob[:n]), f"step {step}: outputs differ"
        assert torch.isnan(oa[n].float()).all(), "padding entry's output was written"
    assert torch.equal(pa.state, pb.state) and torch.equal(pa.window, pb.window)
    assert pa.error() == 0
    win_bytes = pa.window.numel() * pa.window.element_size()
    off = (win_bytes + 255) // 256 * 256 + 256
    ctr = pa._aux_buf[off:off + n_slots * h_k * 4].view(torch.int32)
    assert not ctr.any(), "a roll counter is not back to zero"


@pytest.mark.parametrize("h_k,h_v,d,io,n", [(16, 32, 128, "bf16", 64), (16, 32, 128, "f32", 40),
                                            (4, 16, 64, "bf16", 48), (3, 6, 128, "bf16", 130)])
def test_head_split_decode_and_verify_are_bitwise_group_kernel(h_k, h_v, d, io, n):
    """Batches beyond the row split run one value head per workgroup (the
    q/k window rolled by the last of a group's workgroups).  Decode steps,
    verify of 2, 4 and 8 tokens with mixed acceptance (0 and n_tok
    included), and a commit-only verify (no outputs) equal the
    one-workgroup-per-group kernel bitwise; every roll counter ends at zero."""
    s = syn.Shapes(h_k, h_v, d, d, 4)
    say(f"head-split decode/verify: {s} io={io} n={n}")
    rng = np.random.default_rng(500 + n + d)
    n_slots = n + 9
    ids_np = rng.permutation(n_slots)[:n].astype(np.int32)
    ids_pad = np.concatenate([ids_np[:n // 2], [-1], ids_np[n // 2:]]).astype(np.int32)
    w = dev(syn.draw_conv_weights(rng, s))
    contents = syn.draw_pool_contents(66, ids_np, s, io)
    pa = make_pool(s, n_slots, io)
    pb = make_pool(s, n_slots, io, flags=G.GDN_GROUP_KERNEL)
    for p in (pa, pb):
        scramble_pool(p, 3)
        load_slots(p, contents)
    ids = dev(ids_pad, torch.int32)
    m = len(ids_pad)
    for step in range(2):
        td = tokens_to_dev(syn.draw_tokens(rng, s, (m,), io), io)
        oa, ob = _decode(pa, 0, ids, td, w, io), _decode(pb, 0, ids, td, w, io)
        torch.cuda.synchronize()
        assert torch.equal(torch.nan_to_num(oa, nan=7.0), torch.nan_to_num(ob, nan=7.0)), \
            f"decode {step}"
        assert torch.isnan(oa[n // 2].float()).all(), "padding entry's output was written"
    for n_tok in (2, 4, 8):
        td = tokens_to_dev(syn.draw_tokens(rng, s, (m, n_tok), io), io)
        acc = dev((np.arange(m) * 3 % (n_tok + 1)).astype(np.int32), torch.int32)
        oa, ob = _verify(pa, 0, ids, n_tok, td, w, acc), _verify(pb, 0, ids, n_tok, td, w, acc)
        torch.cuda.synchronize()
        assert torch.equal(torch.nan_to_num(oa, nan=7.0), torch.nan_to_num(ob, nan=7.0)), \
            f"verify n_tok={n_tok}"
        assert torch.equal(pa.state, pb.state) and torch.equal(pa.window, pb.window), \
            f"verify n_tok={n_tok}: slots differ"
    td = tokens_to_dev(syn.draw_tokens(rng, s, (m, 4), io), io)
    acc = dev((np.arange(m) % 5).astype(np.int32), torch.int32)
    for p in (pa, pb):
        p.verify(0, ids, 4, td["q"], td["k"], td["v"], td["a"], td["b"], w, acc, None)
    torch.cuda.synchronize()
    assert torch.equal(pa.state, pb.state) and torch.equal(pa.window, pb.window), "commit-only"
    assert pa.error() == 0 and pb.error() == 0
    win_bytes = pa.window.numel() * pa.window.element_size()
    off = (win_bytes + 255) // 256 * 256 + 256
    ctr = pa._aux_buf[off:off + n_slots * h_k * 4].view(torch.int32)
    assert not ctr.any(), "a roll counter is not back to zero"


def test_padding_and_out_of_range_ids():
    s, io = syn.Shapes(2, 4, 64, 64, 4), "bf16"
    say("padding / out-of-range ids")
    rng = np.random.default_rng(5)
    w = dev(syn.draw_conv_weights(rng, s))
    pool = make_pool(s, 6, io)
    scramble_pool(pool, 3)
    st0, wn0 = pool.state.clone(), pool.window.clone()
    ids_np = np.array([-1, 2, 6, 4], dtype=np.int32)   # 6 is out of range
    tok = syn.draw_tokens(rng, s, (4,), io)
    out = _decode(pool, 0, dev(ids_np, torch.int32), tokens_to_dev(tok, io), w, io)
    assert pool.error() == 1
    assert pool.error() == 0   # cleared by the read
    assert torch.isnan(out[0]).all() and torch.isnan(out[2]).all()
    assert not torch.isnan(out[1]).any() and not torch.isnan(out[3]).any()
    keep = [0, 1, 3, 5]
    assert torch.equal(pool.state[keep], st0[keep]) and torch.equal(pool.window[keep], wn0[keep])


def test_validate_mode_rejects_bad_ids_without_touching_memory():
    import gated_deltanet_state_layer_amd as G
    s, io = syn.Shapes(2, 4, 64, 64, 4), "bf16"
    say("validate mode")
    rng = np.random.default_rng(6)
    w = dev(syn.draw_conv_weights(rng, s))
    pool = make_pool(s, 6, io, flags=G.GDN_VALIDATE)
    scramble_pool(pool, 4)
    st0 = pool.state.clone()
    tok = tokens_to_dev(syn.draw_tokens(rng, s, (3,), io), io)
    for bad in ([1, 1, 2], [0, 9, 2]):
        with pytest.raises(G.GdnError) as ei:
            _decode(pool, 0, dev(np.array(bad, np.int32), torch.int32), tok, w, io)
        assert ei.value.status == -3
        with pytest.raises(G.GdnError):
            pool.reset(dev(np.array(bad, np.int32), torch.int32))
    torch.cuda.synchronize()
    assert torch.equal(pool.state, st0)


def test_reset_zeroes_listed_slots_only():
    s, io = syn.Shapes(2, 4, 64, 64, 4), "bf16"
    say("reset")
    pool = make_pool(s, 7, io, n_layers=2)
    scramble_pool(pool, 5)
    st0, wn0 = pool.state.clone(), pool.window.clone()
    pool.reset(dev(np.array([5, -1, 1], np.int32), torch.int32))
    torch.cuda.synchronize()
    assert not pool.state[[1, 5]].any() and not pool.window[[1, 5]].float().any()
    keep = [0, 2, 3, 4, 6]
    assert torch.equal(pool.state[keep], st0[keep]) and torch.equal(pool.window[keep], wn0[keep])
    fresh = make_pool(s, 7, io, n_layers=2)
    torch.cuda.synchronize()
    assert torch.equal(fresh.state[1], pool.state[1])


# ------------------------------------------------------------------- verify

def _verify(pool, layer, ids, n_tok, td, w, acc):
    s = pool.desc
    out = torch.full((ids.numel(), n_tok, s.h_v, s.d_v), float("nan"), dtype=pool.io_torch,
                     device="cuda")
    pool.verify(layer, ids, n_tok, td["q"], td["k"], td["v"], td["a"], td["b"], w, acc, out)
    return out


def test_verify_128_slots_vs_oracle():
    case = syn.verify_case()
    s, io, n_tok = case["shapes"], case["io"], case["n_tok"]
    ids_np, acc_np = case["slot_ids"], case["accept_len"]
    say(f"verify: {len(ids_np)} slots x {n_tok} tokens")
    pool = make_pool(s, case["n_slots"], io)
    scramble_pool(pool, 11)
    contents = syn.draw_pool_contents(case["pool_seed"], ids_np, s, io)
    load_slots(pool, contents)
    st0, wn0 = pool.state.clone(), pool.window.clone()
    out = _verify(pool, 0, dev(ids_np, torch.int32), n_tok, tokens_to_dev(case["tokens"], io),
                  dev(case["conv_w"]), dev(acc_np, torch.int32))
    torch.cuda.synchronize()
    op = oracle_pool(s, contents, ids_np)
    tok = case["tokens"]
    ref = op.verify(0, np.arange(len(ids_np)), n_tok, tok["q"], tok["k"], tok["v"], tok["a"],
                    tok["b"], case["conv_w"], acc_np)
    check_out("outputs", host(out), ref, io)
    idx = torch.from_numpy(ids_np.astype(np.int64)).cuda()
    check_f32("committed states", host(pool.state[idx]), op.S)
    assert np.array_equal(host(pool.window[idx]), op.X)
    mask = torch.ones(case["n_slots"], dtype=torch.bool, device="cuda")
    mask[idx] = False
    assert torch.equal(pool.state[mask], st0[mask]) and torch.equal(pool.window[mask], wn0[mask])


@pytest.mark.parametrize("n_tok", [1, 3, 4, 8])
def test_verify_is_bitwise_sequential_decode(n_tok):
    """Each position's output, and the state and window committed after
    accept_len tokens, equal those of accept_len decode steps bitwise."""
    s, io = syn.QWEN3_NEXT, "bf16"
    say(f"verify == decode, n_tok={n_tok}")
    rng = np.random.default_rng(40 + n_tok)
    n, n_slots = 12, 20
    ids_np = rng.permutation(n_slots)[:n].astype(np.int32)
    acc_np = np.arange(n, dtype=np.int32) % (n_tok + 1)      # includes 0 and n_tok
    w = dev(syn.draw_conv_weights(rng, s))
    tok = syn.draw_tokens(rng, s, (n, n_tok), io)
    contents = syn.draw_pool_contents(77, ids_np, s, io)
    pv = make_pool(s, n_slots, io)
    load_slots(pv, contents)
    pd = make_pool(s, n_slots, io)
    load_slots(pd, contents)
    ids = dev(ids_np, torch.int32)
    out_v = _verify(pv, 0, ids, n_tok, tokens_to_dev(tok, io), w, dev(acc_np, torch.int32))
    idx = ids.long()
    want_state = pd.state[idx].clone()
    want_win = pd.window[idx].clone()
    for t in range(n_tok):
        tt = tokens_to_dev({m: tok[m][:, t] for m in tok}, io)
        o = _decode(pd, 0, ids, tt, w, io)
        assert torch.equal(o, out_v[:, t]), f"position {t} differs from decode"
        done = torch.from_numpy(acc_np == t + 1).cuda()
        want_state[done] = pd.state[idx][done]
        want_win[done] = pd.window[idx][done]
    torch.cuda.synchronize()
    assert torch.equal(pv.state[idx], want_state)
    assert torch.equal(pv.window[idx], want_win)


def test_verify_then_commit_after_sampling_equals_one_call():
    """Acceptance known only after sampling: verify with accept_len 0 (the
    outputs; slots untouched), then commit with the sampled accept_len and no
    outputs.  Outputs, states and windows equal one verify call with that
    accept_len, bitwise; a commit of 0 changes nothing."""
    s, io, n_tok = syn.QWEN3_NEXT, "bf16", 4
    say("verify, then commit")
    rng = np.random.default_rng(70)
    n, n_slots = 24, 40
    ids_np = rng.permutation(n_slots)[:n].astype(np.int32)
    acc_np = (np.arange(n) % (n_tok + 1)).astype(np.int32)      # 0..4
    w = dev(syn.draw_conv_weights(rng, s))
    tok = syn.draw_tokens(rng, s, (n, n_tok), io)
    td = tokens_to_dev(tok, io)
    contents = syn.draw_pool_contents(88, ids_np, s, io)
    pa, pb = make_pool(s, n_slots, io), make_pool(s, n_slots, io)
    load_slots(pa, contents)
    load_slots(pb, contents)
    st0, wn0 = pb.state.clone(), pb.window.clone()
    ids = dev(ids_np, torch.int32)
    out_a = _verify(pa, 0, ids, n_tok, td, w, dev(acc_np, torch.int32))
    out_b = _verify(pb, 0, ids, n_tok, td, w, dev(np.zeros(n, np.int32), torch.int32))
    torch.cuda.synchronize()
    assert torch.equal(pb.state, st0) and torch.equal(pb.window, wn0), "accept_len 0 touched a slot"
    assert torch.equal(out_a, out_b)
    pb.verify(0, ids, n_tok, td["q"], td["k"], td["v"], td["a"], td["b"], w,
              dev(acc_np, torch.int32), None)
    torch.cuda.synchronize()
    assert torch.equal(pa.state, pb.state) and torch.equal(pa.window, pb.window)
    assert pb.error() == 0


def test_repeated_verify_rounds_match_oracle():
    """Several verify rounds with mixed acceptance on the same slots."""
    s, io = syn.Shapes(4, 8, 128, 128, 4), "bf16"
    say("verify rounds")
    rng = np.random.default_rng(99)
    n, n_tok, rounds = 6, 4, 5
    ids_np = np.array([4, 0, 7, 2, 5, 1], np.int32)
    w_np = syn.draw_conv_weights(rng, s)
    w = dev(w_np)
    contents = syn.draw_pool_contents(5, ids_np, s, io)
    pool = make_pool(s, 8, io)
    load_slots(pool, contents)
    op = oracle_pool(s, contents, ids_np)
    ids = dev(ids_np, torch.int32)
    outs, refs = [], []
    for r in range(rounds):
        tok = syn.draw_tokens(rng, s, (n, n_tok), io)
        acc = rng.integers(0, n_tok + 1, size=n).astype(np.int32)
        outs.append(host(_verify(pool, 0, ids, n_tok, tokens_to_dev(tok, io), w,
                                 dev(acc, torch.int32))))
        refs.append(op.verify(0, np.arange(n), n_tok, tok["q"], tok["k"], tok["v"], tok["a"],
                              tok["b"], w_np, acc))
    check_out("outputs", np.array(outs), np.array(refs), io)
    check_f32("states", host(pool.state[ids.long()]), op.S)
    assert np.array_equal(host(pool.window[ids.long()]), op.X)
