"""GPU parity: chunked prefill through the C ABI against the fp64 token-by-
token oracle, plus the chunk/scheduler-split invariants and the bookkeeping
guarantees (untouched slots, windows, zero-length and padding sequences,
malformed cu_seqlens)."""
import numpy as np
import pytest

import gdn_synth as syn
from oracle import gdn_oracle as O
from gpu_util import (check_f32, check_f32_dev, check_out, dev, group_slice, host, load_slots, make_pool,
                      oracle_pool, rel_err, say, scramble_pool, slice_tokens, tokens_to_dev)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_state_layer_amd import binding
    binding.load_library()


def run_prefill(pool, layer, cu_np, ids_np, tok, w, chunk, io):
    s = pool.desc
    T = int(cu_np[-1])
    td = tokens_to_dev(tok, io)
    out = torch.full((T, s.h_v, s.d_v), float("nan"), dtype=pool.io_torch, device="cuda")
    nbytes = pool.prefill_workspace_bytes(len(ids_np), T, chunk)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    pool.prefill(layer, dev(cu_np, torch.int32), dev(ids_np, torch.int32), T, chunk, td["q"],
                 td["k"], td["v"], td["a"], td["b"], w, out, ws)
    return out


def test_tiny_layer_prefill_then_decode():
    """64-token prefill (chunk 16) then 16 decode steps on the tiny fp32 layer."""
    case = syn.tiny_layer_case()
    s = case["shapes"]
    say("tiny layer: prefill 64 (chunk 16) + 16 decode")
    pool = make_pool(s, 3, "f32")
    w = dev(case["conv_w"])
    pre, dec = case["prefill"], case["decode"]
    out = run_prefill(pool, 0, np.array([0, 64], np.int32), np.array([1], np.int32), pre, w, 16, "f32")
    op = O.OraclePool(1, 1, s)
    ref = op.prefill(0, [0, 64], [0], pre["q"], pre["k"], pre["v"], pre["a"], pre["b"], case["conv_w"])
    check_f32("prefill outputs", host(out), ref)
    check_f32("state after prefill", host(pool.state[1]), op.S[0])
    assert np.array_equal(host(pool.window[1]), op.X[0])
    ids = dev(np.array([1], np.int32), torch.int32)
    outs, refs = [], []
    for t in range(16):
        tt = {n: dec[n][t:t + 1] for n in dec}
        td = tokens_to_dev(tt, "f32")
        o = torch.empty((1, s.h_v, s.d_v), device="cuda")
        pool.decode(0, ids, td["q"], td["k"], td["v"], td["a"], td["b"], w, o)
        outs.append(host(o))
        refs.append(op.decode(0, [0], tt["q"], tt["k"], tt["v"], tt["a"], tt["b"], case["conv_w"]))
    check_f32("decode outputs", np.array(outs), np.array(refs))
    check_f32("final state", host(pool.state[1]), op.S[0])
    assert not host(pool.state[[0, 2]]).any()


def _oracle_groups(s, groups, tok, w, cu, ids_order, contents=None, form="rank1"):
    """Run the oracle on q/k head groups `groups` only; returns per group
    (outputs [T, G, d], oracle pool)."""
    res = {}
    for g in groups:
        ch, hs, sub = group_slice(s, g)
        sub_contents = None
        if contents is not None:
            sub_contents = {sl: (st[:, hs], wn[..., ch]) for sl, (st, wn) in contents.items()}
        op = oracle_pool(sub, sub_contents, ids_order, form=form)
        tk = slice_tokens(tok, s, g)
        out = op.prefill(0, cu, np.arange(len(ids_order)), tk["q"], tk["k"], tk["v"], tk["a"],
                         tk["b"], w[ch])
        res[g] = (out, op, hs, ch)
    return res


def _check_groups(pool, res, out, ids_np, io, cu=None):
    idx = torch.from_numpy(ids_np.astype(np.int64)).cuda()
    for g, (ref, op, hs, ch) in res.items():
        o = host(out[:, hs])
        if cu is not None:   # skip rows of padding sequences
            keep = np.zeros(o.shape[0], bool)
            for j in range(len(cu) - 1):
                if ids_np[j] >= 0:
                    keep[cu[j]:cu[j + 1]] = True
            o, ref = o[keep], ref[keep]
        check_out(f"group {g} outputs", o, ref, io)
        check_f32(f"group {g} final states", host(pool.state[idx][:, :, hs]), op.S)
        assert np.array_equal(host(pool.window[idx][..., ch]), op.X), f"group {g} windows"


def _check_layer(pool, out, ids_np, ref, io, rows=None, what=""):
    """Whole-layer comparison with the oracle: every output row of the
    listed rows (all by default), every final state and every window of the
    sequences' slots; the worst q/k group is printed too."""
    out_ref, S_ref, X_ref = ref
    s = pool.desc
    o = host(out)
    if rows is not None:
        o, out_ref = o[rows], out_ref[rows]
    check_out(f"{what}outputs, all {s.h_k} groups", o, out_ref, io)
    G = s.h_v // s.h_k
    worst = max(range(s.h_k), key=lambda g: rel_err(o[:, g * G:(g + 1) * G],
                                                    out_ref[:, g * G:(g + 1) * G]))
    say(f"  worst group {worst}: {rel_err(o[:, worst * G:(worst + 1) * G], out_ref[:, worst * G:(worst + 1) * G]):.3e}")
    idx = torch.from_numpy(ids_np.astype(np.int64)).cuda()
    check_f32(f"{what}final states, all {s.h_v} heads", host(pool.state[idx]), S_ref)
    assert np.array_equal(host(pool.window[idx]), X_ref), f"{what}windows"


_REF_8192 = {}


def _oracle_8192(workers, case):
    """Oracle over the whole layer for the 8192-token sequence (computed
    once, shared by the one-call and the split test)."""
    if "ref" not in _REF_8192:
        tok = case["tokens"]
        T = tok["q"].shape[0]
        _REF_8192["ref"] = workers.prefill_all_groups(case["shapes"], tok, case["conv_w"],
                                                      np.array([0, T]), np.array([0]))
    return _REF_8192["ref"]


def test_prefill_8192_tokens_all_groups(oracle_pool_workers):
    """One 8192-token sequence, chunk 64, Qwen3-Next shapes, in the launch the
    benchmark times: outputs, final state and window compared with the
    oracle on every q/k group and value head of the layer."""
    case = syn.prefill_case()
    s, io, tok = case["shapes"], case["io"], case["tokens"]
    T = tok["q"].shape[0]
    say(f"prefill T={T} chunk 64, all groups")
    pool = make_pool(s, 4, io)
    scramble_pool(pool, 21)
    pool.reset(dev(np.array([2], np.int32), torch.int32))
    st0, wn0 = pool.state.clone(), pool.window.clone()
    out = run_prefill(pool, 0, np.array([0, T], np.int32), np.array([2], np.int32), tok,
                      dev(case["conv_w"]), 64, io)
    torch.cuda.synchronize()
    assert pool.error() == 0
    _check_layer(pool, out, np.array([2], np.int32), _oracle_8192(oracle_pool_workers, case), io)
    keep = [0, 1, 3]
    assert torch.equal(pool.state[keep], st0[keep]) and torch.equal(pool.window[keep], wn0[keep])


@pytest.mark.parametrize("T", [300, 1000])
def test_prefill_factor_grid_sizes_all_groups(oracle_pool_workers, T):
    """The first T tokens of the 8192-token sequence in one call, against the
    oracle on every group: 300 tokens give 6 x 16 (chunk, q/k head) work items
    (at most one factor workgroup per CU: eight waves, two value heads side
    by side), 1000 tokens 17 x 16 (one round of four-wave workgroups, q|k
    staged in one pass)."""
    case = syn.prefill_case()
    s, io = case["shapes"], case["io"]
    tok = {n: x[:T] for n, x in case["tokens"].items()}
    say(f"prefill T={T} chunk 64, all groups")
    pool = make_pool(s, 4, io)
    scramble_pool(pool, 23)
    pool.reset(dev(np.array([1], np.int32), torch.int32))
    st0, wn0 = pool.state.clone(), pool.window.clone()
    out = run_prefill(pool, 0, np.array([0, T], np.int32), np.array([1], np.int32), tok,
                      dev(case["conv_w"]), 64, io)
    torch.cuda.synchronize()
    assert pool.error() == 0
    ref = oracle_pool_workers.prefill_all_groups(s, tok, case["conv_w"], np.array([0, T]),
                                                 np.array([0]))
    _check_layer(pool, out, np.array([1], np.int32), ref, io)
    keep = [0, 2, 3]
    assert torch.equal(pool.state[keep], st0[keep]) and torch.equal(pool.window[keep], wn0[keep])


def test_prefill_scheduler_split_matches_unsplit(oracle_pool_workers):
    """The same 8192 tokens as 16 calls of 512 tokens carrying state and
    window: equal to the single call (within tolerance) and to the oracle on
    every group of the layer."""
    case = syn.prefill_case()
    s, io, tok = case["shapes"], case["io"], case["tokens"]
    T = tok["q"].shape[0]
    say("prefill split 16 x 512, all groups")
    w = dev(case["conv_w"])
    p1 = make_pool(s, 2, io)
    o1 = run_prefill(p1, 0, np.array([0, T], np.int32), np.array([1], np.int32), tok, w, 64, io)
    p2 = make_pool(s, 2, io)
    parts = []
    for c0 in range(0, T, 512):
        sl = {n: tok[n][c0:c0 + 512] for n in tok}
        parts.append(run_prefill(p2, 0, np.array([0, 512], np.int32), np.array([1], np.int32), sl,
                                 w, 64, io))
    o2 = torch.cat(parts)
    torch.cuda.synchronize()
    assert p2.error() == 0
    check_out("split vs unsplit outputs", host(o2), host(o1), io)
    check_f32("split vs unsplit state", host(p2.state[1]), host(p1.state[1]))
    assert torch.equal(p2.window[1], p1.window[1])
    _check_layer(p2, o2, np.array([1], np.int32), _oracle_8192(oracle_pool_workers, case), io,
                 what="split: ")


def _varlen_setup(case, contents):
    """Pool for the varlen workload: every slot scrambled, the continuing
    sequences' slots holding `contents`, the others reset."""
    s, io, ids_np, cont = case["shapes"], case["io"], case["slot_ids"], case["continuing"]
    pool = make_pool(s, case["n_slots"], io)
    scramble_pool(pool, 31)
    load_slots(pool, contents)
    pool.reset(dev(ids_np[~cont], torch.int32))
    return pool


def _start_contents(case, contents):
    """Oracle starting states/windows per sequence (zero for reset slots)."""
    s, ids_np = case["shapes"], case["slot_ids"]
    n = len(ids_np)
    st = np.zeros((n, 1, s.h_v, s.d_v, s.d_k))
    wn = np.zeros((n, 1, s.conv_k - 1, s.c_conv))
    for j, sl in enumerate(ids_np):
        if int(sl) in contents:
            st[j], wn[j] = contents[int(sl)]
    return st, wn


def test_varlen_batched_prefill_into_slots(oracle_pool_workers):
    """16 packed sequences of 128..4096 tokens; 12 into reset slots, 4
    continuing from pre-filled states and windows; every group, state and
    window of the layer against the oracle, other slots bitwise untouched."""
    case = syn.varlen_case()
    s, io, tok = case["shapes"], case["io"], case["tokens"]
    cu, ids_np, cont = case["cu_seqlens"], case["slot_ids"], case["continuing"]
    say(f"varlen: {len(ids_np)} seqs, {int(cu[-1])} tokens, all groups")
    contents = syn.draw_pool_contents(case["pool_seed"], ids_np[cont], s, io)
    pool = _varlen_setup(case, contents)
    st0, wn0 = pool.state.clone(), pool.window.clone()
    out = run_prefill(pool, 0, cu, ids_np, tok, dev(case["conv_w"]), 64, io)
    torch.cuda.synchronize()
    assert pool.error() == 0
    st, wn = _start_contents(case, contents)
    ref = oracle_pool_workers.prefill_all_groups(s, tok, case["conv_w"], cu, np.arange(len(ids_np)),
                                                 st, wn)
    _check_layer(pool, out, ids_np, ref, io)
    mask = torch.ones(case["n_slots"], dtype=torch.bool, device="cuda")
    mask[torch.from_numpy(ids_np.astype(np.int64)).cuda()] = False
    assert torch.equal(pool.state[mask], st0[mask]) and torch.equal(pool.window[mask], wn0[mask])


def test_varlen_continuing_slots_from_a_prefix_prefill(oracle_pool_workers):
    """The varlen workload whose 4 continuing slots got their state and
    window from an earlier prefill (prefixes of 64..512 tokens, one call),
    as a scheduler's earlier chunk would leave them: the prefix and the
    varlen call are both run by the oracle, every group compared."""
    case = syn.varlen_case()
    s, io, tok = case["shapes"], case["io"], case["tokens"]
    cu, ids_np, cont = case["cu_seqlens"], case["slot_ids"], case["continuing"]
    rng = np.random.default_rng(1013)
    plen = rng.integers(64, 513, size=int(cont.sum()))
    pcu = np.concatenate([[0], np.cumsum(plen)]).astype(np.int32)
    ptok = syn.draw_tokens(rng, s, (int(pcu[-1]),), io)
    pids = ids_np[cont]
    say(f"varlen after prefixes {plen.tolist()} into slots {pids.tolist()}")
    pool = make_pool(s, case["n_slots"], io)
    scramble_pool(pool, 33)
    pool.reset(dev(ids_np, torch.int32))
    w = dev(case["conv_w"])
    run_prefill(pool, 0, pcu, pids, ptok, w, 64, io)
    out = run_prefill(pool, 0, cu, ids_np, tok, w, 64, io)
    torch.cuda.synchronize()
    assert pool.error() == 0
    _, S1, X1 = oracle_pool_workers.prefill_all_groups(s, ptok, case["conv_w"], pcu,
                                                       np.arange(len(pids)))
    n = len(ids_np)
    st = np.zeros((n, 1, s.h_v, s.d_v, s.d_k))
    wn = np.zeros((n, 1, s.conv_k - 1, s.c_conv))
    st[cont], wn[cont] = S1, X1
    ref = oracle_pool_workers.prefill_all_groups(s, tok, case["conv_w"], cu, np.arange(n), st, wn)
    _check_layer(pool, out, ids_np, ref, io)


def test_one_sequence_with_outputs_beyond_2gib(oracle_pool_workers):
    """One fp32 sequence whose output rows run past 2^31 bytes (h_v = 64,
    d = 128: 32 KiB per token, 66,236 tokens) in one call: equal to the
    same tokens as 512-token calls, and the last q/k group against the
    oracle over the whole sequence."""
    s, io = syn.Shapes(16, 64, 128, 128, 4), "f32"
    T = 65536 + 700
    say(f"one sequence of {T} tokens, {s}, outputs {T * s.h_v * s.d_v * 4 / 2**30:.2f} GiB")
    g = torch.Generator(device="cuda").manual_seed(2024)
    qk = torch.randn((T, 2, s.h_k, s.d_k), generator=g, device="cuda")
    qk = qk / qk.norm(dim=-1, keepdim=True)
    td = {"q": qk[:, 0].contiguous(), "k": qk[:, 1].contiguous()}
    del qk
    td["v"] = torch.randn((T, s.h_v, s.d_v), generator=g, device="cuda")
    td["b"] = torch.sigmoid(torch.randn((T, s.h_v), generator=g, device="cuda"))
    td["a"] = torch.exp(-torch.nn.functional.softplus(torch.randn((T, s.h_v), generator=g,
                                                                   device="cuda")))
    w_np = syn.draw_conv_weights(np.random.default_rng(2025), s)
    w = dev(w_np)
    p1 = make_pool(s, 2, io)
    o1 = torch.full((T, s.h_v, s.d_v), float("nan"), device="cuda")
    ws = torch.empty(p1.prefill_workspace_bytes(1, T, 64), dtype=torch.uint8, device="cuda")
    one = dev(np.array([1], np.int32), torch.int32)
    p1.prefill(0, dev(np.array([0, T], np.int32), torch.int32), one, T, 64, td["q"], td["k"],
               td["v"], td["a"], td["b"], w, o1, ws)
    del ws
    p2 = make_pool(s, 2, io)
    o2 = torch.full_like(o1, float("nan"))
    ws = torch.empty(p2.prefill_workspace_bytes(1, 512, 64), dtype=torch.uint8, device="cuda")
    for c0 in range(0, T, 512):
        c1 = min(c0 + 512, T)
        p2.prefill(0, dev(np.array([0, c1 - c0], np.int32), torch.int32), one, c1 - c0, 64,
                   *(td[n][c0:c1] for n in "qkvab"), w, o2[c0:c1], ws)
    torch.cuda.synchronize()
    assert p1.error() == 0 and p2.error() == 0
    assert torch.isfinite(o1).all(), "rows of the one-call run were not written"
    past = 2 ** 31 // (s.h_v * s.d_v * 4)     # first token whose row starts at 2 GiB
    check_f32_dev("rows past 2 GiB: one call vs 512-token calls", o1[past:], o2[past:])
    check_f32_dev("all rows: one call vs 512-token calls", o1, o2)
    check_f32_dev("state: one call vs 512-token calls", p1.state[1], p2.state[1])
    gq = s.h_k - 1
    G = s.group
    hs = slice(gq * G, (gq + 1) * G)
    tok = {"q": host(td["q"][:, gq:gq + 1]).astype(np.float32),
           "k": host(td["k"][:, gq:gq + 1]).astype(np.float32),
           "v": host(td["v"][:, hs]).astype(np.float32),
           "a": host(td["a"][:, hs]).astype(np.float32), "b": host(td["b"][:, hs]).astype(np.float32)}
    sub = syn.Shapes(1, G, s.d_k, s.d_v, s.conv_k)
    ch = oracle_pool_workers.group_channels(s, gq)
    ref, S, X = oracle_pool_workers.prefill_all_groups(sub, tok, w_np[ch], np.array([0, T]),
                                                       np.array([0]))
    check_out(f"group {gq} outputs vs oracle", host(o1[:, hs]), ref, io)
    check_f32(f"group {gq} state vs oracle", host(p1.state[1][:, hs]), S[0])


@pytest.mark.parametrize("d,chunk,lens,io", [
    (32, 16, [2000, 704, 1500], "f32"),
    (64, 64, [5000, 4500], "bf16"),
])
def test_long_unequal_sequences_vs_oracle(d, chunk, lens, io):
    """Long packed sequences of unequal length (hundreds of chunk steps, one
    a whole number of chunks) with a continuing slot, against the oracle on
    every head of the layer."""
    s = syn.Shapes(1, 2, d, d, 4)
    say(f"long sequences: d={d} chunk={chunk} lens={lens} io={io}")
    rng = np.random.default_rng(7 * d + chunk)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    tok = syn.draw_tokens(rng, s, (T,), io)
    w_np = syn.draw_conv_weights(rng, s)
    ids_np = np.array([3, 0, 5][:len(lens)], np.int32)
    pool = make_pool(s, 6, io)
    scramble_pool(pool, 41)
    contents = syn.draw_pool_contents(99, np.array([0]), s, io)   # slot 0 continues
    load_slots(pool, contents)
    pool.reset(dev(ids_np[ids_np != 0], torch.int32))
    st0, wn0 = pool.state.clone(), pool.window.clone()
    out = run_prefill(pool, 0, cu, ids_np, tok, dev(w_np), chunk, io)
    torch.cuda.synchronize()
    assert pool.error() == 0
    res = _oracle_groups(s, [0], tok, w_np, cu, ids_np,
                         contents={int(k): v for k, v in contents.items()})
    _check_groups(pool, res, out, ids_np, io)
    untouched = [i for i in range(6) if i not in ids_np]
    assert torch.equal(pool.state[untouched], st0[untouched])
    assert torch.equal(pool.window[untouched], wn0[untouched])


@pytest.mark.parametrize("h_k,h_v,d,chunk,io", [
    (2, 2, 32, 16, "f32"), (1, 4, 64, 32, "bf16"), (2, 4, 128, 64, "bf16"), (1, 2, 128, 32, "f32"),
    (2, 2, 64, 64, "f32")])
def test_ragged_edges_vs_oracle(h_k, h_v, d, chunk, io):
    """Ragged chunk tails, sequences shorter than the conv window (lengths
    1, 2), a zero-length sequence, a padding entry, continuing slots, on the
    full layer (every head) against the oracle."""
    s = syn.Shapes(h_k, h_v, d, d, 4)
    say(f"ragged edges: {s} chunk={chunk} io={io}")
    rng = np.random.default_rng(d + chunk + h_v)
    lens = np.array([1, chunk + 3, 0, 2, 3 * chunk - 1, 5, chunk])
    ids_np = np.array([4, 0, 2, 7, -1, 3, 6], np.int32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    w_np = syn.draw_conv_weights(rng, s)
    tok = syn.draw_tokens(rng, s, (T,), io)
    n_slots = 8
    pool = make_pool(s, n_slots, io)
    contents = syn.draw_pool_contents(3, [0, 3, 7, 2], s, io)
    load_slots(pool, contents)
    pool.reset(dev(np.array([4, 6], np.int32), torch.int32))
    st0, wn0 = pool.state.clone(), pool.window.clone()
    out = run_prefill(pool, 0, cu, ids_np, tok, dev(w_np), chunk, io)
    torch.cuda.synchronize()
    assert pool.error() == 0
    valid = ids_np >= 0
    op = oracle_pool(s, contents, np.where(valid, ids_np, 0), form="rank1")
    op.S[~valid] = 0.0
    ref = op.prefill(0, cu, np.where(valid, np.arange(len(ids_np)), -1), tok["q"], tok["k"],
                     tok["v"], tok["a"], tok["b"], w_np)
    rows = np.concatenate([np.arange(cu[j], cu[j + 1]) for j in range(len(lens)) if valid[j]])
    check_out("outputs", host(out)[rows], ref[rows], io)
    assert torch.isnan(out[cu[4]:cu[5]].float()).all(), "padding sequence rows were written"
    for jj, sl in enumerate(ids_np):
        if sl < 0:
            continue
        check_f32(f"state of slot {sl}", host(pool.state[int(sl)]), op.S[jj])
        assert np.array_equal(host(pool.window[int(sl)]), op.X[jj]), f"window of slot {sl}"
    for sl in (1, 5):
        assert torch.equal(pool.state[sl], st0[sl]) and torch.equal(pool.window[sl], wn0[sl])
    # zero-length sequence into slot 2 left it bitwise unchanged
    assert torch.equal(pool.state[2], st0[2]) and torch.equal(pool.window[2], wn0[2])


@pytest.mark.parametrize("conv_k,chunk", [(2, 32), (3, 64), (8, 16), (6, 64)])
def test_other_conv_widths_vs_oracle(conv_k, chunk):
    """Prefill, then decode and verify, with conv widths other than 4 (the
    runtime-width kernels), continuing from pre-filled slots."""
    s, io = syn.Shapes(2, 4, 64, 64, conv_k), "bf16"
    say(f"conv_k={conv_k} chunk={chunk}")
    rng = np.random.default_rng(60 + conv_k)
    w_np = syn.draw_conv_weights(rng, s)
    w = dev(w_np)
    lens = np.array([3, chunk + 5, 2 * chunk, 1])
    ids_np = np.array([1, 3, 0, 2], np.int32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tok = syn.draw_tokens(rng, s, (int(cu[-1]),), io)
    contents = syn.draw_pool_contents(9, ids_np, s, io)
    pool = make_pool(s, 4, io)
    load_slots(pool, contents)
    out = run_prefill(pool, 0, cu, ids_np, tok, w, chunk, io)
    op = oracle_pool(s, contents, ids_np, form="rank1")
    ref = op.prefill(0, cu, np.arange(4), tok["q"], tok["k"], tok["v"], tok["a"], tok["b"], w_np)
    check_out("prefill outputs", host(out), ref, io)
    d1 = syn.draw_tokens(rng, s, (4,), io)
    o = torch.empty((4, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda")
    td = tokens_to_dev(d1, io)
    pool.decode(0, dev(ids_np, torch.int32), td["q"], td["k"], td["v"], td["a"], td["b"], w, o)
    r1 = op.decode(0, np.arange(4), d1["q"], d1["k"], d1["v"], d1["a"], d1["b"], w_np)
    check_out("decode outputs", host(o), r1, io)
    idx = torch.from_numpy(ids_np.astype(np.int64)).cuda()
    check_f32("states", host(pool.state[idx]), op.S)
    assert np.array_equal(host(pool.window[idx]), op.X)


def test_malformed_cu_seqlens_is_flagged_and_touches_nothing():
    s, io = syn.Shapes(2, 4, 64, 64, 4), "bf16"
    say("malformed cu_seqlens")
    rng = np.random.default_rng(12)
    w = dev(syn.draw_conv_weights(rng, s))
    pool = make_pool(s, 4, io)
    scramble_pool(pool, 13)
    st0, wn0 = pool.state.clone(), pool.window.clone()
    tok = syn.draw_tokens(rng, s, (40,), io)
    for cu in ([0, 30, 20, 40], [0, 10, 41, 40], [1, 20, 30, 40]):
        out = run_prefill(pool, 0, np.array(cu, np.int32), np.array([0, 1, 2], np.int32), tok, w,
                          32, io)
        assert pool.error() == 2
        assert torch.isnan(out.float()).all()
    assert torch.equal(pool.state, st0) and torch.equal(pool.window, wn0)


@pytest.mark.parametrize("n", [64, 65, 100])
def test_many_sequences_vs_oracle(n):
    """Up to 64 sequences the factor kernel books the chunks itself; beyond,
    the separate prep kernel builds the chunk map (64 and 65 sit on either
    side of that boundary): short sequences, some empty, two padding
    entries, slots continuing from pre-filled contents."""
    s, io, chunk = syn.Shapes(1, 2, 32, 32, 4), "f32", 16
    say(f"{n} sequences: {s} chunk={chunk}")
    rng = np.random.default_rng(77 + n)
    n_slots = 128
    lens = rng.integers(0, 41, n)
    ids_np = rng.permutation(n_slots)[:n].astype(np.int32)
    ids_np[[5, 50]] = -1
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    w_np = syn.draw_conv_weights(rng, s)
    tok = syn.draw_tokens(rng, s, (T,), io)
    pool = make_pool(s, n_slots, io)
    contents = syn.draw_pool_contents(8, ids_np[ids_np >= 0][:12], s, io)
    load_slots(pool, contents)
    st0, wn0 = pool.state.clone(), pool.window.clone()
    out = run_prefill(pool, 0, cu, ids_np, tok, dev(w_np), chunk, io)
    torch.cuda.synchronize()
    assert pool.error() == 0
    valid = ids_np >= 0
    op = oracle_pool(s, contents, np.where(valid, ids_np, 0), form="rank1")
    op.S[~valid] = 0.0
    ref = op.prefill(0, cu, np.where(valid, np.arange(n), -1), tok["q"], tok["k"], tok["v"],
                     tok["a"], tok["b"], w_np)
    rows = np.concatenate([np.arange(cu[j], cu[j + 1]) for j in range(n) if valid[j]])
    check_out("outputs", host(out)[rows], ref[rows], io)
    for jj, sl in enumerate(ids_np):
        if sl < 0:
            continue
        if lens[jj] == 0:   # a zero-length sequence leaves its slot bitwise unchanged
            assert torch.equal(pool.state[int(sl)], st0[int(sl)]), f"state of slot {sl}"
        else:
            check_f32(f"state of slot {sl}", host(pool.state[int(sl)]), op.S[jj])
        assert np.array_equal(host(pool.window[int(sl)]), op.X[jj]), f"window of slot {sl}"
    untouched = np.setdiff1d(np.arange(n_slots), ids_np[valid])
    idx = torch.from_numpy(untouched.astype(np.int64)).cuda()
    assert torch.equal(pool.state[idx], st0[idx]) and torch.equal(pool.window[idx], wn0[idx])


def test_malformed_cu_seqlens_many_sequences_is_flagged():
    """The same check on the prep kernel's path (more than 64 sequences)."""
    s, io = syn.Shapes(1, 2, 32, 32, 4), "f32"
    say("malformed cu_seqlens, 70 sequences")
    rng = np.random.default_rng(14)
    w = dev(syn.draw_conv_weights(rng, s))
    pool = make_pool(s, 80, io)
    scramble_pool(pool, 15)
    st0, wn0 = pool.state.clone(), pool.window.clone()
    tok = syn.draw_tokens(rng, s, (140,), io)
    good = np.arange(0, 141, 2, dtype=np.int32)   # 70 sequences of 2 tokens
    bad_a = good.copy()
    bad_a[40] = bad_a[38]                           # decreasing
    bad_b = good.copy()
    bad_b[0] = 1                                    # does not start at 0
    for cu in (bad_a, bad_b):
        out = run_prefill(pool, 0, cu, np.arange(70, dtype=np.int32), tok, w, 16, io)
        assert pool.error() == 2
        assert torch.isnan(out.float()).all()
    assert torch.equal(pool.state, st0) and torch.equal(pool.window, wn0)


def test_prefill_then_verify_and_decode_continue_the_sequence():
    """Prefill a prompt, then decode and verify steps continue from the
    prefilled state and window (Qwen3-Next shapes, one group checked)."""
    s, io = syn.QWEN3_NEXT, "bf16"
    say("prefill -> decode -> verify continuity")
    rng = np.random.default_rng(50)
    w_np = syn.draw_conv_weights(rng, s)
    w = dev(w_np)
    T = 300
    tok = syn.draw_tokens(rng, s, (T,), io)
    pool = make_pool(s, 3, io)
    ids = np.array([2], np.int32)
    out = run_prefill(pool, 0, np.array([0, T], np.int32), ids, tok, w, 64, io)
    g = 7
    ch, hs, sub = group_slice(s, g)
    op = O.OraclePool(1, 1, sub, form="rank1")
    tk = slice_tokens(tok, s, g)
    ref = op.prefill(0, [0, T], [0], tk["q"], tk["k"], tk["v"], tk["a"], tk["b"], w_np[ch])
    check_out("prefill outputs", host(out[:, hs]), ref, io)
    d1 = syn.draw_tokens(rng, s, (1,), io)
    o = torch.empty((1, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda")
    td = tokens_to_dev(d1, io)
    pool.decode(0, dev(ids, torch.int32), td["q"], td["k"], td["v"], td["a"], td["b"], w, o)
    t1 = slice_tokens(d1, s, g)
    r1 = op.decode(0, [0], t1["q"], t1["k"], t1["v"], t1["a"], t1["b"], w_np[ch])
    check_out("decode after prefill", host(o[:, hs]), r1, io)
    v4 = syn.draw_tokens(rng, s, (1, 4), io)
    ov = torch.empty((1, 4, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda")
    tv = tokens_to_dev(v4, io)
    pool.verify(0, dev(ids, torch.int32), 4, tv["q"], tv["k"], tv["v"], tv["a"], tv["b"], w,
                dev(np.array([3], np.int32), torch.int32), ov)
    t4 = slice_tokens(v4, s, g)
    r4 = op.verify(0, [0], 4, t4["q"], t4["k"], t4["v"], t4["a"], t4["b"], w_np[ch], np.array([3]))
    check_out("verify after prefill", host(ov[:, :, hs]), r4, io)
    check_f32("state", host(pool.state[2][:, hs]), op.S[0])
    assert np.array_equal(host(pool.window[2][..., ch]), op.X[0])
