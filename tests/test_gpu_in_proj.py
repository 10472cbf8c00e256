"""GPU parity of the input projection (gdn_in_proj) against the fp64 oracle:
the raw q, k, v and the activated gates, on the skinny path (up to 64
tokens), the split-hidden path, the 128-token-tile path and the 256-token-tile
path (from 512 tokens; 1000 and 2100 tokens leave ragged row tiles and a
partial band; 8192 tokens is the prefill workload's length), with ragged token and channel counts, and the projection
feeding a decode step."""
import numpy as np
import pytest

import gdn_synth as syn
from gpu_util import check_f32, check_out, dev, host, load_slots, make_pool, oracle_pool, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from oracle import gdn_oracle as O  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_state_layer_amd import binding
    binding.load_library()


def _project(pool, s, x_np, w_np, io):
    n = x_np.shape[0]
    t = torch.bfloat16 if io == "bf16" else torch.float32
    x = dev(x_np, torch.bfloat16)
    w = dev(w_np, torch.bfloat16)
    q = torch.full((n, s.h_k, s.d_k), float("nan"), dtype=t, device="cuda")
    k = torch.full_like(q, float("nan"))
    v = torch.full((n, s.h_v, s.d_v), float("nan"), dtype=t, device="cuda")
    a = torch.full((n, s.h_v), float("nan"), device="cuda")
    b = torch.full_like(a, float("nan"))
    nb = pool.in_proj_workspace_bytes(n, x_np.shape[1])
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda") if nb else None
    pool.in_proj(x, w, q, k, v, a, b, ws)
    torch.cuda.synchronize()
    return q, k, v, a, b, nb


@pytest.mark.parametrize("n_tok", [1, 64, 300, 1024, 1000, 2100, 8192])
def test_in_proj_qwen3_next_vs_oracle(n_tok):
    s, io, hidden = syn.QWEN3_NEXT, "bf16", syn.QWEN3_NEXT_HIDDEN
    rng = np.random.default_rng(1100 + n_tok)
    x = syn.draw_hidden(rng, (n_tok,), hidden)
    w = syn.draw_in_proj_weight(rng, s, hidden)
    pool = make_pool(s, 1, io)
    q, k, v, a, b, nb = _project(pool, s, x, w, io)
    say(f"in_proj: {n_tok} tokens, hidden {hidden}, workspace {nb} B "
        f"({'split' if nb else 'one pass'})")
    rq, rk, rv, ra, rb = O.in_projection(x, w, s)
    check_out("q", host(q), rq, io)
    check_out("k", host(k), rk, io)
    check_out("v", host(v), rv, io)
    check_f32("a", host(a), ra)
    check_f32("b", host(b), rb)
    assert pool.error() == 0


@pytest.mark.parametrize("h_k,h_v,d,hidden,n_tok,io", [
    (2, 2, 32, 96, 7, "f32"),        # 196 output channels: a ragged 16-channel tile
    (1, 3, 64, 160, 70, "bf16"),     # 3 gates each: gate rows straddle a tile
    (2, 4, 128, 4096, 5, "bf16"),    # long hidden, split 16 ways
    (2, 4, 64, 96, 700, "f32"),      # 256-token tiles: ragged rows, an 8-channel last tile
    (1, 2, 128, 32, 600, "bf16"),    # 256-token tiles over a single k-block
    (1, 2, 128, 64, 530, "f32"),     # 256-token tiles over two k-blocks
    (1, 1, 32, 96, 600, "bf16"),     # many tokens, fewer than 256 channels: the 128-tile path
    (1, 2, 128, 2048, 600, "f32"),   # 256-token tiles, then the 4 gate channels 32 tokens per workgroup
])
def test_in_proj_other_shapes(h_k, h_v, d, hidden, n_tok, io):
    s = syn.Shapes(h_k, h_v, d, d, 4)
    rng = np.random.default_rng(1200 + hidden)
    x = syn.draw_hidden(rng, (n_tok,), hidden)
    w = syn.draw_in_proj_weight(rng, s, hidden)
    pool = make_pool(s, 1, io)
    q, k, v, a, b, nb = _project(pool, s, x, w, io)
    say(f"in_proj: {s} hidden {hidden} tokens {n_tok} io {io} workspace {nb}")
    rq, rk, rv, ra, rb = O.in_projection(x, w, s)
    check_out("q", host(q), rq, io)
    check_out("k", host(k), rk, io)
    check_out("v", host(v), rv, io)
    check_f32("a", host(a), ra)
    check_f32("b", host(b), rb)


@pytest.mark.parametrize("h_k,h_v,d,hidden,n_tok,io", [
    (16, 32, 128, 2048, 17, "f32"),   # 8256 channels, fp32 io, ragged tokens
    (2, 4, 64, 1024, 64, "bf16"),     # 520 channels: an 8-channel last tile of gates
    (4, 8, 64, 2048, 33, "bf16"),     # 1040 channels
    (4, 20, 64, 1024, 9, "f32"),      # 1832 channels: 40 gate channels across a tile edge
])
def test_in_proj_few_tokens_repeated_calls(h_k, h_v, d, hidden, n_tok, io):
    """Decode-sized batches (up to 64 tokens) at hidden 1024 and 2048, the
    two step counts of the few-token kernel, with ragged last tiles: three
    calls in a row, each matching the oracle, and a repeated input giving
    bitwise the same outputs."""
    s = syn.Shapes(h_k, h_v, d, d, 4)
    rng = np.random.default_rng(1250 + hidden + n_tok)
    w = syn.draw_in_proj_weight(rng, s, hidden)
    pool = make_pool(s, 1, io)
    xs = [syn.draw_hidden(rng, (n_tok,), hidden) for _ in range(2)]
    outs = []
    for call, x in enumerate(xs + xs[:1]):
        q, k, v, a, b, nb = _project(pool, s, x, w, io)
        say(f"in_proj few tokens: {s} hidden {hidden} tokens {n_tok} io {io} call {call} workspace {nb}")
        rq, rk, rv, ra, rb = O.in_projection(x, w, s)
        check_out("q", host(q), rq, io)
        check_out("k", host(k), rk, io)
        check_out("v", host(v), rv, io)
        check_f32("a", host(a), ra)
        check_f32("b", host(b), rb)
        outs.append((q, k, v, a, b))
    for t0, t2 in zip(outs[0], outs[2]):
        assert torch.equal(t0, t2), "the same input gave different outputs"
    assert pool.error() == 0


@pytest.mark.parametrize("n_tok,io", [(64, "bf16"), (1000, "bf16"), (300, "f32")])
def test_in_proj_unaligned_outputs_equal_aligned(n_tok, io):
    """q, k, v starting one element into their buffers (not 16-byte aligned)
    go out element by element instead of as 16-byte vectors; the values are
    bitwise those of the aligned call, on the few-token, 128-token-tile and
    256-token-tile paths."""
    s, hidden = syn.QWEN3_NEXT, syn.QWEN3_NEXT_HIDDEN
    say(f"in_proj unaligned outputs: {n_tok} tokens io {io}")
    rng = np.random.default_rng(1400 + n_tok)
    x = dev(syn.draw_hidden(rng, (n_tok,), hidden), torch.bfloat16)
    w = dev(syn.draw_in_proj_weight(rng, s, hidden), torch.bfloat16)
    pool = make_pool(s, 1, io)
    t = torch.bfloat16 if io == "bf16" else torch.float32

    def outs(off):
        def view(shape):
            n = int(np.prod(shape))
            return torch.full((n + off,), float("nan"), dtype=t, device="cuda")[off:].view(shape)
        return (view((n_tok, s.h_k, s.d_k)), view((n_tok, s.h_k, s.d_k)), view((n_tok, s.h_v, s.d_v)),
                torch.full((n_tok, s.h_v), float("nan"), device="cuda"),
                torch.full((n_tok, s.h_v), float("nan"), device="cuda"))

    nb = pool.in_proj_workspace_bytes(n_tok, hidden)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda") if nb else None
    al, un = outs(0), outs(1)
    assert all(o.data_ptr() % 16 != 0 for o in un[:3])
    pool.in_proj(x, w, *al, ws)
    pool.in_proj(x, w, *un, ws)
    torch.cuda.synchronize()
    for name, u, v_ in zip("qkvab", al, un):
        assert torch.equal(u, v_), f"{name} differs between aligned and unaligned outputs"
    assert not torch.isnan(al[0].float()).any()
    assert pool.error() == 0


def test_in_proj_feeds_decode():
    """Hidden states -> projection -> decode step, on both sides."""
    s, io, hidden = syn.QWEN3_NEXT, "bf16", syn.QWEN3_NEXT_HIDDEN
    rng = np.random.default_rng(1300)
    n, n_slots = 8, 12
    ids_np = rng.permutation(n_slots)[:n].astype(np.int32)
    contents = syn.draw_pool_contents(1301, ids_np, s, io)
    pool = make_pool(s, n_slots, io)
    load_slots(pool, contents)
    w_conv = syn.draw_conv_weights(rng, s)
    x = syn.draw_hidden(rng, (n,), hidden)
    w = syn.draw_in_proj_weight(rng, s, hidden)
    q, k, v, a, b, _ = _project(pool, s, x, w, io)
    out = torch.empty((n, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda")
    pool.decode(0, dev(ids_np, torch.int32), q, k, v, a, b, dev(w_conv), out)
    torch.cuda.synchronize()
    rq, rk, rv, ra, rb = O.in_projection(x, w, s)
    # the decode consumes the projection rounded to the io dtype, as stored
    rq, rk, rv = (syn.bf16_round(t).astype(np.float64) for t in (rq, rk, rv))
    op = oracle_pool(s, contents, ids_np)
    ref = op.decode(0, np.arange(n), rq, rk, rv, ra, rb, w_conv)
    check_out("decode outputs", host(out), ref, io)
    check_f32("states", host(pool.state[torch.from_numpy(ids_np.astype(np.int64)).cuda()]), op.S)


def test_in_proj_rejects_unsupported_hidden():
    import gated_deltanet_state_layer_amd as G
    s = syn.Shapes(2, 2, 32, 32, 4)
    pool = make_pool(s, 1, "f32")
    with pytest.raises(G.GdnError) as ei:
        pool.in_proj_workspace_bytes(4, 100)
    assert ei.value.status == -2


@pytest.mark.parametrize("i", range(24))
def test_in_proj_random_configuration_vs_oracle(i):
    """24 seeded random configurations: q/k heads 1-4, 1-4 value heads per
    group, d 32/64/128, hidden sizes 32-4096 (multiples of 32), 1 to 3000
    tokens (the skinny, split-hidden, 128-tile and 256-tile paths, ragged
    rows and channels), bf16 and fp32 io, against the oracle."""
    rng = np.random.default_rng(777 + 8191 * i)
    h_k = int(rng.integers(1, 5))
    d = int(rng.choice([32, 64, 128]))
    s = syn.Shapes(h_k, h_k * int(rng.choice([1, 2, 3, 4])), d, d, 4)
    hidden = 32 * int(rng.integers(1, 129))
    n_tok = int(rng.choice([1, 5, 64, 65, 200, 511, 512, 700, 1500, 3000]))
    io = str(rng.choice(["bf16", "f32"]))
    x = syn.draw_hidden(rng, (n_tok,), hidden)
    w = syn.draw_in_proj_weight(rng, s, hidden)
    pool = make_pool(s, 1, io)
    q, k, v, a, b, nb = _project(pool, s, x, w, io)
    say(f"in_proj sweep {i}: {s} hidden {hidden} tokens {n_tok} io {io} workspace {nb}")
    rq, rk, rv, ra, rb = O.in_projection(x, w, s)
    check_out("q", host(q), rq, io)
    check_out("k", host(k), rk, io)
    check_out("v", host(v), rv, io)
    check_f32("a", host(a), ra)
    check_f32("b", host(b), rb)
    assert pool.error() == 0
