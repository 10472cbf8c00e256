"""GPU: the calls recorded into a HIP graph (they enqueue kernels only, no
memset nodes, no host synchronisation) and replayed several times, with
eager work and synchronisations between replays, equal the same calls made
eagerly on a twin pool, bitwise, at every replay."""
from __future__ import annotations

import numpy as np
import pytest

import gdn_synth as syn
from gpu_util import dev, load_slots, make_pool, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_state_layer_amd import binding
    binding.load_library()


def _twins(s, n_slots, ids_np, io, seed):
    contents = syn.draw_pool_contents(seed, ids_np, s, io)
    pa, pb = make_pool(s, n_slots, io), make_pool(s, n_slots, io)
    load_slots(pa, contents)
    load_slots(pb, contents)
    return pa, pb


def _capture(fn):
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("n", [4, 64])
def test_graph_replayed_decode_equals_eager(n):
    s, io = syn.QWEN3_NEXT, "bf16"
    say(f"graph decode: N={n}")
    rng = np.random.default_rng(900 + n)
    n_slots = n + 8
    ids_np = rng.permutation(n_slots)[:n].astype(np.int32)
    pa, pb = _twins(s, n_slots, ids_np, io, 61)
    w = dev(syn.draw_conv_weights(rng, s))
    ids = dev(ids_np, torch.int32)
    shapes = {"q": (n, s.h_k, s.d_k), "k": (n, s.h_k, s.d_k), "v": (n, s.h_v, s.d_v),
              "a": (n, s.h_v), "b": (n, s.h_v)}
    buf = {m: torch.zeros(sh, dtype=torch.bfloat16 if m in "qkv" else torch.float32,
                          device="cuda") for m, sh in shapes.items()}
    out_a = torch.zeros((n, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda")
    out_b = torch.zeros_like(out_a)
    g = _capture(lambda: pa.decode(0, ids, buf["q"], buf["k"], buf["v"], buf["a"], buf["b"], w,
                                   out_a))
    # the capture itself ran nothing: the pools are still equal
    assert torch.equal(pa.state, pb.state) and torch.equal(pa.window, pb.window)
    for r in range(4):
        tok = syn.draw_tokens(rng, s, (n,), io)
        for m in buf:
            buf[m].copy_(torch.from_numpy(tok[m]).to(buf[m].dtype))
        torch.cuda.synchronize()
        g.replay()
        pb.decode(0, ids, buf["q"], buf["k"], buf["v"], buf["a"], buf["b"], w, out_b)
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b), f"replay {r}: outputs differ"
        assert torch.equal(pa.state, pb.state), f"replay {r}: states differ"
        assert torch.equal(pa.window, pb.window), f"replay {r}: windows differ"
    assert pa.error() == 0


def test_graph_replayed_verify_and_prefill_equal_eager():
    s, io = syn.QWEN3_NEXT, "bf16"
    say("graph verify + prefill")
    rng = np.random.default_rng(950)
    n, n_tok, n_slots = 16, 4, 24
    ids_np = rng.permutation(n_slots)[:n].astype(np.int32)
    pa, pb = _twins(s, n_slots, ids_np, io, 62)
    w = dev(syn.draw_conv_weights(rng, s))
    ids = dev(ids_np, torch.int32)
    acc = dev((np.arange(n) % (n_tok + 1)).astype(np.int32), torch.int32)
    vb = {m: torch.zeros((n, n_tok) + sh, dtype=torch.bfloat16 if m in "qkv" else torch.float32,
                         device="cuda")
          for m, sh in {"q": (s.h_k, s.d_k), "k": (s.h_k, s.d_k), "v": (s.h_v, s.d_v),
                        "a": (s.h_v,), "b": (s.h_v,)}.items()}
    vo_a = torch.zeros((n, n_tok, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda")
    vo_b = torch.zeros_like(vo_a)
    # prefill of two sequences (200 and 130 tokens) into two of the slots
    cu_np = np.array([0, 200, 330], np.int32)
    T = int(cu_np[-1])
    p_ids = dev(ids_np[:2], torch.int32)
    cu = dev(cu_np, torch.int32)
    pbuf = {m: torch.zeros((T,) + sh, dtype=torch.bfloat16 if m in "qkv" else torch.float32,
                           device="cuda")
            for m, sh in {"q": (s.h_k, s.d_k), "k": (s.h_k, s.d_k), "v": (s.h_v, s.d_v),
                          "a": (s.h_v,), "b": (s.h_v,)}.items()}
    po_a = torch.zeros((T, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda")
    po_b = torch.zeros_like(po_a)
    ws_a = torch.empty(pa.prefill_workspace_bytes(2, T, 64), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty_like(ws_a)

    def calls(pool, vo, po, ws):
        pool.verify(0, ids, n_tok, vb["q"], vb["k"], vb["v"], vb["a"], vb["b"], w, acc, vo)
        pool.prefill(0, cu, p_ids, T, 64, pbuf["q"], pbuf["k"], pbuf["v"], pbuf["a"], pbuf["b"],
                     w, po, ws)

    g = _capture(lambda: calls(pa, vo_a, po_a, ws_a))
    for r in range(3):
        tv = syn.draw_tokens(rng, s, (n, n_tok), io)
        tp = syn.draw_tokens(rng, s, (T,), io)
        for m in vb:
            vb[m].copy_(torch.from_numpy(tv[m]).to(vb[m].dtype))
            pbuf[m].copy_(torch.from_numpy(tp[m]).to(pbuf[m].dtype))
        torch.cuda.synchronize()
        g.replay()
        calls(pb, vo_b, po_b, ws_b)
        torch.cuda.synchronize()
        assert torch.equal(vo_a, vo_b), f"replay {r}: verify outputs differ"
        assert torch.equal(po_a, po_b), f"replay {r}: prefill outputs differ"
        assert torch.equal(pa.state, pb.state), f"replay {r}: states differ"
        assert torch.equal(pa.window, pb.window), f"replay {r}: windows differ"
    assert pa.error() == 0


@pytest.mark.parametrize("n,n_slots", [(16, 24), (40, 48)])
def test_graph_replayed_ring_cycle_equals_eager(n, n_slots):
    """A verify-ring cycle (ring_verify then ring_commit with acceptance
    read from device memory) recorded once and replayed through appends and
    folds; ring counts, records, states, windows and outputs equal the eager
    twin at every replay.  With 40 entries (1280 commit items) the commit
    runs persistent."""
    s, io, n_tok = syn.QWEN3_NEXT, "bf16", 4
    say(f"graph ring cycle, {n} entries")
    rng = np.random.default_rng(970 + n)
    ids_np = rng.permutation(n_slots)[:n].astype(np.int32)
    contents = syn.draw_pool_contents(63, ids_np, s, io)
    pa, pb = make_pool(s, n_slots, io, ring_len=8), make_pool(s, n_slots, io, ring_len=8)
    load_slots(pa, contents)
    load_slots(pb, contents)
    w = dev(syn.draw_conv_weights(rng, s))
    ids = dev(ids_np, torch.int32)
    acc = torch.zeros(n, dtype=torch.int32, device="cuda")
    vb = {m: torch.zeros((n, n_tok) + sh, dtype=torch.bfloat16 if m in "qkv" else torch.float32,
                         device="cuda")
          for m, sh in {"q": (s.h_k, s.d_k), "k": (s.h_k, s.d_k), "v": (s.h_v, s.d_v),
                        "a": (s.h_v,), "b": (s.h_v,)}.items()}
    out_a = torch.zeros((n, n_tok, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda")
    out_b = torch.zeros_like(out_a)

    def cycle(pool, out):
        pool.ring_verify(0, ids, n_tok, vb["q"], vb["k"], vb["v"], vb["a"], vb["b"], w, out)
        pool.ring_commit(0, ids, n_tok, vb["q"], vb["k"], vb["v"], vb["a"], vb["b"], w, acc)

    g = _capture(lambda: cycle(pa, out_a))
    assert torch.equal(pa.state, pb.state) and torch.equal(pa.ring_count, pb.ring_count)
    folded = False
    for r in range(6):
        tv = syn.draw_tokens(rng, s, (n, n_tok), io)
        for m in vb:
            vb[m].copy_(torch.from_numpy(tv[m]).to(vb[m].dtype))
        acc.copy_(torch.from_numpy(rng.integers(1, n_tok + 1, size=n).astype(np.int32)))
        torch.cuda.synchronize()
        before = pa.ring_count.clone()
        g.replay()
        cycle(pb, out_b)
        torch.cuda.synchronize()
        folded |= bool(((pa.ring_count < before) & (before > 0)).any())
        assert torch.equal(out_a, out_b), f"replay {r}: outputs differ"
        assert torch.equal(pa.ring_count, pb.ring_count), f"replay {r}: ring counts differ"
        assert torch.equal(pa.ring_records, pb.ring_records), f"replay {r}: ring records differ"
        assert torch.equal(pa.state, pb.state), f"replay {r}: states differ"
        assert torch.equal(pa.window, pb.window), f"replay {r}: windows differ"
    assert folded, "no replay folded a ring"
    assert pa.error() == 0


@pytest.mark.parametrize("n_tok", [64, 300, 1000])
def test_graph_replayed_in_proj_equals_eager(n_tok):
    """The input projection on each of its paths (skinny; split hidden with
    the partial-sum kernel; 256-token tiles plus the skinny gate strip),
    recorded once and replayed with new hidden states, equals eager calls
    bitwise at every replay."""
    s, hidden = syn.QWEN3_NEXT, syn.QWEN3_NEXT_HIDDEN
    say(f"graph in_proj: {n_tok} tokens")
    rng = np.random.default_rng(970 + n_tok)
    pool = make_pool(s, 1, "bf16")
    w = dev(syn.draw_in_proj_weight(rng, s, hidden), torch.bfloat16)
    x = torch.zeros((n_tok, hidden), dtype=torch.bfloat16, device="cuda")
    nb = pool.in_proj_workspace_bytes(n_tok, hidden)

    def outs():
        return {"q": torch.zeros((n_tok, s.h_k, s.d_k), dtype=torch.bfloat16, device="cuda"),
                "k": torch.zeros((n_tok, s.h_k, s.d_k), dtype=torch.bfloat16, device="cuda"),
                "v": torch.zeros((n_tok, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda"),
                "a": torch.zeros((n_tok, s.h_v), device="cuda"),
                "b": torch.zeros((n_tok, s.h_v), device="cuda"),
                "ws": torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda") if nb else None}

    oa, ob = outs(), outs()
    g = _capture(lambda: pool.in_proj(x, w, oa["q"], oa["k"], oa["v"], oa["a"], oa["b"], oa["ws"]))
    for r in range(3):
        x.copy_(torch.from_numpy(syn.draw_hidden(rng, (n_tok,), hidden)).to(torch.bfloat16))
        torch.cuda.synchronize()
        g.replay()
        pool.in_proj(x, w, ob["q"], ob["k"], ob["v"], ob["a"], ob["b"], ob["ws"])
        torch.cuda.synchronize()
        for m in "qkvab":
            assert torch.equal(oa[m], ob[m]), f"replay {r}: {m} differs"
    assert pool.error() == 0
