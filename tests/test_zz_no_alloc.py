"""The no-allocation prefill entry point (gdn_prefill_chunked_static),
called through the C ABI, against gdn_prefill_chunked with a caller-owned
workspace: two calls in a row on the same pools, the second smaller, so a
call that read stale contents of the shared device array would show."""
import numpy as np
import pytest

import gdn_synth as syn
from gpu_util import check_f32, check_out, dev, host, load_slots, make_pool, say, tokens_to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_state_layer_amd import binding
    binding.load_library()


def _pair(s, io, lens, ids, seed, contents, chunk=64):
    """The same prefill on two identical pools, one per entry point."""
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    rng = np.random.default_rng(seed)
    tok = syn.draw_tokens(rng, s, (T,), io)
    w = dev(syn.draw_conv_weights(rng, s))
    td = tokens_to_dev(tok, io)
    outs = []
    for pool, static in ((_POOLS[0], False), (_POOLS[1], True)):
        out = torch.full((T, s.h_v, s.d_v), float("nan"), dtype=pool.io_torch, device="cuda")
        args = (0, dev(cu, torch.int32), dev(ids, torch.int32), T, chunk, td["q"], td["k"], td["v"],
                td["a"], td["b"], w, out)
        if static:
            pool.prefill_static(*args)
        else:
            ws = torch.empty(max(pool.prefill_workspace_bytes(len(ids), T, chunk), 256),
                             dtype=torch.uint8, device="cuda")
            pool.prefill(*args, ws)
        outs.append(out)
    torch.cuda.synchronize()
    return outs


_POOLS = []


def test_static_prefill_equals_workspace_prefill_twice():
    from gated_deltanet_state_layer_amd import binding as G
    s, io = syn.QWEN3_NEXT, "bf16"
    _POOLS[:] = [make_pool(s, 8, io), make_pool(s, 8, io)]
    contents = syn.draw_pool_contents(5, [1, 4, 6], s, io)
    for p in _POOLS:
        load_slots(p, contents)
    # first call: 3 sequences filling about 3/4 of the array
    cap = G.GDN_STATIC_SCRATCH_BYTES
    per_tok = _POOLS[1].prefill_workspace_bytes(1, 6400, 64) / 6400
    n1 = int(0.75 * cap / per_tok)
    lens, ids = np.array([n1 * 6 // 10, 33, n1 - n1 * 6 // 10 - 33]), np.array([1, 4, 6], np.int32)
    need = _POOLS[1].prefill_workspace_bytes(3, int(lens.sum()), 64)
    say(f"call 1: {lens.tolist()} tokens, workspace {need} of {G.GDN_STATIC_SCRATCH_BYTES} B")
    assert need <= G.GDN_STATIC_SCRATCH_BYTES
    o_ws, o_st = _pair(s, io, lens, ids, 11, contents)
    check_out("call 1 outputs, static vs workspace", host(o_st), host(o_ws), io)
    assert torch.equal(o_st, o_ws), "call 1: outputs differ bitwise"
    assert torch.equal(_POOLS[1].state, _POOLS[0].state) and torch.equal(_POOLS[1].window, _POOLS[0].window)
    # second call, smaller: 2 sequences, 150 tokens, continuing slot 4 and a fresh slot 2
    lens, ids = np.array([90, 60]), np.array([4, 2], np.int32)
    say(f"call 2: {lens.tolist()} tokens")
    o_ws, o_st = _pair(s, io, lens, ids, 12, contents)
    check_out("call 2 outputs, static vs workspace", host(o_st), host(o_ws), io)
    check_f32("call 2 states, static vs workspace", host(_POOLS[1].state), host(_POOLS[0].state))
    assert torch.equal(o_st, o_ws), "call 2: outputs differ bitwise"
    assert torch.equal(_POOLS[1].state, _POOLS[0].state) and torch.equal(_POOLS[1].window, _POOLS[0].window)
    assert _POOLS[0].error() == 0 and _POOLS[1].error() == 0


def test_static_prefill_rejects_a_call_beyond_the_array():
    from gated_deltanet_state_layer_amd import binding as G
    s, io = syn.QWEN3_NEXT, "bf16"
    pool = make_pool(s, 2, io)
    T = 64
    while pool.prefill_workspace_bytes(1, T, 64) <= G.GDN_STATIC_SCRATCH_BYTES:
        T += 64
    st0 = pool.state.clone()
    td = tokens_to_dev(syn.draw_tokens(np.random.default_rng(3), s, (T,), io), io)
    w = dev(syn.draw_conv_weights(np.random.default_rng(4), s))
    out = torch.full((T, s.h_v, s.d_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(G.GdnError) as e:
        pool.prefill_static(0, dev(np.array([0, T], np.int32), torch.int32),
                            dev(np.array([1], np.int32), torch.int32), T, 64, td["q"], td["k"],
                            td["v"], td["a"], td["b"], w, out)
    assert e.value.status == G.GDN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.equal(pool.state, st0) and torch.isnan(out.float()).all()
