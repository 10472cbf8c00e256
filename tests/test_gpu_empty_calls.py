"""GPU: calls with nothing to do (no entries, no sequences, sequences of no
tokens, no tokens to project) return OK, enqueue nothing that touches the
pool, and leave every slot, window and ring bitwise unchanged."""
import numpy as np
import pytest

import gdn_synth as syn
from gpu_util import dev, make_pool, say, scramble_pool

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_state_layer_amd import binding
    binding.load_library()


def _snapshot(pool):
    torch.cuda.synchronize()
    return pool.state.clone(), pool.window.clone()


def _unchanged(pool, snap):
    torch.cuda.synchronize()
    return torch.equal(pool.state, snap[0]) and torch.equal(pool.window, snap[1])


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_empty_calls_are_no_ops(io):
    s = syn.Shapes(2, 4, 64, 64, 4)
    say(f"empty calls: {s} io={io}")
    t = torch.bfloat16 if io == "bf16" else torch.float32
    pool = make_pool(s, 6, io, ring_len=8)
    scramble_pool(pool, 5)
    snap = _snapshot(pool)
    w = dev(syn.draw_conv_weights(np.random.default_rng(3), s))
    none = torch.empty(0, dtype=torch.int32, device="cuda")

    # no entries
    def tok(n, n_tok=None):
        lead = (n,) if n_tok is None else (n, n_tok)
        return (torch.empty(lead + (s.h_k, s.d_k), dtype=t, device="cuda"),
                torch.empty(lead + (s.h_k, s.d_k), dtype=t, device="cuda"),
                torch.empty(lead + (s.h_v, s.d_v), dtype=t, device="cuda"),
                torch.empty(lead + (s.h_v,), device="cuda"),
                torch.empty(lead + (s.h_v,), device="cuda"))
    q, k, v, a, b = tok(0)
    pool.decode(0, none, q, k, v, a, b, w, torch.empty((0, s.h_v, s.d_v), dtype=t, device="cuda"))
    q, k, v, a, b = tok(0, 4)
    pool.verify(0, none, 4, q, k, v, a, b, w, none,
                torch.empty((0, 4, s.h_v, s.d_v), dtype=t, device="cuda"))
    pool.ring_verify(0, none, 4, q, k, v, a, b, w,
                     torch.empty((0, 4, s.h_v, s.d_v), dtype=t, device="cuda"))
    pool.ring_commit(0, none, 4, q, k, v, a, b, w, none)
    pool.ring_flush(0, none)
    pool.reset(none)
    pool.copy(none, none)
    assert _unchanged(pool, snap), "a call with no entries changed the pool"

    # no sequences, then sequences of no tokens (their slots untouched)
    ws = torch.empty(max(pool.prefill_workspace_bytes(2, 0, 64), 256), dtype=torch.uint8,
                     device="cuda")
    q, k, v, a, b = tok(0)
    out = torch.empty((0, s.h_v, s.d_v), dtype=t, device="cuda")
    pool.prefill(0, dev(np.array([0], np.int32), torch.int32), none, 0, 64, q, k, v, a, b, w,
                 out, ws)
    pool.prefill(0, dev(np.array([0, 0, 0], np.int32), torch.int32),
                 dev(np.array([1, 4], np.int32), torch.int32), 0, 64, q, k, v, a, b, w, out, ws)
    assert _unchanged(pool, snap), "a prefill of no tokens changed the pool"

    # no tokens to project
    hidden = 64
    x = torch.empty((0, hidden), dtype=torch.bfloat16, device="cuda")
    wp = torch.empty((s.h_k * s.d_k * 2 + s.h_v * s.d_v + 2 * s.h_v, hidden),
                     dtype=torch.bfloat16, device="cuda")
    q, k, v, a, b = tok(0)
    pool.in_proj(x, wp, q, k, v, a, b)
    assert _unchanged(pool, snap)
    assert pool.error() == 0


def test_binding_rejects_undersized_or_mistyped_tensors():
    """The binding checks each tensor argument on the host (device,
    contiguity, dtype, element count against the call's shapes) before it
    becomes a raw pointer; a bad one raises ValueError and nothing runs."""
    s, io = syn.Shapes(2, 4, 64, 64, 4), "bf16"
    say("binding argument checks")
    pool = make_pool(s, 4, io)
    scramble_pool(pool, 6)
    snap = _snapshot(pool)
    n = 2
    ids = dev(np.array([0, 1], np.int32), torch.int32)
    w = dev(syn.draw_conv_weights(np.random.default_rng(4), s))
    good = {"q": torch.zeros((n, s.h_k, s.d_k), dtype=torch.bfloat16, device="cuda"),
            "k": torch.zeros((n, s.h_k, s.d_k), dtype=torch.bfloat16, device="cuda"),
            "v": torch.zeros((n, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda"),
            "a": torch.ones((n, s.h_v), device="cuda"),
            "b": torch.zeros((n, s.h_v), device="cuda")}
    out = torch.zeros((n, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda")
    bad_cases = {
        "v": good["v"][:1],                                   # too few elements
        "q": good["q"].float(),                               # wrong dtype
        "a": torch.ones((s.h_v, n), device="cuda").t(),       # not contiguous
        "b": good["b"].cpu(),                                 # not on the device
    }
    for name, bad in bad_cases.items():
        args = dict(good)
        args[name] = bad
        with pytest.raises(ValueError):
            pool.decode(0, ids, args["q"], args["k"], args["v"], args["a"], args["b"], w, out)
    with pytest.raises(ValueError):
        pool.decode(0, ids.long(), good["q"], good["k"], good["v"], good["a"], good["b"], w, out)
    with pytest.raises(ValueError):
        pool.decode(0, ids, good["q"], good["k"], good["v"], good["a"], good["b"], w, out[:1])
    assert _unchanged(pool, snap)
    pool.decode(0, ids, good["q"], good["k"], good["v"], good["a"], good["b"], w, out)
    assert pool.error() == 0
