"""GPU parity sweep: a decode step and then a verify call through the C ABI
against the fp64 oracle on 40 seeded random configurations (q/k heads 1-2,
1-4 value heads per group, d 32/64/128, conv widths 2-8, bf16 and fp32 io,
1 to 130 entries over pools of up to 300 pre-filled slots, padding entries,
1-8 verify tokens, accepted lengths 0..n_tok).  The entry counts cover the
decode kernels' row-split, per-head and one-workgroup-per-group paths.

Each step checks the outputs (the io dtype's criterion), the states (1e-3
relative to their RMS: decode and verify are fp32 throughout), the windows
bitwise and every slot the call does not name bitwise."""
import numpy as np
import pytest

import gdn_synth as syn
from gpu_util import (check_f32, check_out, dev, host, load_slots, make_pool, oracle_pool, say,
                      scramble_pool, tokens_to_dev)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

N_CASES = 40


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_state_layer_amd import binding
    binding.load_library()


def _check_slots(pool, op, ids_np, valid, st0, wn0, n_slots, what):
    idx = [int(x) for x in ids_np[valid]]
    rows = np.nonzero(valid)[0]
    if idx:
        t = torch.tensor(idx, dtype=torch.int64, device="cuda")
        check_f32(f"{what} states", host(pool.state[t]), op.S[rows])
        assert np.array_equal(host(pool.window[t]), op.X[rows]), f"{what} windows"
    for sl in range(n_slots):
        if sl not in idx:
            assert torch.equal(pool.state[sl], st0[sl]) and torch.equal(pool.window[sl], wn0[sl]), \
                f"{what}: slot {sl} changed"


@pytest.mark.parametrize("i", range(N_CASES))
def test_decode_then_verify_random_configuration_vs_oracle(i):
    rng = np.random.default_rng(31337 + 104729 * i)
    h_k = int(rng.integers(1, 3))
    h_v = h_k * int(rng.choice([1, 2, 3, 4]))
    d = int(rng.choice([32, 64, 128]))
    s = syn.Shapes(h_k, h_v, d, d, int(rng.choice([2, 3, 4, 4, 4, 6, 8])))
    io = str(rng.choice(["bf16", "f32"]))
    n = int(rng.choice([1, 2, 4, 7, 16, 33, 64, 130]))
    n_slots = int(min(300, n + rng.integers(0, 2 * n + 8)))
    ids_np = rng.permutation(n_slots)[:n].astype(np.int32)
    ids_np[rng.random(n) < 0.1] = -1
    valid = ids_np >= 0
    n_tok = int(rng.integers(1, 9))
    acc_np = rng.integers(0, n_tok + 1, n).astype(np.int32)
    say(f"sweep {i}: {s} io={io} entries={n} of {n_slots} slots pads={int((~valid).sum())} "
        f"verify n_tok={n_tok}")
    w_np = syn.draw_conv_weights(rng, s)
    w = dev(w_np)
    pool = make_pool(s, n_slots, io)
    scramble_pool(pool, int(rng.integers(1 << 30)))
    named = [int(x) for x in ids_np[valid]]
    contents = syn.draw_pool_contents(int(rng.integers(1 << 30)), np.array(named, np.int64), s, io) \
        if named else {}
    if contents:
        load_slots(pool, contents)
    op = oracle_pool(s, contents, np.where(valid, ids_np, 0), form="rank1")
    ids = dev(ids_np, torch.int32)

    # one decode step
    st0, wn0 = pool.state.clone(), pool.window.clone()
    d1 = syn.draw_tokens(rng, s, (n,), io)
    td = tokens_to_dev(d1, io)
    out = torch.full((n, s.h_v, s.d_v), float("nan"), dtype=pool.io_torch, device="cuda")
    pool.decode(0, ids, td["q"], td["k"], td["v"], td["a"], td["b"], w, out)
    torch.cuda.synchronize()
    assert pool.error() == 0
    ref = op.decode(0, np.where(valid, np.arange(n), -1), d1["q"], d1["k"], d1["v"], d1["a"],
                    d1["b"], w_np)
    if valid.any():
        check_out("decode outputs", host(out)[valid], ref[valid], io)
    assert torch.isnan(out[torch.from_numpy(~valid).cuda()].float()).all(), "padding rows written"
    _check_slots(pool, op, ids_np, valid, st0, wn0, n_slots, "decode")

    # then a verify call on the same entries
    st0, wn0 = pool.state.clone(), pool.window.clone()
    d2 = syn.draw_tokens(rng, s, (n, n_tok), io)
    td = tokens_to_dev(d2, io)
    out = torch.full((n, n_tok, s.h_v, s.d_v), float("nan"), dtype=pool.io_torch, device="cuda")
    pool.verify(0, ids, n_tok, td["q"], td["k"], td["v"], td["a"], td["b"], w,
                dev(acc_np, torch.int32), out)
    torch.cuda.synchronize()
    assert pool.error() == 0
    ref = op.verify(0, np.where(valid, np.arange(n), -1), n_tok, d2["q"], d2["k"], d2["v"], d2["a"],
                    d2["b"], w_np, acc_np)
    if valid.any():
        check_out("verify outputs", host(out)[valid], ref[valid], io)
    _check_slots(pool, op, ids_np, valid, st0, wn0, n_slots, "verify")
