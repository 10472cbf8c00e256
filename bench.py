#!/usr/bin/env python3
"""Benchmark of the GDN state layer on one MI355X.

Headline workload: one multi-slot decode step of a Qwen3-Next-shaped GDN
layer (h_k=16, h_v=32, d_k=d_v=128, conv_k=4, bf16 io, fp32 state) for 64
active slots of a 256-slot pool.  Consecutive steps rotate over four
disjoint 64-slot subsets (512 MiB of state in total, twice the 256 MB
last-level cache), so every step streams its state from HBM.

Printed: one JSON line.  `value` is decode tokens/s at 64 slots; the line
also carries the state bandwidth, the roofline of the decode kernel (HIP
events on the launch stream), the speculative-verify and chunked-prefill
figures measured in the same run, and the CPU oracle baseline.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu] [--no-prefill]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published

# HBM traffic of the decode kernel (decode_heads_kernel, in decode_rows.hip)
# from two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per
# dispatch, averaged over the timed launches), each scaled by bytes / counter
# of torch's copy kernel over 512 MiB measured the same way
# (profiles/decode_hbm_traffic.txt).  Valid only for the kernel source they
# were taken on: DECODE_SRC_SHA256 is checked at run time and the traffic is
# reported as null when the source has changed since.
DECODE_TRAFFIC = {"fetch_kib": 68900.93, "write_kib": 134753.09,
                  "copy_fetch_scale": 536870912 / (262155.93 * 1024),
                  "copy_write_scale": 536870912 / (524288.0 * 1024)}
DECODE_SRC_SHA256 = "e5a23a53c65d1cf4245f064aad40c171f2ead96029a3935eab7040e4be21e843"


# Executed bf16 MFMA flops of the prefill kernels per token, from rocprofv3
# counter runs (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512, factor + scan, median
# dispatch; profiles/prefill_mfma_counters.txt): the hi/lo bf16 split and the
# padded tiles make them ~3.2x the algorithmic flops.  Valid for the prefill
# source they were taken on (PREFILL_SRC_SHA256), else reported as null.
PREFILL_MFMA_FLOP_PER_TOKEN = {"single": (1.573e7 + 2.013e8) * 512 / 8192,
                               "varlen": (7.016e7 + 8.981e8) * 512 / 36080}
# (profiles/prefill_mfma_counters.txt; profiles/prefill_hbm_traffic.txt has the bytes)
PREFILL_SRC_SHA256 = "84b624e214c3583cb0e7844ac956ad3cd8863a806430b2bcce5e5a9c7cb0c167"


def prefill_exec_flop_per_token(case):
    import hashlib
    src = os.path.join(ROOT, "gated_deltanet_state_layer_amd", "csrc", "prefill.hip")
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != PREFILL_SRC_SHA256:
        return None
    return PREFILL_MFMA_FLOP_PER_TOKEN.get(case)


def decode_traffic_bytes():
    """Counter-based HBM bytes per decode launch, or None if unmeasured or stale."""
    import hashlib
    if not DECODE_TRAFFIC or not DECODE_SRC_SHA256:
        return None
    src = os.path.join(ROOT, "gated_deltanet_state_layer_amd", "csrc", "decode_rows.hip")
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != DECODE_SRC_SHA256:
        return None
    t = DECODE_TRAFFIC
    return (t["fetch_kib"] * 1024 * t["copy_fetch_scale"] +
            t["write_kib"] * 1024 * t["copy_write_scale"])


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-verify", action="store_true")
    p.add_argument("--no-ring", action="store_true")
    p.add_argument("--no-in-proj", action="store_true")
    p.add_argument("--only", choices=["decode", "verify", "ring", "in_proj", "prefill", "copy",
                                      "gemm", "stream"],
                   default=None,
                   help="run one workload only (for profiling)")
    p.add_argument("--prefill-case", choices=["single", "split512", "varlen", "all"], default="all",
                   help="prefill workloads to run (for profiling one of them)")
    return p.parse_args()


def decode_bytes_per_slot(s, io_size=2):
    state = 2 * s.h_v * s.d_v * s.d_k * 4
    qkv = (2 * s.h_k * s.d_k + s.h_v * s.d_v) * io_size
    ab = 2 * s.h_v * 4
    win = (s.conv_k - 1) * s.c_conv * io_size + s.c_conv * io_size   # read window, write new column
    out = s.h_v * s.d_v * io_size
    return state + qkv + ab + win + out + 4


def verify_bytes_per_slot(s, n_tok, io_size=2):
    state = 2 * s.h_v * s.d_v * s.d_k * 4
    qkv = n_tok * (2 * s.h_k * s.d_k + s.h_v * s.d_v) * io_size
    ab = n_tok * 2 * s.h_v * 4
    win = 2 * (s.conv_k - 1) * s.c_conv * io_size
    out = n_tok * s.h_v * s.d_v * io_size
    return state + qkv + ab + win + out + 8


def time_launches(fn, steps, warmup, torch):
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(i)
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps * 1e-3   # seconds per launch


def time_graph(fn, n_inner, replays, torch):
    """Seconds per call of fn, captured n_inner times into one HIP graph and
    replayed: the device-side rate without the host launch cost."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            for _ in range(n_inner):
                fn()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / (replays * n_inner)


def launch_percentiles(fn, n, torch):
    """Per-launch durations (events around each launch on the current
    stream): p10 / median / p90 in microseconds."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (a, b) in enumerate(ev):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    d = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    return {"p10_us": float(np.percentile(d, 10)), "median_us": float(np.median(d)),
            "p90_us": float(np.percentile(d, 90))}


def bench_decode(args, torch, G, syn):
    s = syn.QWEN3_NEXT
    n_slots, N, n_sets = 256, 64, 4
    pool = G.Pool(G.make_desc(n_slots, 1, s.h_k, s.h_v, s.d_k, s.d_v, s.conv_k, G.GDN_BF16))
    gen = torch.Generator(device="cuda").manual_seed(1234)
    pool.state.normal_(generator=gen)
    pool.window.copy_(torch.randn(pool.window.shape, generator=gen, device="cuda").bfloat16())
    rng = np.random.default_rng(1001)
    perm = rng.permutation(n_slots).astype(np.int32)
    sets = []
    w = torch.from_numpy(syn.draw_conv_weights(rng, s)).cuda()
    for j in range(n_sets):
        tok = syn.draw_tokens(rng, s, (N,), "bf16")
        d = {n: torch.from_numpy(tok[n]).cuda() for n in "ab"}
        d.update({n: torch.from_numpy(tok[n]).bfloat16().cuda() for n in "qkv"})
        d["ids"] = torch.from_numpy(perm[j * N:(j + 1) * N].copy()).cuda()
        sets.append(d)
    out = torch.empty((N, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda")

    def step(i):
        d = sets[i % n_sets]
        pool.decode(0, d["ids"], d["q"], d["k"], d["v"], d["a"], d["b"], w, out)

    t = time_launches(step, args.steps, args.warmup, torch)
    per_slot = decode_bytes_per_slot(s)
    bytes_launch = N * per_slot + s.c_conv * s.conv_k * 4
    state_bytes = N * 2 * s.h_v * s.d_v * s.d_k * 4
    res = {"sec": t, "n": N, "bytes": bytes_launch, "gbps": bytes_launch / t / 1e9,
           "state_gbps": state_bytes / t / 1e9}
    if args.only == "decode":   # profiling run: the timed loop only
        return res
    res["per_launch"] = launch_percentiles(step, max(200, args.steps), torch)
    # Hot-cache figure: the same 64 slots every step.
    t_hot = time_launches(lambda i: step(0), max(20, args.steps // 4), 5, torch)
    # Small batches (latency-bound at N=1): launched from the Python loop
    # (host launch rate included) and replayed from a captured HIP graph of
    # 50 steps (device time per step).
    small, small_graph = {}, {}
    for n in (1, 4, 16):
        d = sets[0]
        ids = d["ids"][:n].clone()
        qq, kk, vv, aa, bb = (d[m][:n].contiguous() for m in "qkvab")
        o = out[:n]
        fn = lambda: pool.decode(0, ids, qq, kk, vv, aa, bb, w, o)
        small[n] = time_launches(lambda i: fn(), max(50, args.steps // 4), 10, torch)
        small_graph[n] = time_graph(fn, 50, 4, torch)
    # The step's cost does not depend on how long the context is: decode the
    # same 64 slots after a 64-token and after an 8192-token prefill of each
    # (context tokens drawn on the device; timing only).
    ctx = {}
    d0 = sets[0]
    for L in (64, 8192):
        cu = torch.arange(0, (N + 1) * L, L, dtype=torch.int32, device="cuda")
        T = N * L
        qk = torch.randn((T, 2, s.h_k, s.d_k), generator=gen, device="cuda")
        qk = qk / qk.norm(dim=-1, keepdim=True)
        qc, kc = qk[:, 0].bfloat16().contiguous(), qk[:, 1].bfloat16().contiguous()
        vc = torch.randn((T, s.h_v, s.d_v), generator=gen, device="cuda").bfloat16()
        bc = torch.sigmoid(torch.randn((T, s.h_v), generator=gen, device="cuda"))
        ac = torch.exp(-torch.nn.functional.softplus(torch.randn((T, s.h_v), generator=gen, device="cuda")))
        oc = torch.empty((T, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(pool.prefill_workspace_bytes(N, T, 64), dtype=torch.uint8, device="cuda")
        pool.reset(d0["ids"])
        pool.prefill(0, cu, d0["ids"], T, 64, qc, kc, vc, ac, bc, w, oc, ws)
        del qk, qc, kc, vc, bc, ac, oc, ws
        ctx[str(L)] = time_launches(lambda i: step(0), max(50, args.steps // 4), 10, torch) * 1e6
    assert pool.error() == 0
    res.update({
        "after_context_us": ctx,
        "sec_hot": t_hot, "hot_gbps": bytes_launch / t_hot / 1e9,
        "small": {str(n): {"us": small[n] * 1e6, "graph_us": small_graph[n] * 1e6,
                           "tok_s": n / small[n], "graph_tok_s": n / small_graph[n],
                           "gbps": (n * per_slot + s.c_conv * s.conv_k * 4) / small[n] / 1e9}
                  for n in small},
    })
    return res


def bench_verify(args, torch, G, syn):
    s = syn.QWEN3_NEXT
    n_slots, N, n_tok = 256, 128, 4
    pool = G.Pool(G.make_desc(n_slots, 1, s.h_k, s.h_v, s.d_k, s.d_v, s.conv_k, G.GDN_BF16))
    gen = torch.Generator(device="cuda").manual_seed(4321)
    pool.state.normal_(generator=gen)
    case = syn.verify_case()
    tok = case["tokens"]
    d = {n: torch.from_numpy(tok[n]).cuda() for n in "ab"}
    d.update({n: torch.from_numpy(tok[n]).bfloat16().cuda() for n in "qkv"})
    w = torch.from_numpy(case["conv_w"]).cuda()
    # Two disjoint 128-slot halves alternate so each launch streams from HBM.
    perm = np.random.default_rng(7).permutation(n_slots).astype(np.int32)
    ids = [torch.from_numpy(perm[:N].copy()).cuda(), torch.from_numpy(perm[N:].copy()).cuda()]
    acc = torch.from_numpy(case["accept_len"]).cuda()
    out = torch.empty((N, n_tok, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda")

    def step(i):
        pool.verify(0, ids[i % 2], n_tok, d["q"], d["k"], d["v"], d["a"], d["b"], w, acc, out)

    t = time_launches(step, max(50, args.steps // 2), 10, torch)
    assert pool.error() == 0
    b = N * verify_bytes_per_slot(s, n_tok) + s.c_conv * s.conv_k * 4
    return {"sec": t, "n": N, "n_tok": n_tok, "bytes": b, "gbps": b / t / 1e9,
            "tok_s": N * n_tok / t,
            "accepted_tok_s": float(case["accept_len"].sum()) / t}


def ring_record_bytes(s):
    """Bytes of one committed token in the verify ring: k^ per q/k head, v
    per value head, a and b per value head (fp32)."""
    return (s.h_k * s.d_k + s.h_v * s.d_v + 2 * s.h_v) * 4


def bench_ring(args, torch, G, syn):
    """Speculative decoding with acceptance known only after sampling, on
    the verify ring (ring of 8 = twice the 4-token speculation): per cycle,
    gdn_ring_verify (outputs) then gdn_ring_commit (the sampled accept_len).
    Same slots, tokens and alternating 128-slot halves as the one-call verify
    leg; beside it, the same cycle done with the one-call kernel (verify with
    accept_len 0, then a commit-only call)."""
    s = syn.QWEN3_NEXT
    n_slots, N, n_tok, L = 256, 128, 4, 8
    case = syn.verify_case()
    tok = case["tokens"]
    d = {n: torch.from_numpy(tok[n]).cuda() for n in "ab"}
    d.update({n: torch.from_numpy(tok[n]).bfloat16().cuda() for n in "qkv"})
    w = torch.from_numpy(case["conv_w"]).cuda()
    perm = np.random.default_rng(7).permutation(n_slots).astype(np.int32)
    ids = [torch.from_numpy(perm[:N].copy()).cuda(), torch.from_numpy(perm[N:].copy()).cuda()]
    rng = np.random.default_rng(11)
    accs_np = [rng.integers(1, n_tok + 1, size=N).astype(np.int32) for _ in range(8)]
    accs = [torch.from_numpy(x).cuda() for x in accs_np]
    zeros = torch.zeros(N, dtype=torch.int32, device="cuda")
    out = torch.empty((N, n_tok, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda")
    pool = G.Pool(G.make_desc(n_slots, 1, s.h_k, s.h_v, s.d_k, s.d_v, s.conv_k, G.GDN_BF16,
                              ring_len=L))
    pool.state.normal_(generator=torch.Generator(device="cuda").manual_seed(4321))

    def cycle(i):
        h, a_ = ids[i % 2], accs[(i // 2) % len(accs)]
        pool.ring_verify(0, h, n_tok, d["q"], d["k"], d["v"], d["a"], d["b"], w, out)
        pool.ring_commit(0, h, n_tok, d["q"], d["k"], d["v"], d["a"], d["b"], w, a_)

    steps, warm = max(50, args.steps // 2), 20
    t_cycle = time_launches(cycle, steps, warm, torch)
    # ring fill at each verify and folds at each commit, replayed on the host
    # for the same call sequence (warm-up cycles 0.., then timed cycles 0..)
    cnt = [np.zeros(N, np.int64), np.zeros(N, np.int64)]
    fill, folds, fold_fill, n_acc = 0, 0, 0, 0
    for phase, n_cyc in (("warm", warm), ("timed", steps)):
        for i in range(n_cyc):
            c, a_ = cnt[i % 2], accs_np[(i // 2) % len(accs_np)]
            f = c + a_ > L
            if phase == "timed":
                fill += int(c.sum())
                folds += int(f.sum())
                fold_fill += int((c + a_)[f].sum())
                n_acc += int(a_.sum())
            cnt[i % 2] = np.where(f, 0, c + a_)
    # verify alone at the rings' final fill (repeatable: it writes nothing)
    t_ver = time_launches(lambda i: pool.ring_verify(0, ids[i % 2], n_tok, d["q"], d["k"], d["v"],
                                                    d["a"], d["b"], w, out), steps, 10, torch)
    assert pool.error() == 0
    rec = ring_record_bytes(s)
    state = s.h_v * s.d_v * s.d_k * 4
    per_ver = verify_bytes_per_slot(s, n_tok) - state - (s.conv_k - 1) * s.c_conv * 2  # no state or window write
    ver_bytes = N * per_ver + int(cnt[0].sum() + cnt[1].sum()) // 2 * rec + s.c_conv * s.conv_k * 4
    # the same cycle with the one-call kernel: outputs (accept_len 0), then commit only
    plain = G.Pool(G.make_desc(n_slots, 1, s.h_k, s.h_v, s.d_k, s.d_v, s.conv_k, G.GDN_BF16))
    plain.state.normal_(generator=torch.Generator(device="cuda").manual_seed(4321))

    def split_cycle(i):
        h, a_ = ids[i % 2], accs[(i // 2) % len(accs)]
        plain.verify(0, h, n_tok, d["q"], d["k"], d["v"], d["a"], d["b"], w, zeros, out)
        plain.verify(0, h, n_tok, d["q"], d["k"], d["v"], d["a"], d["b"], w, a_, None)

    t_split = time_launches(split_cycle, steps, warm, torch)
    assert plain.error() == 0
    return {"workload": f"{N} slots x {n_tok} draft tokens, accept_len U{{1..{n_tok}}} after "
                        f"sampling, ring of {L}",
            "cycle_us": t_cycle * 1e6, "verify_us": t_ver * 1e6,
            "commit_us": (t_cycle - t_ver) * 1e6,
            "accepted_tok_s": n_acc / steps / t_cycle,
            "fold_rate": folds / (steps * N),
            "mean_ring_fill": fill / (steps * N),
            "verify_GBps": ver_bytes / t_ver / 1e9,
            "verify_hbm_frac": ver_bytes / t_ver / 1e9 / HBM_PEAK_GBPS,
            "one_call_kernel_split_cycle_us": t_split * 1e6}


def bench_in_proj(args, torch, G, syn):
    """The input projection (hidden 2048 -> q|k|v|a|b, 8256 channels) at a
    decode batch (64 tokens: streams the 33.8 MB weight) and at a prefill
    length (8192 tokens: a 277 GFLOP bf16 GEMM)."""
    s, H = syn.QWEN3_NEXT, syn.QWEN3_NEXT_HIDDEN
    n_out = s.c_conv + 2 * s.h_v
    pool = G.Pool(G.make_desc(1, 1, s.h_k, s.h_v, s.d_k, s.d_v, s.conv_k, G.GDN_BF16))
    w = (torch.randn((n_out, H), device="cuda") / H ** 0.5).bfloat16()
    res = {}
    for n_tok, label in ((64, "decode_64"), (8192, "prefill_8192")):
        x = torch.randn((n_tok, H), device="cuda").bfloat16()
        q = torch.empty((n_tok, s.h_k, s.d_k), dtype=torch.bfloat16, device="cuda")
        k = torch.empty_like(q)
        v = torch.empty((n_tok, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda")
        a = torch.empty((n_tok, s.h_v), device="cuda")
        b = torch.empty_like(a)
        nb = pool.in_proj_workspace_bytes(n_tok, H)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda") if nb else None
        reps = max(20, args.steps // 4) if n_tok <= 64 else 20
        t = time_launches(lambda i: pool.in_proj(x, w, q, k, v, a, b, ws), reps, 5, torch)
        flops = 2.0 * n_tok * H * n_out
        bytes_ = n_out * H * 2 + n_tok * H * 2 + n_tok * (s.c_conv * 2 + 2 * s.h_v * 4)
        res[label] = {"tokens": n_tok, "us": t * 1e6, "GBps": bytes_ / t / 1e9,
                      "hbm_frac": bytes_ / t / 1e9 / HBM_PEAK_GBPS,
                      "TFLOPs": flops / t / 1e12, "mfma_frac": flops / t / 1e12 / BF16_PEAK_TFLOPS,
                      "split_hidden": nb > 0}
    assert pool.error() == 0
    res["workload"] = f"hidden {H} -> {n_out} channels (q|k|v|a|b), bf16 x and W, synthetic"
    return res


def prefill_flops_per_token(s, C, kernel_form=False):
    """Algorithmic flops per token of the chunked form (2 per multiply-add,
    triangular products counted as triangles, incl. the diagonal), per chunk
    divided by C, in the WY form of the chunked delta rule:
      per q/k head:   K K^T and Q K^T (lower triangles)         2 * C(C+1)/2 * d_k * 2
      per value head: (I+A)^-1 by substitution                    C^3 / 3
                      W = T diag(b gamma) K, U_v = T diag(b) V,
                      P U (triangles)                             3 * C(C+1)/2 * d * 2
                      W S0^T, Q S0^T, U^T K' (dense)              3 * C * d_k * d_v * 2
    (4.254 MFLOP per token at the Qwen3-Next shapes, chunk 64).  The kernels
    form U = T'(V - diag(gamma) K S0^T) instead of W and U_v, one triangular
    product fewer per value head (3.988 MFLOP per token: kernel_form=True)."""
    dk, dv = s.d_k, s.d_v
    tri = C * (C + 1) / 2
    per_k = 2 * tri * dk * 2
    n_tri = 2 if kernel_form else 3
    per_v = C ** 3 / 3.0 + n_tri * tri * dv * 2 + 3 * C * dk * dv * 2
    return (s.h_k * per_k + s.h_v * per_v) / C


def _prefill_inputs(torch, tok):
    d = {n: torch.from_numpy(tok[n]).cuda() for n in "ab"}
    d.update({n: torch.from_numpy(tok[n]).bfloat16().cuda() for n in "qkv"})
    return d


def _time_prefill(args, torch, pool, cu_list, ids, d, w, out, C, reps):
    """Time one prefill pass made of the given calls (each (t0, t1, cu) over
    the packed token range [t0, t1)).  The slots keep their state between
    repetitions: the kernels do the same work for zero and non-zero states."""
    calls = []
    for (t0, t1, cu) in cu_list:
        wsb = pool.prefill_workspace_bytes(int(ids.numel()), t1 - t0, C)
        ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device="cuda")
        cu_d = torch.tensor(cu, dtype=torch.int32, device="cuda")
        calls.append((t0, t1, cu_d, ws))

    def step(i):
        for (t0, t1, cu_d, ws) in calls:
            pool.prefill(0, cu_d, ids, t1 - t0, C, d["q"][t0:t1], d["k"][t0:t1], d["v"][t0:t1],
                         d["a"][t0:t1], d["b"][t0:t1], w, out[t0:t1], ws)

    return time_launches(step, reps, 3, torch)


def bench_prefill(args, torch, G, syn):
    s = syn.QWEN3_NEXT
    C = 64
    res = {}
    io = 2
    tok_bytes = (2 * s.h_k * s.d_k + s.h_v * s.d_v) * io + 2 * s.h_v * 4 + s.h_v * s.d_v * io
    # per sequence: state read + write, conv window read + write
    state_rw = 2 * s.h_v * s.d_v * s.d_k * 4 + 2 * (s.conv_k - 1) * s.c_conv * io
    fl_tok = prefill_flops_per_token(s, C)
    # One 8192-token sequence: one call, and 16 scheduler chunks of 512.
    case = syn.prefill_case()
    T = case["tokens"]["q"].shape[0]
    pool = G.Pool(G.make_desc(4, 1, s.h_k, s.h_v, s.d_k, s.d_v, s.conv_k, G.GDN_BF16))
    d = _prefill_inputs(torch, case["tokens"])
    w = torch.from_numpy(case["conv_w"]).cuda()
    out = torch.empty((T, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda")
    ids = torch.tensor([1], dtype=torch.int32, device="cuda")
    reps = max(10, args.steps // 10)
    want = lambda c: args.prefill_case in ("all", c)
    if want("single"):
        t1 = _time_prefill(args, torch, pool, [(0, T, [0, T])], ids, d, w, out, C, reps)
        b = T * tok_bytes + state_rw
        res["single"] = {"workload": "one 8192-token sequence, chunk 64", "us": t1 * 1e6,
                         "tok_s": T / t1, "GBps": b / t1 / 1e9, "hbm_frac": b / t1 / 1e9 / HBM_PEAK_GBPS,
                         "alg_TFLOPs": fl_tok * T / t1 / 1e12,
                         "mfma_frac_alg": fl_tok * T / t1 / 1e12 / BF16_PEAK_TFLOPS}
        ex = prefill_exec_flop_per_token("single")
        res["single"]["mfma_frac_exec"] = None if ex is None else ex * T / t1 / 1e12 / BF16_PEAK_TFLOPS
    if want("split512"):
        t16 = _time_prefill(args, torch, pool, [(c0, c0 + 512, [0, 512]) for c0 in range(0, T, 512)],
                            ids, d, w, out, C, reps)
        res["split512"] = {"workload": "the same sequence as 16 calls of 512 tokens", "us": t16 * 1e6,
                           "tok_s": T / t16}
    assert pool.error() == 0
    del pool, d, out
    if not want("varlen"):
        return res
    # Varlen: 16 sequences, lengths uniform in [128, 4096].
    case = syn.varlen_case()
    cu = case["cu_seqlens"]
    Tv = int(cu[-1])
    pool = G.Pool(G.make_desc(case["n_slots"], 1, s.h_k, s.h_v, s.d_k, s.d_v, s.conv_k, G.GDN_BF16))
    d = _prefill_inputs(torch, case["tokens"])
    w = torch.from_numpy(case["conv_w"]).cuda()
    out = torch.empty((Tv, s.h_v, s.d_v), dtype=torch.bfloat16, device="cuda")
    ids = torch.from_numpy(case["slot_ids"]).cuda()
    tv = _time_prefill(args, torch, pool, [(0, Tv, [int(x) for x in cu])], ids, d, w, out, C, reps)
    bv = Tv * tok_bytes + (len(cu) - 1) * state_rw
    res["varlen"] = {"workload": f"16 packed sequences, {Tv} tokens (lengths U[128,4096])",
                     "us": tv * 1e6, "tok_s": Tv / tv, "GBps": bv / tv / 1e9,
                     "hbm_frac": bv / tv / 1e9 / HBM_PEAK_GBPS,
                     "alg_TFLOPs": fl_tok * Tv / tv / 1e12,
                     "mfma_frac_alg": fl_tok * Tv / tv / 1e12 / BF16_PEAK_TFLOPS}
    ex = prefill_exec_flop_per_token("varlen")
    res["varlen"]["mfma_frac_exec"] = None if ex is None else ex * Tv / tv / 1e12 / BF16_PEAK_TFLOPS
    assert pool.error() == 0
    return res


def bench_stream_ceiling(args, torch):
    """The state stream of the decode step with nothing else, through the
    bandwidth probe (libgdn_probe.so, not part of the libgdn ABI): the same
    256-slot fp32 pool, the same four rotating sets of 64 slot ids in random
    order, each slot's 2 MiB read once and written once in place with the
    decode kernel's access pattern.  Its rate is the ceiling the decode state
    traffic can reach on this machine; decode, verify and the ring are reported
    against it beside the published 8 TB/s."""
    import ctypes
    from gated_deltanet_state_layer_amd import build as B
    if not os.path.exists(B.PROBE_LIB):
        raise RuntimeError(f"{B.PROBE_LIB} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(B.PROBE_LIB)
    lib.gdn_probe_stream_tiles.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.c_int, ctypes.c_float, ctypes.c_int,
                                           ctypes.c_void_p]
    lib.gdn_probe_stream_tiles.restype = ctypes.c_int
    n_slots, heads, N = 256, 32, 64
    state = torch.empty(n_slots * heads * 128 * 128, dtype=torch.float32, device="cuda")
    state.normal_(generator=torch.Generator(device="cuda").manual_seed(99))
    perm = np.random.default_rng(1001).permutation(n_slots).astype(np.int32)
    sets = [torch.from_numpy(perm[j * N:(j + 1) * N].copy()).cuda() for j in range(4)]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    names = ["2 tiles/workgroup, default loads", "2 tiles/workgroup, non-temporal loads",
             "1 tile/workgroup, default loads", "1 tile/workgroup, non-temporal loads"]
    b = N * 2 * heads * 128 * 128 * 4
    rates = {}
    for variant, name in enumerate(names):
        def step(i):
            rc = lib.gdn_probe_stream_tiles(ctypes.c_void_p(state.data_ptr()), heads,
                                            ctypes.c_void_p(sets[i % 4].data_ptr()), N, 1.0,
                                            variant, stream)
            if rc != 0:
                raise RuntimeError(f"gdn_probe_stream_tiles: hipError {rc}")
        rates[name] = b / time_launches(step, max(100, args.steps), 20, torch) / 1e9
    best = max(rates, key=rates.get)
    return {"workload": "state stream of the decode step alone: 64 of 256 slots (rotating 4 "
                        "disjoint sets, random order), 2 MiB read + 2 MiB written per slot",
            "bytes": b, "GBps": rates[best], "us": b / rates[best] / 1e3, "best": best,
            "hbm_frac": rates[best] / HBM_PEAK_GBPS, "variants_GBps": rates}


def bench_gemm(args, torch):
    """torch's bf16 GEMM (8192^3, hipBLASLt): the measured dense-MFMA
    reference next to the published peak."""
    n = 8192
    g = torch.Generator(device="cuda").manual_seed(5)
    x = torch.randn((n, n), generator=g, device="cuda").bfloat16()
    y = torch.randn((n, n), generator=g, device="cuda").bfloat16()
    z = torch.empty((n, n), device="cuda", dtype=torch.bfloat16)
    t = time_launches(lambda i: torch.matmul(x, y, out=z), max(10, args.steps // 20), 3, torch)
    return {"shape": [n, n, n], "us": t * 1e6, "TFLOPs": 2 * n ** 3 / t / 1e12}


def bench_copy(args, torch):
    """torch's plain copy kernel over 512 MiB: the achievable-bandwidth
    reference and the byte count used to scale the HBM counters."""
    n = 128 * 1024 * 1024
    src = torch.empty(n, dtype=torch.float32, device="cuda").normal_()
    dst = torch.empty_like(src)
    t = time_launches(lambda i: dst.copy_(src), max(20, args.steps // 10), 5, torch)
    return {"bytes": 2 * n * 4, "us": t * 1e6, "GBps": 2 * n * 4 / t / 1e9}


def cpu_threads():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "host"


def _threaded(jobs, fn, nthr):
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(nthr) as ex:
        return list(ex.map(fn, jobs))


def _timed_rounds(round_fn, seconds, min_rounds=1):
    round_fn()                       # warm-up
    n, t0 = 0, time.perf_counter()
    while n < min_rounds or time.perf_counter() - t0 < seconds:
        round_fn()
        n += 1
    return n, time.perf_counter() - t0


def cpu_baseline(syn):
    """The oracle's fp32 variant (rank-1 form), as it stands, on the host:
    decode steps of the 64-of-256-slot workload with the slots split over
    one thread per available core (NumPy releases the GIL in the state
    arithmetic; BLAS threads are held at 1 inside each thread), for about 6 s.
    Returns (cpu_baseline, details), the details being bounded samples of the
    other workloads run the same way."""
    from oracle import gdn_oracle as O
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(1)
    except Exception:
        limiter = None
    s, io = syn.QWEN3_NEXT, "bf16"
    nthr = cpu_threads()
    f32 = np.float32

    def slot_pools(ids, contents, shards):
        pools = []
        for sh in shards:
            op = O.OraclePool(len(sh), 1, s, form="rank1", dtype=f32)
            for j, i in enumerate(sh):
                op.S[j], op.X[j] = contents[int(ids[i])]
            pools.append((op, sh))
        return pools

    # decode, N slots
    def decode_rate(N, seconds):
        case = syn.decode_case(N)
        ids, tok, w = case["slot_ids"], case["tokens"], case["conv_w"]
        contents = syn.draw_pool_contents(case["pool_seed"], ids, s, io)
        k = min(nthr, N)
        pools = slot_pools(ids, contents, [sh for sh in np.array_split(np.arange(N), k) if len(sh)])
        run = lambda p: p[0].decode(0, np.arange(len(p[1])), *(tok[m][p[1]] for m in "qkvab"), w)
        n, dt = _timed_rounds(lambda: _threaded(pools, run, k), seconds)
        return N * n / dt, n, dt, k

    value, n64, dt64, k64 = decode_rate(64, 5.0)
    detail = {"decode_tok_s": {"64": value}}
    for N in (1, 4, 16):
        detail["decode_tok_s"][str(N)] = decode_rate(N, 0.7)[0]
    # verify: 128 slots x 4 tokens, accept_len U{1..4}
    vc = syn.verify_case()
    vids, vt = vc["slot_ids"], vc["tokens"]
    contents = syn.draw_pool_contents(vc["pool_seed"], vids, s, io)
    pools = slot_pools(vids, contents, np.array_split(np.arange(len(vids)), nthr))
    run = lambda p: p[0].verify(0, np.arange(len(p[1])), 4, *(vt[m][p[1]] for m in "qkvab"),
                                vc["conv_w"], vc["accept_len"][p[1]])
    n, dt = _timed_rounds(lambda: _threaded(pools, run, nthr), 2.0)
    detail["verify_tok_s"] = 128 * 4 * n / dt
    # prefill, one 8192-token sequence token by token (one thread; the
    # oracle's step is vectorised over the layer's heads): the first 256 tokens
    case = syn.prefill_case()
    tok, w = case["tokens"], case["conv_w"]
    t0 = time.perf_counter()
    O.OraclePool(1, 1, s, form="rank1", dtype=f32).prefill(0, [0, 256], [0],
                                                           *(tok[m][:256] for m in "qkvab"), w)
    detail["prefill_token_loop_tok_s"] = 256 / (time.perf_counter() - t0)
    # the same 256 tokens in the chunked form (chunk 64, fp64, one thread)
    t0 = time.perf_counter()
    O.chunked_sequence(np.zeros((s.h_v, s.d_v, s.d_k)), np.zeros((s.conv_k - 1, s.c_conv)),
                       *(tok[m][:256] for m in "qkvab"), w, s, 64)
    detail["prefill_chunked_fp64_one_thread_tok_s"] = 256 / (time.perf_counter() - t0)
    # varlen: 16 sequences, one thread per sequence, the first 64 tokens of each
    vc3 = syn.varlen_case()
    cu, vtok = vc3["cu_seqlens"], vc3["tokens"]
    seqs = [{m: vtok[m][cu[j]:cu[j] + 64] for m in "qkvab"} for j in range(len(cu) - 1)]
    run = lambda t: O.OraclePool(1, 1, s, form="rank1", dtype=f32).prefill(
        0, [0, 64], [0], *(t[m] for m in "qkvab"), vc3["conv_w"])
    t0 = time.perf_counter()
    _threaded(seqs, run, min(nthr, len(seqs)))
    detail["varlen_tok_s"] = 64 * len(seqs) / (time.perf_counter() - t0)
    if limiter is not None:
        limiter.restore_original_limits()
    detail["threads"] = nthr
    detail["sample"] = ("decode of 1/4/16 slots ~0.7 s each (slots over up to one thread per "
                        "core); verify 128 slots x 4 tokens ~2 s (slots over threads); prefill: "
                        "the first 256 of the 8192 tokens on one thread, token by token (fp32) "
                        "and in the chunked form (fp64, chunk 64); varlen: the first 64 tokens "
                        "of each of the 16 sequences, one thread per sequence; fp32 rank-1 "
                        "oracle unless stated")
    base = {"value": value, "unit": "tokens/s", "cores": k64, "kind": "oracle",
            "sample": f"{n64} decode steps of 64 of 256 slots (Qwen3-Next shapes) in {dt64:.1f} s, "
                      f"fp32 rank-1 oracle, slots over {k64} threads on {cpu_model()}"}
    return base, detail


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the GDN state layer benchmark runs on one GPU; --gpus must be 1"}))
        sys.exit(2)
    import torch
    import gated_deltanet_state_layer_amd as G
    import gdn_synth as syn
    G.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    res = {}
    if args.only in (None, "decode"):
        res["decode"] = bench_decode(args, torch, G, syn)
        print(f"# decode done: {res['decode']['sec'] * 1e6:.1f} us/step", file=sys.stderr, flush=True)
    if args.only in (None, "verify") and not args.no_verify:
        res["verify"] = bench_verify(args, torch, G, syn)
        print(f"# verify done: {res['verify']['sec'] * 1e6:.1f} us", file=sys.stderr, flush=True)
    if args.only in (None, "ring") and not args.no_ring:
        res["ring"] = bench_ring(args, torch, G, syn)
        print(f"# ring done: {res['ring']['cycle_us']:.1f} us/cycle", file=sys.stderr, flush=True)
    if args.only in (None, "in_proj") and not args.no_in_proj:
        res["in_proj"] = bench_in_proj(args, torch, G, syn)
        print("# in_proj done", file=sys.stderr, flush=True)
    if args.only in (None, "prefill") and not args.no_prefill:
        res["prefill"] = bench_prefill(args, torch, G, syn)
        print("# prefill done", file=sys.stderr, flush=True)
    if args.only in (None, "stream"):
        res["stream"] = bench_stream_ceiling(args, torch)
        print(f"# stream ceiling done: {res['stream']['GBps']:.0f} GB/s", file=sys.stderr, flush=True)
    if args.only in (None, "copy"):
        res["copy"] = bench_copy(args, torch)
        print("# copy done", file=sys.stderr, flush=True)
    if args.only in (None, "gemm"):
        res["gemm"] = bench_gemm(args, torch)
        print("# gemm done", file=sys.stderr, flush=True)
    cpu = cpu_more = None
    if not args.no_cpu and args.only is None:
        cpu, cpu_more = cpu_baseline(syn)
        print("# cpu baseline done", file=sys.stderr, flush=True)
    if "decode" not in res:
        print(json.dumps(res))
        return
    dec = res["decode"]
    line = {
        "metric": "GDN decode tokens/s at 64 slots (state-GB/s, %HBM peak); prefill tok/s (%MFMA)",
        "value": dec["n"] / dec["sec"],
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": dec["sec"] * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "multi-slot decode step, 64 of 256 slots (rotating 4 disjoint "
                               "sets), h_k=16 h_v=32 d_k=d_v=128 conv_k=4, bf16 io, fp32 state",
                   "n_slots": 256, "active_slots": 64},
        "state_GBps": dec["state_gbps"],
        "hbm_frac": dec["gbps"] / HBM_PEAK_GBPS,
        "roofline": {"bound": "hbm", "achieved": dec["gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": dec["gbps"] / HBM_PEAK_GBPS, "traffic": decode_traffic_bytes(),
                     "kernel": "decode_heads_kernel<128,bf16,4,1,true>",
                     "bytes_per_launch": dec["bytes"], "us_per_launch": dec["sec"] * 1e6},
        "decode_per_launch": dec.get("per_launch"),
        "decode_hot_cache_GBps": dec.get("hot_gbps"),
        "decode_small_batches": dec.get("small"),
        "decode_after_context_us": dec.get("after_context_us"),
    }
    if "verify" in res:
        v = res["verify"]
        line["verify"] = {"workload": "128 slots x 4 tokens, accept_len U{1..4}",
                          "kernel": "decode_heads_kernel<128,bf16,4,4,false>",
                          "us": v["sec"] * 1e6, "tok_s": v["tok_s"],
                          "accepted_tok_s": v["accepted_tok_s"], "GBps": v["gbps"],
                          "hbm_frac": v["gbps"] / HBM_PEAK_GBPS}
    if res.get("ring"):
        line["verify_ring"] = res["ring"]
    if res.get("in_proj"):
        line["in_proj"] = res["in_proj"]
    if res.get("prefill"):
        pf = res["prefill"]
        one = pf.get("single", {})
        flat = {"workload": "one 8192-token sequence, chunk 64, h_k=16 h_v=32 d=128, bf16 io, "
                            "fp32 state (one call)",
                "alg_MFLOP_per_token": prefill_flops_per_token(syn.QWEN3_NEXT, 64) / 1e6}
        for k in ("us", "tok_s", "GBps", "hbm_frac", "mfma_frac_alg", "mfma_frac_exec"):
            if k in one:
                flat[k] = one[k]
        if "split512" in pf:
            flat["split512_us"] = pf["split512"]["us"]
            if "us" in one:
                flat["split512_over_single"] = pf["split512"]["us"] / one["us"]
        if "varlen" in pf:
            for k in ("us", "tok_s", "mfma_frac_alg", "mfma_frac_exec", "hbm_frac"):
                flat["varlen_" + k] = pf["varlen"].get(k)
        line["prefill"] = flat
        line["prefill_detail"] = pf
    if res.get("stream"):
        st = dict(res["stream"])
        st["decode_frac_of_ceiling"] = dec["gbps"] / st["GBps"]
        if "verify" in line:
            st["verify_frac_of_ceiling"] = line["verify"]["GBps"] / st["GBps"]
        if "verify_ring" in line:
            st["ring_verify_frac_of_ceiling"] = line["verify_ring"]["verify_GBps"] / st["GBps"]
        line["stream_ceiling"] = st
    if res.get("copy"):
        line["copy_reference"] = res["copy"]
    if res.get("gemm"):
        line["mfma_reference"] = res["gemm"]
    if cpu:
        line["cpu_baseline"] = cpu
        line["cpu_baseline_detail"] = cpu_more
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
