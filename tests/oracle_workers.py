"""Host worker processes that run the CPU oracle on q/k head groups in
parallel, for parity checks over whole Qwen3-Next-sized layers.

Value heads of different q/k groups never interact (each group has its own
q, k and v channels, conv taps and state tiles), so the oracle runs each
group as a layer of its own (h_k = 1, h_v = G) and the results are put back
together.  The workers are plain Python processes started with the "spawn"
method before the test process first touches the GPU (tests/conftest.py
starts them once per session); they import only NumPy, the seeded
generators and the oracle.  Nothing here imports torch.
"""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

_POOL = None


def n_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _ping(_):
    return os.getpid()


def start():
    """Start the worker pool (idempotent).  All workers exist when this
    returns, so no process is started after the GPU is in use."""
    global _POOL
    if _POOL is None:
        n = n_workers()
        pool = mp.get_context("spawn").Pool(n, initializer=_init)
        try:
            # a worker that cannot start is replaced for ever by the pool:
            # bound the wait instead of hanging
            pool.map_async(_ping, range(n), chunksize=1).get(timeout=120)
        except BaseException:
            pool.terminate()
            raise
        _POOL = pool
    return _POOL


def stop():
    global _POOL
    if _POOL is not None:
        _POOL.terminate()
        _POOL.join()
        _POOL = None


def group_channels(s, g):
    """Conv channels of q/k group g: its q head, its k head and its value
    heads, in the layer's channel order."""
    D, G = s.d_k, s.group
    return np.concatenate([np.arange(g * D, (g + 1) * D),
                           s.h_k * D + np.arange(g * D, (g + 1) * D),
                           2 * s.h_k * D + np.arange(g * G * D, (g + 1) * G * D)])


def _prefill_group(job):
    """One group: oracle pool with n_seq slots (slot j <- sequence j's
    starting contents), then the packed prefill.  Returns (outputs [T][G][d],
    final states [n_seq][1][G][d][d], windows [n_seq][1][K-1][ch])."""
    import gdn_synth as syn
    from oracle import gdn_oracle as O
    (h_k, h_v, d, K), cu, order, tok, w, start_states, start_windows = job
    sub = syn.Shapes(1, h_v // h_k, d, d, K)
    n = len(order)
    op = O.OraclePool(n, 1, sub, form="rank1")
    if start_states is not None:
        op.S[:] = start_states
        op.X[:] = start_windows
    out = op.prefill(0, cu, order, tok["q"], tok["k"], tok["v"], tok["a"], tok["b"], w)
    return out, op.S, op.X


def prefill_all_groups(s, tok, conv_w, cu, order, start_states=None, start_windows=None):
    """Oracle prefill of a whole layer, one q/k group per job.

    tok: raw inputs of the packed tokens (q, k [T][h_k][d], v [T][h_v][d],
    a, b [T][h_v]); conv_w [C_conv][K]; cu: cu_seqlens; order[j]: the oracle
    slot of sequence j (-1: padding); start_states [n_seq][1][h_v][d][d] and
    start_windows [n_seq][1][K-1][C_conv] (None: every slot from zero).
    Returns (outputs [T][h_v][d], states, windows) in the layer's layout."""
    pool = start()
    G = s.group
    jobs = []
    for g in range(s.h_k):
        ch = group_channels(s, g)
        hs = slice(g * G, (g + 1) * G)
        sub_tok = {"q": tok["q"][:, g:g + 1], "k": tok["k"][:, g:g + 1], "v": tok["v"][:, hs],
                   "a": tok["a"][:, hs], "b": tok["b"][:, hs]}
        st = None if start_states is None else np.ascontiguousarray(start_states[:, :, hs])
        wn = None if start_windows is None else np.ascontiguousarray(start_windows[..., ch])
        jobs.append(((s.h_k, s.h_v, s.d_k, s.conv_k), np.asarray(cu), np.asarray(order),
                     sub_tok, np.ascontiguousarray(conv_w[ch]), st, wn))
    res = pool.map_async(_prefill_group, jobs, chunksize=1).get(timeout=900)
    T, n = tok["q"].shape[0], len(order)
    out = np.full((T, s.h_v, s.d_v), np.nan)
    S = np.zeros((n, 1, s.h_v, s.d_v, s.d_k))
    X = np.zeros((n, 1, s.conv_k - 1, s.c_conv))
    for g, (o, sg, xg) in enumerate(res):
        hs = slice(g * G, (g + 1) * G)
        out[:, hs] = o
        S[:, :, hs] = sg
        X[..., group_channels(s, g)] = xg
    return out, S, X
