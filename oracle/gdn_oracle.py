"""CPU oracle for the Gated DeltaNet state layer -- TEST INFRASTRUCTURE ONLY.

This is the plain, slow, obviously-correct definition of what the layer
computes, in float64 NumPy, one token at a time.  Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import it.  It shares no
code with the GPU library (no kernels, headers, helpers or constants) and
imports nothing from it.

Sources (pages, by title and section):
  [P1] baseRT issue #31, "GDN keeps a single recurrent state, so requests
       serialise" -- sections "Why this looks tractable" (one constant-size
       recurrent state per sequence, an outer slot dimension, a slot index in
       the kernels; conv window sized by conv_k) and "Scope note" (N
       independent states).
  [P2] "Plan (research-based): Qwen3.6-35B-A3B -- parity fix + path to >150
       tok/s", section "What the research found" (the state is a full
       [V,K] matrix; prefill in chunked delta-rule form via the (I+A)^-1 UT
       transform; verify commits only what is accepted).
  [P3] "Project: adding the hybrid model Qwen3.5", table "What to do", row
       "State" (one conv cache and one recurrent state per request slot; a
       new request starts from zero; chunked prefill carries the state from
       chunk to chunk), and "Why it is worth doing" (state is cleared on slot
       reuse, copied whole, never truncated).

The recurrence itself (the gated delta rule) is the layer's definition:
    S_t = a_t * S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t
with S a [d_v, d_k] matrix per value head ([P2] "[V,K]" state).  The pages
name the rule but do not print it; every reading taken where they are silent
is listed below and repeated next to the code it affects:

  R1  conv: depthwise causal, all q, k and v channels, no bias; tap
      conv_k-1 multiplies the current token, tap 0 the oldest; the window
      holds the last conv_k-1 raw inputs, oldest first; a fresh window is 0.
  R2  SiLU after the conv: silu(z) = z / (1 + exp(-z)).
  R3  q and k are L2-normalised per head after conv+SiLU,
      x / sqrt(|x|^2 + eps) with eps = 1e-6; then q is multiplied by
      q_scale (default d_k^-1/2).
  R4  grouped heads: value head h uses q/k head floor(h / (h_v / h_k)).
  R5  a, b are given per token and value head, already activated.
  R6  verify runs n_tok tokens on a copy of the slot, returns every
      position's output and commits the copy taken after accept_len tokens
      (0 leaves the slot untouched).
  R7  a negative slot id marks a padding entry: skipped, its output unwritten.
  R14 the input projection: y = x W^T; rows of W in the order q | k | v |
      a logits | b logits; a = exp(-softplus(y_a)), b = sigmoid(y_b).

Parity of these readings against an external implementation is unpinned (no
implementation exists to compare against); the oracle itself is pinned by the
closed forms and invariants in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "silu", "conv_silu_token", "l2norm", "expand_groups", "delta_rule_step",
    "token_step", "OraclePool", "unit_lower_inverse", "chunked_sequence",
    "split_channels", "in_projection",
]


# ---------------------------------------------------------------------------
# Front end: depthwise causal conv1d + SiLU, then q/k normalisation.
# ---------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """SiLU (reading R2): z * sigmoid(z)."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def conv_silu_token(window: np.ndarray, x: np.ndarray, w: np.ndarray):
    """One token of the depthwise causal conv + SiLU ([P1] conv_k-sized conv
    cache, [P3] one conv cache per request; reading R1).

    window: [conv_k-1, C] raw inputs, oldest first.  x: [C] current raw input.
    w: [C, conv_k].  Returns (y [C], new window [conv_k-1, C]).
    y_c = silu( sum_j w[c, j] * X[j, c] ),  X = [window; x]  (row conv_k-1 = x).
    """
    X = np.concatenate([window, x[None, :]], axis=0)
    z = np.zeros(x.shape[0], dtype=X.dtype)
    for j in range(X.shape[0]):
        z += w[:, j] * X[j]
    return silu(z), X[1:].copy()


def l2norm(x: np.ndarray, eps: float) -> np.ndarray:
    """Per-head L2 normalisation over the last axis (reading R3)."""
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def split_channels(y: np.ndarray, dims):
    """Split conv channels [q heads | k heads | v heads] into (q, k, v)."""
    nq = dims.h_k * dims.d_k
    q = y[..., :nq].reshape(y.shape[:-1] + (dims.h_k, dims.d_k))
    k = y[..., nq:2 * nq].reshape(y.shape[:-1] + (dims.h_k, dims.d_k))
    v = y[..., 2 * nq:].reshape(y.shape[:-1] + (dims.h_v, dims.d_v))
    return q, k, v


def in_projection(x: np.ndarray, W: np.ndarray, dims):
    """The input projection in front of the conv ([P1] "Why this looks
    tractable": the layer's kernels include an input projection beside the
    conv).  Reading R14: y = x W^T over the hidden size, W's rows being the
    output channels in the order q heads | k heads | v heads | h_v gate
    logits for a | h_v gate logits for b; the raw q, k, v are the first
    C_conv channels of y, and the gates are activated as the layer's inputs
    are distributed: a = exp(-softplus(y_a)), b = sigmoid(y_b).

    x: [..., hidden]; W: [C_conv + 2 h_v, hidden].  Returns (q, k, v, a, b)
    with q, k [..., h_k, d_k], v [..., h_v, d_v], a, b [..., h_v]."""
    y = np.asarray(x, np.float64) @ np.asarray(W, np.float64).T
    c_conv = 2 * dims.h_k * dims.d_k + dims.h_v * dims.d_v
    q, k, v = split_channels(y[..., :c_conv], dims)
    ya = y[..., c_conv:c_conv + dims.h_v]
    yb = y[..., c_conv + dims.h_v:c_conv + 2 * dims.h_v]
    a = np.exp(-np.logaddexp(0.0, ya))          # softplus(y) = log(1 + e^y)
    with np.errstate(over="ignore"):
        b = 1.0 / (1.0 + np.exp(-yb))
    return q, k, v, a, b


def expand_groups(x: np.ndarray, h_v: int) -> np.ndarray:
    """q/k head g serves value heads g*G .. g*G+G-1 (reading R4)."""
    G = h_v // x.shape[-2]
    return np.repeat(x, G, axis=-2)


# ---------------------------------------------------------------------------
# The recurrence.
# ---------------------------------------------------------------------------

def delta_rule_step(S, q, k, v, a, b, form: str = "matrix"):
    """One gated delta-rule step for every value head ([P2] delta rule with a
    [V,K] state).

    S: [H, d_v, d_k]; q, k: [H, d_k]; v: [H, d_v]; a, b: [H].
    form="matrix": S' = a S (I - b k k^T) + b v k^T, written out literally.
    form="rank1":  S' = a S + b (v - a S k) k^T, its expansion (same value;
                   the two agree to rounding, pinned in the tests).
    Output o = S' q (the updated state).
    """
    H, dv, dk = S.shape
    if form == "matrix":
        eye = np.eye(dk)
        S_new = np.empty_like(S)
        for h in range(H):
            P = eye - b[h] * np.outer(k[h], k[h])
            S_new[h] = a[h] * (S[h] @ P) + b[h] * np.outer(v[h], k[h])
    elif form == "rank1":
        Sk = np.einsum("hij,hj->hi", S, k)
        delta = b[:, None] * (v - a[:, None] * Sk)
        S_new = a[:, None, None] * S + delta[:, :, None] * k[:, None, :]
    else:
        raise ValueError(form)
    o = np.einsum("hij,hj->hi", S_new, q)
    return S_new, o


def front_end(window, xq, xk, xv, conv_w, dims, q_scale, eps, dtype=np.float64):
    """conv+SiLU on the concatenated raw input, then the q/k normalisation.
    Returns (q_hat [h_k,d_k], k_hat [h_k,d_k], v_hat [h_v,d_v], new window).
    All arithmetic in `dtype` (float64 for parity; float32 only for timing)."""
    x = np.concatenate([xq.reshape(-1), xk.reshape(-1), xv.reshape(-1)]).astype(dtype)
    window = np.asarray(window, dtype)
    conv_w = np.asarray(conv_w, dtype)
    y, window = conv_silu_token(window, x, conv_w)
    q, k, v = split_channels(y, dims)
    q = l2norm(q, eps) * q_scale
    k = l2norm(k, eps)
    return q, k, v, window


def token_step(S, window, xq, xk, xv, a, b, conv_w, dims, q_scale, eps, form="matrix",
               dtype=np.float64):
    """One token through the layer core: conv+SiLU, normalisation, grouped
    heads, recurrence.  Returns (S', window', o [h_v, d_v])."""
    q, k, v, window = front_end(window, xq, xk, xv, conv_w, dims, q_scale, eps, dtype)
    S, o = delta_rule_step(S, expand_groups(q, dims.h_v), expand_groups(k, dims.h_v), v,
                           np.asarray(a, dtype), np.asarray(b, dtype), form)
    return S, window, o


# ---------------------------------------------------------------------------
# The slot pool and its calls.
# ---------------------------------------------------------------------------

class OraclePool:
    """N independent fixed-size slots, each with a recurrent state per layer and
    value head and a conv window per layer ([P1] "Why this looks tractable":
    an outer slot dimension; [P3] "State": one conv cache and one state per
    request slot, new requests start from zero).

    S: [n_slots, n_layers, h_v, d_v, d_k] float64
    X: [n_slots, n_layers, conv_k-1, C_conv] float64 (raw inputs, oldest first)

    dtype=np.float32 runs the same steps in fp32: a timing variant only (the
    CPU baseline of the benchmark), never a parity reference.
    """

    def __init__(self, n_slots, n_layers, dims, q_scale=None, eps=1e-6, form="matrix",
                 dtype=np.float64):
        self.dims = dims
        self.n_slots, self.n_layers = n_slots, n_layers
        self.q_scale = dims.d_k ** -0.5 if q_scale is None else q_scale
        self.eps = eps
        self.form = form
        self.dtype = dtype
        c_conv = 2 * dims.h_k * dims.d_k + dims.h_v * dims.d_v
        self.S = np.zeros((n_slots, n_layers, dims.h_v, dims.d_v, dims.d_k), dtype)
        self.X = np.zeros((n_slots, n_layers, dims.conv_k - 1, c_conv), dtype)

    # -- bookkeeping -------------------------------------------------------
    def reset(self, slot_ids):
        """A reused slot starts from zero state and zero window ([P3] "State",
        "Why it is worth doing")."""
        for s in slot_ids:
            if s >= 0:
                self.S[s] = 0.0
                self.X[s] = 0.0

    def _step(self, slot, layer, xq, xk, xv, a, b, conv_w):
        S, X, o = token_step(self.S[slot, layer], self.X[slot, layer], xq, xk, xv, a, b,
                             np.asarray(conv_w, self.dtype), self.dims, self.q_scale,
                             self.eps, self.form, self.dtype)
        self.S[slot, layer] = S
        self.X[slot, layer] = X
        return o

    # -- calls ---------------------------------------------------------------
    def decode(self, layer, slot_ids, q, k, v, a, b, conv_w):
        """One token for each listed slot; entry i goes to slot slot_ids[i]
        ([P1] "Why this looks tractable": a slot index in the GDN kernels).
        q, k: [n, h_k, d_k]; v: [n, h_v, d_v]; a, b: [n, h_v]."""
        n = len(slot_ids)
        out = np.full((n, self.dims.h_v, self.dims.d_v), np.nan)
        for i, s in enumerate(slot_ids):
            if s < 0:
                continue
            out[i] = self._step(s, layer, q[i], k[i], v[i], a[i], b[i], conv_w)
        return out

    def prefill(self, layer, cu_seqlens, slot_ids, q, k, v, a, b, conv_w):
        """Packed sequences, token by token, each on its own slot; the state
        and window carry over from whatever the slot holds ([P3] "State":
        chunked prefill passes the state on).  q, k: [T, h_k, d_k] etc."""
        T = q.shape[0]
        out = np.full((T, self.dims.h_v, self.dims.d_v), np.nan)
        for i, s in enumerate(slot_ids):
            if s < 0:
                continue
            for t in range(int(cu_seqlens[i]), int(cu_seqlens[i + 1])):
                out[t] = self._step(s, layer, q[t], k[t], v[t], a[t], b[t], conv_w)
        return out

    def verify(self, layer, slot_ids, n_tok, q, k, v, a, b, conv_w, accept_len):
        """Speculative verify (reading R6; [P2] "What the research found":
        only the accepted prefix's state is kept, no per-draft snapshots).
        q, k: [n, n_tok, h_k, d_k]; v: [n, n_tok, h_v, d_v]; a, b: [n, n_tok, h_v]."""
        n = len(slot_ids)
        out = np.full((n, n_tok, self.dims.h_v, self.dims.d_v), np.nan)
        for i, s in enumerate(slot_ids):
            if s < 0:
                continue
            S = self.S[s, layer].copy()
            X = self.X[s, layer].copy()
            keep = None
            if accept_len[i] == 0:
                keep = (S.copy(), X.copy())
            for t in range(n_tok):
                S, X, out[i, t] = token_step(S, X, q[i, t], k[i, t], v[i, t], a[i, t], b[i, t],
                                             np.asarray(conv_w, self.dtype), self.dims,
                                             self.q_scale, self.eps, self.form, self.dtype)
                if t + 1 == accept_len[i]:
                    keep = (S.copy(), X.copy())
            self.S[s, layer], self.X[s, layer] = keep
        return out


# ---------------------------------------------------------------------------
# Chunked form ([P2] "What the research found": chunked delta rule with the
# (I+A)^-1 UT transform; [P3] "State": state passed chunk to chunk).
# Used by the tests to show that the chunked equations reproduce the token
# loop; it is a template for the GPU prefill, not shared code.
# ---------------------------------------------------------------------------

def unit_lower_inverse(A: np.ndarray) -> np.ndarray:
    """(I + A)^-1 for strictly lower-triangular A, by forward substitution:
    row t of T = (I+A)^-1 satisfies T[t] = e_t - sum_{j<t} A[t, j] T[j]."""
    n = A.shape[0]
    T = np.zeros_like(A)
    for t in range(n):
        T[t, t] = 1.0
        for j in range(t):
            T[t] -= A[t, j] * T[j]
    return T


def chunked_sequence(S0, window0, q, k, v, a, b, conv_w, dims, chunk,
                     q_scale=None, eps=1e-6):
    """One sequence in chunks of `chunk` tokens (the last may be short).

    Per token: the same conv+SiLU and normalisation as the token loop.  Per
    chunk of L tokens and value head (g = cumulative sum of log a within the
    chunk, gamma = exp(g)):
        A[t,s] = b_t exp(g_t - g_s) (k_t . k_s)         for s < t
        T      = (I + A)^-1                              (the UT transform)
        U      = T diag(b) (V - diag(gamma) K S0^T)      (new values)
        O      = diag(gamma) Q S0^T + (QK^T * exp(g_t - g_s), s <= t) U
        S      = gamma_L S0 + U^T diag(exp(g_L - g)) K
    S0: [h_v, d_v, d_k]; window0: [conv_k-1, C]; returns (O [T,h_v,d_v], S, window).
    """
    q_scale = dims.d_k ** -0.5 if q_scale is None else q_scale
    Tn = q.shape[0]
    W = np.asarray(conv_w, np.float64)
    # Front end, token by token (exactly the token loop's front end).
    Q = np.zeros((Tn, dims.h_k, dims.d_k))
    K = np.zeros((Tn, dims.h_k, dims.d_k))
    V = np.zeros((Tn, dims.h_v, dims.d_v))
    X = np.asarray(window0, np.float64).copy()
    for t in range(Tn):
        Q[t], K[t], V[t], X = front_end(X, q[t], k[t], v[t], W, dims, q_scale, eps)
    G = dims.h_v // dims.h_k
    S = np.asarray(S0, np.float64).copy()
    O = np.zeros((Tn, dims.h_v, dims.d_v))
    la = np.log(np.asarray(a, np.float64))
    bb = np.asarray(b, np.float64)
    for c0 in range(0, Tn, chunk):
        c1 = min(c0 + chunk, Tn)
        L = c1 - c0
        for h in range(dims.h_v):
            gk = h // G
            Kc, Qc, Vc = K[c0:c1, gk], Q[c0:c1, gk], V[c0:c1, h]
            g = np.cumsum(la[c0:c1, h])
            gam = np.exp(g)
            beta = bb[c0:c1, h]
            decay = np.exp(g[:, None] - g[None, :])
            KK = Kc @ Kc.T
            A = np.tril(beta[:, None] * decay * KK, -1)
            T = unit_lower_inverse(A)
            U = T @ (beta[:, None] * (Vc - gam[:, None] * (Kc @ S[h].T)))
            P = np.tril((Qc @ Kc.T) * decay, 0)
            O[c0:c1, h] = gam[:, None] * (Qc @ S[h].T) + P @ U
            S[h] = gam[L - 1] * S[h] + U.T @ (np.exp(g[L - 1] - g)[:, None] * Kc)
    return O, S, X
