"""Seeded synthetic inputs for the Gated DeltaNet state layer.

This module is shared by the tests, the benchmark and the smoke check.  It
draws random numbers and shapes them into the distributions the workloads
use; it holds none of the layer's arithmetic (no convolution, no SiLU, no
normalisation of activations, no recurrence).  Both the CPU oracle and the
GPU path are fed from the arrays it returns.

Distributions (the same for every workload):
  * raw q, k: i.i.d. N(0, 1) per element, then each head vector is scaled to
    unit L2 norm, then rounded to the io dtype (round-to-nearest-even);
  * raw v: i.i.d. N(0, 1), rounded to the io dtype;
  * b = sigmoid(N(0, 1)), a = exp(-softplus(N(0, 1))), kept in fp32;
  * depthwise conv weights: N(0, 0.5^2) in fp32 (0.5 read as the standard
    deviation);
  * pre-filled slot states: N(0, 1) fp32; pre-filled conv windows: rows of
    raw inputs drawn as above.

Every generator takes an explicit seed and draws in a fixed order, written
next to each function.  Arrays are float32 (bf16 values are float32 arrays
whose low 16 bits are zero) and int32 for indices.
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = [
    "Shapes", "TINY", "QWEN3_NEXT", "bf16_round", "conv_channels",
    "draw_tokens", "draw_conv_weights", "draw_slot_state", "draw_slot_window",
    "draw_pool_contents", "tiny_layer_case", "decode_case", "prefill_case",
    "varlen_case", "verify_case", "QWEN3_NEXT_HIDDEN", "draw_hidden", "draw_in_proj_weight",
]


@dataclasses.dataclass(frozen=True)
class Shapes:
    h_k: int
    h_v: int
    d_k: int
    d_v: int
    conv_k: int

    @property
    def group(self) -> int:
        return self.h_v // self.h_k

    @property
    def c_conv(self) -> int:
        return conv_channels(self)


# Tiny single-slot layer: 2 heads of width 32, 4-tap conv.
TINY = Shapes(h_k=2, h_v=2, d_k=32, d_v=32, conv_k=4)
# Qwen3-Next-like GDN layer: 16 q/k heads, 32 v heads, width 128, 4-tap conv.
QWEN3_NEXT = Shapes(h_k=16, h_v=32, d_k=128, d_v=128, conv_k=4)


def conv_channels(s: Shapes) -> int:
    """Number of conv channels: q heads, then k heads, then v heads."""
    return 2 * s.h_k * s.d_k + s.h_v * s.d_v


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); float32 out."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out = np.where(nan, np.float32(np.nan), out)
    return out.reshape(x.shape)


def _io_cast(x: np.ndarray, io: str) -> np.ndarray:
    x = x.astype(np.float32)
    if io == "bf16":
        return bf16_round(x)
    if io == "f32":
        return x
    raise ValueError(f"unknown io dtype {io!r}")


def _unit_heads(rng: np.random.Generator, lead: tuple, h: int, d: int) -> np.ndarray:
    x = rng.standard_normal(lead + (h, d))
    x /= np.linalg.norm(x, axis=-1, keepdims=True)
    return x


def draw_tokens(rng: np.random.Generator, s: Shapes, lead: tuple, io: str) -> dict:
    """Raw per-token inputs with leading shape `lead` (e.g. (T,) or (n, n_tok)).

    Draw order: q, k, v, then the pre-activation of b, then that of a.
    """
    q = _unit_heads(rng, lead, s.h_k, s.d_k)
    k = _unit_heads(rng, lead, s.h_k, s.d_k)
    v = rng.standard_normal(lead + (s.h_v, s.d_v))
    zb = rng.standard_normal(lead + (s.h_v,))
    za = rng.standard_normal(lead + (s.h_v,))
    b = 1.0 / (1.0 + np.exp(-zb))
    a = np.exp(-np.logaddexp(0.0, za))
    return {
        "q": _io_cast(q, io), "k": _io_cast(k, io), "v": _io_cast(v, io),
        "a": a.astype(np.float32), "b": b.astype(np.float32),
    }


def draw_conv_weights(rng: np.random.Generator, s: Shapes) -> np.ndarray:
    """[C_conv][conv_k] fp32; tap conv_k-1 multiplies the current token."""
    return (0.5 * rng.standard_normal((s.c_conv, s.conv_k))).astype(np.float32)


# Hidden size of the layer's input for the Qwen3-Next-shaped workloads (the
# model's width; the pages give the GDN head shapes only).
QWEN3_NEXT_HIDDEN = 2048


def draw_hidden(rng: np.random.Generator, lead: tuple, hidden: int) -> np.ndarray:
    """Hidden states x ~ N(0, 1), rounded to bf16 (float32 values)."""
    return bf16_round(rng.standard_normal(lead + (hidden,)))


def draw_in_proj_weight(rng: np.random.Generator, s: Shapes, hidden: int) -> np.ndarray:
    """Synthetic input-projection weights [C_conv + 2 h_v][hidden], entries
    N(0, 1/hidden) rounded to bf16 (float32 values), so that with N(0,1) hidden states every
    projected channel is about N(0,1), the distribution of the layer's raw
    inputs and gate pre-activations."""
    n_out = s.c_conv + 2 * s.h_v
    return bf16_round(rng.standard_normal((n_out, hidden)) / np.sqrt(hidden))


def draw_slot_state(seed: int, slot: int, s: Shapes, n_layers: int = 1) -> np.ndarray:
    """A pre-filled slot state [n_layers][h_v][d_v][d_k] fp32, N(0,1)."""
    rng = np.random.default_rng([seed, slot, 1])
    return rng.standard_normal((n_layers, s.h_v, s.d_v, s.d_k), dtype=np.float32)


def draw_slot_window(seed: int, slot: int, s: Shapes, io: str, n_layers: int = 1) -> np.ndarray:
    """A pre-filled conv window [n_layers][conv_k-1][C_conv] of raw inputs."""
    rng = np.random.default_rng([seed, slot, 2])
    rows = draw_tokens(rng, s, (n_layers, s.conv_k - 1), io)
    n = (n_layers, s.conv_k - 1)
    return np.concatenate(
        [rows["q"].reshape(n + (-1,)), rows["k"].reshape(n + (-1,)),
         rows["v"].reshape(n + (-1,))], axis=-1)


def draw_pool_contents(seed: int, slots, s: Shapes, io: str, n_layers: int = 1):
    """States and windows for the listed slots (dict slot -> (state, window))."""
    return {int(i): (draw_slot_state(seed, int(i), s, n_layers),
                     draw_slot_window(seed, int(i), s, io, n_layers)) for i in slots}


# --------------------------------------------------------------------------
# Workloads.  Each returns a dict of numpy arrays plus the shapes.
# --------------------------------------------------------------------------

def tiny_layer_case(seed: int = 1000) -> dict:
    """One sequence on the tiny layer: 64-token prefill (chunk 16), then 16
    decode steps; fp32 io; slot state starts at zero.

    Draw order: conv weights, prefill tokens (64), decode tokens (16).
    """
    rng = np.random.default_rng(seed)
    s = TINY
    w = draw_conv_weights(rng, s)
    pre = draw_tokens(rng, s, (64,), "f32")
    dec = draw_tokens(rng, s, (16,), "f32")
    return {"shapes": s, "io": "f32", "conv_w": w, "prefill": pre, "decode": dec,
            "chunk": 16}


def decode_case(n_active: int, seed: int = 1001, n_slots: int = 256,
                s: Shapes = QWEN3_NEXT, io: str = "bf16") -> dict:
    """Multi-slot decode step: `n_active` distinct slots drawn at random from
    an `n_slots` pool, one token each.

    Draw order: conv weights, slot permutation, tokens [n_active].
    Slot contents come from draw_pool_contents(seed, ...) per slot.
    """
    rng = np.random.default_rng([seed, n_active])
    w = draw_conv_weights(rng, s)
    slots = rng.permutation(n_slots)[:n_active].astype(np.int32)
    tok = draw_tokens(rng, s, (n_active,), io)
    return {"shapes": s, "io": io, "conv_w": w, "slot_ids": slots, "n_slots": n_slots,
            "tokens": tok, "pool_seed": seed}


def prefill_case(T: int = 8192, seed: int = 1002, s: Shapes = QWEN3_NEXT,
                 io: str = "bf16") -> dict:
    """One sequence of T tokens into a fresh slot.

    Draw order: conv weights, tokens [T].
    """
    rng = np.random.default_rng([seed, T])
    w = draw_conv_weights(rng, s)
    tok = draw_tokens(rng, s, (T,), io)
    return {"shapes": s, "io": io, "conv_w": w, "tokens": tok}


def varlen_case(n_seq: int = 16, lo: int = 128, hi: int = 4096, n_continue: int = 4,
                seed: int = 1003, n_slots: int = 64, s: Shapes = QWEN3_NEXT,
                io: str = "bf16") -> dict:
    """Packed variable-length prefill into slots.

    Lengths are uniform integers on [lo, hi]; `n_continue` of the sequences
    (chosen at random) continue from pre-filled slot contents, the rest go
    into freshly reset slots.

    Draw order: conv weights, lengths, slot permutation, continuing subset,
    tokens [sum(lengths)].
    """
    rng = np.random.default_rng([seed, n_seq, lo, hi])
    w = draw_conv_weights(rng, s)
    lens = rng.integers(lo, hi + 1, size=n_seq)
    slots = rng.permutation(n_slots)[:n_seq].astype(np.int32)
    cont = np.zeros(n_seq, dtype=bool)
    if n_continue:
        cont[rng.choice(n_seq, size=n_continue, replace=False)] = True
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tok = draw_tokens(rng, s, (int(cu[-1]),), io)
    return {"shapes": s, "io": io, "conv_w": w, "cu_seqlens": cu, "slot_ids": slots,
            "continuing": cont, "n_slots": n_slots, "tokens": tok, "pool_seed": seed}


def verify_case(n_active: int = 128, n_tok: int = 4, seed: int = 1004, n_slots: int = 256,
                s: Shapes = QWEN3_NEXT, io: str = "bf16") -> dict:
    """Speculative verify: n_active slots, n_tok tokens each, accepted prefix
    lengths uniform on {1..n_tok}.

    Draw order: conv weights, slot permutation, accepted lengths,
    tokens [n_active][n_tok].
    """
    rng = np.random.default_rng([seed, n_active, n_tok])
    w = draw_conv_weights(rng, s)
    slots = rng.permutation(n_slots)[:n_active].astype(np.int32)
    acc = rng.integers(1, n_tok + 1, size=n_active).astype(np.int32)
    tok = draw_tokens(rng, s, (n_active, n_tok), io)
    return {"shapes": s, "io": io, "conv_w": w, "slot_ids": slots, "accept_len": acc,
            "n_tok": n_tok, "n_slots": n_slots, "tokens": tok, "pool_seed": seed}
