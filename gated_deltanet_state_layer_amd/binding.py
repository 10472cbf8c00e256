"""Thin ctypes binding over libgdn (include/gdn.h): argument marshalling only.

Every step of the layer runs in the HIP kernels of libgdn.so.  PyTorch is
used for device memory (tensors are passed by data_ptr) and for the current
HIP stream.  There is no fallback: if the library is missing or fails to
load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_OK = 0
GDN_ERR_INVALID_ARG = -1
GDN_ERR_UNSUPPORTED = -2
GDN_ERR_BAD_INDEX = -3
GDN_ERR_WORKSPACE = -4
GDN_ERR_HIP = -5
GDN_ERR_RING = -6
GDN_ERR_HOST = -7
GDN_F32 = 0
GDN_BF16 = 1
GDN_VALIDATE = 1
GDN_GROUP_KERNEL = 2
GDN_STATIC_SCRATCH_BYTES = 64 << 20

EXPORTED = (
    "gdn_pool_bytes", "gdn_pool_create", "gdn_pool_destroy", "gdn_slot_reset",
    "gdn_decode_step", "gdn_verify_step", "gdn_prefill_workspace_bytes",
    "gdn_prefill_chunked", "gdn_prefill_chunked_static", "gdn_prefill_chunked_ckpt",
    "gdn_slot_copy", "gdn_ring_verify",
    "gdn_ring_commit", "gdn_ring_flush", "gdn_in_proj_workspace_bytes", "gdn_in_proj",
    "gdn_pool_error", "gdn_status_string",
)


class GdnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class PoolDesc(ctypes.Structure):
    _fields_ = [
        ("n_slots", ctypes.c_int32), ("n_layers", ctypes.c_int32),
        ("h_k", ctypes.c_int32), ("h_v", ctypes.c_int32),
        ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("conv_k", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
        ("q_scale", ctypes.c_float), ("norm_eps", ctypes.c_float),
        ("flags", ctypes.c_uint32), ("ring_len", ctypes.c_int32),
    ]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libgdn.so not found at {path}; build it with "
                           "`python -m gated_deltanet_state_layer_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    PSZ = ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "gdn_pool_bytes": [ctypes.POINTER(PoolDesc), PSZ, PSZ],
        "gdn_pool_create": [ctypes.POINTER(PoolDesc), P, P, P, ctypes.POINTER(P)],
        "gdn_pool_destroy": [P],
        "gdn_slot_reset": [P, I32, P, P],
        "gdn_slot_copy": [P, I32, P, P, P],
        "gdn_decode_step": [P, I32, I32, P, P, P, P, P, P, P, P, P],
        "gdn_verify_step": [P, I32, I32, P, I32, P, P, P, P, P, P, P, P, P],
        "gdn_prefill_workspace_bytes": [P, I32, I64, I32, PSZ],
        "gdn_prefill_chunked": [P, I32, I32, P, P, I64, I32, P, P, P, P, P, P, P, P, SZ, P],
        "gdn_prefill_chunked_static": [P, I32, I32, P, P, I64, I32, P, P, P, P, P, P, P, P],
        "gdn_prefill_chunked_ckpt": [P, I32, I32, P, P, I64, I32, P, P, P, P, P, P, P, I32, P, P,
                                     P, SZ, P],
        "gdn_ring_verify": [P, I32, I32, P, I32, P, P, P, P, P, P, P, P],
        "gdn_ring_commit": [P, I32, I32, P, I32, P, P, P, P, P, P, P, P],
        "gdn_ring_flush": [P, I32, I32, P, P],
        "gdn_in_proj_workspace_bytes": [P, I64, I32, PSZ],
        "gdn_in_proj": [P, I64, I32, P, P, P, P, P, P, P, P, SZ, P],
        "gdn_pool_error": [P, P, ctypes.POINTER(I32)],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = I32
    lib.gdn_status_string.argtypes = [I32]
    lib.gdn_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().gdn_status_string(status).decode()


def _check(status: int, what: str):
    if status != GDN_OK:
        raise GdnError(status, what)


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _need(t, name, numel, dtype):
    """Host-side check of a tensor argument before it becomes a raw pointer:
    a contiguous device tensor of `dtype` with at least `numel` elements, so
    that no kernel reads or writes past it.  A call that touches no element
    of it (numel 0) accepts anything, None included."""
    if numel <= 0:
        return
    if t is None:
        raise ValueError(f"{name}: missing")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: not a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: not contiguous")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, the call needs {numel}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _io_torch(io_dtype: int):
    return torch.bfloat16 if io_dtype == GDN_BF16 else torch.float32


def make_desc(n_slots, n_layers, h_k, h_v, d_k, d_v, conv_k, io_dtype=GDN_BF16,
              q_scale=0.0, norm_eps=0.0, flags=0, ring_len=0) -> PoolDesc:
    return PoolDesc(n_slots, n_layers, h_k, h_v, d_k, d_v, conv_k, io_dtype,
                    q_scale, norm_eps, flags, ring_len)


def ring_layout(desc: PoolDesc):
    """Byte offsets of the verify ring inside the aux buffer (the layout
    include/gdn.h documents): (count offset, record offset, floats per
    (slot, layer) record block), or None without a ring."""
    if desc.ring_len == 0:
        return None
    up = lambda x, a: (x + a - 1) // a * a
    io = 2 if desc.io_dtype == GDN_BF16 else 4
    sl = desc.n_slots * desc.n_layers
    c_conv = 2 * desc.h_k * desc.d_k + desc.h_v * desc.d_v
    win = sl * (desc.conv_k - 1) * c_conv * io
    cnt = up(win, 256) + 256 + up(sl * desc.h_k * 4, 256)
    rec = cnt + 2 * up(sl * 4, 256)
    stride = up(desc.ring_len * (desc.h_k * desc.d_k + desc.h_v * desc.d_v + 2 * desc.h_v), 64)
    return cnt, rec, stride


def pool_bytes(desc: PoolDesc):
    lib = load_library()
    sb, ab = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib.gdn_pool_bytes(ctypes.byref(desc), ctypes.byref(sb), ctypes.byref(ab)),
           "gdn_pool_bytes")
    return sb.value, ab.value


class Pool:
    """A slot pool over torch-owned device buffers.

    Attributes `state` ([n_slots, n_layers, h_v, d_v, d_k] fp32) and `window`
    ([n_slots, n_layers, conv_k-1, C_conv] io dtype) are views of the pool's
    device memory in the library's documented layout.
    """

    def __init__(self, desc: PoolDesc, device="cuda", stream=None):
        lib = load_library()
        self.desc = desc
        self.device = torch.device(device)
        sb, ab = pool_bytes(desc)
        self._state_buf = torch.empty(sb // 4, dtype=torch.float32, device=self.device)
        self._aux_buf = torch.empty(ab, dtype=torch.uint8, device=self.device)
        h = ctypes.c_void_p()
        _check(lib.gdn_pool_create(ctypes.byref(desc), _ptr(self._state_buf), _ptr(self._aux_buf),
                                   _stream(stream), ctypes.byref(h)), "gdn_pool_create")
        self._h = h
        self.c_conv = 2 * desc.h_k * desc.d_k + desc.h_v * desc.d_v
        self.io_torch = _io_torch(desc.io_dtype)
        self.state = self._state_buf.view(desc.n_slots, desc.n_layers, desc.h_v, desc.d_v, desc.d_k)
        io_size = 2 if desc.io_dtype == GDN_BF16 else 4
        nwin = desc.n_slots * desc.n_layers * (desc.conv_k - 1) * self.c_conv
        self.window = self._aux_buf[: nwin * io_size].view(self.io_torch).view(
            desc.n_slots, desc.n_layers, desc.conv_k - 1, self.c_conv)
        rl = ring_layout(desc)
        self.ring_count = self.ring_records = None
        if rl is not None:
            cnt, rec, stride = rl
            sl = desc.n_slots * desc.n_layers
            self.ring_count = self._aux_buf[cnt: cnt + 4 * sl].view(torch.int32).view(
                desc.n_slots, desc.n_layers)
            self.ring_records = self._aux_buf[rec: rec + 4 * sl * stride].view(torch.float32).view(
                desc.n_slots, desc.n_layers, stride)

    def close(self):
        if getattr(self, "_h", None):
            load_library().gdn_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- argument checks (shapes follow include/gdn.h) ----------------------
    def _tokens(self, rows, q, k, v, a, b, conv_w):
        d, io = self.desc, self.io_torch
        _need(q, "q", rows * d.h_k * d.d_k, io)
        _need(k, "k", rows * d.h_k * d.d_k, io)
        _need(v, "v", rows * d.h_v * d.d_v, io)
        _need(a, "a", rows * d.h_v, torch.float32)
        _need(b, "b", rows * d.h_v, torch.float32)
        _need(conv_w, "conv_w", self.c_conv * d.conv_k if rows else 0, torch.float32)

    def _out(self, rows, out):
        _need(out, "out", rows * self.desc.h_v * self.desc.d_v, self.io_torch)

    # -- calls -------------------------------------------------------------
    def reset(self, slot_ids, stream=None):
        lib = load_library()
        _need(slot_ids, "slot_ids", slot_ids.numel(), torch.int32)
        _check(lib.gdn_slot_reset(self._h, int(slot_ids.numel()), _ptr(slot_ids), _stream(stream)),
               "gdn_slot_reset")

    def copy(self, src_ids, dst_ids, stream=None):
        lib = load_library()
        _need(src_ids, "src_ids", src_ids.numel(), torch.int32)
        _need(dst_ids, "dst_ids", src_ids.numel(), torch.int32)
        _check(lib.gdn_slot_copy(self._h, int(src_ids.numel()), _ptr(src_ids), _ptr(dst_ids),
                                 _stream(stream)), "gdn_slot_copy")

    def decode(self, layer, slot_ids, q, k, v, a, b, conv_w, out, stream=None):
        lib = load_library()
        n = int(slot_ids.numel())
        _need(slot_ids, "slot_ids", n, torch.int32)
        self._tokens(n, q, k, v, a, b, conv_w)
        self._out(n, out)
        _check(lib.gdn_decode_step(self._h, layer, int(slot_ids.numel()), _ptr(slot_ids), _ptr(q),
                                   _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(conv_w), _ptr(out),
                                   _stream(stream)), "gdn_decode_step")
        return out

    def verify(self, layer, slot_ids, n_tok, q, k, v, a, b, conv_w, accept_len, out, stream=None):
        lib = load_library()
        n = int(slot_ids.numel())
        _need(slot_ids, "slot_ids", n, torch.int32)
        self._tokens(n * n_tok, q, k, v, a, b, conv_w)
        if accept_len is not None:
            _need(accept_len, "accept_len", n, torch.int32)
        if out is not None:   # None: commit only
            self._out(n * n_tok, out)
        _check(lib.gdn_verify_step(self._h, layer, int(slot_ids.numel()), _ptr(slot_ids), n_tok,
                                   _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(conv_w),
                                   _ptr(accept_len), _ptr(out), _stream(stream)),
               "gdn_verify_step")
        return out

    def ring_verify(self, layer, slot_ids, n_tok, q, k, v, a, b, conv_w, out, stream=None):
        lib = load_library()
        n = int(slot_ids.numel())
        _need(slot_ids, "slot_ids", n, torch.int32)
        self._tokens(n * n_tok, q, k, v, a, b, conv_w)
        self._out(n * n_tok, out)
        _check(lib.gdn_ring_verify(self._h, layer, int(slot_ids.numel()), _ptr(slot_ids), n_tok,
                                   _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(conv_w),
                                   _ptr(out), _stream(stream)), "gdn_ring_verify")
        return out

    def ring_commit(self, layer, slot_ids, n_tok, q, k, v, a, b, conv_w, accept_len, stream=None):
        lib = load_library()
        n = int(slot_ids.numel())
        _need(slot_ids, "slot_ids", n, torch.int32)
        self._tokens(n * n_tok, q, k, v, a, b, conv_w)
        _need(accept_len, "accept_len", n, torch.int32)
        _check(lib.gdn_ring_commit(self._h, layer, int(slot_ids.numel()), _ptr(slot_ids), n_tok,
                                   _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(conv_w),
                                   _ptr(accept_len), _stream(stream)), "gdn_ring_commit")

    def ring_flush(self, layer, slot_ids, stream=None):
        lib = load_library()
        _need(slot_ids, "slot_ids", slot_ids.numel(), torch.int32)
        _check(lib.gdn_ring_flush(self._h, layer, int(slot_ids.numel()), _ptr(slot_ids),
                                  _stream(stream)), "gdn_ring_flush")

    def in_proj_workspace_bytes(self, n_tok, hidden):
        lib = load_library()
        n = ctypes.c_size_t()
        _check(lib.gdn_in_proj_workspace_bytes(self._h, n_tok, hidden, ctypes.byref(n)),
               "gdn_in_proj_workspace_bytes")
        return n.value

    def in_proj(self, x, w, q, k, v, a, b, workspace=None, stream=None):
        """x [n_tok][hidden] bf16, w [C_conv + 2 h_v][hidden] bf16 -> q, k, v, a, b."""
        lib = load_library()
        n_tok, hidden = int(x.shape[0]), int(x.shape[1])
        d = self.desc
        _need(x, "x", n_tok * hidden, torch.bfloat16)
        _need(w, "w", (self.c_conv + 2 * d.h_v) * hidden if n_tok else 0, torch.bfloat16)
        _need(q, "q", n_tok * d.h_k * d.d_k, self.io_torch)
        _need(k, "k", n_tok * d.h_k * d.d_k, self.io_torch)
        _need(v, "v", n_tok * d.h_v * d.d_v, self.io_torch)
        _need(a, "a", n_tok * d.h_v, torch.float32)
        _need(b, "b", n_tok * d.h_v, torch.float32)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check(lib.gdn_in_proj(self._h, n_tok, hidden, _ptr(x), _ptr(w), _ptr(q), _ptr(k), _ptr(v),
                               _ptr(a), _ptr(b), _ptr(workspace), ws_bytes, _stream(stream)),
               "gdn_in_proj")

    def prefill_workspace_bytes(self, n_seq, total_tokens, chunk):
        lib = load_library()
        n = ctypes.c_size_t()
        _check(lib.gdn_prefill_workspace_bytes(self._h, n_seq, total_tokens, chunk,
                                               ctypes.byref(n)), "gdn_prefill_workspace_bytes")
        return n.value

    def prefill(self, layer, cu_seqlens, slot_ids, total_tokens, chunk, q, k, v, a, b, conv_w,
                out, workspace=None, stream=None):
        lib = load_library()
        n_seq = int(slot_ids.numel())
        self._prefill_args(n_seq, cu_seqlens, slot_ids, total_tokens, q, k, v, a, b, conv_w, out)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check(lib.gdn_prefill_chunked(self._h, layer, n_seq, _ptr(cu_seqlens), _ptr(slot_ids),
                                       total_tokens, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                       _ptr(b), _ptr(conv_w), _ptr(out), _ptr(workspace), ws_bytes,
                                       _stream(stream)), "gdn_prefill_chunked")
        return out

    def prefill_static(self, layer, cu_seqlens, slot_ids, total_tokens, chunk, q, k, v, a, b,
                       conv_w, out, stream=None):
        """gdn_prefill_chunked_static: the workspace is the library's own
        device array (no allocation)."""
        lib = load_library()
        n_seq = int(slot_ids.numel())
        self._prefill_args(n_seq, cu_seqlens, slot_ids, total_tokens, q, k, v, a, b, conv_w, out)
        _check(lib.gdn_prefill_chunked_static(self._h, layer, n_seq, _ptr(cu_seqlens),
                                              _ptr(slot_ids), total_tokens, chunk, _ptr(q),
                                              _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(conv_w),
                                              _ptr(out), _stream(stream)),
               "gdn_prefill_chunked_static")
        return out

    def prefill_ckpt(self, layer, cu_seqlens, slot_ids, total_tokens, chunk, q, k, v, a, b,
                     conv_w, out, ckpt_every, ckpt_offsets, ckpt_slots, workspace=None,
                     stream=None):
        lib = load_library()
        n_seq = int(slot_ids.numel())
        self._prefill_args(n_seq, cu_seqlens, slot_ids, total_tokens, q, k, v, a, b, conv_w, out)
        if ckpt_every > 0:
            _need(ckpt_offsets, "ckpt_offsets", n_seq + 1, torch.int32)
            _need(ckpt_slots, "ckpt_slots", 0 if ckpt_slots is None else ckpt_slots.numel(),
                  torch.int32)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check(lib.gdn_prefill_chunked_ckpt(self._h, layer, n_seq, _ptr(cu_seqlens),
                                            _ptr(slot_ids), total_tokens, chunk, _ptr(q), _ptr(k),
                                            _ptr(v), _ptr(a), _ptr(b), _ptr(conv_w), _ptr(out),
                                            ckpt_every, _ptr(ckpt_offsets), _ptr(ckpt_slots),
                                            _ptr(workspace), ws_bytes, _stream(stream)),
               "gdn_prefill_chunked_ckpt")
        return out

    def _prefill_args(self, n_seq, cu_seqlens, slot_ids, total_tokens, q, k, v, a, b, conv_w,
                      out):
        _need(slot_ids, "slot_ids", n_seq, torch.int32)
        _need(cu_seqlens, "cu_seqlens", n_seq + 1 if n_seq else 0, torch.int32)
        self._tokens(int(total_tokens), q, k, v, a, b, conv_w)
        self._out(int(total_tokens), out)

    def error(self, stream=None) -> int:
        lib = load_library()
        e = ctypes.c_int32()
        _check(lib.gdn_pool_error(self._h, _stream(stream), ctypes.byref(e)), "gdn_pool_error")
        return e.value
