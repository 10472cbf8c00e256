"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every call include/gdn.h declares, sizes pools as documented and rejects bad
arguments before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


@pytest.fixture(scope="module")
def lib():
    from gated_deltanet_state_layer_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libgdn.so is not built (run __graft_entry__.build())")
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_header_declares_the_documented_calls():
    names = declared_functions()
    for want in ("gdn_pool_create", "gdn_slot_reset", "gdn_decode_step", "gdn_prefill_chunked",
                 "gdn_verify_step"):
        assert want in names


def test_binding_constants_match_the_header():
    """Every GDN_ constant of the binding has the value include/gdn.h gives."""
    from gated_deltanet_state_layer_amd import binding as B
    text = open(HEADER).read()
    seen = 0
    for name, expr in re.findall(r"^#define (GDN_\w+) (.+?)\s*(?:/\*.*)?$", text, re.M):
        if not hasattr(B, name):
            continue
        expr = re.sub(r"\(size_t\)", "", expr)
        expr = re.sub(r"(\d+)u\b", r"\1", expr)
        assert getattr(B, name) == eval(expr, {}), name
        seen += 1
    assert seen >= 12


def test_library_exports_every_declared_symbol(lib):
    from gated_deltanet_state_layer_amd import binding
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(binding.EXPORTED)


def test_pool_bytes_layout(lib):
    from gated_deltanet_state_layer_amd import binding as B
    d = B.make_desc(256, 1, 16, 32, 128, 128, 4, B.GDN_BF16)
    sb, ab = B.pool_bytes(d)
    assert sb == 256 * 32 * 128 * 128 * 4
    win = 256 * 3 * (2 * 16 * 128 + 32 * 128) * 2
    assert ab == (win + 255) // 256 * 256 + 256 + (256 * 1 * 16 * 4 + 255) // 256 * 256
    d = B.make_desc(3, 2, 2, 2, 32, 32, 4, B.GDN_F32)
    sb, ab = B.pool_bytes(d)
    assert sb == 3 * 2 * 2 * 32 * 32 * 4
    assert ab == (3 * 2 * 3 * 192 * 4 + 255) // 256 * 256 + 256 + 256   # 3*2*2 counters


def test_pool_bytes_layout_with_a_verify_ring(lib):
    from gated_deltanet_state_layer_amd import binding as B
    base = B.pool_bytes(B.make_desc(256, 1, 16, 32, 128, 128, 4, B.GDN_BF16))[1]
    d = B.make_desc(256, 1, 16, 32, 128, 128, 4, B.GDN_BF16, ring_len=8)
    sb, ab = B.pool_bytes(d)
    assert sb == 256 * 32 * 128 * 128 * 4                 # the state buffer does not change
    per_tok = 16 * 128 + 32 * 128 + 2 * 32                # k^, v, a, b
    stride = (8 * per_tok + 63) // 64 * 64
    assert ab == base + 2 * 1024 + 256 * stride * 4       # counts, commit counters, records
    cnt, rec, st = B.ring_layout(d)
    assert (cnt, rec, st) == (base, base + 2048, stride)
    assert rec % 256 == 0 and ab == rec + 256 * stride * 4
    assert B.ring_layout(B.make_desc(4, 1, 2, 4, 64, 64, 4)) is None
    # tiny shapes: the record block is padded to 64 floats (256 bytes)
    d = B.make_desc(3, 2, 1, 1, 32, 32, 2, B.GDN_F32, ring_len=1)
    cnt, rec, st = B.ring_layout(d)
    assert st == 128 and B.pool_bytes(d)[1] == rec + 3 * 2 * 128 * 4


@pytest.mark.parametrize("field,value,status", [
    ("n_slots", 0, -1), ("h_v", 3, -1), ("d_k", 96, -2), ("d_v", 32, -2), ("conv_k", 0, -1), ("conv_k", 1, -2),
    ("conv_k", 9, -2), ("io_dtype", 7, -1), ("flags", 4, -1), ("flags", 8, -1), ("q_scale", -1.0, -1),
    ("ring_len", -1, -1), ("ring_len", 25, -2),
])
def test_bad_descriptor_is_rejected(lib, field, value, status):
    from gated_deltanet_state_layer_amd import binding as B
    d = B.make_desc(4, 1, 2, 4, 64, 64, 4)
    setattr(d, field, value)
    sb, ab = ctypes.c_size_t(7), ctypes.c_size_t(7)
    assert lib.gdn_pool_bytes(ctypes.byref(d), ctypes.byref(sb), ctypes.byref(ab)) == status
    assert sb.value == 7 and ab.value == 7


def test_known_flags_are_accepted(lib):
    from gated_deltanet_state_layer_amd import binding as B
    for flags in (B.GDN_VALIDATE, B.GDN_GROUP_KERNEL, B.GDN_VALIDATE | B.GDN_GROUP_KERNEL):
        d = B.make_desc(4, 1, 2, 4, 64, 64, 4, flags=flags)
        sb, ab = ctypes.c_size_t(0), ctypes.c_size_t(0)
        assert lib.gdn_pool_bytes(ctypes.byref(d), ctypes.byref(sb), ctypes.byref(ab)) == 0
        assert (sb.value, ab.value) == B.pool_bytes(B.make_desc(4, 1, 2, 4, 64, 64, 4))


def test_null_arguments_are_rejected_before_any_device_work(lib):
    from gated_deltanet_state_layer_amd import binding as B
    d = B.make_desc(4, 1, 2, 4, 64, 64, 4)
    h = ctypes.c_void_p()
    assert lib.gdn_pool_create(ctypes.byref(d), None, None, None, ctypes.byref(h)) == -1
    assert lib.gdn_pool_create(None, None, None, None, ctypes.byref(h)) == -1
    # Misaligned buffers are refused without a launch.
    assert lib.gdn_pool_create(ctypes.byref(d), ctypes.c_void_p(16), ctypes.c_void_p(256), None,
                               ctypes.byref(h)) == -1
    nul = None
    assert lib.gdn_slot_reset(nul, 1, nul, nul) == -1
    assert lib.gdn_decode_step(nul, 0, 1, *([nul] * 9)) == -1
    assert lib.gdn_verify_step(nul, 0, 1, nul, 2, *([nul] * 9)) == -1
    assert lib.gdn_prefill_chunked(nul, 0, 1, nul, nul, 8, 64, *([nul] * 8), 0, nul) == -1
    assert lib.gdn_prefill_chunked_ckpt(nul, 0, 1, nul, nul, 8, 64, *([nul] * 7), 64, nul, nul,
                                        nul, 0, nul) == -1
    assert lib.gdn_slot_copy(nul, 1, nul, nul, nul) == -1
    assert lib.gdn_ring_verify(nul, 0, 1, nul, 2, *([nul] * 8)) == -1
    assert lib.gdn_ring_commit(nul, 0, 1, nul, 2, *([nul] * 8)) == -1
    assert lib.gdn_ring_flush(nul, 0, 1, nul, nul) == -1
    assert lib.gdn_in_proj(nul, 4, 64, *([nul] * 8), 0, nul) == -1
    assert lib.gdn_in_proj_workspace_bytes(nul, 4, 64, ctypes.byref(ctypes.c_size_t())) == -1
    n = ctypes.c_size_t()
    assert lib.gdn_prefill_workspace_bytes(nul, 1, 8, 64, ctypes.byref(n)) == -1
    e = ctypes.c_int32()
    assert lib.gdn_pool_error(nul, nul, ctypes.byref(e)) == -1
    assert lib.gdn_pool_destroy(nul) == -1


def test_status_strings(lib):
    from gated_deltanet_state_layer_amd import binding as B
    assert B.status_string(0) == "ok"
    for s in (-1, -2, -3, -4, -5, -6):
        assert B.status_string(s) != "unknown status"
    assert B.status_string(42) == "unknown status"


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: asked for more it prints a JSON error line
    and exits with status 2 before touching a device."""
    import json
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "--gpus must be 1" in json.loads(r.stdout.strip().splitlines()[-1])["error"]
