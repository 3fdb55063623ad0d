"""Host-side checks of the C-ABI library that need no GPU: it loads, exports every symbol the
header declares, and validates configurations before touching the device."""
import ctypes
import os
import re

import pytest

import workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    import adaptive_depth_recursive_amd as mor
    if not os.path.exists(mor.LIB_PATH):
        pytest.fail("libmor.so is not built (run __graft_entry__.build())")
    return mor


def test_header_symbols_exported():
    mor = _lib()
    text = open(os.path.join(ROOT, "include", "mor.h")).read()
    declared = set(re.findall(r"\b(mor_[a-z_]+)\s*\(", text))
    assert {"mor_init", "mor_prefill", "mor_route", "mor_workspace_bytes"} <= declared
    L = ctypes.CDLL(mor.LIB_PATH)
    for name in sorted(declared):
        assert hasattr(L, name), f"{name} declared in mor.h but not exported"
    assert set(mor.EXPORTED) == declared


def test_abi_version():
    mor = _lib()
    assert mor.lib().mor_abi_version() == 3


@pytest.mark.parametrize("name", sorted(workload.CONFIGS))
def test_workspace_bytes_for_every_config(name):
    mor = _lib()
    cfg = workload.get_config(name)
    n = mor.workspace_bytes(mor.make_config(cfg))
    assert n > 0
    if name == "smol360m_bf16":
        # packed weights (12 blocks x 9.83 M params x 2 B) + KV caches (32 streams) + activations
        assert 1.0e9 < n < 2.0e9


@pytest.mark.parametrize("field,value", [
    ("d_model", 100), ("head_dim", 48), ("n_layers", 9), ("n_kv_heads", 7), ("cap_den", 0),
    ("max_seq", 9000), ("n_rec", 9), ("sharing", 4), ("sharing", -1)])
def test_invalid_configs_rejected(field, value):
    mor = _lib()
    c = mor.make_config(workload.get_config("small_bf16"))
    setattr(c, field, value)
    assert mor.lib().mor_workspace_bytes(ctypes.byref(c)) == 0
    assert mor.lib().mor_last_error()


@pytest.mark.parametrize("scheme,L,ok", [
    ("middle_cycle", 8, True), ("middle_sequence", 8, True), ("cycle", 9, True), ("sequence", 9, True),
    ("cycle", 8, False), ("sequence", 10, False), ("middle_sequence", 9, False), ("cycle", 3, True),
    ("cycle", 2, False)])
def test_sharing_scheme_layer_counts(scheme, L, ok):
    """Middle schemes need L - 2 = N_r n_s, the others L = N_r n_s (n_s >= 1)."""
    mor = _lib()
    cfg = workload.get_config("small_bf16", sharing=scheme, n_layers=L)
    n = mor.lib().mor_workspace_bytes(ctypes.byref(mor.make_config(cfg)))
    assert (n > 0) == ok, mor.lib().mor_last_error()


def test_increasing_capacities_rejected():
    mor = _lib()
    c = mor.make_config(workload.get_config("small_bf16"))
    c.cap_num[1] = 3
    c.cap_num[0] = 2
    assert mor.lib().mor_workspace_bytes(ctypes.byref(c)) == 0


def test_init_checks_workspace_before_any_device_work():
    mor = _lib()
    L = mor.lib()
    c = mor.make_config(workload.get_config("tiny_f32"))
    w = mor.mor_weights()
    h = ctypes.c_void_p()
    dummy = ctypes.create_string_buffer(64)
    w.router_w = ctypes.addressof(dummy)
    shared = (mor.mor_block_weights * 1)()
    w.shared = shared
    st = L.mor_init(ctypes.byref(c), ctypes.byref(w), ctypes.addressof(dummy), 64, None,
                    ctypes.byref(h))
    assert st == mor.MOR_E_WORKSPACE
    assert b"needs" in L.mor_last_error()
    st = L.mor_init(ctypes.byref(c), None, ctypes.addressof(dummy), 64, None, ctypes.byref(h))
    assert st == mor.MOR_E_INVALID


def test_null_handle_calls_rejected():
    mor = _lib()
    L = mor.lib()
    assert L.mor_prefill(None, None, 1, 1, None, None, None, None, None, None) == mor.MOR_E_INVALID
    assert L.mor_route(None, None, None, None, 1, 1, 1, None, None, None, None) == mor.MOR_E_INVALID
    assert L.mor_route_noalloc(None, None, None, None, 1, 1, 1, None, None, None, None) == mor.MOR_E_INVALID
    assert L.mor_timing_clock(None, None) == mor.MOR_E_INVALID
    L.mor_destroy(None)


@pytest.mark.parametrize("field,value", [
    ("max_slots", 65), ("kv_page_tokens", 48), ("routing", 0), ("max_requests", 0), ("kv_pages", -1),
    ("d_model", 4160), ("sharing", 1), ("sharing", 2)])
def test_invalid_decode_configs_rejected(field, value):
    mor = _lib()
    c = mor.make_config(workload.get_config("small_thr_bf16"), max_slots=5, kv_page_tokens=16,
                        max_requests=4)
    assert mor.lib().mor_workspace_bytes(ctypes.byref(c)) > 0
    setattr(c, field, value)
    assert mor.lib().mor_workspace_bytes(ctypes.byref(c)) == 0
    assert mor.lib().mor_last_error()


def test_decode_workspace_includes_page_pool():
    """The default pool holds max_slots requests of max_seq tokens at full depth: pages of one
    layer's K and V (2 x Hkv x P x hd elements) for the 2 unique and N_r x n_s shared layer streams."""
    mor = _lib()
    cfg = workload.get_config("smol360m_mor4_decode")
    base = mor.workspace_bytes(mor.make_config(cfg, max_batch=1))
    c = mor.make_config(cfg, max_batch=1, max_slots=51, kv_page_tokens=64, max_requests=1024)
    full = mor.workspace_bytes(c)
    page_bytes = 2 * 5 * 64 * 64 * 2
    pages = 51 * (2 + 4 * 7) * (2048 // 64)
    assert pages * page_bytes < full - base < pages * page_bytes + 64 * 2 ** 20
    c.kv_pages = 100
    assert mor.workspace_bytes(c) < base + 100 * page_bytes + 64 * 2 ** 20


def test_decode_calls_rejected_without_handle():
    mor = _lib()
    L = mor.lib()
    assert L.mor_decode_submit(None, 1, None, None, None, None, None, None, None) == mor.MOR_E_INVALID
    assert L.mor_decode_step(None, 1, None, None) == mor.MOR_E_INVALID
