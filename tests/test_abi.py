"""The C ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any HIP call (runs without a GPU)."""
import ctypes
import os
import re

import pytest

from long_context_decode_ada_amd import ska

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ska.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(ska_[a-z_]+)\s*\(", txt)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert set(names) == set(ska.SYMBOLS), names
    L = ska.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for s in range(5):
        assert ska.status_string(s)


def _desc(**kw):
    base = dict(d=128, num_kv_heads=8, page_size=16, num_pages=4, radius_mode=1, radius_bits=8,
                tier_mask=1 << 4, query_mode=0, kcode=16, page_off=None, rcode=16, v=16, page_bits=16,
                head_tiers=0)
    base.update(kw)
    return ska.PoolDesc(*[base[f] for f, _ in ska.PoolDesc._fields_])


def _enc(desc, n=1, keys=16, slot=16, rr=None, cache=None):
    h = ctypes.c_void_p(cache)
    return ska.lib().ska_encode_keys(ctypes.byref(h), ctypes.byref(desc), keys, None, slot, n, rr, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(d=96), ska.SKA_ERR_UNSUPPORTED),
    (dict(d=3), ska.SKA_ERR_INVALID),
    (dict(page_size=32), ska.SKA_ERR_INVALID),
    (dict(num_kv_heads=0), ska.SKA_ERR_INVALID),
    (dict(num_pages=0), ska.SKA_ERR_INVALID),
    (dict(radius_mode=5), ska.SKA_ERR_INVALID),
    (dict(radius_bits=4), ska.SKA_ERR_UNSUPPORTED),
    (dict(tier_mask=0), ska.SKA_ERR_INVALID),
    (dict(tier_mask=1 << 5), ska.SKA_ERR_INVALID),
    (dict(tier_mask=(1 << 4) | 1), ska.SKA_ERR_INVALID),
    (dict(query_mode=2), ska.SKA_ERR_INVALID),
    (dict(kcode=None), ska.SKA_ERR_INVALID),
    (dict(v=None), ska.SKA_ERR_INVALID),
    (dict(page_bits=None), ska.SKA_ERR_INVALID),
    (dict(head_tiers=2), ska.SKA_ERR_INVALID),
    (dict(head_tiers=1), ska.SKA_ERR_INVALID),          # per-head tiers need the offsets
])
def test_encode_rejects_bad_pool(kw, expect):
    assert _enc(_desc(**kw)) == expect


def test_encode_rejects_bad_arguments():
    L = ska.lib()
    d = _desc()
    assert L.ska_encode_keys(None, ctypes.byref(d), 16, None, 16, 1, None, None) == ska.SKA_ERR_INVALID
    h = ctypes.c_void_p(None)
    assert L.ska_encode_keys(ctypes.byref(h), None, 16, None, 16, 1, None, None) == ska.SKA_ERR_INVALID
    assert _enc(d, n=-1) == ska.SKA_ERR_INVALID
    assert _enc(d, keys=None) == ska.SKA_ERR_INVALID
    assert _enc(d, slot=None) == ska.SKA_ERR_INVALID
    assert _enc(d, n=0) == ska.SKA_ERR_INVALID           # nothing to calibrate on
    import numpy as np
    bad = np.array([[2.0, 1.0]] * 8)                       # R_lo > R_hi
    assert _enc(d, rr=bad.ctypes.data_as(ctypes.c_void_p)) == ska.SKA_ERR_INVALID
    nan = np.array([[0.0, float("nan")]] * 8)
    assert _enc(d, rr=nan.ctypes.data_as(ctypes.c_void_p)) == ska.SKA_ERR_INVALID


def test_decode_rejects_bad_arguments_without_a_cache():
    L = ska.lib()
    assert L.ska_decode_attention(None, 16, 1, 32, 16, 4, 16, 0.0, 0, 16, None, None) == ska.SKA_ERR_INVALID


def test_append_rejects_bad_arguments_without_a_cache():
    L = ska.lib()
    assert L.ska_append_decode_attention(None, 16, 16, 16, 1, 32, 16, 4, 16, 0.0, 0, 16, None,
                                         None) == ska.SKA_ERR_INVALID


def test_null_free_and_queries():
    L = ska.lib()
    L.ska_free(None)
    assert L.ska_get_radius_range(None, None) == ska.SKA_ERR_INVALID
    v = ctypes.c_uint32()
    assert L.ska_device_errors(None, None, ctypes.byref(v)) == ska.SKA_ERR_INVALID


def test_baseline_entry_points_reject_bad_arguments_without_a_cache():
    L = ska.lib()
    assert L.ska_dense_decode_attention(None, 16, 16, 1, 32, 16, 4, 16, 0.0, 0, 16, None, None) == ska.SKA_ERR_INVALID
    assert L.ska_decompress_keys(None, 16, 1, 4, 16, 16, None) == ska.SKA_ERR_INVALID


def test_binding_refuses_tensors_it_cannot_pass_through():
    """The binding checks dtype, device, layout and shape before any call:
    the C ABI would read a wrong tensor as garbage."""
    import types
    import torch
    fake = types.SimpleNamespace(pools=types.SimpleNamespace(d=64, hkv=1, num_pages=4), handle=None)
    q = torch.zeros((2, 1, 64))
    bt = torch.zeros((2, 4), dtype=torch.int32)
    sl = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="device"):
        ska.decode_attention(fake, q, bt, sl)
    with pytest.raises(ValueError, match="shape"):
        ska.decode_attention(fake, torch.zeros((2, 1, 32)), bt, sl)
    with pytest.raises(ValueError):
        ska.rdr_plan(torch.zeros((2, 8)), torch.zeros((2, 8)), torch.zeros((2, 8), dtype=torch.uint8),
                     torch.zeros(2, dtype=torch.int32), torch.zeros(2, dtype=torch.int64), [4], [0.1], [100], 0.1)
