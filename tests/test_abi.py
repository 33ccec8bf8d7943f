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
                head_tiers=0, query_precision=0, max_batch=4, max_heads_q=32, max_pages=8, max_splits=0)
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
    (dict(query_precision=2), ska.SKA_ERR_INVALID),
    (dict(max_batch=0), ska.SKA_ERR_INVALID),            # the workspace maxima
    (dict(max_heads_q=0), ska.SKA_ERR_INVALID),
    (dict(max_heads_q=12), ska.SKA_ERR_INVALID),         # not a multiple of Hkv
    (dict(max_pages=0), ska.SKA_ERR_INVALID),
    (dict(max_splits=-1), ska.SKA_ERR_INVALID),
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


def test_decode_path_never_allocates():
    """The decode's workspace is allocated when the cache is created: nothing
    reachable from a decode call allocates, frees or synchronises."""
    src = open(os.path.join(ROOT, "long_context_decode_ada_amd", "csrc", "ska_api.cpp")).read()
    bodies = []
    for fn in ("ska_status prepare_decode(", "ska_status decode_impl("):
        i = src.index(fn)
        j = src.index("\n}\n", i)
        bodies.append(src[i:j])
    for b in bodies:
        for call in ("hipMalloc", "hipFree", "hipDeviceSynchronize", "hipStreamSynchronize", "hipMemset",
                     "ensure_", "launch_zero"):
            assert call not in b, call
    launch = open(os.path.join(ROOT, "long_context_decode_ada_amd", "csrc", "k_decode.hip")).read()
    i = launch.index("hipError_t launch_decode(")
    body = launch[i:launch.index("\n}\n", i)]
    assert "hipMalloc" not in body and "hipFree" not in body


@pytest.mark.gpu
def test_decode_outside_the_reserved_maxima_is_rejected():
    """A decode call beyond the batch, query heads, block-table width or
    explicit split count the cache was created for returns SKA_ERR_INVALID
    and enqueues nothing; within them it runs."""
    import numpy as np
    import torch
    from long_context_decode_ada_amd import workloads as W
    w = W.make("gqa_t32k", 1 / 64, batch=3)
    dev = "cuda"
    pools = ska.DevicePools.for_workload(w, device=dev, max_batch=2, max_splits=4)
    cache = ska.Cache(pools)
    ska.encode_keys(cache, torch.from_numpy(w.keys).to(dev), torch.from_numpy(w.values.view(np.int16)).to(dev),
                    torch.from_numpy(w.slot).to(dev))
    q = torch.from_numpy(w.q).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    out = torch.full((3, w.hq, w.d), 7.0, device=dev)
    with pytest.raises(ska.SkaError) as e:                 # batch 3 > 2
        ska.decode_attention(cache, q, bt, sl, out=out)
    assert e.value.status == ska.SKA_ERR_INVALID
    with pytest.raises(ska.SkaError) as e:                 # 8 splits > 4
        ska.decode_attention(cache, q[:2], bt[:2], sl[:2], num_splits=8, out=out[:2])
    assert e.value.status == ska.SKA_ERR_INVALID
    wide = torch.zeros((2, w.max_pages + 1), dtype=torch.int32, device=dev)
    wide[:, : w.max_pages] = bt[:2]
    with pytest.raises(ska.SkaError) as e:                 # a wider block table
        ska.decode_attention(cache, q[:2], wide, sl[:2], out=out[:2])
    assert e.value.status == ska.SKA_ERR_INVALID
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())                        # nothing ran
    ska.decode_attention(cache, q[:2], bt[:2], sl[:2], num_splits=4, out=out[:2])
    ska.decode_attention(cache, q[:2], bt[:2], sl[:2], out=out[:2])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out[:2]).all()) and bool((out[2] == 7.0).all())
    assert ska.device_errors(cache) == 0
    cache.free()


@pytest.mark.gpu
def test_prepared_decode_call_matches_the_plain_call():
    """The prepared call (arguments checked and marshalled once) enqueues the
    same library call: identical outputs, coded and dense, on every call."""
    import numpy as np
    import torch
    from long_context_decode_ada_amd import workloads as W
    w = W.make("gqa_t32k", 1 / 64, batch=2)
    dev = "cuda"
    cache = ska.Cache(ska.DevicePools.for_workload(w, device=dev))
    ska.encode_keys(cache, torch.from_numpy(w.keys).to(dev), torch.from_numpy(w.values.view(np.int16)).to(dev),
                    torch.from_numpy(w.slot).to(dev))
    q = torch.from_numpy(w.q).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    kd = torch.zeros((w.num_pages, w.hkv, 16, w.d), dtype=torch.int16, device=dev)
    ska.decompress_keys(cache, bt, sl, kd)
    ref = ska.decode_attention(cache, q, bt, sl, num_splits=3)
    ref_d = ska.dense_decode_attention(cache, kd, q, bt, sl, num_splits=3)
    out = torch.full_like(ref, 7.0)
    call = ska.prepared_decode(cache, q, bt, sl, out, num_splits=3)
    dcall = ska.prepared_decode(cache, q, bt, sl, out, num_splits=3, k_dense=kd)
    for _ in range(3):
        out.fill_(7.0)
        call()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        out.fill_(7.0)
        dcall()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_d)
    with pytest.raises(ValueError):                        # checked once, at preparation
        ska.prepared_decode(cache, q, bt, sl, out[:1])
    assert ska.device_errors(cache) == 0
    cache.free()


@pytest.mark.gpu
def test_profile_records_one_duration_per_decode_call():
    """ska_profile_begin/ska_profile_read: one finite positive duration per
    decode call while recording is on, none after it is turned off, and the
    outputs unchanged by the events."""
    import numpy as np
    import torch
    from long_context_decode_ada_amd import workloads as W
    w = W.make("gqa_t32k", 1 / 64, batch=2)
    dev = "cuda"
    cache = ska.Cache(ska.DevicePools.for_workload(w, device=dev))
    ska.encode_keys(cache, torch.from_numpy(w.keys).to(dev), torch.from_numpy(w.values.view(np.int16)).to(dev),
                    torch.from_numpy(w.slot).to(dev))
    q = torch.from_numpy(w.q).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    ref = ska.decode_attention(cache, q, bt, sl)
    ska.profile_begin(cache, 8)
    outs = [ska.decode_attention(cache, q, bt, sl) for _ in range(3)]
    ms = ska.profile_read(cache, 8)
    assert ms.shape == (3,) and np.all(np.isfinite(ms)) and np.all(ms > 0), ms
    assert all(torch.equal(o, ref) for o in outs)
    ska.profile_begin(cache, 0)
    ska.decode_attention(cache, q, bt, sl)
    assert ska.profile_read(cache, 8).shape == (0,)
    assert ska.device_errors(cache) == 0
    cache.free()
