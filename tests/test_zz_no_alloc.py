"""The decode entry point that allocates nothing (ska_decode_attention_noalloc,
split workspace in the library's static device array) against
ska_decode_attention and the oracle: two calls in a row, the second on a
smaller batch with shorter sequences, then a call whose workspace would not
fit the array (rejected, nothing enqueued)."""
import numpy as np
import pytest

from long_context_decode_ada_amd import workloads as W
from oracle import oracle as O
from tests.parity_util import OUT_TOL, oracle_run, say

pytestmark = pytest.mark.gpu


def test_noalloc_decode_matches_the_decode_and_the_oracle():
    import torch
    from long_context_decode_ada_amd import ska
    dev = "cuda"
    w = W.make("gqa_t32k", 1 / 16)                     # B = 8, T = 2048, 32/8 heads, b = 4
    rng = O.calibrate(w.keys)
    pools = ska.DevicePools.for_workload(w, device=dev)
    cache = ska.Cache(pools)
    ska.encode_keys(cache, torch.from_numpy(w.keys).to(dev), torch.from_numpy(w.values.view(np.int16)).to(dev),
                    torch.from_numpy(w.slot).to(dev))
    q = torch.from_numpy(w.q).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    hp = W.host_pools(w)
    O.encode(hp, w.keys, w.values, w.slot, w.radius_mode, rng)
    cases = [(w.B, w.seq_lens, 0),                                          # the whole batch
             (3, np.array([700, 1, 2048 // 3], np.int32), 3)]               # smaller, explicit splits
    for B, lens, ns in cases:
        say("[noalloc] B=%d lens=%s splits=%d" % (B, lens.tolist(), ns))
        sl = torch.from_numpy(np.ascontiguousarray(lens[:B])).to(dev)
        out_na = torch.full((B, w.hq, w.d), float("nan"), device=dev)
        ska.decode_attention_noalloc(cache, q[:B].contiguous(), bt[:B].contiguous(), sl, num_splits=ns, out=out_na)
        out_ref = ska.decode_attention(cache, q[:B].contiguous(), bt[:B].contiguous(), sl, num_splits=ns)
        torch.cuda.synchronize()
        a, b = out_na.cpu().numpy(), out_ref.cpu().numpy()
        assert np.isfinite(a).all()
        diff = float(np.abs(a - b).max())
        pairs = [(s, h) for s in range(B) for h in range(w.hq)]
        o = O.decode(hp, w.radius_mode, rng, w.q, w.block_table, np.pad(lens[:B], (0, w.B - B)), pairs=pairs)
        err = float(np.abs(a - o[:B]).max())
        say("   max|noalloc - decode| %.3g, max|noalloc - oracle| %.3g" % (diff, err))
        assert diff <= 1e-6
        assert err <= OUT_TOL
    assert ska.device_errors(cache) == 0
    cache.free()


def test_noalloc_multi_round_batch_matches_the_decode():
    """A ragged batch that runs in several rounds (compacted grid, units in
    decreasing size through the unit table, which the no-alloc call keeps in
    its static array): equal to ska_decode_attention, two calls in a row."""
    import torch
    from long_context_decode_ada_amd import ska
    dev = "cuda"
    w = W.make("ragged_b64", 1 / 16)
    pools = ska.DevicePools.for_workload(w, device=dev)
    cache = ska.Cache(pools)
    ska.encode_keys(cache, torch.from_numpy(w.keys).to(dev), torch.from_numpy(w.values.view(np.int16)).to(dev),
                    torch.from_numpy(w.slot).to(dev))
    q = torch.from_numpy(w.q).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    for B in (w.B, w.B // 2):
        say("[noalloc] ragged_b64 1/16, B=%d" % B)
        sl = torch.from_numpy(np.ascontiguousarray(w.seq_lens[:B])).to(dev)
        out_na = torch.full((B, w.hq, w.d), float("nan"), device=dev)
        ska.decode_attention_noalloc(cache, q[:B].contiguous(), bt[:B].contiguous(), sl, out=out_na)
        out_ref = ska.decode_attention(cache, q[:B].contiguous(), bt[:B].contiguous(), sl)
        torch.cuda.synchronize()
        a, b = out_na.cpu().numpy(), out_ref.cpu().numpy()
        assert np.isfinite(a).all()
        assert np.array_equal(a, b)
    assert ska.device_errors(cache) == 0
    cache.free()


def test_noalloc_rejects_a_workspace_beyond_its_array():
    import torch
    from long_context_decode_ada_amd import ska
    dev = "cuda"
    w = W.make("gqa_t32k", 1 / 64)
    pools = ska.DevicePools.for_workload(w, device=dev, max_pages=1024, max_splits=128)
    cache = ska.Cache(pools)
    ska.encode_keys(cache, torch.from_numpy(w.keys).to(dev), None, torch.from_numpy(w.slot).to(dev))
    # 8 sequences x 32 heads x 128 splits of (128 + 2) floats: 17 MB of partials
    bt = torch.zeros((w.B, 1024), dtype=torch.int32, device=dev)
    sl = torch.full((w.B,), 16384, dtype=torch.int32, device=dev)
    q = torch.from_numpy(w.q).to(dev)
    out = torch.full((w.B, w.hq, w.d), 7.0, device=dev)
    with pytest.raises(ska.SkaError) as e:
        ska.decode_attention_noalloc(cache, q, bt, sl, num_splits=128, out=out)
    assert e.value.status == ska.SKA_ERR_INVALID
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    cache.free()
