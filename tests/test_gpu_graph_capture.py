"""The no-alloc decode (ska_decode_attention_noalloc) inside a captured HIP
graph, the use it exists for: the step is captured once with static input
and output buffers and replayed with new queries and lengths written into
those buffers between replays.  Every replay is checked against an eager
ska_decode_attention call on the same inputs (same kernels, same split
layout: equal bit for bit) and, on sampled rows, against the oracle.  The
replays are separated by eager work and device synchronisations.  Two
batches: one that runs in one round (one kernel per step) and a ragged one
that runs in several (the unit-order kernel and the decode kernel)."""
import numpy as np
import pytest

from long_context_decode_ada_amd import workloads as W
from oracle import oracle as O
from tests.parity_util import OUT_TOL, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,scale", [("gqa_t32k", 1 / 16), ("ragged_b64", 1 / 16)])
def test_noalloc_decode_replayed_from_a_graph(name, scale):
    import torch
    from long_context_decode_ada_amd import ska
    dev = "cuda"
    w = W.make(name, scale)
    rng = O.calibrate(w.keys)
    pools = ska.DevicePools.for_workload(w, device=dev)
    cache = ska.Cache(pools)
    ska.encode_keys(cache, torch.from_numpy(w.keys).to(dev), torch.from_numpy(w.values.view(np.int16)).to(dev),
                    torch.from_numpy(w.slot).to(dev))
    hp = W.host_pools(w)
    O.encode(hp, w.keys, w.values, w.slot, w.radius_mode, rng)

    # static buffers the graph reads and writes
    q = torch.from_numpy(w.q).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    out = torch.full((w.B, w.hq, w.d), float("nan"), device=dev)

    # an eager call first: the library looks up its static array on the first call
    ska.decode_attention_noalloc(cache, q, bt, sl, out=out)
    torch.cuda.synchronize()
    say("[graph] %s %.4g: capture" % (name, scale))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ska.decode_attention_noalloc(cache, q, bt, sl, out=out)
    torch.cuda.synchronize()

    gen = np.random.default_rng(20261204)
    for rep in range(4):
        # new inputs in the static buffers: fresh queries; from the second
        # replay on, every sequence also loses a random number of tokens
        qn = gen.standard_normal(w.q.shape).astype(np.float32)
        lens = w.seq_lens.copy()
        if rep > 0:
            lens = np.maximum(0, lens - gen.integers(0, 40, size=lens.shape)).astype(np.int32)
        q.copy_(torch.from_numpy(qn))
        sl.copy_(torch.from_numpy(lens))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        # eager work between replays: the same step through the plain entry point
        ref = ska.decode_attention(cache, q, bt, sl).cpu().numpy()
        assert np.isfinite(got).all(), rep
        assert np.array_equal(got, ref), (rep, float(np.nanmax(np.abs(got - ref))))
        rows = gen.choice(w.B, size=min(2, w.B), replace=False)
        pairs = [(int(s), h) for s in rows for h in range(w.hq)]
        o = O.decode(hp, w.radius_mode, rng, qn, w.block_table, lens, pairs=pairs)
        err = max(float(np.abs(got[s] - o[s]).max()) for s in rows)
        say("   replay %d: rows %s, max|graph - oracle| %.3g" % (rep, rows.tolist(), err))
        assert err <= OUT_TOL, (rep, err)
    assert ska.device_errors(cache) == 0
    del g
    cache.free()
