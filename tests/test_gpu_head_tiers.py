"""GPU parity for pools with a tier per (page, KV head) (section 2.2 of the
page allocates tiers per token, head and layer): the encode writes each KV
head's records at that head's tier and offset, bit for bit as the oracle; the
decode, the decode step with append and the decompress baseline read them
at parity."""
import numpy as np
import pytest

from long_context_decode_ada_amd import workloads as W
from oracle import oracle as O
from tests.parity_util import compare, gpu_run, oracle_run, say

pytestmark = pytest.mark.gpu

PAGE = W.PAGE


@pytest.mark.parametrize("scale,batch,splits", [(1 / 16, 4, 0), (1 / 64, 3, 5), (1 / 8, 2, 0)])
def test_head_tier_pool_encode_and_decode(scale, batch, splits):
    w = W.make("mixed_tiers", scale, batch=batch, head_tiers=True)
    hb = w.page_bits.reshape(w.num_pages, w.hkv)
    say("[head tiers] B=%d lens %s, %d pages, %d of them with mixed head tiers" %
        (w.B, w.seq_lens.tolist(), w.num_pages, int(sum(len(set(r)) > 1 for r in hb))))
    rng = O.calibrate(w.keys)
    g = gpu_run(w, num_splits=splits)
    assert np.array_equal(g["range"], rng)
    o = oracle_run(w, rng)
    for k in ("kcode", "rcode", "v"):
        assert np.array_equal(g["pools"][k], o["pools"][k]), k
    assert g["errors"] == 0
    compare(w, g, o, rng, label="head tiers %g" % scale)


def test_head_tier_pool_append_step():
    import torch
    from long_context_decode_ada_amd import ska
    w = W.make("mixed_tiers", 1 / 16, batch=3, head_tiers=True)
    rng = O.calibrate(w.keys)
    dev = "cuda"
    pools = ska.DevicePools.for_workload(w, device=dev, poison=True)
    cache = ska.Cache(pools)
    starts = np.cumsum(np.concatenate([[0], w.seq_lens[:-1]])).astype(np.int64)
    last = starts + w.seq_lens.astype(np.int64) - 1
    keep = np.setdiff1d(np.arange(w.n_tokens), last)
    ska.encode_keys(cache, torch.from_numpy(w.keys[keep]).to(dev),
                    torch.from_numpy(np.ascontiguousarray(w.values[keep]).view(np.int16)).to(dev),
                    torch.from_numpy(w.slot[keep]).to(dev), radius_range=rng)
    out = ska.append_decode_attention(cache, torch.from_numpy(np.ascontiguousarray(w.keys[last])).to(dev),
                                      torch.from_numpy(np.ascontiguousarray(w.values[last]).view(np.int16)).to(dev),
                                      torch.from_numpy(w.q).to(dev), torch.from_numpy(w.block_table).to(dev),
                                      torch.from_numpy(w.seq_lens).to(dev))
    torch.cuda.synchronize()
    assert ska.device_errors(cache) == 0
    o = oracle_run(w, rng, want_logits=False)
    host = pools.to_host()
    for k in ("kcode", "rcode", "v"):
        assert np.array_equal(host[k], o["pools"][k]), k
    err = float(np.abs(out.cpu().numpy() - o["out"]).max())
    say("[head tiers append] max|out err| %.3g" % err)
    assert err <= 2e-3


def test_head_tier_pool_decompress():
    import torch
    from long_context_decode_ada_amd import ska
    w = W.make("mixed_tiers", 1 / 16, batch=3, head_tiers=True)
    g = gpu_run(w, want_logits=False)
    cache, rng = g["cache"], g["range"]
    dev = "cuda"
    kd = torch.full((w.num_pages, w.hkv, PAGE, w.d), 0x7FC0, dtype=torch.int16, device=dev)
    ska.decompress_keys(cache, torch.from_numpy(w.block_table).to(dev), torch.from_numpy(w.seq_lens).to(dev), kd)
    torch.cuda.synchronize()
    assert ska.device_errors(cache) == 0
    got = kd.cpu().numpy().view(np.uint16)
    hp = W.host_pools(w)
    hp["kcode"], hp["rcode"] = g["pools"]["kcode"], g["pools"]["rcode"]
    used = np.unique(w.slot // PAGE).astype(np.int32)
    want = O.decoded_keys(hp, w.radius_mode, rng, used)                  # [n][hkv][16][d]
    gv = (got[used].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ulp = np.maximum(np.abs(want), 1e-30) * 2.0 ** -7
    bad = int(np.count_nonzero(np.abs(gv - want) > ulp))
    say("[head tiers decompress] %d of %d values off by more than one bf16 ulp" % (bad, want.size))
    assert bad == 0
