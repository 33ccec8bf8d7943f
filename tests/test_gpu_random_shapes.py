"""GPU parity on seeded random shapes beyond the five workloads: head
dimension, KV heads, group size, batch, lengths (zero, page boundaries,
odd tails), one tier or mixed tiers (fixed stride or packed pages, tiers per
page or per (page, KV head)), radius mode, query mode and split count are
drawn per case, and so is the precision of the query direction (binary16 or
binary32).  Every case checks the encode bit for bit and the decode
(outputs and logits) against the oracle; every other case also runs the
decode step with append."""
import os

import numpy as np
import pytest

from long_context_decode_ada_amd import workloads as W
from oracle import oracle as O
from tests.parity_util import compare, gpu_run, oracle_run, say

pytestmark = pytest.mark.gpu

PAGE = W.PAGE
TIERS = [2, 3, 4, 6, 8]


def _case(seed):
    r = np.random.default_rng(1000 + seed)
    d = int(r.choice([64, 128]))
    hkv = int(r.choice([1, 2, 4, 8]))
    g = int(r.choice([1, 2, 4]))
    B = int(r.integers(1, 7))
    lens = r.integers(0, 700, B)
    for s in range(B):                      # some lengths on or next to a page boundary
        if r.random() < 0.4:
            lens[s] = int(r.integers(0, 40)) * PAGE + int(r.choice([-1, 0, 1]))
    lens = (np.clip(lens, 0, None) * LEN_SCALE).astype(np.int32)
    if r.random() < 0.4:
        tiers = [int(r.choice(TIERS))]
    else:
        tiers = sorted(int(t) for t in r.choice(TIERS, size=int(r.integers(2, 6)), replace=False))
    head_tiers = len(tiers) > 1 and r.random() < 0.4
    packed = len(tiers) > 1 and (head_tiers or r.random() < 0.7)
    npg = [(int(n) + PAGE - 1) // PAGE for n in lens]
    num_pages = sum(npg) + int(r.integers(0, 5))
    perm = r.permutation(num_pages)
    max_pages = max(1, max(npg))
    bt = np.zeros((B, max_pages), np.int32)
    k = 0
    for s in range(B):
        bt[s, : npg[s]] = perm[k: k + npg[s]]
        k += npg[s]
    pb = r.choice(tiers, size=(num_pages * hkv) if head_tiers else num_pages).astype(np.uint8)
    bstride = max(tiers)
    if packed:
        per = PAGE if head_tiers else hkv * PAGE
        sizes = per * np.array([W.record_bytes(d, int(b)) for b in pb], np.uint64)
        off = np.zeros(pb.shape[0], np.uint64)
        off[1:] = np.cumsum(sizes)[:-1]
        kcode_bytes = int(sizes.sum())
    else:
        pb[:] = bstride if len(tiers) == 1 else pb    # fixed stride: any tier, the widest's room
        off = None
        kcode_bytes = num_pages * hkv * PAGE * W.record_bytes(d, bstride)
    n = int(lens.sum())
    keys = (r.standard_normal((n, hkv, d)) * r.lognormal(0, 0.5, (1, hkv, d))).astype(np.float32)
    values = W._bf16_bits(r.standard_normal((n, hkv, d)).astype(np.float32))
    q = r.standard_normal((B, hkv * g, d)).astype(np.float32)
    slot = np.empty(n, np.int64)
    o = 0
    for s in range(B):
        t = np.arange(int(lens[s]))
        slot[o: o + len(t)] = bt[s, t // PAGE].astype(np.int64) * PAGE + t % PAGE
        o += len(t)
    w = W.Workload(name="random%d" % seed, d=d, hq=hkv * g, hkv=hkv, B=B,
                   radius_mode=int(r.choice([W.UNIFORM, W.LOG])), tier_mask=sum(1 << t for t in tiers),
                   seq_lens=lens, block_table=bt, num_pages=num_pages, page_bits=pb, page_off=off,
                   bstride=bstride, kcode_bytes=kcode_bytes, keys=keys, values=values, slot=slot, q=q,
                   head_tiers=head_tiers)
    splits, qmode = int(r.choice([0, 1, 3, 7])), int(r.choice([0, 0, 1]))
    qprec = int(r.random() < 0.5)          # query direction in binary16 or binary32
    return w, splits, qmode, qprec


# 40 seeds by default; SKA_RANDOM_SEEDS=<n> runs seeds 0..n-1 (a longer sweep);
# SKA_RANDOM_LEN_SCALE=<k> multiplies the drawn lengths by k (longer rows:
# several 64-page chunks per wave and more splits)
NSEEDS = int(os.environ.get("SKA_RANDOM_SEEDS", "40"))
LEN_SCALE = int(os.environ.get("SKA_RANDOM_LEN_SCALE", "1"))


@pytest.mark.parametrize("seed", range(NSEEDS))
def test_random_shape_parity(seed):
    w, splits, qmode, qprec = _case(seed)
    say("[random %d] d=%d hkv=%d G=%d B=%d lens=%s tiers=%s head_tiers=%s packed=%s splits=%d query_mode=%d "
        "query_precision=%d" %
        (seed, w.d, w.hkv, w.hq // w.hkv, w.B, w.seq_lens.tolist(), sorted(t for t in range(9) if w.tier_mask >> t & 1),
         w.head_tiers, w.page_off is not None, splits, qmode, qprec))
    if w.n_tokens == 0:
        pytest.skip("no token in this draw")
    rng = O.calibrate(w.keys)
    g = gpu_run(w, num_splits=splits, query_mode=qmode, query_precision=qprec)
    assert np.array_equal(g["range"], rng)
    o = oracle_run(w, rng, query_mode=qmode)
    for k in ("kcode", "rcode", "v"):
        assert np.array_equal(g["pools"][k], o["pools"][k]), k
    assert g["errors"] == 0
    compare(w, g, o, rng, label="random %d" % seed)
    if seed % 2 == 0:
        _append_check(w, rng, splits, qmode, qprec, o)


def _append_check(w, rng, splits, qmode, qprec, o):
    import torch
    from long_context_decode_ada_amd import ska
    dev = "cuda"
    pools = ska.DevicePools.for_workload(w, device=dev, poison=True, query_mode=qmode, query_precision=qprec)
    cache = ska.Cache(pools)
    starts = np.concatenate([[0], np.cumsum(w.seq_lens)[:-1]]).astype(np.int64)
    last = np.where(w.seq_lens > 0, starts + w.seq_lens - 1, -1)
    keep = np.setdiff1d(np.arange(w.n_tokens), last[last >= 0])
    ska.encode_keys(cache, torch.from_numpy(np.ascontiguousarray(w.keys[keep])).to(dev),
                    torch.from_numpy(np.ascontiguousarray(w.values[keep]).view(np.int16)).to(dev),
                    torch.from_numpy(np.ascontiguousarray(w.slot[keep])).to(dev), radius_range=rng)
    nk = np.zeros((w.B, w.hkv, w.d), np.float32)
    nv = np.zeros((w.B, w.hkv, w.d), np.uint16)
    for s in range(w.B):
        if last[s] >= 0:
            nk[s], nv[s] = w.keys[last[s]], w.values[last[s]]
    out = ska.append_decode_attention(cache, torch.from_numpy(nk).to(dev), torch.from_numpy(nv.view(np.int16)).to(dev),
                                      torch.from_numpy(w.q).to(dev), torch.from_numpy(w.block_table).to(dev),
                                      torch.from_numpy(w.seq_lens).to(dev), num_splits=splits)
    torch.cuda.synchronize()
    assert ska.device_errors(cache) == 0
    host = pools.to_host()
    for k in ("kcode", "rcode", "v"):
        assert np.array_equal(host[k], o["pools"][k]), k
    err = float(np.abs(out.cpu().numpy() - o["out"]).max())
    say("   append: max|out err| %.3g" % err)
    assert err <= 2e-3
