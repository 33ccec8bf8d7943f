"""GPU parity of the two baselines the codes are set against (section 1 of the
page): dense bf16 paged attention, and decompress-then-dot (the dense keys
r~ * u(c) written to HBM, then dense attention).  Both run through the C ABI
on the same pools as the coded kernels and are checked against the CPU
oracle: the decompressed keys within one bf16 unit in the last place of the
oracle's binary64 keys, the dense decode's outputs within 2e-3 and its logits
within 1e-4 of their bound scale * |q| * |k| (the query enters the MFMA as an
exact bf16 hi + lo pair)."""
import math

import numpy as np
import pytest

from long_context_decode_ada_amd import workloads as W
from oracle import oracle as O
from tests.parity_util import OUT_TOL, say

pytestmark = pytest.mark.gpu

PAGE = W.PAGE
CASES = [
    ("tiny", 1.0, None),
    ("gqa_t32k", 1 / 32, None),
    ("long_t128k", 1 / 128, None),
    ("ragged_b64", 1 / 32, None),
    ("mixed_tiers", 1 / 16, 4),
]


def _bf16(x):
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _bf16_to_f64(h):
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _setup(w):
    """Coded pools (values shared with the dense path) and a dense key pool
    holding the keys in bf16, NaN in every slot no token uses."""
    import torch
    from long_context_decode_ada_amd import ska
    dev = "cuda"
    pools = ska.DevicePools.for_workload(w, device=dev, poison=True)
    cache = ska.Cache(pools)
    ska.encode_keys(cache, torch.from_numpy(w.keys).to(dev), torch.from_numpy(w.values.view(np.int16)).to(dev),
                    torch.from_numpy(w.slot).to(dev))
    kd_host = np.full((w.num_pages, w.hkv, PAGE, w.d), 0x7FC0, np.uint16)
    kd_host[w.slot // PAGE, :, w.slot % PAGE, :] = _bf16(w.keys)
    kd = torch.from_numpy(kd_host.view(np.int16)).to(dev)
    return cache, pools, kd, kd_host


def _dense_run(cache, kd, w, num_splits=0):
    import torch
    from long_context_decode_ada_amd import ska
    dev = "cuda"
    q = torch.from_numpy(w.q).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    out = ska.dense_decode_attention(cache, kd, q, bt, sl, num_splits=num_splits)
    lg = torch.full((w.B, w.hq, w.max_pages * PAGE), float("nan"), device=dev)
    out_dbg = ska.dense_decode_attention(cache, kd, q, bt, sl, num_splits=num_splits, logits=lg)
    torch.cuda.synchronize()
    return out.cpu().numpy(), out_dbg.cpu().numpy(), lg.cpu().numpy()


def _check_dense(w, kd_host, v_host, out, out_dbg, lg, label):
    ref, ref_lg = O.dense_decode(kd_host, v_host, w.q, w.block_table, w.seq_lens, want_logits=True)
    oe = max(np.abs(out - ref).max(), np.abs(out_dbg - ref).max())
    scale = 1.0 / math.sqrt(w.d)
    qn = np.linalg.norm(w.q.astype(np.float64), axis=2)
    kn = np.linalg.norm(_bf16_to_f64(kd_host), axis=3)          # [num_pages][hkv][16]
    le = 0.0
    g = w.hq // w.hkv
    for s in range(w.B):
        n = int(w.seq_lens[s])
        t = np.arange(n)
        phys = w.block_table[s, t // PAGE]
        for h in range(w.hq):
            bound = scale * qn[s, h] * kn[phys, h // g, t % PAGE]
            le = max(le, float((np.abs(lg[s, h, :n] - ref_lg[s, h, :n]) / np.maximum(bound, 1e-30)).max()))
    say("[%s] dense decode: max|out err| %.3g  max logit err/bound %.3g" % (label, oe, le))
    assert oe <= OUT_TOL
    assert le <= 1e-4


@pytest.mark.parametrize("name,scale,batch", CASES)
def test_dense_decode_matches_oracle(name, scale, batch):
    w = W.make(name, scale, batch=batch)
    cache, pools, kd, kd_host = _setup(w)
    out, out_dbg, lg = _dense_run(cache, kd, w)
    v_host = pools.to_host()["v"].reshape(w.num_pages, w.hkv, w.d, PAGE)
    _check_dense(w, kd_host, v_host, out, out_dbg, lg, name)
    from long_context_decode_ada_amd import ska
    assert ska.device_errors(cache) == 0


def test_dense_decode_split_counts_agree():
    w = W.make("gqa_t32k", 1 / 32, batch=3)
    cache, pools, kd, kd_host = _setup(w)
    base, _, _ = _dense_run(cache, kd, w, num_splits=1)
    for ns in (3, 16):
        out, _, _ = _dense_run(cache, kd, w, num_splits=ns)
        assert np.abs(out - base).max() < 1e-4


@pytest.mark.parametrize("name,scale,batch", CASES)
def test_decompress_then_dot(name, scale, batch):
    """ska_decompress_keys writes r~ u(c) of every resident slot within one
    bf16 ulp of the oracle's binary64 dense keys (the kernel forms them in
    binary32, so a value within a few binary32 roundings of a bf16 rounding
    boundary may round the other way) and leaves the other slots untouched;
    the dense decode over them then matches the oracle's dense attention over
    the same bf16 keys."""
    import torch
    from long_context_decode_ada_amd import ska
    w = W.make(name, scale, batch=batch)
    cache, pools, _, _ = _setup(w)
    dev = "cuda"
    kd = torch.full((w.num_pages, w.hkv, PAGE, w.d), 0x7FC0, dtype=torch.int16, device=dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    ska.decompress_keys(cache, bt, sl, kd)
    torch.cuda.synchronize()
    got = kd.cpu().numpy().view(np.uint16)
    host = pools.to_host()
    rng = ska.radius_range(cache)
    hp = W.host_pools(w)
    hp["kcode"], hp["rcode"] = host["kcode"], host["rcode"]
    phys = np.arange(w.num_pages, dtype=np.int32)
    want = O.decoded_keys(hp, w.radius_mode, rng, phys)          # [num_pages][hkv][16][d]
    used = np.zeros((w.num_pages, PAGE), bool)
    for s in range(w.B):
        for p in range((int(w.seq_lens[s]) + PAGE - 1) // PAGE):
            used[w.block_table[s, p], :] = True                   # whole resident pages are written
    g = _bf16_to_f64(got)[used.nonzero()[0], :, used.nonzero()[1], :]
    r = want[used.nonzero()[0], :, used.nonzero()[1], :]
    ulp = np.maximum(np.abs(r), 1e-30) * 2.0 ** -7
    bad = int(np.count_nonzero(np.abs(g - r) > ulp))
    say("[%s] decompressed keys: %d of %d values off by more than one bf16 ulp; max rel %.3g" %
        (name, bad, g.size, float((np.abs(g - r) / np.maximum(np.abs(r), 1e-30)).max())))
    assert bad == 0
    assert (got[~used.any(1)] == 0x7FC0).all()                    # untouched pages
    assert ska.device_errors(cache) == 0
    out, out_dbg, lg = _dense_run(cache, kd, w)
    v_host = host["v"].reshape(w.num_pages, w.hkv, w.d, PAGE)
    _check_dense(w, got, v_host, out, out_dbg, lg, name + " decompressed")
