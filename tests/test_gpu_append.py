"""GPU parity of the decode step with append (ska_append_decode_attention):
the step's new token of each sequence is encoded into its page slot (the
write path of section 2.3 of the page, dense key -> spherical codes -> paged
store) and then decoded with the rest.  The pools after the step must equal,
bit for bit, the oracle's encode of every token at once (with the same radius
range), and the output and logits must match the oracle's decode over all
tokens to the decode tolerances.  Sequences of length 0 append nothing; the
new token may open a new page; pools of mixed tiers encode it at its page's
tier."""
import numpy as np
import pytest

from long_context_decode_ada_amd import workloads as W
from oracle import oracle as O
from tests.parity_util import compare, oracle_run, say

pytestmark = pytest.mark.gpu

CASES = [
    ("tiny", 1.0, None),
    ("gqa_t32k", 1 / 32, None),
    ("ragged_b64", 1 / 32, None),
    ("mixed_tiers", 1 / 16, 4),
    ("ragged_b64", 1 / 4, 40),    # several rounds: doubling splits, compacted grid
]


def _rows(w):
    """Per sequence: its key rows in position order."""
    return [np.arange(W.token_keys(w, s).start, W.token_keys(w, s).stop) for s in range(w.B)]


def _setup(w, rng, upto):
    """Pools holding, per sequence s, the tokens at positions < upto[s]."""
    import torch
    from long_context_decode_ada_amd import ska
    dev = "cuda"
    pools = ska.DevicePools.for_workload(w, device=dev, poison=True)
    cache = ska.Cache(pools)
    rows = _rows(w)
    sel = np.concatenate([r[: int(upto[s])] for s, r in enumerate(rows)]).astype(np.int64)
    keys = torch.from_numpy(np.ascontiguousarray(w.keys[sel])).to(dev)
    vals = torch.from_numpy(np.ascontiguousarray(w.values[sel]).view(np.int16)).to(dev)
    slot = torch.from_numpy(np.ascontiguousarray(w.slot[sel])).to(dev)
    ska.encode_keys(cache, keys, vals, slot, radius_range=rng)
    torch.cuda.synchronize()
    return pools, cache, rows


def _step(w, cache, rows, lens, want_logits):
    """One append step: sequence s gains its token at position lens[s] - 1."""
    import torch
    from long_context_decode_ada_amd import ska
    dev = "cuda"
    nk = np.zeros((w.B, w.hkv, w.d), np.float32)
    nv = np.zeros((w.B, w.hkv, w.d), np.uint16)
    for s in range(w.B):
        if lens[s] > 0:
            nk[s] = w.keys[rows[s][lens[s] - 1]]
            nv[s] = w.values[rows[s][lens[s] - 1]]
    args = (torch.from_numpy(nk).to(dev), torch.from_numpy(nv.view(np.int16)).to(dev),
            torch.from_numpy(w.q).to(dev), torch.from_numpy(w.block_table).to(dev),
            torch.from_numpy(np.asarray(lens, np.int32)).to(dev))
    out = ska.append_decode_attention(cache, *args)
    lg = out_dbg = None
    if want_logits:
        # the same step again with the logits written: the append stores the
        # same token in the same slot, so the pools do not change
        lg = torch.full((w.B, w.hq, w.max_pages * W.PAGE), float("nan"), device=dev)
        out_dbg = ska.append_decode_attention(cache, *args, logits=lg).cpu().numpy()
        lg = lg.cpu().numpy()
    torch.cuda.synchronize()
    return {"out": out.cpu().numpy(), "out_dbg": out_dbg, "logits": lg}


@pytest.mark.parametrize("name,scale,batch", CASES)
def test_append_step_matches_full_encode_and_decode(name, scale, batch):
    from long_context_decode_ada_amd import ska
    w = W.make(name, scale, batch=batch)
    rng = O.calibrate(w.keys)
    lens = w.seq_lens.astype(np.int64)
    pools, cache, rows = _setup(w, rng, np.maximum(lens - 1, 0))
    say("[append %s] B=%d lengths %s..." % (name, w.B, lens[:6].tolist()))
    g = _step(w, cache, rows, lens, want_logits=True)
    assert ska.device_errors(cache) == 0
    o = oracle_run(w, rng)
    host = pools.to_host()
    for k in ("kcode", "rcode", "v"):
        assert np.array_equal(host[k], o["pools"][k]), k
    compare(w, g, o, rng, label="append " + name)


def test_append_steps_one_token_at_a_time():
    """Three steps in a row, each checked against the oracle at its length:
    sequence 0 starts empty, sequence 1 crosses from page 0 into page 1
    (lengths 15 -> 18), sequence 2 ends at its full length.  The pools after
    the three steps equal the oracle's encode of the same tokens."""
    from long_context_decode_ada_amd import ska
    w = W.make("gqa_t32k", 1 / 64, batch=3)
    lens_full = w.seq_lens.astype(np.int64)
    assert (lens_full >= 18).all()
    rng = O.calibrate(w.keys)
    start = np.array([0, 15, lens_full[2] - 3], np.int64)
    pools, cache, rows = _setup(w, rng, start)
    o_full = oracle_run(w, rng, want_logits=False)
    for k in range(1, 4):
        lens = start + k
        g = _step(w, cache, rows, lens, want_logits=False)
        assert ska.device_errors(cache) == 0
        o = oracle_run(w, rng, seq_lens=lens.astype(np.int32), want_logits=False, pools=o_full["pools"])
        err = float(np.abs(g["out"] - o["out"]).max())
        say("[append step %d] lengths %s max|out err| %.3g" % (k, lens.tolist(), err))
        assert err <= 2e-3
    sel = np.concatenate([r[: int(start[s]) + 3] for s, r in enumerate(rows)]).astype(np.int64)
    want = W.host_pools(w)
    O.encode(want, w.keys[sel], w.values[sel], w.slot[sel], w.radius_mode, rng)
    host = pools.to_host()
    for key in ("kcode", "rcode", "v"):
        assert np.array_equal(host[key], want[key]), key


def test_append_edges_empty_row_and_out_of_row():
    """seq_len 0 appends nothing and gives a zero row while the other rows
    append; a length past the block-table row sets the slot error and stores
    nothing.  (A new token at slot 0 of a fresh page: ragged_b64 above has
    such rows.)"""
    import torch
    from long_context_decode_ada_amd import ska
    w = W.make("ragged_b64", 1 / 32, batch=4)
    rng = O.calibrate(w.keys)
    lens = w.seq_lens.astype(np.int64).copy()
    pools, cache, rows = _setup(w, rng, np.maximum(lens - 1, 0))
    before = pools.to_host()
    # sequence 0: empty; the others as in the workload
    lens0 = lens.copy()
    lens0[0] = 0
    g = _step(w, cache, rows, lens0, want_logits=False)
    assert np.all(g["out"][0] == 0)
    assert ska.device_errors(cache) == 0
    o = oracle_run(w, rng, seq_lens=lens0.astype(np.int32), want_logits=False)
    assert float(np.abs(g["out"][1:] - o["out"][1:]).max()) <= 2e-3
    after = pools.to_host()
    r0 = rows[0]
    if len(r0):
        p0 = int(w.slot[r0[-1]])                       # sequence 0's last slot stays untouched
        phys, s = p0 // W.PAGE, p0 % W.PAGE
        for kv in range(w.hkv):
            i = (phys * w.hkv + kv) * W.PAGE + s
            assert after["rcode"][i] == before["rcode"][i]
    # a length one past the row: slot error, nothing stored
    over = lens.copy()
    over[:] = 0
    over[-1] = w.max_pages * W.PAGE + 1
    nk = torch.ones((w.B, w.hkv, w.d), device="cuda")
    nv = torch.zeros((w.B, w.hkv, w.d), dtype=torch.int16, device="cuda")
    snap = pools.to_host()
    ska.append_decode_attention(cache, nk, nv, torch.from_numpy(w.q).cuda(), torch.from_numpy(w.block_table).cuda(),
                                torch.from_numpy(over.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    assert ska.device_errors(cache) & ska.DEVERR_SLOT
    snap2 = pools.to_host()
    for k in ("kcode", "rcode", "v"):
        assert np.array_equal(snap[k], snap2[k]), k


def test_append_at_full_size_gqa_t32k():
    """The benchmark's configuration (8 x 32K tokens, automatic splits, the
    production kernel): every sequence's last token appended by the step;
    every pool byte and every output compared with the oracle."""
    import time
    from long_context_decode_ada_amd import ska
    t0 = time.time()
    w = W.make("gqa_t32k")
    rng = O.calibrate(w.keys)
    lens = w.seq_lens.astype(np.int64)
    say("[append full] generated (%.1fs)" % (time.time() - t0))
    pools, cache, rows = _setup(w, rng, lens - 1)
    g = _step(w, cache, rows, lens, want_logits=False)
    assert ska.device_errors(cache) == 0
    say("[append full] GPU done (%.1fs)" % (time.time() - t0))
    o = oracle_run(w, rng, want_logits=False)
    say("[append full] oracle done (%.1fs)" % (time.time() - t0))
    host = pools.to_host()
    for k in ("kcode", "rcode", "v"):
        nd = int(np.count_nonzero(host[k] != o["pools"][k]))
        say("[append full] %s mismatching bytes: %d" % (k, nd))
        assert nd == 0
    err = float(np.abs(g["out"] - o["out"]).max())
    say("[append full] max|out err| %.3g" % err)
    assert err <= 2e-3
