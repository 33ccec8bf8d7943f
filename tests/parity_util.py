"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and the CPU oracle on the same seeded workload, and compare them."""
import math
import sys

import numpy as np

from long_context_decode_ada_amd import workloads as W
from oracle import oracle as O

OUT_TOL = 2e-3          # max |out_gpu - out_ref|, fp32 outputs vs the fp64 oracle
LOGIT_TOL = 1e-3        # max |l_gpu - l_ref| / (scale * |q| * r~), the bound on |l|


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_run(w, num_splits=0, want_logits=True, poison=True, radius_range=None, query_mode=0,
            seq_lens=None, q=None, repeat=1):
    import torch
    from long_context_decode_ada_amd import ska
    dev = "cuda"
    pools = ska.DevicePools.for_workload(w, device=dev, poison=poison, query_mode=query_mode)
    cache = ska.Cache(pools)
    keys = torch.from_numpy(w.keys).to(dev)
    vals = torch.from_numpy(w.values.view(np.int16)).to(dev)
    slot = torch.from_numpy(w.slot).to(dev)
    ska.encode_keys(cache, keys, vals, slot, radius_range=radius_range)
    del keys, vals
    qh = w.q if q is None else q
    qd = torch.from_numpy(np.ascontiguousarray(qh)).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(np.asarray(w.seq_lens if seq_lens is None else seq_lens, np.int32)).to(dev)
    outs, lgs = [], []
    for _ in range(repeat):
        # production kernel (no logits written)
        out = ska.decode_attention(cache, qd, bt, sl, num_splits=num_splits)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    out_dbg = lg = None
    if want_logits:
        # debug kernel variant: also writes the logits
        lg = torch.full((qh.shape[0], qh.shape[1], w.max_pages * W.PAGE), float("nan"), device=dev)
        out_dbg = ska.decode_attention(cache, qd, bt, sl, num_splits=num_splits, logits=lg)
        torch.cuda.synchronize()
        out_dbg = out_dbg.cpu().numpy()
        lg = lg.cpu().numpy()
    res = {"out": outs[0], "out_dbg": out_dbg, "logits": lg, "outs": outs,
           "range": ska.radius_range(cache), "errors": ska.device_errors(cache),
           "pools": pools.to_host(), "cache": cache}
    return res


def oracle_run(w, rng, pairs=None, want_logits=True, query_mode=0, seq_lens=None, q=None, encode=True,
               pools=None):
    if pools is None:
        pools = W.host_pools(w)
        O.encode(pools, w.keys, w.values, w.slot, w.radius_mode, rng)
    qh = w.q if q is None else q
    sl = w.seq_lens if seq_lens is None else np.asarray(seq_lens, np.int32)
    r = O.decode(pools, w.radius_mode, rng, qh, w.block_table, sl, pairs=pairs,
                 want_logits=want_logits, query_mode=query_mode)
    out, lg = (r if want_logits else (r, None))
    return {"out": out, "logits": lg, "pools": pools}


def logit_bounds(w, rcode, rng, q=None, seq_lens=None):
    """scale * |q| * r~_t at every resident position (NaN elsewhere)."""
    qh = w.q if q is None else q
    sl = w.seq_lens if seq_lens is None else seq_lens
    B, hq, d = qh.shape
    g = hq // w.hkv
    scale = 1.0 / math.sqrt(d)
    lev = np.stack([O.radius_tables(w.radius_mode, rng[k, 0], rng[k, 1])[0] for k in range(w.hkv)])
    qn = np.linalg.norm(qh.astype(np.float64), axis=2)
    out = np.full((B, hq, w.max_pages * W.PAGE), np.nan)
    for s in range(B):
        n = int(sl[s])
        t = np.arange(n)
        phys = w.block_table[s, t // W.PAGE].astype(np.int64)
        for kv in range(w.hkv):
            r = lev[kv][rcode[(phys * w.hkv + kv) * W.PAGE + t % W.PAGE]]
            for h in range(kv * g, (kv + 1) * g):
                out[s, h, :n] = scale * qn[s, h] * r
    return out


def compare(w, g, o, rng, q=None, seq_lens=None, pairs=None, label=""):
    """Assert parity and return (max out err, max normalised logit err)."""
    def out_err(go):
        if pairs is None:
            return float(np.abs(go - o["out"]).max()) if go.size else 0.0
        return max(float(np.abs(go[s, h] - o["out"][s, h]).max()) for s, h in pairs)
    oe = out_err(g["out"])
    if g.get("out_dbg") is not None:
        oe = max(oe, out_err(g["out_dbg"]))
    le = 0.0
    if o["logits"] is not None and g["logits"] is not None:
        bnd = logit_bounds(w, o["pools"]["rcode"], rng, q=q, seq_lens=seq_lens)
        gl, ol = g["logits"], o["logits"]
        if pairs is not None:
            idx = tuple(np.array(pairs).T)
            gl, ol, bnd = gl[idx], ol[idx], bnd[idx]
        res = ~np.isnan(bnd)
        assert np.array_equal(res, ~np.isnan(gl)), "GPU wrote logits outside the resident positions"
        zero = res & (bnd == 0)
        assert np.all(gl[zero] == 0) and np.all(ol[zero] == 0)
        nz = res & (bnd > 0)
        if nz.any():
            le = float((np.abs(gl[nz] - ol[nz]) / bnd[nz]).max())
    say("%s max|out err| %.3g  max logit err/bound %.3g" % (label, oe, le))
    assert oe <= OUT_TOL, (label, oe)
    assert le <= LOGIT_TOL, (label, le)
    return oe, le
