"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and the CPU oracle on the same seeded workload, and compare them."""
import math
import sys

import numpy as np

from long_context_decode_ada_amd import workloads as W
from oracle import oracle as O

OUT_TOL = 2e-3          # max |out_gpu - out_ref|, fp32 outputs vs the fp64 oracle
LOGIT_TOL = 1e-3        # max |l_gpu - l_ref| / (scale * |q| * r~), the bound on |l|
# The logits come from the debug variant of the kernel that produces `out`
# (the same template with the logit store added), so its output must equal
# the production output: same codes, same arithmetic, same merge.
DBG_TOL = 1e-6

# (test id, label, max out err, max logit err / bound, max |out - out_dbg|),
# written out at the end of the session (conftest.py)
MARGINS = []
CURRENT_TEST = [""]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_run(w, num_splits=0, want_logits=True, poison=True, radius_range=None, query_mode=0,
            seq_lens=None, q=None, repeat=1, query_precision=0, max_splits=64):
    import torch
    from long_context_decode_ada_amd import ska
    dev = "cuda"
    pools = ska.DevicePools.for_workload(w, device=dev, poison=poison, query_mode=query_mode,
                                         query_precision=query_precision, max_splits=max(max_splits, num_splits))
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
            # resident: the slot below the page's count (header's high four bits: empty slots)
            hdr = w.page_bits[phys * w.hkv + kv] if w.head_tiers else w.page_bits[phys]
            res = (t % W.PAGE) < (W.PAGE - (hdr.astype(np.int64) >> 4))
            r = lev[kv][rcode[(phys * w.hkv + kv) * W.PAGE + t % W.PAGE]]
            for h in range(kv * g, (kv + 1) * g):
                out[s, h, t[res]] = scale * qn[s, h] * r[res]
    return out


def compare(w, g, o, rng, q=None, seq_lens=None, pairs=None, label="", out_tol=OUT_TOL):
    """Assert parity and return (max out err, max normalised logit err).
    out_tol None checks the logits (and the production/logits variants'
    agreement) only, recording the output error."""
    def out_err(go):
        if pairs is None:
            return float(np.abs(go - o["out"]).max()) if go.size else 0.0
        return max(float(np.abs(go[s, h] - o["out"][s, h]).max()) for s, h in pairs)
    oe = out_err(g["out"])
    de = None
    if g.get("out_dbg") is not None:
        oe = max(oe, out_err(g["out_dbg"]))
        if pairs is None:
            de = float(np.abs(g["out"] - g["out_dbg"]).max()) if g["out"].size else 0.0
        else:
            de = max(float(np.abs(g["out"][s, h] - g["out_dbg"][s, h]).max()) for s, h in pairs)
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
    say("%s max|out err| %.3g  max logit err/bound %.3g  max|out - out_dbg| %s" %
        (label, oe, le, "-" if de is None else "%.3g" % de))
    MARGINS.append((CURRENT_TEST[0], label + ("" if out_tol is not None else " (output recorded, not asserted)"),
                    oe, le if g["logits"] is not None else None, de))
    if out_tol is not None:
        assert oe <= out_tol, (label, oe)
    assert le <= LOGIT_TOL, (label, le)
    if de is not None:
        assert de <= DBG_TOL, (label, "production and logits variants differ", de)
    return oe, le


def write_margins(path):
    """The recorded parity margins as a Markdown table (fractions of the
    tolerances in the last two columns)."""
    if not MARGINS:
        return
    import os
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write("# Parity margins (GPU path vs the CPU oracle)\n\n")
        f.write("Written by the GPU test run (`python -u -m pytest tests -m gpu -x -v --timeout 120 --timeout-method "
                "thread` on one MI355X; tests/conftest.py writes every check that tests/parity_util.py recorded).\n\n")
        f.write("Tolerances: output %.0e absolute, logit %.0e of the bound scale*|q|*r~; the production\n"
                "kernel's output must equal its logits variant's within %.0e.\n\n" % (OUT_TOL, LOGIT_TOL, DBG_TOL))
        f.write("| test | case | max out err | max logit err / bound | max out - out_dbg | out / tol | logit / tol |\n")
        f.write("|---|---|---|---|---|---|---|\n")
        for t, lab, oe, le, de in MARGINS:
            f.write("| %s | %s | %.3g | %s | %s | %.2f | %s |\n" % (
                t, lab, oe, "-" if le is None else "%.3g" % le, "-" if de is None else "%.3g" % de,
                oe / OUT_TOL, "-" if le is None else "%.2f" % (le / LOGIT_TOL)))


def planned_workloads(inp):
    """The RDR controller on the GPU (ska_rdr_plan) and in the oracle on the
    same inputs: the plans must agree bit for bit; each side's plan is laid
    out on its own (workloads.planned_workload) and the layouts must agree.
    Returns (workload from the GPU plan, workload from the oracle's plan)."""
    import torch
    from long_context_decode_ada_amd import ska
    dev = "cuda"
    B, T = inp.utility.shape
    g = ska.rdr_plan(torch.from_numpy(inp.utility).to(dev), torch.from_numpy(inp.key_norm).to(dev),
                     torch.from_numpy(inp.protect).to(dev), torch.from_numpy(inp.num_states).to(dev),
                     torch.from_numpy(inp.budget).to(dev), inp.tiers, inp.eps, inp.bytes_per_tier, inp.sigma)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in g.items()}
    o_tier = np.zeros((B, T), np.uint8)
    o_page = np.full((B, T), -1, np.int32)
    o_slot = np.full((B, T), -1, np.int32)
    o_hdr, o_np = [], []
    for s in range(B):
        n = int(inp.num_states[s])
        r = O.rdr_plan(inp.utility[s, :n], inp.key_norm[s, :n], inp.protect[s, :n], inp.tiers, inp.eps,
                       inp.bytes_per_tier, int(inp.budget[s]), inp.sigma)
        o_tier[s, :n], o_page[s, :n], o_slot[s, :n] = r["tier"], r["page"], r["slot"]
        o_hdr.append(r["page_tier"])
        o_np.append(len(r["page_tier"]))
        assert g["status"][s] == r["status"] and g["lambda"][s] == r["lambda"], s
        assert g["npages"][s] == len(r["page_tier"]), s
        assert np.array_equal(g["page_tier"][s, : len(r["page_tier"])], r["page_tier"]), s
        for k, v in (("tier", r["tier"]), ("page", r["page"]), ("slot", r["slot"])):
            assert np.array_equal(g[k][s, :n], v), (s, k)
    g_hdr = [g["page_tier"][s, : int(g["npages"][s])] for s in range(B)]
    wg = W.planned_workload(inp, g["tier"], g["page"], g["slot"], g_hdr, g["npages"])
    wo = W.planned_workload(inp, o_tier, o_page, o_slot, o_hdr, np.array(o_np))
    for f in ("seq_lens", "block_table", "page_bits", "page_off", "slot", "keys", "values", "q"):
        assert np.array_equal(getattr(wg, f), getattr(wo, f)), f
    return wg, wo
