"""Oracle pins for pages that hold fewer than 16 tokens anywhere in a row.

The page header carries the tier in its low four bits and the number of
empty slots at the end of the page in its high four bits (0: a full page).
This lets the RDR controller's tier-homogeneous pages, one partial page per
tier (the page's section 2.2 groups retained states into pages of one
tier), be read as a single row under one softmax.  Pinned by:
  * brute-force dense attention over exactly the resident tokens, on keys
    and queries on the code lattice (where ADA is exact), with poison in
    every empty slot;
  * the log-sum-exp merge of per-tier rows in the full-page format (pinned
    elsewhere) against the single row over all pages;
  * the RDR plan's headers against its own tier, page and slot outputs.
"""
import math

import numpy as np
import pytest

from oracle import oracle as O
from tests.test_oracle_pipeline import PAGE, _bf16, _brute, _lattice_vector


def _packed_pools(page_hdr, hkv, d):
    """Host pools with a variable-size code block per page (page_off), every
    byte poisoned."""
    sizes = hkv * PAGE * np.array([O.kb(d, int(h) & 15) for h in page_hdr], np.uint64)
    off = np.zeros(len(page_hdr), np.uint64)
    off[1:] = np.cumsum(sizes)[:-1]
    n = len(page_hdr)
    return {"d": d, "hkv": hkv, "bstride": 8, "page_bits": np.asarray(page_hdr, np.uint8), "page_off": off,
            "kcode": np.full(int(sizes.sum()), 0xFF, np.uint8),
            "rcode": np.full(n * hkv * PAGE, 0xFF, np.uint8),
            "v": np.full(n * hkv * d * PAGE, 0x7FC0, np.uint16)}


@pytest.mark.parametrize("d,hq,hkv", [(64, 2, 1), (128, 8, 2)])
def test_partial_pages_equal_brute_force_over_resident_tokens(d, hq, hkv):
    rng = np.random.default_rng(7 * d + hq)
    B, npg = 3, [5, 1, 7]
    R = 10.0
    levels = np.array([j * R / 255 for j in range(256)])
    total = sum(npg)
    tiers = rng.choice([3, 4, 8], size=total)
    counts = rng.integers(1, 17, size=total)
    counts[rng.integers(0, total)] = 16
    hdr = (tiers | ((16 - counts) << 4)).astype(np.uint8)
    perm = rng.permutation(total)
    bt = np.zeros((B, max(npg)), np.int32)
    k = 0
    for s in range(B):
        bt[s, : npg[s]] = perm[k: k + npg[s]]
        k += npg[s]
    pools = _packed_pools(hdr, hkv, d)
    q = np.zeros((B, hq, d), np.float32)
    for s in range(B):
        for h in range(hq):
            q[s, h], _ = _lattice_vector(rng, d, 8, rng.uniform(0.5, 2.0))
    # one lattice key per resident slot, at its page's tier; the query is on
    # the 8-bit lattice, which contains every coarser tier's centres only for
    # the key side, so the queries are coded exactly (query mode exact)
    keys, vals, slots, by_seq_k, by_seq_v = [], [], [], [], []
    for s in range(B):
        ks, vs = [], []
        for p in range(npg[s]):
            phys = int(bt[s, p])
            b = int(tiers[phys])
            for t in range(int(counts[phys])):
                kk = np.zeros((hkv, d), np.float32)
                for g in range(hkv):
                    kk[g], _ = _lattice_vector(rng, d, b, levels[rng.integers(20, 256)])
                vv = _bf16(rng.standard_normal((hkv, d)).astype(np.float32))
                keys.append(kk)
                vals.append(vv)
                slots.append(phys * PAGE + t)
                ks.append(kk)
                vs.append(vv)
        by_seq_k.append(np.stack(ks))
        by_seq_v.append(np.stack(vs))
    rg = np.tile([0.0, R], (hkv, 1))
    O.encode(pools, np.stack(keys), np.stack(vals), np.array(slots, np.int64), O.UNIFORM, rg)
    lens = np.array([16 * n for n in npg], np.int32)      # every page walked; headers mask the slots
    out, lg = O.decode(pools, O.UNIFORM, rg, q, bt, lens, query_mode=O.Q_EXACT, want_logits=True)
    ref = _brute(q, by_seq_k, by_seq_v, hkv, 1.0 / math.sqrt(d))
    assert np.abs(out - ref).max() < 2e-6
    # logits exactly at the resident positions 16 p + slot
    for s in range(B):
        res = np.zeros(bt.shape[1] * PAGE, bool)
        for p in range(npg[s]):
            res[p * PAGE: p * PAGE + int(counts[bt[s, p]])] = True
        for h in range(hq):
            assert np.array_equal(~np.isnan(lg[s, h]), res)


def test_one_row_equals_the_merge_of_per_tier_rows():
    """A planned sequence read as one row (its tiers' pages, each tier's last
    page partial) equals the per-tier rows in the full-page format merged by
    their softmax masses: out = sum_r L_r out_r / sum_r L_r, L_r = sum over
    row r of exp(l_t - M)."""
    rng = np.random.default_rng(11)
    d, hq, hkv = 128, 8, 2
    per_tier = {2: 37, 4: 16, 6: 5, 8: 20}
    hdr, rows = [], {}
    for b, n in per_tier.items():
        np_t = (n + PAGE - 1) // PAGE
        rows[b] = list(range(len(hdr), len(hdr) + np_t))
        for p in range(np_t):
            empty = np_t * PAGE - n if p == np_t - 1 else 0
            hdr.append(b | (empty << 4))
    total = len(hdr)
    pools = _packed_pools(hdr, hkv, d)
    keys, vals, slots = [], [], []
    for b, n in per_tier.items():
        for i in range(n):
            phys = rows[b][i // PAGE]
            keys.append((rng.standard_normal((hkv, d)) * rng.lognormal(0, 0.5, (hkv, d))).astype(np.float32))
            vals.append(_bf16(rng.standard_normal((hkv, d)).astype(np.float32)))
            slots.append(phys * PAGE + i % PAGE)
    keys = np.stack(keys)
    rg = O.calibrate(keys)
    O.encode(pools, keys, np.stack(vals), np.array(slots, np.int64), O.LOG, rg)
    q = rng.standard_normal((1, hq, d)).astype(np.float32)
    one, lg1 = O.decode(pools, O.LOG, rg, q, np.arange(total, dtype=np.int32)[None], np.array([16 * total], np.int32),
                        want_logits=True)
    outs, masses = [], []
    for b, n in per_tier.items():
        bt = np.array([rows[b]], np.int32)
        o, lg = O.decode(pools, O.LOG, rg, q, bt, np.array([n], np.int32), want_logits=True)
        outs.append(o[0].astype(np.float64))
        masses.append(lg[0])
    M = np.nanmax(np.concatenate([m for m in masses], axis=1), axis=1)            # [hq]
    L = np.stack([np.nansum(np.exp(m - M[:, None]), axis=1) for m in masses])     # [rows][hq]
    merged = (L[:, :, None] * np.stack(outs)).sum(0) / L.sum(0)[:, None]
    assert np.abs(one[0] - merged).max() < 1e-6
    # the single row's logits are the per-tier rows' logits at their places
    for b, n in per_tier.items():
        for i in range(n):
            p = rows[b][i // PAGE]
            assert np.all(lg1[0, :, p * PAGE + i % PAGE] == masses[list(per_tier).index(b)][:, i])


def test_rdr_plan_page_headers():
    """The plan's page headers: each page's tier in the low bits, and the
    slots its states fill: full pages, except each tier's last page, whose
    empty slots the high bits count."""
    rng = np.random.default_rng(5)
    tiers, eps, byts = [2, 4, 6, 8], [0.27, 0.058, 0.0145, 0.0037], [8 * 289, 8 * 321, 8 * 353, 8 * 385]
    for n in (0, 1, 15, 16, 17, 300, 1000):
        u = rng.exponential(1.0, n).astype(np.float32)
        kn = rng.uniform(3, 40, n).astype(np.float32)
        prot = np.zeros(n, np.uint8)
        prot[:2] = 1
        r = O.rdr_plan(u, kn, prot, tiers, eps, byts, int(0.4 * n * byts[-1]), 0.04)
        hdr = r["page_tier"].astype(int)
        fill = np.zeros(len(hdr), int)
        for i in np.nonzero(r["tier"])[0]:
            p = r["page"][i]
            assert hdr[p] & 15 == r["tier"][i]
            assert r["slot"][i] == fill[p]            # states fill their page's slots in order
            fill[p] += 1
        assert np.array_equal(fill, 16 - (hdr >> 4))
        for b in tiers:
            pages = np.nonzero((hdr & 15) == b)[0]
            if len(pages):
                assert np.all(hdr[pages[:-1]] >> 4 == 0)
