"""Pins of the oracle's rate-distortion retention (RDR) plan, the page's
section 2.2: per state a residency and a tier under a byte budget, protected
states at the widest tier, retained states in tier-homogeneous pages.

The plan is a Lagrangian relaxation of a multiple-choice knapsack.  Everett's
theorem pins it against brute force: a plan that minimises D + lambda * bytes
state by state is optimal among all plans that use no more bytes, so on tiny
inputs no enumerated plan may beat it.  Other pins: the budget is met, a
larger budget never raises the distortion, protection and infeasibility
behave as stated, zero-utility states go first, and the page packing is
tier-homogeneous, dense and in state order.
"""
import itertools
import os

import numpy as np

from oracle import oracle as O

TIERS = [2, 4, 6, 8]


def _eps_table():
    """eps(b) from tests/golden/rdr_eps_d128.txt (written by make_rdr_eps.py, oracle only)."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "rdr_eps_d128.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    return {int(b): float(e) for b, e in rows}


EPS = [_eps_table()[b] for b in TIERS]
D, HKV = 128, 8
BYTES = [HKV * (16 * (((D - 1) * b + 127) // 128) + 1 + 2 * D) for b in TIERS]


def _distortion(u, kn, tier, sigma, tiers=TIERS, eps=EPS):
    tot = 0.0
    for ui, ki, t in zip(u.astype(np.float64), kn.astype(np.float64), tier):
        if t == 0:
            tot += ui
        else:
            tot += ui * min(1.0, sigma * ki * eps[tiers.index(int(t))])
    return tot


def _bytes(tier, tiers=TIERS, bpt=BYTES):
    return sum(bpt[tiers.index(int(t))] for t in tier if t)


def _inputs(seed, n):
    rng = np.random.default_rng(seed)
    u = rng.exponential(1.0, n).astype(np.float32)
    kn = rng.uniform(4.0, 30.0, n).astype(np.float32)
    return u, kn


def test_eps_table_is_what_its_generator_writes():
    import importlib.util
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "make_rdr_eps.py")
    spec = importlib.util.spec_from_file_location("make_rdr_eps", path)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    fresh = m.eps_table()
    stored = _eps_table()
    for b, e in fresh.items():
        assert abs(stored[b] - e) <= 1e-6 * e
    # the angular error roughly halves per bit
    for b0, b1 in ((2, 3), (3, 4), (4, 6), (6, 8)):
        ratio = stored[b0] / stored[b1]
        assert 1.6 ** (b1 - b0) < ratio < 2.6 ** (b1 - b0)


def test_lagrangian_plan_beats_every_plan_with_no_more_bytes():
    tiers, eps = [2, 4, 8], [EPS[0], EPS[1], EPS[3]]
    bpt = [BYTES[0], BYTES[1], BYTES[3]]
    for seed in range(6):
        n = 7
        u, kn = _inputs(seed, n)
        prot = np.zeros(n, np.uint8)
        full = n * bpt[-1]
        for frac in (0.15, 0.35, 0.6, 0.85):
            r = O.rdr_plan(u, kn, prot, tiers, eps, bpt, int(frac * full), 0.03)
            d_plan = _distortion(u, kn, r["tier"], 0.03, tiers, eps)
            b_plan = _bytes(r["tier"], tiers, bpt)
            assert b_plan <= int(frac * full)
            for choice in itertools.product([0] + tiers, repeat=n):
                if _bytes(choice, tiers, bpt) <= b_plan:
                    assert _distortion(u, kn, choice, 0.03, tiers, eps) >= d_plan - 1e-9


def test_budget_is_met_and_more_budget_never_hurts():
    n = 3000
    u, kn = _inputs(11, n)
    prot = np.zeros(n, np.uint8)
    prot[:4] = 1
    prot[-128:] = 1
    full = n * BYTES[-1]
    last_d, last_b = None, None
    for frac in (0.15, 0.25, 0.4, 0.6, 0.8, 1.0):
        budget = int(frac * full)
        r = O.rdr_plan(u, kn, prot, TIERS, EPS, BYTES, budget, 0.05)
        assert r["status"] == 0
        b = _bytes(r["tier"])
        dist = _distortion(u, kn, r["tier"], 0.05)
        assert b <= budget
        if last_d is not None:
            assert dist <= last_d + 1e-9 and b >= last_b
        last_d, last_b = dist, b
    # with room for everything at the widest tier, nothing is evicted or narrowed
    r = O.rdr_plan(u, kn, prot, TIERS, EPS, BYTES, full, 0.05)
    assert (r["tier"] == 8).all() and r["lambda"] == 0.0


def test_protection_and_infeasible_budget():
    n = 200
    u, kn = _inputs(12, n)
    u[:10] = 0.0                                     # useless but protected
    prot = np.zeros(n, np.uint8)
    prot[:10] = 1
    r = O.rdr_plan(u, kn, prot, TIERS, EPS, BYTES, int(0.3 * n * BYTES[-1]), 0.05)
    assert (r["tier"][:10] == 8).all()
    # protected states alone over budget: they stay, everything else goes
    r = O.rdr_plan(u, kn, prot, TIERS, EPS, BYTES, 5 * BYTES[-1], 0.05)
    assert r["status"] == 2
    assert (r["tier"][:10] == 8).all() and (r["tier"][10:] == 0).all()


def test_zero_utility_states_are_evicted_first():
    n = 400
    u, kn = _inputs(13, n)
    u[::5] = 0.0
    prot = np.zeros(n, np.uint8)
    r = O.rdr_plan(u, kn, prot, TIERS, EPS, BYTES, int(0.7 * n * BYTES[-1]), 0.05)
    assert (r["tier"][::5] == 0).all()


def test_pages_are_tier_homogeneous_dense_and_in_state_order():
    n = 1234
    u, kn = _inputs(14, n)
    prot = np.zeros(n, np.uint8)
    prot[:4] = 1
    r = O.rdr_plan(u, kn, prot, TIERS, EPS, BYTES, int(0.45 * n * BYTES[-1]), 0.05)
    tier, page, slot, pt = r["tier"], r["page"], r["slot"], r["page_tier"]
    kept = tier > 0
    assert ((page >= 0) == kept).all() and ((slot >= 0) == kept).all()
    assert np.all(pt[page[kept]] & 15 == tier[kept])                # homogeneous (the header's tier bits)
    keys = page[kept].astype(np.int64) * 16 + slot[kept]
    assert len(np.unique(keys)) == kept.sum()                         # one state per slot
    expect_pages = sum((int((tier == t).sum()) + 15) // 16 for t in TIERS)
    assert len(pt) == expect_pages
    for t in TIERS:                                                   # index order, filled from slot 0
        idx = np.nonzero(tier == t)[0]
        pos = page[idx].astype(np.int64) * 16 + slot[idx]
        assert np.all(np.diff(pos) == 1)
        if len(idx):
            assert slot[idx[0]] == 0
