"""Synthetic workload generator: determinism and structure (CPU only)."""
import numpy as np
import pytest

from long_context_decode_ada_amd import workloads as W
from oracle import oracle as O


@pytest.mark.parametrize("name,scale", [("tiny", 1.0), ("gqa_t32k", 1 / 256), ("long_t128k", 1 / 1024),
                                        ("ragged_b64", 1 / 64), ("mixed_tiers", 1 / 128)])
def test_same_seed_same_bytes(name, scale):
    a = W.make(name, scale)
    b = W.make(name, scale)
    for f in ("keys", "values", "q", "slot", "block_table", "seq_lens", "page_bits"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    # every resident slot is distinct and inside the pool
    assert len(np.unique(a.slot)) == len(a.slot)
    assert a.slot.max() < a.num_pages * W.PAGE
    assert a.keys.shape == (a.n_tokens, a.hkv, a.d)
    c = W.make(name, scale, data=False)
    for f in ("slot", "block_table", "seq_lens", "page_bits"):
        assert np.array_equal(getattr(a, f), getattr(c, f)), f


def test_ragged_lengths_follow_the_recipe():
    w = W.make("ragged_b64", data=False)
    assert w.B == 64 and w.seq_lens.min() >= 512 and w.seq_lens.max() <= 65536
    npg = ((w.seq_lens + 15) // 16).sum()
    assert w.num_pages == int(np.ceil(1.25 * npg))
    used = np.concatenate([w.block_table[s, : (w.seq_lens[s] + 15) // 16] for s in range(w.B)])
    assert len(np.unique(used)) == len(used)


def test_mixed_tiers_structure():
    w = W.make("mixed_tiers", scale=1 / 16)   # T = 2048: 128 logical pages per sequence
    npg_logical = 2048 // 16
    resident_pages = (w.seq_lens + 15) // 16
    assert np.all(resident_pages == npg_logical - (npg_logical - 1) // 2)
    for s in range(w.B):
        assert w.page_bits[w.block_table[s, 0]] == 8         # sink page at b_max
    assert set(np.unique(w.page_bits)) <= {2, 4, 6, 8}
    sizes = [w.hkv * 16 * W.record_bytes(w.d, int(b)) for b in w.page_bits]
    assert np.array_equal(w.page_off[1:], np.cumsum(sizes)[:-1])


def test_full_size_shapes_are_the_stated_ones():
    # sizes only (no key generation): the headline workload
    w = W.make("tiny")
    assert (w.B, w.hq, w.hkv, w.d, int(w.seq_lens[0])) == (1, 1, 1, 64, 256)
    assert w.num_pages == 16 and np.array_equal(w.block_table[0], np.arange(16))


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.1415927], np.float32)
    h = W._bf16_bits(x)
    back = (h.astype(np.uint32) << 16).view(np.float32)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.015625 and back[3] == -2.5
    assert abs(back[4] - 3.140625) < 1e-7


def test_small_workloads_run_through_the_oracle():
    for name, scale in (("tiny", 1.0), ("mixed_tiers", 1 / 256)):
        w = W.make(name, scale, batch=2)
        pools = W.host_pools(w)
        rg = O.calibrate(w.keys)
        O.encode(pools, w.keys, w.values, w.slot, w.radius_mode, rg)
        out = O.decode(pools, w.radius_mode, rg, w.q, w.block_table, w.seq_lens)
        assert np.isfinite(out).all()


def test_head_tier_layout_is_packed_per_page_and_head():
    w = W.make("mixed_tiers", 1 / 64, batch=2, head_tiers=True)
    assert w.page_bits.shape == (w.num_pages * w.hkv,) and w.page_off.shape == (w.num_pages * w.hkv,)
    sizes = W.PAGE * np.array([W.record_bytes(w.d, int(b)) for b in w.page_bits], np.uint64)
    assert w.page_off[0] == 0 and np.array_equal(np.diff(w.page_off), sizes[:-1])
    assert w.kcode_bytes == int(sizes.sum())
    hb = w.page_bits.reshape(w.num_pages, w.hkv)
    assert set(np.unique(hb)) <= {2, 4, 6, 8}
    for s in range(w.B):                      # the sink page: every head at the widest tier
        assert (hb[w.block_table[s, 0]] == 8).all()
    w0 = W.make("mixed_tiers", 1 / 64, batch=2)
    assert np.array_equal(w0.seq_lens, w.seq_lens) and np.array_equal(w0.block_table, w.block_table)


def test_outlier_channels():
    """Keys with a few outlier channels: seeded, and the chosen channels
    carry norms far above the rest."""
    a = W.make("gqa_t32k", 1 / 256, outliers=4)
    b = W.make("gqa_t32k", 1 / 256, outliers=4)
    assert np.array_equal(a.keys, b.keys)
    plain = W.make("gqa_t32k", 1 / 256)
    assert np.array_equal(a.values, plain.values) and np.array_equal(a.q, plain.q)
    ra = np.linalg.norm(a.keys.astype(np.float64), axis=2)
    rp = np.linalg.norm(plain.keys.astype(np.float64), axis=2)
    assert ra.mean() > 3 * rp.mean()          # the outlier channels dominate the norms
    assert ra.max() / ra.min() > rp.max() / rp.min()
    with pytest.raises(ValueError):
        W.make("tiny", outliers=2)


def test_rdr_parameters_match_the_measured_table():
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "rdr_eps_d128.txt")
    rows = {int(a): float(b) for a, b in (ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#"))}
    assert W.RDR_EPS == tuple(rows[b] for b in W.RDR_TIERS)


def oracle_plans(inp):
    B, T = inp.utility.shape
    tier = np.zeros((B, T), np.uint8)
    page = np.full((B, T), -1, np.int32)
    slot = np.full((B, T), -1, np.int32)
    hdr, npg = [], []
    for s in range(B):
        n = int(inp.num_states[s])
        r = O.rdr_plan(inp.utility[s, :n], inp.key_norm[s, :n], inp.protect[s, :n], inp.tiers, inp.eps,
                       inp.bytes_per_tier, int(inp.budget[s]), inp.sigma)
        tier[s, :n], page[s, :n], slot[s, :n] = r["tier"], r["page"], r["slot"]
        hdr.append(r["page_tier"])
        npg.append(len(r["page_tier"]))
    return tier, page, slot, hdr, np.array(npg)


def test_rdr_planned_workload_layout():
    """The planned workload holds exactly the retained tokens, each at its
    planned slot of a physical page whose header carries the plan's tier and
    count; rows end at their last page's last token."""
    inp = W.rdr_inputs(1 / 64)
    tier, page, slot, hdr, npg = oracle_plans(inp)
    w = W.planned_workload(inp, tier, page, slot, hdr, npg)
    kept = int((tier > 0).sum())
    assert w.keys.shape[0] == kept == len(w.slot) == w.n_tokens
    assert len(np.unique(w.slot)) == kept
    assert 0.3 < kept / tier.size < 0.7                   # about half evicted
    assert w.num_pages == int(npg.sum())
    for s in range(w.B):
        n = int(inp.num_states[s])
        rows = W.token_keys(inp.base, s)
        idx = np.nonzero(tier[s, :n])[0]
        start = int((tier[:s] > 0).sum())
        assert np.array_equal(w.keys[start: start + len(idx)], inp.base.keys[rows][idx])
        for j, i in enumerate(idx[:50]):
            phys = int(w.slot[start + j]) // 16
            assert phys == w.block_table[s, page[s, i]] and int(w.slot[start + j]) % 16 == slot[s, i]
            assert w.page_bits[phys] & 15 == tier[s, i]
            assert slot[s, i] < 16 - (w.page_bits[phys] >> 4)
        last = int(w.block_table[s, npg[s] - 1])
        assert w.seq_lens[s] == 16 * (npg[s] - 1) + 16 - (w.page_bits[last] >> 4)
    # the sinks are kept at the widest tier
    assert np.all(tier[:, : W.RDR_SINKS] == max(W.RDR_TIERS))
