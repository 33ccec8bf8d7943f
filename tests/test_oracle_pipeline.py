"""Whole-pipeline pins of the oracle: encode -> paged store -> ADA decode.

The decode is pinned against a plain numpy brute force of dense attention,
softmax(scale * q.K) V, on keys and queries placed exactly on the code
lattice (radius levels times decoded bin-centre directions).  On that lattice
the spherical code is lossless, so the logit estimator of the page's section
2.1 (|q| * r~ * f_b(c_q, c_k)) must equal the dense dot product, and the whole
pipeline (packing, page walk, block table, GQA grouping, softmax, value sum)
must equal the brute force.  Other tests pin invariances the paged layout of
sections 2.2-2.3 implies: physical placement, eviction as absence from the
block table, variable-size tier pages.
"""
import math

import numpy as np
import pytest

from oracle import oracle as O

PAGE = 16


def _bf16(x):
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _bf16_to_f64(h):
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _lattice_vector(rng, d, b, radius):
    """A vector exactly on the lattice: radius * u(centres(c)).  Polar codes
    stay in the middle half of [0, pi] so that no component underflows fp32."""
    c = np.empty(d - 1, np.int64)
    c[:-1] = rng.integers(1 << (b - 2), 3 << (b - 2), d - 2)
    c[-1] = rng.integers(0, 1 << b)
    return (radius * O.direction(c, d, b)).astype(np.float32), c


def _make_paged(rng, lens, hkv, d, num_pages=None, shuffle=True):
    B = len(lens)
    npg = [(n + PAGE - 1) // PAGE for n in lens]
    total = sum(npg)
    num_pages = num_pages or total + 3
    perm = rng.permutation(num_pages)[:total] if shuffle else np.arange(total)
    bt = np.zeros((B, max(npg)), np.int32)
    k = 0
    for s in range(B):
        bt[s, : npg[s]] = perm[k: k + npg[s]]
        k += npg[s]
    slots = []
    for s in range(B):
        t = np.arange(lens[s])
        slots.append(bt[s, t // PAGE].astype(np.int64) * PAGE + t % PAGE)
    return bt, np.concatenate(slots), num_pages


def _pools(num_pages, hkv, d, bits, page_off=None, kbytes=None):
    page_bits = np.full(num_pages, bits, np.uint8) if np.isscalar(bits) else bits
    bstride = int(page_bits.max())
    if kbytes is None:
        kbytes = num_pages * hkv * PAGE * O.kb(d, bstride)
    return {"d": d, "hkv": hkv, "bstride": bstride, "page_bits": page_bits, "page_off": page_off,
            "kcode": np.full(kbytes, 0xFF, np.uint8),
            "rcode": np.full(num_pages * hkv * PAGE, 0xFF, np.uint8),
            "v": np.full(num_pages * hkv * d * PAGE, 0x7FC0, np.uint16)}


def _brute(q, keys_by_seq, vals_by_seq, hkv, scale):
    """softmax(scale * q.K^T) V with K/V dense fp64; kv head = h // (hq/hkv)."""
    B, hq, d = q.shape
    g = hq // hkv
    out = np.zeros((B, hq, d))
    for s in range(B):
        K = keys_by_seq[s].astype(np.float64)
        V = _bf16_to_f64(vals_by_seq[s])
        for h in range(hq):
            kv = h // g
            lg = scale * (K[:, kv, :] @ q[s, h].astype(np.float64))
            w = np.exp(lg - lg.max())
            out[s, h] = (w[:, None] * V[:, kv, :]).sum(0) / w.sum()
    return out


@pytest.mark.parametrize("d,b,hq,hkv", [(64, 4, 1, 1), (128, 4, 4, 2), (128, 3, 8, 2), (128, 8, 2, 2)])
def test_lattice_pipeline_equals_dense_brute_force(d, b, hq, hkv):
    rng = np.random.default_rng(100 * d + 10 * b + hq)
    lens = [37, 50, 16]
    R = 12.0
    levels = np.array([j * R / 255 for j in range(256)])
    bt, slot, num_pages = _make_paged(rng, lens, hkv, d)
    n = len(slot)
    keys = np.zeros((n, hkv, d), np.float32)
    for i in range(n):
        for g in range(hkv):
            keys[i, g], _ = _lattice_vector(rng, d, b, levels[rng.integers(20, 256)])
    vals = _bf16(rng.standard_normal((n, hkv, d)).astype(np.float32))
    q = np.zeros((len(lens), hq, d), np.float32)
    for s in range(len(lens)):
        for h in range(hq):
            q[s, h], _ = _lattice_vector(rng, d, b, rng.uniform(0.5, 2.0))
    pools = _pools(num_pages, hkv, d, b)
    rg = np.tile([0.0, R], (hkv, 1))
    O.encode(pools, keys, vals, slot, O.UNIFORM, rg)
    # the lattice re-encodes to itself: stored radius levels are exact
    scale = 1.0 / math.sqrt(d)
    out, lg = O.decode(pools, O.UNIFORM, rg, q, bt, np.array(lens, np.int32), scale=0.0,
                       want_logits=True)
    starts = np.cumsum([0] + lens)
    ks = [keys[starts[s]: starts[s + 1]] for s in range(len(lens))]
    vs = [vals[starts[s]: starts[s + 1]] for s in range(len(lens))]
    ref = _brute(q, ks, vs, hkv, scale)
    assert np.abs(out - ref).max() < 2e-6
    # logits equal dense q.k (scaled) on the lattice
    for s in range(len(lens)):
        for h in range(hq):
            dense = scale * (ks[s][:, h // (hq // hkv), :].astype(np.float64) @ q[s, h].astype(np.float64))
            assert np.abs(lg[s, h, : lens[s]] - dense).max() < 1e-5 * max(1.0, np.abs(dense).max())


def test_gqa_grouping_is_consecutive():
    """Query head h reads kv head h // (hq/hkv): with kv heads whose values
    differ by a constant offset, the output reveals the head read."""
    rng = np.random.default_rng(9)
    d, b, hq, hkv = 64, 4, 8, 4
    lens = [40]
    bt, slot, num_pages = _make_paged(rng, lens, hkv, d)
    keys = rng.standard_normal((40, hkv, d)).astype(np.float32)
    base = rng.standard_normal((40, 1, d)).astype(np.float32) * 0.01
    vals = _bf16(base + np.arange(hkv, dtype=np.float32)[None, :, None] * 4.0)
    q = rng.standard_normal((1, hq, d)).astype(np.float32)
    pools = _pools(num_pages, hkv, d, b)
    rg = O.calibrate(keys)
    O.encode(pools, keys, vals, slot, O.LOG, rg)
    out = O.decode(pools, O.LOG, rg, q, bt, np.array(lens, np.int32))
    got = np.round(out[0].mean(axis=1) / 4.0).astype(int)
    assert list(got) == [h // (hq // hkv) for h in range(hq)]


def _encode_decode(rng_seed, lens, shuffle, num_pages_extra=0, page_bits=None, variable=False):
    rng = np.random.default_rng(rng_seed)
    d, hq, hkv = 128, 4, 2
    n = sum(lens)
    keys = (np.random.default_rng(77).standard_normal((n, hkv, d))).astype(np.float32)
    vals = _bf16(np.random.default_rng(78).standard_normal((n, hkv, d)).astype(np.float32))
    q = np.random.default_rng(79).standard_normal((len(lens), hq, d)).astype(np.float32)
    npg = sum((x + PAGE - 1) // PAGE for x in lens)
    bt, slot, num_pages = _make_paged(rng, lens, hkv, d, num_pages=npg + num_pages_extra, shuffle=shuffle)
    if page_bits is None:
        pb = np.full(num_pages, 4, np.uint8)
    else:  # tiers given per logical page, in sequence order
        pb = np.full(num_pages, 8, np.uint8)
        k = 0
        for s in range(len(lens)):
            for p in range((lens[s] + PAGE - 1) // PAGE):
                pb[bt[s, p]] = page_bits[k]
                k += 1
    if variable:
        sizes = np.array([hkv * PAGE * O.kb(d, int(x)) for x in pb], np.uint64)
        off = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.uint64)
        pools = _pools(num_pages, hkv, d, pb, page_off=off, kbytes=int(sizes.sum()))
    else:
        pools = _pools(num_pages, hkv, d, pb)
    rg = np.array([[0.5, 30.0]] * hkv)
    O.encode(pools, keys, vals, slot, O.LOG, rg)
    return O.decode(pools, O.LOG, rg, q, bt, np.array(lens, np.int32), want_logits=True), pools, bt


def test_physical_placement_does_not_change_the_result():
    (o1, l1), _, _ = _encode_decode(1, [70, 33], shuffle=False)
    (o2, l2), _, _ = _encode_decode(2, [70, 33], shuffle=True, num_pages_extra=11)
    assert np.array_equal(o1, o2)
    assert np.array_equal(l1, l2, equal_nan=True)


def test_variable_size_pages_equal_fixed_stride():
    tiers = [2, 4, 6, 8, 3, 4, 2, 8]
    (o1, l1), p1, _ = _encode_decode(3, [70, 33], shuffle=True, page_bits=tiers, variable=False)
    (o2, l2), p2, _ = _encode_decode(3, [70, 33], shuffle=True, page_bits=tiers, variable=True)
    assert np.array_equal(o1, o2)
    assert np.array_equal(l1, l2, equal_nan=True)
    assert len(p2["kcode"]) < len(p1["kcode"])


def test_mixed_tier_logits_equal_single_tier_logits():
    """A page at tier b gives the logits a cache holding every page at b
    would give for those tokens (the query is coded at the page's tier)."""
    tiers = [2, 4, 6, 8, 3, 4, 2, 8]
    (om, lm), _, _ = _encode_decode(4, [70, 33], shuffle=True, page_bits=tiers)
    lens = [70, 33]
    k = 0
    for s in range(2):
        for p in range((lens[s] + PAGE - 1) // PAGE):
            b = tiers[k]
            k += 1
            (_, lb), _, _ = _encode_decode(4, lens, shuffle=True, page_bits=[b] * 8)
            sl = slice(p * PAGE, min((p + 1) * PAGE, lens[s]))
            assert np.array_equal(lm[s, :, sl], lb[s, :, sl])


def test_eviction_is_attention_over_resident_pages():
    """Removing pages from the block table (compacted, seq_len = resident
    tokens) equals the plain softmax over the remaining tokens' logits."""
    (o_full, l_full), pools, bt = _encode_decode(5, [96], shuffle=True)
    keep = [0, 2, 3, 5]
    bt2 = bt[:, keep].copy()
    n2 = PAGE * len(keep)
    q = np.random.default_rng(79).standard_normal((1, 4, 128)).astype(np.float32)
    rg = np.array([[0.5, 30.0]] * 2)
    o2, l2 = O.decode(pools, O.LOG, rg, q, bt2, np.array([n2], np.int32), want_logits=True)
    idx = np.concatenate([np.arange(p * PAGE, (p + 1) * PAGE) for p in keep])
    assert np.array_equal(l2[0, :, :n2], l_full[0, :, idx].T)
    for h in range(4):
        lg = l_full[0, h, idx].astype(np.float64)
        w = np.exp(lg - lg.max())
        V = np.zeros((n2, 128))
        for j, t in enumerate(idx):
            phys, sl = bt[0, t // PAGE], t % PAGE
            base = ((phys * 2 + h // 2) * 128) * PAGE
            V[j] = _bf16_to_f64(pools["v"][base + np.arange(128) * PAGE + sl])
        ref = (w[:, None] * V).sum(0) / w.sum()
        assert np.abs(o2[0, h] - ref).max() < 1e-5


def test_empty_sequence_gives_zeros():
    (o, _), pools, bt = _encode_decode(6, [40, 20], shuffle=True)
    q = np.ones((2, 4, 128), np.float32)
    rg = np.array([[0.5, 30.0]] * 2)
    out = O.decode(pools, O.LOG, rg, q, bt, np.array([0, 20], np.int32))
    assert not out[0].any()
    assert np.isfinite(out[1]).all()


def test_query_exact_mode_uses_the_true_direction():
    """With the query uncoded, logits are |q| r~ <q/|q|, u_k> (scale 1)."""
    rng = np.random.default_rng(12)
    d, b = 64, 6
    R = 9.0
    k, ck = _lattice_vector(rng, d, b, R)
    keys = k[None, None, :]
    vals = _bf16(np.ones((1, 1, d), np.float32))
    bt = np.zeros((1, 1), np.int32)
    pools = _pools(1, 1, d, b)
    rg = np.array([[0.0, R]])
    O.encode(pools, keys, vals, np.array([0], np.int64), O.UNIFORM, rg)
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    _, lg = O.decode(pools, O.UNIFORM, rg, q, bt, np.array([1], np.int32), scale=1.0,
                     query_mode=O.Q_EXACT, want_logits=True)
    dense = float(q[0, 0].astype(np.float64) @ k.astype(np.float64))
    assert abs(lg[0, 0, 0] - dense) < 1e-5 * abs(dense) + 1e-5
