"""Pins of the oracle's two baseline pieces: dense paged attention (what ADA
replaces, the page's section 1) and the decompress step of
decompress-then-dot (the dense keys r~ * u(codes) of section 2.1).

Dense attention is pinned by closed forms and invariances that a dropped
term, a wrong index or a transposed operand breaks: uniform weights give
the mean of the values, one resident token gives its value, basis-vector
keys give logits equal to scaled query components, placement and GQA
grouping behave as the block table says.  The decompress step is pinned by
the code lattice (where the stored code is lossless) and by |k~| equal to
the radius level.  Finally the two meet: ADA's exact-query logits equal the
dense logits over the decompressed keys, up to the keys' bf16 rounding.
"""
import math

import numpy as np

from oracle import oracle as O

PAGE = 16


def _bf16(x):
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _bf16_to_f64(h):
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _paged(rng, lens, hkv, d, extra=3):
    """Random placement of the sequences' pages in a pool; returns the block
    table, the slot of every token (sequence-major) and the pool size."""
    npg = [(n + PAGE - 1) // PAGE for n in lens]
    num_pages = sum(npg) + extra
    perm = rng.permutation(num_pages)
    bt = np.zeros((len(lens), max(npg)), np.int32)
    k = 0
    for s in range(len(lens)):
        bt[s, : npg[s]] = perm[k: k + npg[s]]
        k += npg[s]
    slots = np.concatenate([bt[s, np.arange(lens[s]) // PAGE].astype(np.int64) * PAGE + np.arange(lens[s]) % PAGE
                            for s in range(len(lens))])
    return bt, slots, num_pages


def _scatter(keys, vals, slots, num_pages, hkv, d):
    """Dense pools: K bf16 [num_pages][hkv][16][d] (token-major), V bf16
    [num_pages][hkv][d][16] (dimension-major), unused slots NaN."""
    kd = np.full((num_pages, hkv, PAGE, d), 0x7FC0, np.uint16)
    vd = np.full((num_pages, hkv, d, PAGE), 0x7FC0, np.uint16)
    phys, t = slots // PAGE, slots % PAGE
    kd[phys, :, t, :] = keys
    vd[phys, :, :, t] = vals
    return kd, vd


def _setup(seed, lens, hq, hkv, d, keyfn=None):
    rng = np.random.default_rng(seed)
    bt, slots, num_pages = _paged(rng, lens, hkv, d)
    n = len(slots)
    keys = rng.standard_normal((n, hkv, d)).astype(np.float32) if keyfn is None else keyfn(rng, n)
    kb = _bf16(keys)
    vb = _bf16(rng.standard_normal((n, hkv, d)).astype(np.float32))
    q = rng.standard_normal((len(lens), hq, d)).astype(np.float32)
    kd, vd = _scatter(kb, vb, slots, num_pages, hkv, d)
    return dict(rng=rng, bt=bt, slots=slots, kb=kb, vb=vb, q=q, kd=kd, vd=vd,
                lens=np.array(lens, np.int32), starts=np.cumsum([0] + list(lens)))


def test_identical_keys_and_zero_query_give_the_mean_of_values():
    hq, hkv, d = 4, 2, 64
    same = lambda rng, n: np.broadcast_to(rng.standard_normal((1, hkv, d)), (n, hkv, d)).astype(np.float32)
    c = _setup(1, [37, 16, 5], hq, hkv, d, keyfn=same)
    out = O.dense_decode(c["kd"], c["vd"], c["q"], c["bt"], c["lens"])
    q0 = np.zeros_like(c["q"])
    c2 = _setup(2, [37, 16, 5], hq, hkv, d)
    out0 = O.dense_decode(c2["kd"], c2["vd"], q0, c2["bt"], c2["lens"])
    for cc, o in ((c, out), (c2, out0)):
        for s in range(3):
            vs = _bf16_to_f64(cc["vb"][cc["starts"][s]: cc["starts"][s + 1]])
            for h in range(hq):
                assert np.abs(o[s, h] - vs[:, h // (hq // hkv)].mean(0)).max() < 1e-6


def test_one_resident_token_gives_its_value():
    hq, hkv, d = 2, 1, 32
    c = _setup(3, [1, 17], hq, hkv, d)
    out = O.dense_decode(c["kd"], c["vd"], c["q"], c["bt"], c["lens"])
    v0 = _bf16_to_f64(c["vb"][0, 0])
    assert np.array_equal(out[0, 0], v0.astype(np.float32)) and np.array_equal(out[0, 1], v0.astype(np.float32))


def test_basis_keys_give_scaled_query_components():
    """Key t of a sequence is the basis vector e_(t mod d): its logit is
    scale * q[t mod d], which pins the token-major key layout and the scale."""
    hq, hkv, d = 2, 2, 16
    basis = lambda rng, n: np.stack([np.eye(d, dtype=np.float32)[np.arange(n) % d]] * hkv, 1)
    c = _setup(4, [40, 21], hq, hkv, d, keyfn=basis)
    # basis keys restart per sequence
    n0 = 40
    kb = c["kb"].copy()
    kb[n0:] = _bf16(np.stack([np.eye(d, dtype=np.float32)[np.arange(21) % d]] * hkv, 1))
    kd, _ = _scatter(kb, c["vb"], c["slots"], c["kd"].shape[0], hkv, d)
    scale = 0.37
    _, lg = O.dense_decode(kd, c["vd"], c["q"], c["bt"], c["lens"], scale=scale, want_logits=True)
    for s, n in enumerate([40, 21]):
        for h in range(hq):
            want = scale * c["q"][s, h, np.arange(n) % d].astype(np.float64)
            assert np.abs(lg[s, h, :n] - want).max() < 1e-6


def test_placement_and_gqa_grouping():
    """Moving pages to other physical slots changes nothing; query head h
    reads KV head h // (hq/hkv): making KV head 1's keys identical makes heads
    2 and 3 (and only they) average their values."""
    hq, hkv, d = 4, 2, 32
    c = _setup(5, [33, 48], hq, hkv, d)
    out = O.dense_decode(c["kd"], c["vd"], c["q"], c["bt"], c["lens"])
    # re-place every page one slot further in a larger pool
    num_pages = c["kd"].shape[0]
    bt2 = (c["bt"] + 7) % (num_pages + 7)
    kd2 = np.full((num_pages + 7,) + c["kd"].shape[1:], 0x7FC0, np.uint16)
    vd2 = np.full((num_pages + 7,) + c["vd"].shape[1:], 0x7FC0, np.uint16)
    for s in range(2):
        for p in range((c["lens"][s] + PAGE - 1) // PAGE):
            kd2[bt2[s, p]] = c["kd"][c["bt"][s, p]]
            vd2[bt2[s, p]] = c["vd"][c["bt"][s, p]]
    out2 = O.dense_decode(kd2, vd2, c["q"], bt2, c["lens"])
    assert np.abs(out - out2).max() < 1e-6
    kb = c["kb"].copy()
    kb[:, 1] = kb[0, 1]
    kd3, _ = _scatter(kb, c["vb"], c["slots"], num_pages, hkv, d)
    out3 = O.dense_decode(kd3, c["vd"], c["q"], c["bt"], c["lens"])
    for s in range(2):
        vs = _bf16_to_f64(c["vb"][c["starts"][s]: c["starts"][s + 1]])
        assert np.abs(out3[s, 2] - vs[:, 1].mean(0)).max() < 1e-6
        assert np.abs(out3[s, 3] - vs[:, 1].mean(0)).max() < 1e-6
        assert np.array_equal(out3[s, :2], out[s, :2])


def _ada_pools(seed, lens, hkv, d, b, R=12.0):
    rng = np.random.default_rng(seed)
    bt, slots, num_pages = _paged(rng, lens, hkv, d)
    n = len(slots)
    keys = (rng.standard_normal((n, hkv, d)) * 1.5).astype(np.float32)
    vals = _bf16(rng.standard_normal((n, hkv, d)).astype(np.float32))
    pools = {"d": d, "hkv": hkv, "bstride": b, "page_bits": np.full(num_pages, b, np.uint8), "page_off": None,
             "kcode": np.zeros(num_pages * hkv * PAGE * O.kb(d, b), np.uint8),
             "rcode": np.zeros(num_pages * hkv * PAGE, np.uint8),
             "v": np.zeros(num_pages * hkv * d * PAGE, np.uint16)}
    rg = O.calibrate(keys)
    O.encode(pools, keys, vals, slots, O.LOG, rg)
    return rng, bt, slots, num_pages, keys, vals, pools, rg


def test_decompressed_keys_have_the_radius_level_as_norm_and_lattice_keys_return():
    d, hkv, b = 64, 2, 4
    rng, bt, slots, num_pages, keys, vals, pools, rg = _ada_pools(6, [40, 9], hkv, d, b)
    phys = np.unique(slots // PAGE).astype(np.int32)
    kt = O.decoded_keys(pools, O.LOG, rg, phys)
    levels = []
    for g in range(hkv):
        lv, _ = O.radius_tables(O.LOG, rg[g, 0], rg[g, 1])
        levels.append(lv)
    rc = pools["rcode"].reshape(num_pages, hkv, PAGE)
    for i, p in enumerate(phys):
        for g in range(hkv):
            norms = np.linalg.norm(kt[i, g], axis=1)
            assert np.abs(norms - levels[g][rc[p, g]]).max() < 1e-12 * max(1.0, levels[g].max())
    # keys placed on the lattice (uniform radius levels times bin-centre
    # directions) decompress to themselves
    R = 10.0
    lat_levels = np.array([j * R / 255 for j in range(256)])
    lat = np.zeros_like(keys)
    for i in range(lat.shape[0]):
        for g in range(hkv):
            c = np.empty(d - 1, np.int64)
            c[:-1] = rng.integers(1 << (b - 2), 3 << (b - 2), d - 2)
            c[-1] = rng.integers(0, 1 << b)
            lat[i, g] = (lat_levels[rng.integers(20, 256)] * O.direction(c, d, b)).astype(np.float32)
    rgu = np.tile([0.0, R], (hkv, 1))
    O.encode(pools, lat, vals, slots, O.UNIFORM, rgu)
    kt2 = O.decoded_keys(pools, O.UNIFORM, rgu, phys)
    for i, p in enumerate(phys):
        for sl in range(PAGE):
            hit = np.nonzero(slots == p * PAGE + sl)[0]
            if len(hit):
                assert np.abs(kt2[i, :, sl] - lat[hit[0]]).max() < 1e-5


def test_ada_exact_query_equals_dense_attention_over_decompressed_keys():
    """l = scale * |q| * r~ * <q/|q|, u> = scale * q . (r~ u): ADA's exact-query
    logits are dense logits over k~ = r~ u.  With k~ stored as bf16 the two
    differ by at most scale * |q| * r~ * 2^-8 (relative rounding 2^-9 of each
    component, Cauchy-Schwarz)."""
    d, hkv, hq, b = 128, 2, 4, 4
    lens = [45, 32]
    rng, bt, slots, num_pages, keys, vals, pools, rg = _ada_pools(7, lens, hkv, d, b)
    q = rng.standard_normal((len(lens), hq, d)).astype(np.float32)
    phys = np.arange(num_pages, dtype=np.int32)
    kt = O.decoded_keys(pools, O.LOG, rg, phys)                  # [num_pages][hkv][16][d]
    kd = _bf16(kt.astype(np.float32))
    vd = pools["v"].reshape(num_pages, hkv, d, PAGE)
    scale = 1.0 / math.sqrt(d)
    _, lg_dense = O.dense_decode(kd, vd, q, bt, np.array(lens, np.int32), scale=scale, want_logits=True)
    _, lg_ada = O.decode(pools, O.LOG, rg, q, bt, np.array(lens, np.int32), scale=scale,
                         query_mode=O.Q_EXACT, want_logits=True)
    rc = pools["rcode"].reshape(num_pages, hkv, PAGE)
    for s, n in enumerate(lens):
        for h in range(hq):
            g = h // (hq // hkv)
            t = np.arange(n)
            ph = bt[s, t // PAGE]
            r = np.array([O.radius_tables(O.LOG, rg[g, 0], rg[g, 1])[0][rc[p, g, x]] for p, x in zip(ph, t % PAGE)])
            bound = scale * np.linalg.norm(q[s, h].astype(np.float64)) * r
            err = np.abs(lg_dense[s, h, :n].astype(np.float64) - lg_ada[s, h, :n])
            assert (err <= bound * 2.0 ** -8 + 1e-6).all()
