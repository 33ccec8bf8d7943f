"""Pins of the oracle's per-(page, KV head) tiers (the page's section 2.2
allocates a tier per token, head and layer; here one header per page and KV
head).  Two reductions to the pinned per-page format: a head-tier pool whose
heads all carry their page's tier, with each head's records at the offset the
per-page layout gives them, holds the same bytes and decodes to the same
outputs; and in a pool of mixed per-head tiers, KV head g decodes (and
decompresses) exactly as a per-page pool whose pages all carry head g's
tiers."""
import numpy as np

from long_context_decode_ada_amd import workloads as W
from oracle import oracle as O

PAGE = W.PAGE


def _per_page_pools(w, bits):
    """Host pools of per-page format for w's pages with page tiers `bits`."""
    sizes = w.hkv * PAGE * np.array([O.kb(w.d, int(b)) for b in bits], np.uint64)
    off = np.zeros(w.num_pages, np.uint64)
    off[1:] = np.cumsum(sizes)[:-1]
    return {"d": w.d, "hkv": w.hkv, "bstride": 8, "page_bits": np.ascontiguousarray(bits, np.uint8),
            "page_off": off, "kcode": np.full(int(sizes.sum()), 0xFF, np.uint8),
            "rcode": np.full(w.num_pages * w.hkv * PAGE, 0xFF, np.uint8),
            "v": np.full(w.num_pages * w.hkv * w.d * PAGE, 0x7FC0, np.uint16)}


def test_uniform_head_tiers_equal_the_per_page_format():
    w = W.make("mixed_tiers", 1 / 64, batch=2)
    rng = O.calibrate(w.keys)
    pp = W.host_pools(w)
    O.encode(pp, w.keys, w.values, w.slot, w.radius_mode, rng)
    # the same tiers, per head, with each head's records where the per-page
    # layout puts them
    hb = np.repeat(w.page_bits, w.hkv)
    kb = np.array([O.kb(w.d, int(b)) for b in w.page_bits], np.uint64)
    hoff = (w.page_off[:, None] + np.arange(w.hkv, dtype=np.uint64)[None, :] * PAGE * kb[:, None]).reshape(-1)
    hp = dict(pp, page_bits=hb, page_off=hoff, head_tiers=True,
              kcode=np.full_like(pp["kcode"], 0xFF), rcode=np.full_like(pp["rcode"], 0xFF),
              v=np.full_like(pp["v"], 0x7FC0))
    O.encode(hp, w.keys, w.values, w.slot, w.radius_mode, rng)
    for k in ("kcode", "rcode", "v"):
        assert np.array_equal(hp[k], pp[k]), k
    a = O.decode(pp, w.radius_mode, rng, w.q, w.block_table, w.seq_lens)
    b = O.decode(hp, w.radius_mode, rng, w.q, w.block_table, w.seq_lens)
    assert np.array_equal(a, b)


def test_each_head_decodes_as_a_per_page_pool_of_its_tiers():
    w = W.make("mixed_tiers", 1 / 64, batch=2, head_tiers=True)
    hb = w.page_bits.reshape(w.num_pages, w.hkv)
    assert len({tuple(r) for r in hb}) > 1 and any(len(set(r)) > 1 for r in hb)   # tiers really differ per head
    rng = O.calibrate(w.keys)
    hp = W.host_pools(w)
    O.encode(hp, w.keys, w.values, w.slot, w.radius_mode, rng)
    out, lg = O.decode(hp, w.radius_mode, rng, w.q, w.block_table, w.seq_lens, want_logits=True)
    g_sz = w.hq // w.hkv
    used = np.unique(w.slot // PAGE).astype(np.int32)
    dk = O.decoded_keys(hp, w.radius_mode, rng, used)
    for g in range(w.hkv):
        pp = _per_page_pools(w, hb[:, g])
        O.encode(pp, w.keys, w.values, w.slot, w.radius_mode, rng)
        pairs = [(s, h) for s in range(w.B) for h in range(g * g_sz, (g + 1) * g_sz)]
        o2, l2 = O.decode(pp, w.radius_mode, rng, w.q, w.block_table, w.seq_lens, pairs=pairs, want_logits=True)
        for s, h in pairs:
            assert np.array_equal(out[s, h], o2[s, h]), (g, s, h)
            n = int(w.seq_lens[s])
            assert np.array_equal(lg[s, h, :n], l2[s, h, :n]), (g, s, h)
        assert np.array_equal(dk[:, g], O.decoded_keys(pp, w.radius_mode, rng, used)[:, g]), g
        # head g's radius bytes and values sit where the per-page layout has them
        r1 = hp["rcode"].reshape(w.num_pages, w.hkv, PAGE)[:, g]
        r2 = pp["rcode"].reshape(w.num_pages, w.hkv, PAGE)[:, g]
        assert np.array_equal(r1, r2)


def test_head_tiers_need_offsets():
    w = W.make("mixed_tiers", 1 / 64, batch=1, head_tiers=True)
    hp = W.host_pools(w)
    hp["page_off"] = None
    try:
        O.encode(hp, w.keys, w.values, w.slot, w.radius_mode, O.calibrate(w.keys))
    except ValueError:
        return
    raise AssertionError("head tiers without offsets accepted")
