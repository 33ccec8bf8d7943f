"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs, at sizes the oracle finishes in seconds.

Bars: encoded pools (angle-code records, radius codes, scattered values)
bit-exact, including bytes that must stay untouched; radius range bit-exact;
logits within 1e-3 of their bound scale*|q|*r~; outputs within 2e-3."""
import numpy as np
import pytest

from long_context_decode_ada_amd import workloads as W
from oracle import oracle as O
from tests.parity_util import compare, gpu_run, oracle_run, say

pytestmark = pytest.mark.gpu

SMALL = [
    ("tiny", 1.0, None),
    ("gqa_t32k", 1 / 32, None),       # T = 1024, B = 8, 32/8 heads, b = 4
    ("long_t128k", 1 / 128, None),    # T = 1024, B = 1, b = 3
    ("ragged_b64", 1 / 32, None),     # lengths 16..2048
    ("mixed_tiers", 1 / 16, 4),       # 65 resident pages of mixed tiers per sequence
]


@pytest.fixture(scope="module")
def runs():
    cache = {}

    def get(name, scale, batch):
        key = (name, scale, batch)
        if key not in cache:
            say("[gpu parity] workload", key)
            w = W.make(name, scale, batch=batch)
            g = gpu_run(w)
            rng = O.calibrate(w.keys)
            o = oracle_run(w, rng)
            cache[key] = (w, g, o, rng)
        return cache[key]
    return get


@pytest.mark.parametrize("name,scale,batch", SMALL)
def test_encode_is_bit_exact(runs, name, scale, batch):
    w, g, o, rng = runs(name, scale, batch)
    assert np.array_equal(g["range"], rng), (g["range"], rng)
    for k in ("kcode", "rcode", "v"):
        a, b = g["pools"][k], o["pools"][k]
        nd = int(np.count_nonzero(a != b))
        say("[%s] %s mismatching bytes: %d of %d" % (name, k, nd, a.size))
        assert nd == 0
    assert g["errors"] == 0


@pytest.mark.parametrize("name,scale,batch", SMALL)
def test_decode_matches_oracle(runs, name, scale, batch):
    w, g, o, rng = runs(name, scale, batch)
    compare(w, g, o, rng, label=name)


def test_split_count_and_determinism():
    w = W.make("gqa_t32k", 1 / 32, batch=3)
    rng = O.calibrate(w.keys)
    o = oracle_run(w, rng)
    base = None
    for ns in (1, 3, 16, 64):
        g = gpu_run(w, num_splits=ns, repeat=2)
        assert np.array_equal(g["outs"][0], g["outs"][1]), "run-to-run difference at %d splits" % ns
        compare(w, g, o, rng, label="splits=%d" % ns)
        if base is None:
            base = g
        else:
            assert np.array_equal(g["logits"], base["logits"], equal_nan=True)
            assert np.array_equal(g["out"], g["out_dbg"]) or np.abs(g["out"] - g["out_dbg"]).max() < 1e-6
            # P enters P.V as hi + lo bf16 (16 significant bits, relative
            # error <= 2^-16), and a different split count rescales P against
            # different running maxima, so outputs may move by up to about
            # 2^-16 * max|v| (|v| <= ~5 here) between split counts
            assert np.abs(g["out"] - base["out"]).max() < 1e-4


@pytest.mark.parametrize("name,scale,counts,qprec", [
    # 128 pages per row: explicit counts giving 4, 5, 8, 9, 16, 19, 32 and 43
    # non-empty splits, on both sides of each size of the one-round merge
    # (4, 8, 16, 32 loads per thread) and past it (the LDS weight pass)
    ("gqa_t32k", 1 / 16, (4, 5, 8, 9, 16, 19, 32, 43), 0),
    ("mixed_tiers", 1 / 8, (4, 5, 8, 9, 16, 19, 32, 43), 0),
    # the mixed-tier kernel with binary32 directions (query_precision 1) merges
    # up to 8 splits in one round
    ("mixed_tiers", 1 / 8, (5, 8, 9, 12), 1),
])
def test_merge_paths_at_their_split_count_boundaries(name, scale, counts, qprec):
    w = W.make(name, scale, batch=2)
    rng = O.calibrate(w.keys)
    o = oracle_run(w, rng)
    base = None
    for ns in counts:
        g = gpu_run(w, num_splits=ns, repeat=2, query_precision=qprec)
        assert np.array_equal(g["outs"][0], g["outs"][1]), "run-to-run difference at %d splits" % ns
        compare(w, g, o, rng, label="%s splits=%d" % (name, ns))
        if base is None:
            base = g
        else:
            assert np.array_equal(g["logits"], base["logits"], equal_nan=True)
            assert np.abs(g["out"] - base["out"]).max() < 1e-4


def test_ragged_edges_zero_one_and_page_boundaries():
    w = W.make("gqa_t32k", 1 / 32, batch=8)          # 1024 tokens encoded per sequence
    lens = np.array([0, 1, 15, 16, 17, 31, 33, 1024], np.int32)
    rng = O.calibrate(w.keys)
    g = gpu_run(w, seq_lens=lens)
    o = oracle_run(w, rng, seq_lens=lens)
    assert not g["out"][0].any()
    compare(w, g, o, rng, seq_lens=lens, label="edge lengths")


@pytest.mark.parametrize("hq", [8, 16])
def test_group_sizes_one_and_two(hq):
    w = W.make("gqa_t32k", 1 / 64, batch=2)
    q = np.ascontiguousarray(w.q[:, :hq])
    rng = O.calibrate(w.keys)
    g = gpu_run(w, q=q)
    o = oracle_run(w, rng, q=q)
    compare(w, g, o, rng, q=q, label="G=%d" % (hq // 8))


def test_query_exact_variant():
    w = W.make("mixed_tiers", 1 / 32, batch=2)
    rng = O.calibrate(w.keys)
    g = gpu_run(w, query_mode=1)
    o = oracle_run(w, rng, query_mode=1)
    compare(w, g, o, rng, label="exact query")


def test_given_radius_range_and_uniform_d128():
    w = W.make("gqa_t32k", 1 / 64, batch=2)
    w.radius_mode = W.UNIFORM
    rng = np.tile([0.0, 25.0], (w.hkv, 1))           # some keys exceed R_hi: code 255
    g = gpu_run(w, radius_range=rng)
    assert np.array_equal(g["range"], rng)
    o = oracle_run(w, rng)
    for k in ("kcode", "rcode", "v"):
        assert np.array_equal(g["pools"][k], o["pools"][k]), k
    compare(w, g, o, rng, label="uniform radius, given range")


def test_no_poison_read_from_unused_pages():
    """With NaN/0xFF poison everywhere outside the written slots (shared pool
    with unused pages and partial last pages), outputs are finite."""
    w = W.make("ragged_b64", 1 / 64, batch=16)
    g = gpu_run(w, poison=True)
    assert np.isfinite(g["out"]).all()


def test_queries_and_keys_on_bin_edges():
    """Rows whose angles sit exactly on bin edges (pi/4 and 3pi/4 are edges at
    every b >= 2; zero tails give zero sub-vectors): ties go to the upper bin
    on both sides, and the query codes take the exact path, not the margin
    test (their sums are exact, so the margin test cannot accept them)."""
    for name, scale in (("gqa_t32k", 1 / 64), ("mixed_tiers", 1 / 32)):
        w = W.make(name, scale, batch=2)
        d = w.d
        edge = [np.r_[1.0, 1.0, np.zeros(d - 2)], np.r_[-1.0, 1.0, np.zeros(d - 2)],
                np.r_[np.zeros(d - 2), -1.0, 0.0], np.r_[1.0, 0.0, 1.0, np.zeros(d - 3)]]
        q = w.q.copy()
        for i, e in enumerate(edge):
            q[:, (5 * i) % w.hq] = e.astype(np.float32)
        keys = w.keys.copy()
        for t in range(16):
            keys[t, t % w.hkv] = (edge[t % len(edge)] * (1 + t)).astype(np.float32)
        w.keys = keys
        rng = O.calibrate(w.keys)
        g = gpu_run(w, q=q)
        o = oracle_run(w, rng, q=q)
        for k in ("kcode", "rcode", "v"):
            assert np.array_equal(g["pools"][k], o["pools"][k]), (name, k)
        compare(w, g, o, rng, q=q, label="%s edges" % name)


def test_mixed_pool_with_all_five_tiers():
    """A pool holding pages of every width {2, 3, 4, 6, 8}: the mixed-tier
    kernel's loads are the same for every width (a 3-bit page has 12-byte
    slices, read with the same 32 bytes per lane as the others)."""
    w = W.make("mixed_tiers", 1 / 16, batch=4, tiers=(2, 3, 4, 6, 8))
    assert set(np.unique(w.page_bits).tolist()) == {2, 3, 4, 6, 8}
    rng = O.calibrate(w.keys)
    g = gpu_run(w)
    o = oracle_run(w, rng)
    for k in ("kcode", "rcode", "v"):
        assert np.array_equal(g["pools"][k], o["pools"][k]), k
    assert g["errors"] == 0
    compare(w, g, o, rng, label="five tiers")


def test_more_splits_than_one_merge_round():
    """64 splits of one (sequence, KV head) group: the merging workgroup folds
    the partials in two rounds of requests; the result matches the oracle and
    the default split count."""
    w = W.make("long_t128k", 1 / 8)                 # B = 1, T = 16384: 1024 pages
    rng = O.calibrate(w.keys)
    o = oracle_run(w, rng)
    g64 = gpu_run(w, num_splits=64)
    compare(w, g64, o, rng, label="64 splits")
    g0 = gpu_run(w)
    assert np.abs(g64["out"] - g0["out"]).max() < 1e-4


def test_multi_round_batch_split_layout():
    """A batch whose (sequence, KV head) groups alone fill the CUs runs in
    rounds of workgroups: by default its splits are 384, 384, then 768 pages
    each, handed out in decreasing size through the unit table.  Ragged
    lengths up to 1773 pages, with an empty row, a one-token row and rows on
    and next to the split boundaries (384, 768 pages; the longest row crosses
    1536), match the oracle, and equal splits give the same output."""
    w = W.make("ragged_b64", 1 / 2, batch=40)                 # 40 x 8 groups, up to 28360 tokens
    lens = w.seq_lens.copy()
    order = np.argsort(-lens, kind="stable")                   # longest first
    for i, n in zip(order[1:5], [768 * 16 + 16, 768 * 16 - 1, 384 * 16 + 1, 384 * 16]):
        assert lens[i] >= n
        lens[i] = n
    lens[order[-1]], lens[order[-2]] = 0, 1
    say("[rounds] B=%d max_pages=%d lengths %s" % (w.B, w.max_pages, lens.tolist()))
    assert lens.max() > 1536 * 16
    rng = O.calibrate(w.keys)
    g = gpu_run(w, seq_lens=lens)
    o = oracle_run(w, rng, seq_lens=lens)
    assert not g["out"][order[-1]].any()
    assert g["errors"] == 0
    compare(w, g, o, rng, seq_lens=lens, label="rounds")
    g4 = gpu_run(w, seq_lens=lens, num_splits=4, want_logits=False)
    assert np.abs(g4["out"] - g["out"]).max() < 1e-4


@pytest.mark.parametrize("scale,batch", [(1 / 8, 130), (1 / 32, 512), (1 / 512, 600)])
def test_multi_round_batches_past_one_wave_of_lengths(scale, batch):
    """Multi-round batches of 130 sequences and of 512, the compaction limit
    (compacted grid, units in size order through the unit table), and of 600
    short sequences, past it (the multi-round layout without compaction).
    All match the oracle."""
    w = W.make("ragged_b64", scale, batch=batch)
    say("[rounds] B=%d max_pages=%d tokens=%d" % (w.B, w.max_pages, w.n_tokens))
    rng = O.calibrate(w.keys)
    g = gpu_run(w)
    o = oracle_run(w, rng)
    assert g["errors"] == 0
    compare(w, g, o, rng, label="rounds B=%d" % batch)


@pytest.mark.parametrize("batch,pages", [(256, 2048), (257, 2048), (512, 2048), (255, 1024)])
def test_multi_round_batches_of_one_row_repeated(batch, pages):
    """`batch` rows over the same pages with the same query rows (one
    block-table row of long_t128k at 1/4 repeated, read to `pages` pages): a
    multi-round batch of 4 units per row at 2048 pages (splits of 384, 384,
    768, 512), 3 at 1024.  1024 units at 256 rows are the most the
    unit-order kernel ranks by counting, 765 an odd count of them; 1028 and
    2048 units go through its bitonic sort, with and without padding keys.
    Every row matches the oracle's decode of the row, and all rows are equal
    bit for bit (the same computation on the same inputs, whichever
    workgroups ran it)."""
    import dataclasses
    base = W.make("long_t128k", 1 / 4)
    assert base.B == 1 and int(base.seq_lens[0]) == 2048 * W.PAGE
    lens1 = np.array([pages * W.PAGE], np.int32)
    w = dataclasses.replace(base, B=batch, block_table=np.repeat(base.block_table, batch, 0),
                            seq_lens=np.repeat(lens1, batch), q=np.repeat(base.q, batch, 0))
    rng = O.calibrate(base.keys)
    o1 = oracle_run(base, rng, want_logits=False, seq_lens=lens1)
    g = gpu_run(w, want_logits=False)
    assert g["errors"] == 0
    assert np.array_equal(g["out"], np.repeat(g["out"][:1], batch, 0)), "rows differ"
    o = {"out": np.repeat(o1["out"], batch, 0), "logits": None, "pools": o1["pools"]}
    compare(w, g, o, rng, label="%d rows of one %d-page row repeated" % (batch, pages))


@pytest.mark.parametrize("name,scale,batch", [("gqa_t32k", 1 / 16, None), ("mixed_tiers", 1 / 16, 4)])
def test_high_dynamic_range_keys(name, scale, batch):
    """Keys with four outlier channels per KV head (scales x20..x50 on top of
    the LogNormal channel scales): norms span a wide range and the logit
    bound scale*|q|*r~ grows several-fold.  With the query direction in
    binary16 the logits stay within their bar (their error is relative to the
    bound) but, scaled by the large radii through a sharp softmax, move the
    outputs by more than 2e-3; with the binary32 direction (query_precision)
    both bars hold."""
    from long_context_decode_ada_amd import ska
    w = W.make(name, scale, batch=batch, outliers=4)
    rng = O.calibrate(w.keys)
    o = oracle_run(w, rng)
    g = gpu_run(w, query_precision=ska.QDIR_F32)
    for k in ("kcode", "rcode", "v"):
        assert np.array_equal(g["pools"][k], o["pools"][k]), k
    compare(w, g, o, rng, label="%s, outlier channels, binary32 query direction" % name)
    g16 = gpu_run(w)
    oe, _ = compare(w, g16, o, rng, label="%s, outlier channels, binary16 query direction" % name, out_tol=None)
    say("   binary16 direction: output error %.3g (bar 2e-3 not required here)" % oe)


@pytest.mark.parametrize("name,scale,batch,splits", [("gqa_t32k", 1 / 32, 3, 0), ("gqa_t32k", 1 / 32, 3, 5),
                                                     ("mixed_tiers", 1 / 16, 3, 0), ("tiny", 1.0, None, 0)])
def test_partial_pages_inside_rows(name, scale, batch, splits):
    """Page headers that count fewer than 16 tokens on pages anywhere in the
    rows (the high four bits: empty slots at the page's end): the tokens in
    those slots are still stored, so a decode that read them would differ;
    single-tier pools run the tier-specialised kernel, mixed pools the
    header-dispatched one."""
    w = W.make(name, scale, batch=batch)
    r = np.random.default_rng(77)
    used = np.unique(np.concatenate([w.block_table[s, : (int(w.seq_lens[s]) + 15) // 16] for s in range(w.B)]))
    pick = r.choice(used, size=max(1, len(used) // 3), replace=False)
    w.page_bits[pick] = (w.page_bits[pick] & 15) | (r.integers(1, 16, size=len(pick)) << 4).astype(np.uint8)
    g = gpu_run(w, num_splits=splits)
    rng = O.calibrate(w.keys)
    o = oracle_run(w, rng)
    assert g["errors"] == 0
    compare(w, g, o, rng, label="%s, partial pages inside rows, splits=%d" % (name, splits))


def test_more_splits_than_the_weight_pass_holds():
    """512 splits of one (sequence, KV head): more than the merge's LDS weight
    pass holds (256), so the merge folds the partials element by element;
    against the oracle and the automatic split layout."""
    w = W.make("long_t128k", 1 / 2)                   # 4096 pages
    rng = O.calibrate(w.keys)
    o = oracle_run(w, rng, want_logits=False)
    g = gpu_run(w, num_splits=512, want_logits=False)
    compare(w, g, o, rng, label="512 splits")
    g0 = gpu_run(w, want_logits=False)
    assert np.abs(g["out"] - g0["out"]).max() < 1e-4
