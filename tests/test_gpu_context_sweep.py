"""GPU parity at the shapes of the benchmark's context sweep (gqa_t32k's
batch shape, B = 8, 32/8 heads, d = 128, b = 4, at T = 8K and 128K; section
4 of the page reports its gains over 8K / 32K / 128K contexts), in the
launch configuration the sweep times (automatic split count).  At 8K the
oracle computes every output and logit; at 128K (1M tokens) it decodes a
sample of (sequence, query head) rows, one by one, from its own encode of
those sequences."""
import numpy as np
import pytest

from long_context_decode_ada_amd import workloads as W
from oracle import oracle as O
from tests.parity_util import compare, gpu_run, oracle_run, say

pytestmark = pytest.mark.gpu


def test_sweep_t8k_b8():
    w = W.make("gqa_t32k", 0.25)                          # T = 8192
    assert w.B == 8 and int(w.seq_lens.max()) == 8192
    g = gpu_run(w)
    rng = O.calibrate(w.keys)
    o = oracle_run(w, rng)
    for k in ("kcode", "rcode", "v"):
        assert np.array_equal(g["pools"][k], o["pools"][k]), k
    compare(w, g, o, rng, label="sweep T=8K B=8")


def test_sweep_t128k_b8_sampled_rows():
    w = W.make("gqa_t32k", 4.0)                           # T = 131072, 1M tokens
    assert w.B == 8 and int(w.seq_lens.max()) == 131072
    say("[sweep 128K] %d tokens, %d pages" % (w.n_tokens, w.num_pages))
    g = gpu_run(w, want_logits=False)
    rng = O.calibrate(w.keys)
    assert np.array_equal(g["range"], rng)
    seqs = (0, 5)
    pairs = [(s, h) for s in seqs for h in (0, 13, 31)]
    pools = W.host_pools(w)
    for s in seqs:
        rows = W.token_keys(w, s)
        O.encode(pools, w.keys[rows], w.values[rows], w.slot[rows], w.radius_mode, rng)
        pages = w.block_table[s, : (int(w.seq_lens[s]) + 15) // 16].astype(np.int64)
        kb = w.hkv * 16 * W.record_bytes(w.d, 4)
        for k, per in (("kcode", kb), ("rcode", w.hkv * 16), ("v", w.hkv * w.d * 16)):
            idx = (pages[:, None] * per + np.arange(per)[None]).reshape(-1)
            assert np.array_equal(g["pools"][k][idx], pools[k][idx]), (s, k)
    o = oracle_run(w, rng, pairs=pairs, want_logits=False, pools=pools)
    compare(w, g, o, rng, pairs=pairs, label="sweep T=128K B=8, %d sampled rows" % len(pairs))
